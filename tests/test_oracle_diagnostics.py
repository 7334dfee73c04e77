"""Per-position diagnostics in the oracle, pinned against the mathematics.

- alpha = sum_v min(p_v, q_v) is the probability that a token drafted from q
  is accepted (DistillSpec section 3) and equals 1 - TV(p, q) with
  TV = (1/2) sum |p - q| (DistillSpec section 4 uses TV as the acceptance
  proxy); the verify step's empirical acceptance rate must match it.
- Ent(q) and Top_k(q) are the features of DISCO's stopping classifier (DISCO
  section 3, Eq. 2); checked against scipy's entropy, closed forms and
  numpy's sort.
"""
import numpy as np
import pytest
import torch
from scipy import stats

import oracle
import synth
from helpers import pack, run_oracle


def softmax64(z, T=1.0):
    return torch.softmax(torch.from_numpy(np.asarray(z, np.float64)) / float(np.float32(T)),
                         dim=-1).numpy()


def diag(x, k):
    return oracle.position_diagnostics(x.target, x.draft, x.gamma, x.temperature, vocab=x.vocab,
                                       top_k=k)


def rows_of(x):
    """(target row, draft row) float64 logits of every draft position."""
    toff, doff = x.offsets()
    dec = (lambda a: oracle.decode_bf16(a)) if x.dtype == "bf16" else \
        (lambda a: a.astype(np.float64))
    out = []
    for b in range(x.batch):
        for i in range(int(x.gamma[b])):
            out.append((dec(x.target[toff[b] + i]), dec(x.draft[doff[b] + i]),
                        float(x.temperature[b])))
    return out


@pytest.mark.parametrize("name,kw", [("tiny_cpu", dict(rounds=30, vocab=200)),
                                     ("t5xxl_like", dict(rounds=3)),
                                     ("ragged_b256", dict(batch=3))])
def test_alpha_entropy_topk_against_library_routines(name, kw):
    x = synth.by_name(name, **kw)
    k = 8
    d = diag(x, k)
    for j, (zt, zd, T) in enumerate(rows_of(x)):
        p, q = softmax64(zt, T), softmax64(zd, T)
        # alpha = 1 - TV
        assert abs(d.alpha[j] - (1.0 - 0.5 * np.abs(p - q).sum())) < 1e-12
        assert abs(d.entropy[j] - stats.entropy(q)) < 1e-10
        order = np.lexsort((np.arange(len(zd)), -zd))[:k]  # logit desc, index asc
        np.testing.assert_array_equal(d.topk_index[j], order)
        # two float64 sums over V terms in different orders: |error| <= V * 2^-53
        np.testing.assert_allclose(d.topk_prob[j], q[order], rtol=len(zd) * 2.0 ** -53, atol=0)


def test_alpha_is_the_verify_steps_acceptance_rate():
    # fixed rows, fresh drafts per round: position 0 accepts with probability
    # alpha_0, and position k given reached with alpha_k
    x = synth.chi_square_set(rounds=200_000)
    g = x.max_gamma
    one = pack([{"target": x.meta["target_rows"], "draft": x.meta["draft_rows"],
                 "tokens": [0] * g, "T": 1.0}], x.vocab)
    d = diag(one, 0)
    res = run_oracle(x)
    for k in range(g):
        reach = res.n >= k
        acc = (res.n[reach] > k).sum()
        a = d.alpha[k]
        z = (acc - a * reach.sum()) / np.sqrt(reach.sum() * a * (1 - a))
        assert abs(z) < 4.5, (k, z, a)


def test_special_cases():
    V = 8
    # logits on a 1/64 grid, so that adding 5 is exact in float32
    z = (np.round(np.random.default_rng(3).standard_normal((3, V)) * 64) / 64).astype(np.float32)
    disjoint_t = np.full((2, V), -np.inf, np.float32)
    disjoint_t[:, :4] = 0.0
    disjoint_d = np.full((1, V), -np.inf, np.float32)
    disjoint_d[0, 4:] = 1.5
    uni = np.zeros((1, V), np.float32)
    uni[0, 5:] = -np.inf  # uniform on 5 tokens
    seqs = [
        {"target": z, "draft": z[:2], "tokens": [0, 0], "T": 0.7},           # q == p
        {"target": disjoint_t, "draft": disjoint_d, "tokens": [4], "T": 1.0},  # disjoint
        {"target": z[:2], "draft": uni, "tokens": [0], "T": 2.0},              # uniform q
        {"target": z[:2], "draft": z[:1] + 5.0, "tokens": [0], "T": 0.7},      # shifted q
    ]
    x = pack(seqs, V)
    d = diag(x, 6)
    assert abs(d.alpha[0] - 1.0) < 1e-15 and abs(d.alpha[1] - 1.0) < 1e-15
    assert d.alpha[2] == 0.0
    np.testing.assert_allclose(d.entropy[2], np.log(4.0), rtol=1e-15)  # q uniform on 4
    np.testing.assert_allclose(d.entropy[3], np.log(5.0), rtol=1e-15)
    # masked tail: tokens 5..7 of q have probability 0, ranked by index
    np.testing.assert_array_equal(d.topk_index[3], [0, 1, 2, 3, 4, 5])
    np.testing.assert_array_equal(d.topk_prob[3][5:], [0.0])
    np.testing.assert_allclose(d.topk_prob[3][:5], 0.2, rtol=1e-15)
    # a shift of every draft logit changes nothing (position 0 of sequence 0
    # against sequence 3's shifted copy of the same draft row)
    assert abs(d.entropy[4] - d.entropy[0]) < 1e-13
    np.testing.assert_array_equal(d.topk_index[4], d.topk_index[0])


def test_two_token_closed_form():
    # q = (s, 1 - s) with s the logistic of the logit gap: H = -s ln s - (1-s) ln(1-s)
    gaps = np.array([0.0, 0.3, 2.0, -5.0, 12.0], np.float32)
    seqs = []
    for g in gaps:
        t = np.zeros((2, 2), np.float32)
        dr = np.array([[g, 0.0]], np.float32)
        seqs.append({"target": t, "draft": dr, "tokens": [0], "T": 1.0})
    d = diag(pack(seqs, 2), 2)
    s = 1.0 / (1.0 + np.exp(-gaps.astype(np.float64)))
    want = -(s * np.log(s) + (1 - s) * np.log1p(-s))
    np.testing.assert_allclose(d.entropy, want, rtol=1e-12, atol=1e-15)
    # target uniform (0.5, 0.5): alpha = 0.5 + min(s, 1 - s)... = 1 - |s - 0.5|
    np.testing.assert_allclose(d.alpha, 1.0 - np.abs(s - 0.5), rtol=1e-13)
    # equal logits rank the lower index first
    assert list(d.topk_index[0]) == [0, 1]


def test_greedy_limits_and_invalid_rows():
    V = 16
    rng = np.random.default_rng(4)
    t = rng.standard_normal((3, V)).astype(np.float32)
    dr = rng.standard_normal((2, V)).astype(np.float32)
    dr[0, int(np.argmax(t[0]))] = 10.0  # agrees with the target argmax at position 0
    bad = t.copy()
    bad[1, 3] = np.nan
    seqs = [{"target": t, "draft": dr, "tokens": [0, 0], "T": 0.0},
            {"target": bad, "draft": dr, "tokens": [0, 0], "T": 1.0}]
    x = pack(seqs, V)
    d = diag(x, 3)
    assert d.alpha[0] == 1.0 and d.alpha[1] == float(np.argmax(t[1]) == np.argmax(dr[1]))
    assert d.entropy[0] == 0.0 and d.entropy[1] == 0.0
    np.testing.assert_array_equal(d.topk_prob[0], [1.0, 0.0, 0.0])
    np.testing.assert_array_equal(d.topk_index[0], np.lexsort((np.arange(V), -dr[0]))[:3])
    # sequence 1: position 0 usable, position 1 has a NaN target logit
    assert np.isfinite(d.alpha[2]) and np.isnan(d.alpha[3]) and np.isnan(d.entropy[3])
    assert (d.topk_index[3] == -1).all() and np.isnan(d.topk_prob[3]).all()
