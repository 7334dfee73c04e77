"""Hand-worked cases of the verify step with injected uniforms.

The rule (DistillSpec, Appendix A.3, Algorithm A.1, steps 5-11; the 1-indexed
form in the Leviathan et al. summary on "How speculative decoding lets a small
model draft and a large one check"): reject the first i with r_i > p_i(x_i) /
q_i(x_i), then draw from norm(max(0, p_n - q_n)), or from p_gamma if nothing
was rejected. Greedy is exact match with argmax p ("Speculative Decoding and
Distillation", Practical considerations).

The cases use distributions uniform on supports of power-of-two size, so that
every probability, ratio and CDF value is exact in float64 and the expected
outcome is known without any arithmetic error.
"""
import json
from pathlib import Path

import numpy as np
import pytest

import oracle
from helpers import pack, run_oracle, subset
import synth

NINF = -np.inf
EPS24 = 2.0 ** -24
GOLDEN = Path(__file__).parent / "golden"


def uniform_row(V, support):
    z = np.full(V, NINF, np.float32)
    z[list(support)] = 0.0
    return z


def one_step(V, p_support_rows, q_support_rows, tokens, T=1.0):
    t = np.stack([uniform_row(V, s) for s in p_support_rows])
    d = np.stack([uniform_row(V, s) for s in q_support_rows]) if q_support_rows else np.zeros((0, V))
    return {"target": t, "draft": d, "tokens": tokens, "T": T}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ratio_boundary_and_residual(dtype):
    # p_0 uniform on 4 tokens (0.25 each), q_0 uniform on {0, 1} (0.5 each):
    # x_0 = 0 has ratio exactly 0.5; residual (p - q)+ = 0.25 on {2, 3}.
    V = 4
    s = one_step(V, [range(4), range(4)], [[0, 1]], [0])
    x = pack([s] * 8, V, dtype)
    r = np.array([[0.5], [0.5 + EPS24], [0.5], [0.5 + EPS24], [EPS24], [1.0], [0.5 + EPS24],
                  [0.5 + EPS24]], np.float32)
    u = np.array([0.25, 0.5, 0.25 + EPS24, 0.5 + EPS24, 1.0, EPS24, EPS24, 1.0], np.float32)
    res = run_oracle(x, r=r, u=u)
    # equality accepts; then the bonus row (uniform on 4) is drawn by inverse CDF
    assert list(res.n) == [1, 0, 1, 0, 1, 0, 0, 0]
    assert list(res.next_token) == [0, 2, 1, 3, 3, 2, 2, 3]
    np.testing.assert_array_equal(res.ratio[:, 0], 0.5)


def test_p_at_least_q_always_accepts_and_p_zero_always_rejects():
    V = 4
    # x_0 = 2: p = 0.25, q = 0 -> ratio inf; x_1 = 1: p = q = 0.5 -> ratio 1;
    # x_2 = 3: p = 0 -> ratio 0, rejected even by the smallest uniform.
    s = one_step(V, [range(4), [0, 1], [0, 1], range(4)], [[0, 1], [0, 1], [3]], [2, 1, 3])
    x = pack([s], V)
    res = run_oracle(x, r=np.array([[1.0, 1.0, EPS24]], np.float32), u=np.array([1.0], np.float32))
    assert res.n[0] == 2
    assert res.ratio[0, 0] == np.inf and res.ratio[0, 1] == 1.0 and res.ratio[0, 2] == 0.0
    # residual at position 2: (p - q)+ = p = uniform on {0, 1}; u = 1 -> token 1
    assert res.next_token[0] == 1


def test_disco_figure1_trace():
    g = json.loads((GOLDEN / "disco_fig1_trace.json").read_text())
    SL = g["speculation_lookahead"]
    V = 4
    s = one_step(V, [range(4)] * (SL + 1), [[0, 1]] * SL, [0] * SL)  # every ratio is 0.5
    x = pack([s], V)
    r = np.array([[0.25, 0.5, 0.125, 0.75, 0.0625]], np.float32)  # t1..t3 pass, t4 fails
    res = run_oracle(x, r=r, u=np.array([0.5], np.float32))
    assert res.n[0] == g["accepted"]
    assert res.n[0] + 1 == g["tokens_emitted"]
    assert res.next_token[0] in (2, 3)  # the corrected token comes from the residual


def test_bonus_draw_from_last_target_row():
    V = 4
    # all drafts accepted (p = 1, q = 0.5: ratio 2); the bonus row is uniform on {1, 3}
    s = one_step(V, [[0], [0], [1, 3]], [[0, 1], [0, 1]], [0, 0])
    x = pack([s, s], V)
    res = run_oracle(x, r=np.ones((2, 2), np.float32), u=np.array([0.5, 0.5 + EPS24], np.float32))
    assert list(res.n) == [2, 2]
    assert list(res.next_token) == [1, 3]


def test_gamma_zero_draws_from_first_row():
    V = 4
    s = {"target": uniform_row(V, [2])[None, :], "draft": np.zeros((0, V)), "tokens": [], "T": 1.0}
    x = pack([s], V)
    res = run_oracle(x)
    assert res.n[0] == 0 and res.next_token[0] == 2


def test_greedy_exact_match_ties_and_no_rng():
    V = 5
    t = np.array([[1, 4, 4, 0, 2],      # argmax 1 (tie with 2: lowest index)
                  [0, 0, 0, 3, 3],      # argmax 3
                  [9, 1, 1, 1, 1],      # argmax 0
                  [0, 0, 0, 0, 7]], np.float32)
    d = np.full((3, V), np.nan, np.float32)  # greedy never reads draft rows
    seqs = [{"target": t, "draft": d, "tokens": [1, 3, 1], "T": 0.0},   # mismatch at i=2 -> emit 0
            {"target": t, "draft": d, "tokens": [1, 3, 0], "T": 0.0},   # all accepted -> emit 4
            {"target": t, "draft": d, "tokens": [2, 3, 0], "T": 0.0}]   # tie not matched -> n = 0
    x = pack(seqs, V)
    a = run_oracle(x, seed=1)
    b = run_oracle(x, seed=99, row_offset=12345)
    assert list(a.n) == [2, 3, 0] and list(a.next_token) == [0, 4, 1]
    np.testing.assert_array_equal(a.n, b.n)
    np.testing.assert_array_equal(a.next_token, b.next_token)


def test_data_errors_give_sentinels():
    V = 4
    good = one_step(V, [range(4), range(4)], [[0, 1]], [0])
    nan_t = dict(good, target=good["target"].copy())
    nan_t["target"][1, 2] = np.nan
    inf_d = dict(good, draft=good["draft"].copy())
    inf_d["draft"][0, 3] = np.inf
    masked = dict(good, target=good["target"].copy())
    masked["target"][0, :] = NINF
    bad_tok = dict(good, tokens=[4])
    neg_tok = dict(good, tokens=[-1])
    seqs = [good, nan_t, inf_d, masked, bad_tok, neg_tok,
            dict(good, T=-1.0), dict(good, T=np.nan), dict(good, T=np.inf),
            dict(inf_d, T=0.0)]  # greedy does not read the draft row: valid
    res = run_oracle(pack(seqs, V))
    assert res.layout_ok
    assert list(res.n[1:9]) == [-1] * 8 and list(res.next_token[1:9]) == [-1] * 8
    assert res.n[0] >= 0 and res.n[9] >= 0


def test_temperature_domain():
    # sampling needs log2(e)/T finite in fp32: T = 1e-38 (scale 1.44e38) and
    # T = 3e38 are valid, T = 1e-39 (scale 1.44e39 > FLT_MAX) and the
    # smallest subnormal are not; T = 0 stays greedy
    V = 4
    good = one_step(V, [range(4), range(4)], [[0, 1]], [0])
    Ts = [1e-38, 3e38, 1e-39, float(np.float32(1.4e-45)), 0.0]
    res = run_oracle(pack([dict(good, T=T) for T in Ts], V))
    assert list(res.n >= 0) == [True, True, False, False, True]


def test_tiny_temperature_reaches_the_greedy_limit():
    # As T -> 0 each softmax becomes one-hot at its row's maximum, so with
    # unique maxima the sampling step at T = 1e-30 (a valid temperature)
    # gives the greedy outcome for drafts drawn at that T (the draft rows'
    # argmax): accept while x_i == argmax p_i, then emit argmax p_n, since
    # the residual max(0, p_n - q_n) is one-hot there too.
    rng = np.random.default_rng(3)
    V, g, B = 50, 4, 40
    seqs = []
    for _ in range(B):
        t = rng.permutation(V * (g + 1)).reshape(g + 1, V).astype(np.float32)  # unique values
        d = t[:g].copy()
        flip = rng.random(g) < 0.4  # some drafts disagree with the target's argmax
        for i in np.flatnonzero(flip):
            d[i] = rng.permutation(V).astype(np.float32)
        tokens = [int(np.argmax(d[i])) for i in range(g)]
        seqs.append({"target": t, "draft": d, "tokens": tokens, "T": 1e-30})
    x = pack(seqs, V)
    hot = run_oracle(x, seed=5)
    greedy = run_oracle(pack([dict(s_, T=0.0) for s_ in seqs], V), seed=5)
    np.testing.assert_array_equal(hot.n, greedy.n)
    np.testing.assert_array_equal(hot.next_token, greedy.next_token)
    assert (hot.n < g).any() and (hot.n == g).any()


def test_layout_errors_poison_every_sequence():
    V = 4
    good = one_step(V, [range(4), range(4)], [[0, 1]], [0])
    x = pack([good, good], V)
    res = run_oracle(x, max_gamma=0)  # gamma 1 > max_gamma 0
    assert not res.layout_ok and list(res.n) == [-1, -1] and list(res.next_token) == [-1, -1]
    x.gamma[1] = 0  # totals no longer match the row counts
    res = run_oracle(x)
    assert not res.layout_ok and list(res.n) == [-1, -1]


def test_batch_invariance_ragged():
    # A sequence's result depends only on its own rows and its Philox row
    # (row_offset + b): the packed ragged batch equals single-sequence calls.
    x = synth.ragged_b256(batch=12, vocab=257, max_gamma=6)
    x.row_offset = 1000
    full = run_oracle(x)
    for b in range(x.batch):
        one = run_oracle(subset(x, [b]), row_offset=1000 + b)
        assert (one.n[0], one.next_token[0]) == (full.n[b], full.next_token[b])


def test_bounds_and_shared_temperature_scaling():
    x = synth.tiny_cpu(rounds=3000, vocab=257)
    res = run_oracle(x)
    assert ((res.n >= 0) & (res.n <= x.gamma)).all()
    assert ((res.next_token >= 0) & (res.next_token < x.vocab)).all()
    # softmax(z/T) depends on z/T only: doubling both logits and T keeps the
    # outcome up to the near-tie rule (float64 rounding of the scaled rows)
    y = synth.Inputs(x.name, x.vocab, x.max_gamma, x.dtype, x.target * 2, x.draft * 2, x.tokens,
                     x.gamma, x.temperature * 2)
    res2 = run_oracle(y)
    assert res.admits(res2.n, res2.next_token).all()
    keep = ~(res.near_tie | res2.near_tie)
    np.testing.assert_array_equal(res.n[keep], res2.n[keep])
    np.testing.assert_array_equal(res.next_token[keep], res2.next_token[keep])


def test_identical_rows_accept_everything_and_disjoint_reject_first():
    rng = np.random.default_rng(5)
    V, g = 16, 3
    t = rng.standard_normal((g + 1, V)).astype(np.float32)
    same = {"target": t, "draft": t[:g], "tokens": [int(v) for v in rng.integers(0, V, g)], "T": 1.0}
    # disjoint supports: the draft puts all mass on tokens the target masks
    tt = t.copy()
    tt[:, :8] = NINF
    dd = t[:g].copy()
    dd[:, 8:] = NINF
    disj = {"target": tt, "draft": dd, "tokens": [0, 1, 2], "T": 1.0}
    x = pack([same] * 200 + [disj] * 200, V)
    x.row_offset = 77
    res = run_oracle(x)
    assert (res.n[:200] == g).all()
    assert (res.n[200:] == 0).all()
    assert (res.next_token[200:] >= 8).all()  # residual = p on the target support
