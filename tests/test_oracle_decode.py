"""Multi-round decoding with bigram "models", pinned against what the pages fix.

- Sequence-level identity: speculative decoding generates the same
  distribution over sequences as sampling from the target alone (DistillSpec
  section 3; the Leviathan et al. summary; "Speculative Decoding and
  Distillation", Part 1). With bigram models the target's law of a sequence
  is the Markov chain prod_t p(y_t | y_{t-1}), so the joint of the first
  three generated tokens is a closed form to test against (chi-square).
- Tokens per round: E[n + 1] = sum_{k=0}^{gamma} P(the first k drafts are
  accepted) (DistillSpec section 3, block efficiency). With context-dependent
  rows this is a forward recursion over the previous token:
  f_0 = delta_c, f_{i+1}(x) = sum_s f_i(s) min(p(x | s), q(x | s)).
- Greedy decoding emits the target's greedy chain, whatever the draft.
"""
import numpy as np
import pytest
import torch
from scipy import stats

import oracle

P_MIN = 1e-4


def softmax64(z, T=1.0):
    return torch.softmax(torch.from_numpy(np.asarray(z, np.float64)) / float(np.float32(T)),
                         dim=-1).numpy()


def tables(V=5, seed=0, sigma=0.7):
    rng = np.random.default_rng(seed)
    t = (rng.standard_normal((V, V)) * 1.5).astype(np.float32)
    d = (t + rng.standard_normal((V, V)) * sigma).astype(np.float32)
    return t, d


def expected_tokens(P, Q, c, gamma):
    f = np.zeros(P.shape[0])
    f[c] = 1.0
    total = 1.0
    M = np.minimum(P, Q)  # M[s, x] = min(p(x | s), q(x | s))
    for _ in range(gamma):
        f = f @ M
        total += f.sum()
    return total


@pytest.fixture(scope="module")
def run():
    t, d = tables()
    B, g, R, c = 300_000, 3, 3, 2
    res = oracle.decode_bigram(t, d, np.full(B, 1.0, np.float32), np.full(B, c, np.int32),
                               gamma=g, rounds=R, seed=5)
    return t, d, res, c, g, R


def joint3_pvalue(t, res, c, T=1.0):
    P = softmax64(t, T)
    V = P.shape[0]
    y = res.tokens[:, :3].astype(np.int64)
    obs = np.bincount((y[:, 0] * V + y[:, 1]) * V + y[:, 2], minlength=V ** 3)
    # the chain p(y1 | c) p(y2 | y1) p(y3 | y2)
    exp = np.einsum("a,ab,bc->abc", P[c], P, P).reshape(-1) * len(y)
    return stats.chisquare(obs, exp).pvalue


def test_sequence_law_is_the_target_chain(run):
    t, d, res, c, g, R = run
    assert (res.length >= R).all() and (res.length <= R * (g + 1)).all()
    assert ((res.accepted >= 0) & (res.accepted <= g)).all()
    np.testing.assert_array_equal(res.length, (res.accepted + 1).sum(axis=1))
    assert joint3_pvalue(t, res, c) > P_MIN


def test_tokens_per_round_matches_the_recursion(run):
    t, d, res, c, g, R = run
    P, Q = softmax64(t), softmax64(d)
    # start state of every round: the start token, then the last token so far
    B = res.tokens.shape[0]
    ends = np.cumsum(res.accepted + 1, axis=1)
    starts = np.empty((B, R), np.int64)
    starts[:, 0] = c
    for r in range(1, R):
        starts[:, r] = res.tokens[np.arange(B), ends[:, r - 1] - 1]
    E = np.array([expected_tokens(P, Q, s, g) for s in range(P.shape[0])])
    want = E[starts].mean()
    got = (res.accepted + 1.0)
    assert abs(got.mean() - want) < 4.5 * got.std() / np.sqrt(got.size), (got.mean(), want)
    # and a draft from the target itself would accept everything
    assert abs(expected_tokens(P, P, c, g) - (g + 1)) < 1e-12


@pytest.mark.parametrize("which", [oracle.MUTANT_RESIDUAL_IS_P, oracle.MUTANT_N_PLUS_ONE])
def test_sequence_law_has_power_against_planted_mistakes(which):
    t, d = tables()
    B, c = 300_000, 2
    with oracle.mutant(which):
        res = oracle.decode_bigram(t, d, np.full(B, 1.0, np.float32), np.full(B, c, np.int32),
                                   gamma=3, rounds=3, seed=5)
    assert joint3_pvalue(t, res, c) < P_MIN


def test_tokens_per_round_detects_a_wrong_draft():
    # drafting from the wrong table changes the acceptance rate: the recursion
    # with the table actually used must match, the other must not
    t, d = tables(seed=3, sigma=1.5)
    B, g, R, c = 100_000, 4, 2, 1
    res = oracle.decode_bigram(t, d, np.ones(B, np.float32), np.full(B, c, np.int32), gamma=g,
                               rounds=1, seed=9)
    P, Q = softmax64(t), softmax64(d)
    got = res.accepted[:, 0] + 1.0
    se = got.std() / np.sqrt(B)
    assert abs(got.mean() - expected_tokens(P, Q, c, g)) < 4.5 * se
    assert abs(got.mean() - expected_tokens(P, softmax64(t * 0.5), c, g)) > 10 * se


def test_temperature_and_bf16_tables():
    t, d = tables(V=6, seed=4)
    bits = lambda a: (a.view(np.uint32) >> 16).astype(np.uint16)  # truncation: exact bf16 values
    tb, db = bits(t), bits(d)
    tf = (tb.astype(np.uint32) << 16).view(np.float32)
    B, c, T = 300_000, 0, 0.6
    res = oracle.decode_bigram(tb, db, np.full(B, T, np.float32), np.full(B, c, np.int32),
                               gamma=2, rounds=3, seed=2)
    assert joint3_pvalue(tf, res, c, T) > P_MIN


def test_greedy_decoding_is_the_target_greedy_chain():
    t, d = tables(V=64, seed=6, sigma=2.0)
    B, g, R = 64, 4, 6
    start = np.arange(B, dtype=np.int32) % 64
    res = oracle.decode_bigram(t, d, np.zeros(B, np.float32), start, gamma=g, rounds=R)
    for b in range(B):
        y, prev = [], int(start[b])
        for _ in range(res.length[b]):
            prev = int(np.argmax(t[prev]))
            y.append(prev)
        np.testing.assert_array_equal(res.tokens[b, :res.length[b]], y)
    assert (res.first_near == R).all()


def test_bad_start_token_fails_only_its_sequence():
    t, d = tables(V=8)
    res = oracle.decode_bigram(t, d, np.ones(3, np.float32), np.array([1, 8, -1], np.int32),
                               gamma=2, rounds=2)
    assert res.length[0] >= 2 and res.length[1] == -1 and res.length[2] == -1
    assert (res.accepted[1:] == -1).all()
