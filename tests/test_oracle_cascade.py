"""CS Drafting's vertical cascade in the oracle, pinned against what the pages
fix ("Cascade Speculative Drafting for Even Faster LLM Inference", sections
3.1 and 3.4: lenience may speed up the intermediate reviews, and withholding
it at the target review keeps the target's output distribution).

With bigram tables the target's law of a sequence is the Markov chain
prod_t p(y_t | y_{t-1}); the joint of the first three generated tokens is
tested against it (chi-square) with a lenient intermediate review. The
target review must use, at each position, the law the draft token was drawn
from; a planted mistake that uses the intermediate model's own distribution
instead must fail as soon as the intermediate review is lenient.
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


def tables(V=5, seed=0):
    rng = np.random.default_rng(seed)
    t = (rng.standard_normal((V, V)) * 1.5).astype(np.float32)
    m = (t + rng.standard_normal((V, V)) * 0.6).astype(np.float32)
    s = (t + rng.standard_normal((V, V)) * 1.4).astype(np.float32)
    return t, m, s


def joint3_pvalue(t, res, c, T=1.0):
    P = softmax64(t, T)
    V = P.shape[0]
    y = res.tokens[:, :3].astype(np.int64)
    obs = np.bincount((y[:, 0] * V + y[:, 1]) * V + y[:, 2], minlength=V ** 3)
    exp = np.einsum("a,ab,bc->abc", P[c], P, P).reshape(-1) * len(y)
    return stats.chisquare(obs, exp).pvalue


def run(kind, eps, mutant=False, B=300_000, c=2, seed=4, T=1.0, k1=3, k2=2):
    t, m, s = tables()
    res = oracle.cascade_bigram(t, m, s, np.full(B, T, np.float32), np.full(B, c, np.int32),
                                k1=k1, k2=k2, rounds=3, lenience=kind, epsilon=eps, seed=seed,
                                mutant_q_is_p1=mutant)
    return t, res, c


@pytest.mark.parametrize("kind,eps", [("none", 1.0), ("sq", 0.5), ("exp", 0.3), ("lin", 0.2)])
def test_target_law_survives_a_lenient_intermediate_review(kind, eps):
    t, res, c = run(kind, eps)
    assert (res.length >= 3).all() and (res.length <= 3 * 4).all()
    assert ((res.accepted >= 0) & (res.accepted <= 3)).all()
    np.testing.assert_array_equal(res.length, (res.accepted + 1).sum(axis=1))
    assert joint3_pvalue(t, res, c) > P_MIN


def test_target_law_with_more_inner_drafts_than_the_target_reviews():
    # k2 > k1: one inner round already drafts past the k1 tokens the target
    # reviews; the excess is dropped and the law still holds
    t, res, c = run("sq", 0.5, k1=1, k2=3, seed=6)
    assert (res.length >= 3).all() and (res.length <= 3 * 2).all()
    assert ((res.accepted >= 0) & (res.accepted <= 1)).all()
    assert joint3_pvalue(t, res, c) > P_MIN


def test_reviewing_against_the_intermediate_model_is_wrong_when_lenient():
    t, res, c = run("sq", 0.5, mutant=True)
    assert joint3_pvalue(t, res, c) < P_MIN


def test_lenience_raises_the_acceptance_of_the_cascade_draft():
    # a lenient intermediate review lets more of the small model's tokens
    # through; the target then accepts fewer of the cascade's draft tokens
    # (its law drifts away from the intermediate model), but still in range
    _, lossless, _ = run("none", 1.0, B=50_000)
    _, lenient, _ = run("lin", 0.05, B=50_000)
    assert lenient.accepted.mean() < lossless.accepted.mean()


def test_greedy_cascade_is_the_target_greedy_chain():
    t, m, s = tables(V=32, seed=7)
    B = 32
    start = np.arange(B, dtype=np.int32)
    res = oracle.cascade_bigram(t, m, s, np.zeros(B, np.float32), start, k1=4, k2=2, rounds=4,
                                lenience="sq", epsilon=0.5)
    for b in range(B):
        y, prev = [], int(start[b])
        for _ in range(res.length[b]):
            prev = int(np.argmax(t[prev]))
            y.append(prev)
        np.testing.assert_array_equal(res.tokens[b, :res.length[b]], y)


def test_bf16_tables_and_temperature():
    t, m, s = tables(V=6, seed=9)
    bits = lambda a: (a.view(np.uint32) >> 16).astype(np.uint16)
    tb, mb, sb = bits(t), bits(m), bits(s)
    tf = (tb.astype(np.uint32) << 16).view(np.float32)
    B, c, T = 300_000, 1, 0.7
    res = oracle.cascade_bigram(tb, mb, sb, np.full(B, T, np.float32), np.full(B, c, np.int32),
                                k1=3, k2=3, rounds=3, lenience="exp", epsilon=0.5, seed=3)
    assert joint3_pvalue(tf, res, c, T) > P_MIN


def test_bad_start_token_fails_only_its_sequence():
    t, m, s = tables(V=8)
    res = oracle.cascade_bigram(t, m, s, np.ones(3, np.float32), np.array([1, 8, -1], np.int32),
                                k1=3, k2=2, rounds=2)
    assert res.length[0] >= 2 and res.length[1] == -1 and res.length[2] == -1
