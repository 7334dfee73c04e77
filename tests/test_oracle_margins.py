"""The oracle's near-tie rule, pinned on both sides of its 1e-6 window.

The parity bar lets a GPU result differ from the oracle only where a decisive
uniform lies within 1e-6 of its threshold: r_i within 1e-6 relative of the
accept threshold p_i(x_i)/q_i(x_i) (Algorithm A.1 step 7 of DistillSpec,
Appendix A.3), or u * C within 1e-6 * C of a step of the final draw's CDF
(steps 9-11, the inverse CDF in index order). These tests fix what the oracle
reports for that rule with injected uniforms whose distance to the boundary
is known exactly: 5e-7 must be flagged, 2e-6 must not; the token window of a
flagged draw holds exactly the tokens on both sides of the step; and the
outcome reported for the other side of a flagged accept decision equals the
oracle's own outcome when the uniform is moved clearly past the threshold.
The decode loop's and the cascade's first near-tie round are pinned the
same way, with tables built around the Philox uniform that decides them.

Distributions are uniform on supports of power-of-two size wherever possible,
so every probability, ratio and CDF step is exact in float64.
"""
import numpy as np
import pytest

import oracle
from helpers import pack, run_oracle

NINF = -np.inf


def uniform_row(V, support):
    z = np.full(V, NINF, np.float32)
    z[list(support)] = 0.0
    return z


def f32(v):
    return np.float32(v)


# ----------------------------------------------------------------- accept

def accept_case(r0, u0=0.6, dtype="f32"):
    # p_0 uniform on 4 tokens, q_0 uniform on {0, 1}: x_0 = 0 has ratio 0.5
    # exactly; a rejection draws from (p - q)+ = 0.25 on {2, 3}; acceptance
    # draws the bonus token from p_1, uniform on 4 tokens
    V = 4
    s = {"target": np.stack([uniform_row(V, range(4)), uniform_row(V, range(4))]),
         "draft": np.stack([uniform_row(V, [0, 1])]), "tokens": [0], "T": 1.0}
    x = pack([s], V, dtype)
    r = np.array([[r0]], np.float32)
    u = np.array([u0], np.float32)
    return x, r, u, run_oracle(x, r=r, u=u)


@pytest.mark.parametrize("rel,near", [(5e-7, True), (-5e-7, True), (2e-6, False), (-2e-6, False)])
def test_accept_margin_both_sides_of_the_window(rel, near):
    r0 = f32(0.5 * (1 + rel))
    x, r, u, res = accept_case(r0)
    want = abs(float(r0) - 0.5) / 0.5  # the fp32 uniform's exact distance
    assert abs(want - abs(rel)) < 1.3e-7  # fp32 spacing near 0.5 is 6e-8
    assert res.accept_margin[0] == want
    assert bool(res.near_tie[0]) == near
    n_expected = 0 if r0 > 0.5 else 1  # strict >: only r above the ratio rejects
    assert res.n[0] == n_expected
    if near:
        # the other side of the decision: reversed n, with its own draw
        assert res.alt_n[0] == 1 - n_expected
    else:
        assert res.alt_n[0] == -2
    # a draw far from every CDF step: one token in the window
    assert res.tok_lo[0] == res.tok_hi[0] == res.next_token[0]


@pytest.mark.parametrize("u0", [f32(0.1), f32(0.3), f32(0.6), f32(0.9)])
@pytest.mark.parametrize("side", [+1, -1])
def test_reversed_decision_is_the_outcome_past_the_threshold(u0, side):
    # the alternative outcome of a near-tie must be what the step gives when
    # r sits clearly on the other side (same u): reject <-> accept
    x, r, u, res = accept_case(f32(0.5 * (1 + side * 5e-7)), u0)
    assert res.near_tie[0] and res.alt_n[0] >= 0
    clear = f32(0.25) if side > 0 else f32(0.75)
    other = run_oracle(x, r=np.array([[clear]], np.float32), u=u)
    assert other.n[0] == res.alt_n[0]
    assert res.alt_lo[0] <= other.next_token[0] <= res.alt_hi[0]
    assert res.alt_lo[0] == res.alt_hi[0]  # u in {0.1, 0.3, ...} is far from every step


def test_accept_margin_is_the_smallest_over_decisive_positions():
    # three positions with ratio 0.5; r_0 accepts by 4e-7 (near), r_1 accepts
    # far, r_2 rejects far: the margin is position 0's, and the alternative
    # rejects at position 0
    V = 4
    s = {"target": np.stack([uniform_row(V, range(4))] * 4),
         "draft": np.stack([uniform_row(V, [0, 1])] * 3), "tokens": [0, 1, 0], "T": 1.0}
    x = pack([s], V)
    r0 = f32(0.5 * (1 - 4e-7))
    r = np.array([[r0, f32(0.2), f32(0.9)]], np.float32)
    res = run_oracle(x, r=r, u=np.array([0.6], np.float32))
    assert res.n[0] == 2
    assert res.accept_margin[0] == abs(float(r0) - 0.5) / 0.5
    assert res.alt_n[0] == 0
    # positions past the first rejection are not decisive: a near-tie there is
    # not reported
    r = np.array([[f32(0.9), f32(0.5 * (1 + 4e-7)), f32(0.2)]], np.float32)
    res = run_oracle(x, r=r, u=np.array([0.6], np.float32))
    assert res.n[0] == 0 and not res.near_tie[0] and res.alt_n[0] == -2


# ------------------------------------------------------------------- draw

def bonus_case(u0, V=4, support=range(4)):
    # gamma = 0: the token is drawn from p_0 by inverse CDF
    s = {"target": np.stack([uniform_row(V, support)]), "draft": np.zeros((0, V), np.float32),
         "tokens": [], "T": 1.0}
    x = pack([s], V)
    x.max_gamma = 0
    return run_oracle(x, r=np.zeros((1, 0), np.float32), u=np.array([u0], np.float32),
                      max_gamma=0)


@pytest.mark.parametrize("rel,near", [(5e-7, True), (-5e-7, True), (2e-6, False), (-2e-6, False)])
def test_draw_margin_both_sides_of_a_cdf_step(rel, near):
    # p uniform on 4 tokens: C = (1/4, 1/2, 3/4, 1); u * C_3 next to the step
    # C_1 = 1/2 between tokens 1 and 2
    u0 = f32(0.5 * (1 + rel))
    res = bonus_case(u0)
    want = abs(float(u0) - 0.5)  # C_3 = 1
    assert res.draw_margin[0] == want
    assert bool(res.near_tie[0]) == near
    tok = 2 if u0 > 0.5 else 1  # the smallest v with u C_3 <= C_v
    assert res.next_token[0] == tok
    if near:
        assert (res.tok_lo[0], res.tok_hi[0]) == (1, 2)
    else:
        assert res.tok_lo[0] == res.tok_hi[0] == tok
    assert res.alt_n[0] == -2


def test_draw_window_spans_a_masked_token():
    # p uniform on {0, 2, 3} (token 1 masked): the step between tokens 0 and
    # 2 has token 1's empty interval on it; the window reaches from 0 to 2
    res = bonus_case(f32(1 / 3 + 3e-7), support=[0, 2, 3])
    assert res.near_tie[0] and res.next_token[0] == 2
    assert (res.tok_lo[0], res.tok_hi[0]) == (0, 2)
    res = bonus_case(f32(1 / 3 + 3e-6), support=[0, 2, 3])
    assert not res.near_tie[0] and res.tok_lo[0] == res.tok_hi[0] == 2


def test_draw_window_at_the_top_and_bottom():
    # u = 1 draws the last token, u = 2^-24 the first; the window stays inside
    # the support at both ends
    res = bonus_case(f32(1.0))
    assert res.next_token[0] == 3 and (res.tok_lo[0], res.tok_hi[0]) == (3, 3)
    res = bonus_case(f32(2.0 ** -24))
    assert res.next_token[0] == 0 and (res.tok_lo[0], res.tok_hi[0]) == (0, 0)


@pytest.mark.parametrize("rel,near", [(5e-7, True), (2e-6, False)])
def test_residual_draw_margin(rel, near):
    # p_0 uniform on 4 tokens, q_0 one-hot on token 0; x_0 = 0 has ratio 1/4
    # and r = 0.9 rejects; the residual (p - q)+ is 1/4 on {1, 2, 3} (total
    # 3/4), whose first step (between tokens 1 and 2) is at u = 1/3
    V = 4
    s = {"target": np.stack([uniform_row(V, range(4)), uniform_row(V, range(4))]),
         "draft": np.stack([uniform_row(V, [0])]), "tokens": [0], "T": 1.0}
    x = pack([s], V)
    u0 = f32(1 / 3 + rel)
    res = run_oracle(x, r=np.array([[0.9]], np.float32), u=np.array([u0], np.float32))
    assert res.n[0] == 0 and res.next_token[0] == (2 if u0 > 1 / 3 else 1)
    assert abs(res.draw_margin[0] - abs(float(u0) * 0.75 - 0.25) / 0.75) < 1e-15
    assert bool(res.near_tie[0]) == near
    assert (res.tok_lo[0], res.tok_hi[0]) == ((1, 2) if near else (2, 2))


def test_a_residual_below_the_window_admits_every_token():
    # p = (1/2, 1/2); q from logits (0, 1e-6): the residual is about 2.5e-7 on
    # token 0 -- too little for fp32 weights to resolve, so the draw is
    # flagged and every token is admitted; n is still exact
    V = 2
    s = {"target": np.zeros((2, V), np.float32),
         "draft": np.array([[0.0, 1e-6]], np.float32), "tokens": [1], "T": 1.0}
    x = pack([s], V)
    res = run_oracle(x, r=np.array([[1.0]], np.float32), u=np.array([0.5], np.float32))
    assert res.n[0] == 0 and res.next_token[0] == 0
    assert 0 < res.resmass[0] < 1e-6
    assert res.near_tie[0] and res.draw_margin[0] == 0.0
    assert (res.tok_lo[0], res.tok_hi[0]) == (0, V - 1)


def test_greedy_and_failed_sequences_have_exact_windows():
    V = 8
    rng = np.random.default_rng(0)
    t = rng.standard_normal((3, V)).astype(np.float32)
    good = {"target": t, "draft": t[:2].copy(), "tokens": [int(np.argmax(t[0])), 0], "T": 0.0}
    bad = {"target": t, "draft": t[:2].copy(), "tokens": [0, V], "T": 1.0}  # token out of range
    x = pack([good, bad], V)
    res = run_oracle(x)
    assert res.next_token[0] >= 0 and res.tok_lo[0] == res.tok_hi[0] == res.next_token[0]
    assert np.isinf(res.accept_margin[0]) and np.isinf(res.draw_margin[0])
    assert res.n[1] == -1 and res.tok_lo[1] == res.tok_hi[1] == -1 and res.alt_n[1] == -2


def test_admits_checks_n_exactly_and_the_token_against_its_window():
    x, r, u, res = accept_case(f32(0.5 * (1 + 5e-7)), u0=f32(0.6))
    # primary outcome; the alternative; wrong n; a token outside both windows
    assert res.admits([res.n[0]], [res.next_token[0]]).all()
    assert res.admits([res.alt_n[0]], [res.alt_lo[0]]).all()
    assert not res.admits([res.n[0] + 2], [res.next_token[0]]).any()
    out = [v for v in range(4) if not (res.tok_lo[0] <= v <= res.tok_hi[0])
           and not (res.alt_lo[0] <= v <= res.alt_hi[0])]
    for v in out:
        assert not res.admits([res.n[0]], [v]).any()


# ------------------------------------------------ decode loop and cascade

def philox_u(seed, row, pos, word3, word):
    blk = oracle.philox_blocks(seed, np.array([[row & 0xffffffff, row >> 32, pos, word3]],
                                              np.uint32))
    return float(oracle.uniform24(blk[0, word])[0])


def two_token_row(q0):
    # logits (0, z) with softmax (q0, 1 - q0)
    return np.array([0.0, np.log((1 - q0) / q0)], np.float32)


def q0_of(row):
    z = row.astype(np.float64)
    e = np.exp(z - z.max())
    return e[0] / e.sum()


@pytest.mark.parametrize("offset,near", [(5e-7, True), (-5e-7, True), (2e-6, False),
                                         (-2e-6, False)])
def test_decode_first_near_round_from_the_drafting_draw(offset, near):
    # one sequence, gamma = 1, start token 0. Round 0 drafts x_0 by inverse
    # CDF with u_d = U(word 0 of Philox(seed; 0, 0, 0, 1)); the draft table's
    # row 0 puts its only CDF step at u_d + offset. Both tables are equal, so
    # the verification accepts with ratio exactly 1.
    seed = 11
    u_d = philox_u(seed, 0, 0, 1, 0)
    row = two_token_row(u_d + offset)
    assert abs(abs(q0_of(row) - u_d) - abs(offset)) < 1e-7  # the fp32 logits keep the offset
    tab = np.stack([row, row])
    res = oracle.decode_bigram(tab, tab, np.ones(1, np.float32), np.zeros(1, np.int32), gamma=1,
                               rounds=1, seed=seed)
    assert res.accepted[0, 0] == 1
    assert res.first_near[0] == (0 if near else 1)


@pytest.mark.parametrize("offset,near", [(5e-7, True), (2e-6, False)])
def test_cascade_first_near_round_from_the_inner_drafting_draw(offset, near):
    # one sequence, k1 = k2 = 1: inner round 0 drafts with u from Philox block
    # row 1 (= (0 (k1 + 1) + 1 + 0) * batch), counter word 3 = 1; the smallest
    # table's row 0 puts its CDF step there. All three tables are equal, so
    # both reviews accept with ratio exactly 1.
    seed = 5
    u_d = philox_u(seed, 1, 0, 1, 0)
    row = two_token_row(u_d + offset)
    tab = np.stack([row, row])
    res = oracle.cascade_bigram(tab, tab, tab, np.ones(1, np.float32), np.zeros(1, np.int32),
                                k1=1, k2=1, rounds=1, seed=seed)
    assert res.accepted[0, 0] == 1
    assert res.first_near[0] == (0 if near else 1)


# ------------------------------------------------- chance of a flagged row

def test_near_prob_of_a_uniform_bonus_draw():
    # p uniform on 4 tokens: each interval contributes its 2e-6 share
    res = bonus_case(f32(0.6))
    assert abs(res.near_prob[0] - 4 * 2e-6) < 1e-18
    # a residual below the window is flagged whatever u is
    V = 2
    s = {"target": np.zeros((2, V), np.float32),
         "draft": np.array([[0.0, 1e-6]], np.float32), "tokens": [1], "T": 1.0}
    res = run_oracle(pack([s], V), r=np.array([[1.0]], np.float32), u=np.array([0.5], np.float32))
    assert res.near_prob[0] >= 1.0


def test_flagged_count_follows_its_expectation():
    # the near-tie flags come from the margins, near_prob from the weights:
    # over many Philox-drawn sequences the flagged count must agree with the
    # summed probabilities (Poisson, 5 sigma), which pins both
    import synth
    x = synth.tiny_cpu(rounds=20000, gen_seed=3)
    res = oracle.verify(x.target, x.draft, x.tokens, x.gamma, x.temperature, vocab=x.vocab,
                        max_gamma=x.max_gamma, seed=0)
    expect = float(res.near_prob.sum())
    seen = int(res.near_tie.sum())
    assert expect > 20  # V = 1000: about 2e-6 * V per draw
    assert abs(seen - expect) < 5 * np.sqrt(expect) + 2, (seen, expect)
