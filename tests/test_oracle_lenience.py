"""Lossy verification in the oracle, pinned against what the pages fix.

DistillSpec (section 4, the paragraph on DistillSpec with lossy SD; Appendix
A.3, Algorithm A.1): the acceptance probability min(1, p/q) becomes
min(1, f(p, eps)/q) with a lenience function f that increases in p and
decreases in eps; eps = 1 is lossless. The three functions evaluated there
are f_lin = p/eps, f_sq = p/eps^2 and f_exp = p^eps, and f_sq at eps = 0.1
makes a drafted token a hundred times more likely to be accepted. The
residual of the final draw stays norm(max(0, p - q)) as the algorithm prints
it.

With rows that do not depend on earlier tokens, position j accepts with
probability beta_j = sum_x q_j(x) min(1, f(p_j(x))/q_j(x)) = sum_x
min(q_j(x), f(p_j(x))), so P(n = k, y) = prod_{j<k} beta_j (1 - beta_k)
res_k(y) for k < gamma and prod_{j<gamma} beta_j p_gamma(y) for k = gamma.
The brute-force enumeration below derives that from the step itself before
the oracle is held to it.
"""
import itertools

import numpy as np
import pytest
from scipy import stats

import oracle
import synth
from helpers import pack, run_oracle

P_MIN = 1e-4
KINDS = ["lin", "sq", "exp"]


def softmax64(z):
    z = np.asarray(z, np.float64)
    m = z.max(axis=-1, keepdims=True)
    e = np.exp(z - m)
    return e / e.sum(axis=-1, keepdims=True)


def f_len(kind, p, eps):
    eps = float(np.float32(eps))
    return {"none": lambda: p, "lin": lambda: p / eps, "sq": lambda: p / (eps * eps),
            "exp": lambda: np.power(p, eps)}[kind]()


def residual(p, q):
    w = np.maximum(p - q, 0.0)
    return w / w.sum()


def enumerate_law(p, q, kind, eps):
    """Exact joint law of (n, emitted tokens), from the step: every draft
    sequence x ~ q, every position's uniform integrated exactly."""
    g, V = q.shape
    law = {}
    for xs in itertools.product(range(V), repeat=g):
        w = float(np.prod([q[i][xs[i]] for i in range(g)]))
        if w == 0.0:
            continue
        reach = 1.0
        for k in range(g + 1):
            if k == g:
                for y in range(V):
                    key = (g, xs + (y,))
                    law[key] = law.get(key, 0.0) + w * reach * p[g][y]
                break
            a = min(1.0, f_len(kind, p[k][xs[k]], eps) / q[k][xs[k]])
            res = residual(p[k], q[k]) if a < 1.0 else np.zeros(V)
            for y in range(V):
                key = (k, xs[:k] + (y,))
                law[key] = law.get(key, 0.0) + w * reach * (1.0 - a) * res[y]
            reach *= a
    return law


def closed_form_joint(p, q, kind, eps):
    """[gamma + 1, V]: P(n = k, token emitted at position k = y)."""
    g, V = q.shape
    beta = np.minimum(q, f_len(kind, p[:g], eps)).sum(axis=1)
    joint = np.zeros((g + 1, V))
    reach = 1.0
    for k in range(g):
        if beta[k] < 1.0:
            joint[k] = reach * (1.0 - beta[k]) * residual(p[k], q[k])
        reach *= beta[k]
    joint[g] = reach * p[g]
    return joint, beta


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("eps", [1.0, 0.5, 0.1])
def test_enumerated_lenient_law_matches_closed_form(kind, eps):
    rng = np.random.default_rng(7)
    V, g = 3, 2
    p = softmax64(rng.standard_normal((g + 1, V)) * 1.5)
    q = softmax64(rng.standard_normal((g, V)) * 1.5)
    law = enumerate_law(p, q, kind, eps)
    assert abs(sum(law.values()) - 1.0) < 1e-12
    joint = np.zeros((g + 1, V))
    for (n, toks), pr in law.items():
        joint[n, toks[n]] += pr
    want, _ = closed_form_joint(p, q, kind, eps)
    np.testing.assert_allclose(joint, want, atol=1e-12)


def tiny(rounds=400, gen_seed=5):
    return synth.tiny_cpu(rounds=rounds, vocab=64, gamma=6, gen_seed=gen_seed)


@pytest.mark.parametrize("kind", KINDS)
def test_eps_one_is_lossless(kind):
    # f(p, 1) = p for all three functions: outcomes and thresholds identical
    x = tiny()
    base = run_oracle(x)
    res = run_oracle(x, lenience=kind, epsilon=1.0)
    np.testing.assert_array_equal(res.n, base.n)
    np.testing.assert_array_equal(res.next_token, base.next_token)
    np.testing.assert_array_equal(res.ratio, base.ratio)


@pytest.mark.parametrize("kind", KINDS)
def test_acceptance_is_monotone_in_eps(kind):
    # f decreases in eps, and the uniforms are the same at every eps: a
    # smaller eps never accepts fewer draft tokens
    x = tiny()
    prev = None
    for eps in [1.0, 0.9, 0.6, 0.3, 0.1, 0.01]:
        res = run_oracle(x, lenience=kind, epsilon=eps)
        assert (res.n >= 0).all()
        if prev is not None:
            assert (res.n >= prev).all(), eps
        prev = res.n
    # and the lenience actually bites on this workload
    assert prev.mean() > run_oracle(x).n.mean() + 0.5


def test_sq_is_at_least_as_lenient_as_lin():
    # eps^2 <= eps on (0, 1], so f_sq >= f_lin pointwise
    x = tiny()
    for eps in [0.8, 0.4, 0.05]:
        lin = run_oracle(x, lenience="lin", epsilon=eps)
        sq = run_oracle(x, lenience="sq", epsilon=eps)
        assert (sq.n >= lin.n).all()


def test_sq_eps_tenth_is_hundred_times_more_likely():
    # The pages' example: with f_sq and eps = 0.1 the acceptance threshold of
    # a drafted token is a hundred times its lossless value (eps is the
    # float32 nearest 0.1, so the factor is 100 to within 1e-7 relative).
    x = tiny(rounds=50)
    base = run_oracle(x, r=np.full((50, 6), 1e-7, np.float32), u=np.full(50, 0.5, np.float32))
    sq = run_oracle(x, lenience="sq", epsilon=0.1, r=np.full((50, 6), 1e-7, np.float32),
                    u=np.full(50, 0.5, np.float32))
    ok = np.isfinite(base.ratio) & np.isfinite(sq.ratio)
    assert ok.sum() > 100
    np.testing.assert_allclose(sq.ratio[ok] / base.ratio[ok], 100.0, rtol=2e-7)


def test_tiny_eps_accepts_every_possible_token_and_rejects_impossible_ones():
    # f_lin with eps = 1e-30: any token with p(x) > 0 has a threshold far above
    # 1 and is accepted; a token masked in the target (p = 0) keeps
    # threshold 0 and, since r > 0, is always rejected.
    V = 8
    t = np.zeros((3, V), np.float32)
    t[0, 5] = -np.inf
    t[1, 2] = -30.0
    d = np.zeros((2, V), np.float32)
    seqs = [{"target": t, "draft": d, "tokens": [2, 2], "T": 1.0},
            {"target": t, "draft": d, "tokens": [5, 1], "T": 1.0},
            {"target": t, "draft": d, "tokens": [1, 2], "T": 1.0}]
    x = pack(seqs * 20, V)
    res = run_oracle(x, lenience="lin", epsilon=1e-30)
    n = res.n.reshape(20, 3)
    assert (n[:, 0] == 2).all() and (n[:, 1] == 0).all() and (n[:, 2] == 2).all()
    # the lossless step rejects token 2 at position 1 (p = e^-30 / ...) almost surely
    assert (run_oracle(x).n.reshape(20, 3)[:, 2] == 1).all()


def test_greedy_ignores_lenience():
    x = synth.tiny_cpu(rounds=200, vocab=64, gamma=6, gen_seed=5, greedy=True)
    base = run_oracle(x)
    for kind in KINDS:
        res = run_oracle(x, lenience=kind, epsilon=0.05)
        np.testing.assert_array_equal(res.n, base.n)
        np.testing.assert_array_equal(res.next_token, base.next_token)


def dyadic_rows():
    """Target rows uniform on 4 tokens or on 1 token, draft rows uniform on
    2 or 4: p in {1/4, 1}, q in {1/2, 1/4}, so with eps = 1/2 every threshold
    f(p, eps)/q of all three functions (2p/q, 4p/q, sqrt(p)/q) and every
    residual weight is a multiple of 1/8, exact in float64."""
    V = 4
    sup_p = [[0, 1, 2, 3], [2], [0, 1, 2, 3]]
    sup_q = [[0, 1], [1, 2, 3, 0]]

    def rows(sups):
        z = np.full((len(sups), V), -np.inf, np.float32)
        for i, s in enumerate(sups):
            z[i, s] = 0.0
        return z
    return rows(sup_p), rows(sup_q)


@pytest.mark.parametrize("kind", KINDS + ["none"])
def test_oracle_dyadic_quadrature_is_exact(kind):
    # every draft sequence with q(x) > 0 times an 8-point midpoint grid for
    # each uniform: the oracle's outcome frequencies, weighted by q(x), equal
    # the enumerated law exactly
    zt, zd = dyadic_rows()
    p, q = softmax64(zt), softmax64(zd)
    V, g, M, eps = 4, 2, 8, 0.5
    law = enumerate_law(p, q, kind, eps)
    grid = (np.arange(M) + 0.5) / M
    drafts = [xs for xs in itertools.product(range(V), repeat=g)
              if np.prod([q[i][xs[i]] for i in range(g)]) > 0]
    R = np.array(list(itertools.product(grid, repeat=g + 1)))
    seqs, weights = [], []
    for xs in drafts:
        seqs += [{"target": zt, "draft": zd, "tokens": list(xs), "T": 1.0}] * len(R)
        weights.append(np.prod([q[i][xs[i]] for i in range(g)]))
    x = pack(seqs, V)
    r = np.tile(R[:, :g], (len(drafts), 1)).astype(np.float32)
    u = np.tile(R[:, g], len(drafts)).astype(np.float32)
    res = run_oracle(x, r=r, u=u, lenience=kind, epsilon=eps)
    got = {}
    for d, (xs, w) in enumerate(zip(drafts, weights)):
        for j in range(len(R)):
            b = d * len(R) + j
            n, y = int(res.n[b]), int(res.next_token[b])
            key = (n, tuple(xs[:n]) + (y,))
            got[key] = got.get(key, 0.0) + w / len(R)
    for k in set(law) | set(got):
        assert abs(law.get(k, 0.0) - got.get(k, 0.0)) < 1e-15, k


def _joint_pvalue(x, res, p, q, kind, eps):
    g, V = q.shape
    n, y = res.n.astype(np.int64), res.next_token.astype(np.int64)
    joint, _ = closed_form_joint(p, q, kind, eps)
    obs = np.bincount(n * V + y, minlength=(g + 1) * V)
    exp = joint.ravel() * len(n)
    keep = exp > 0
    if obs[~keep].sum() > 0:
        return 0.0
    return stats.chisquare(obs[keep], exp[keep] * obs[keep].sum() / exp[keep].sum()).pvalue


@pytest.fixture(scope="module")
def chi_set():
    return synth.chi_square_set(rounds=400_000)


@pytest.mark.slow
@pytest.mark.parametrize("kind,eps", [("lin", 0.5), ("sq", 0.7), ("exp", 0.3)])
def test_lenient_law_chi_square(chi_set, kind, eps):
    x = chi_set
    p, q = softmax64(x.meta["target_rows"]), softmax64(x.meta["draft_rows"])
    res = run_oracle(x, lenience=kind, epsilon=eps)
    assert _joint_pvalue(x, res, p, q, kind, eps) > P_MIN
    # the lossless law is refuted: lenience changes the output distribution
    assert _joint_pvalue(x, res, p, q, "none", 1.0) < P_MIN


@pytest.mark.slow
def test_lenient_chi_square_has_power_against_planted_mistake(chi_set):
    x = chi_set
    p, q = softmax64(x.meta["target_rows"]), softmax64(x.meta["draft_rows"])
    with oracle.mutant(oracle.MUTANT_LENIENCE_TIMES):
        res = run_oracle(x, lenience="lin", epsilon=0.5)
    assert _joint_pvalue(x, res, p, q, "lin", 0.5) < P_MIN
