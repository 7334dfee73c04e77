"""The oracle's output law, pinned against what the pages fix.

- Identity of the output distribution with the target's: DistillSpec section
  3 (speculative sampling keeps the target distribution), the Leviathan et al.
  summary (identical output distribution for any draft), and "Speculative
  Decoding and Distillation", Part 1 ("Why it's exact").
- Token acceptance rate beta = E_{x~q} min(1, p/q) = sum min(p, q) = 1 - TV:
  DistillSpec section 3 (Eq. 1 context) and section 4 (TVD as proxy).
- Expected tokens per round (1 - alpha^(g+1)) / (1 - alpha) under i.i.d.
  acceptance: DistillSpec section 3 (block efficiency), DISCO Eq. 1, and the
  worked example alpha = 0.8, k = 4 in the study notes ("Speedup math").
- Law of the accepted count alpha^i - alpha^(i+1), and alpha^k for all
  accepted: Cascade Speculative Drafting summary, Appendix C.1.
- Bounds: at least one and at most gamma + 1 tokens per round (Leviathan et
  al. summary).

Rows in these tests do not depend on earlier tokens, so with position-
dependent acceptance rates alpha_j = sum_v min(p_j(v), q_j(v)) the law is
P(n = k, y) = prod_{j<k} alpha_j * (1 - alpha_k) * res_k(y) for k < gamma and
prod_{j<gamma} alpha_j * p_gamma(y) for k = gamma; the brute-force enumeration
below confirms this from the step's definition before the oracle is
compared with it.
"""
import itertools
import json
from pathlib import Path

import numpy as np
import pytest
import torch
from scipy import stats

import oracle
import synth
from helpers import pack, run_oracle

GOLDEN = Path(__file__).parent / "golden"
P_MIN = 1e-4  # chi-square acceptance threshold (fixed seeds: deterministic)


def softmax64(z, T=1.0):
    return torch.softmax(torch.from_numpy(np.asarray(z, np.float64)) / float(np.float32(T)),
                         dim=-1).numpy()


def residual(p, q):
    w = np.maximum(p - q, 0.0)
    return w / w.sum()


def enumerate_law(p, q):
    """Exact joint law of (n, emitted tokens) from the step's definition:
    enumerate every draft sequence x ~ q and integrate the uniforms exactly.
    Returns {(n, tokens_tuple): prob}."""
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
            a = min(1.0, p[k][xs[k]] / q[k][xs[k]])
            res = residual(p[k], q[k]) if a < 1.0 else np.zeros(V)
            for y in range(V):
                key = (k, xs[:k] + (y,))
                law[key] = law.get(key, 0.0) + w * reach * (1.0 - a) * res[y]
            reach *= a
    return law


def closed_form_nk(p, q):
    """P(n = k) for k = 0..gamma with alpha_j = sum min(p_j, q_j)."""
    g = q.shape[0]
    alpha = np.minimum(p[:g], q).sum(axis=1)
    out = np.empty(g + 1)
    reach = 1.0
    for k in range(g):
        out[k] = reach * (1.0 - alpha[k])
        reach *= alpha[k]
    out[g] = reach
    return out, alpha


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_enumerated_law_matches_pages(seed):
    rng = np.random.default_rng(seed)
    V, g = 3, 2
    p = softmax64(rng.standard_normal((g + 1, V)) * 1.5)
    q = softmax64(rng.standard_normal((g, V)) * 1.5)
    law = enumerate_law(p, q)
    assert abs(sum(law.values()) - 1.0) < 1e-12
    # token at position k, given the round reached position k, is ~ p_k
    for k in range(g + 1):
        mass = np.zeros(V)
        for (n, toks), pr in law.items():
            if n >= k:
                mass[toks[k]] += pr
        np.testing.assert_allclose(mass / mass.sum(), p[k], rtol=0, atol=1e-12)
    # P(n = k) = prod alpha_j (1 - alpha_k); alpha = 1 - TV(p, q)
    pn = np.zeros(g + 1)
    for (n, _), pr in law.items():
        pn[n] += pr
    want, alpha = closed_form_nk(p, q)
    np.testing.assert_allclose(pn, want, atol=1e-12)
    np.testing.assert_allclose(alpha, 1.0 - 0.5 * np.abs(p[:g] - q).sum(axis=1), atol=1e-12)


def dyadic_rows():
    """Rows uniform on supports of size 1, 2 or 4: every probability, ratio and
    normalised residual weight is a multiple of 1/8, exact in float64."""
    V = 4
    sup_p = [[0, 1, 2, 3], [0, 2], [1, 3]]
    sup_q = [[0, 1], [1, 2, 3, 0]]
    def rows(sups):
        z = np.full((len(sups), V), -np.inf, np.float32)
        for i, s in enumerate(sups):
            z[i, s] = 0.0
        return z
    return rows(sup_p), rows(sup_q)


def test_oracle_dyadic_quadrature_is_exact():
    # Every draft sequence x with q(x) > 0, times an 8-point midpoint grid for
    # each uniform (r_0, r_1, u): the oracle's outcome frequencies, weighted by
    # q(x), must equal the enumerated law exactly.
    zt, zd = dyadic_rows()
    p, q = softmax64(zt), softmax64(zd)
    V, g, M = 4, 2, 8
    law = enumerate_law(p, q)
    grid = (np.arange(M) + 0.5) / M
    drafts = [xs for xs in itertools.product(range(V), repeat=g) if np.prod([q[i][xs[i]] for i in range(g)]) > 0]
    R = np.array(list(itertools.product(grid, repeat=g + 1)))  # [M^3, 3]
    seqs, weights, toks = [], [], []
    for xs in drafts:
        for row in R:
            seqs.append({"target": zt, "draft": zd, "tokens": list(xs), "T": 1.0})
        weights.append(np.prod([q[i][xs[i]] for i in range(g)]))
        toks.append(xs)
    x = pack(seqs, V)
    r = np.tile(R[:, :g], (len(drafts), 1)).astype(np.float32)
    u = np.tile(R[:, g], len(drafts)).astype(np.float32)
    res = run_oracle(x, r=r, u=u)
    got = {}
    for d, (xs, w) in enumerate(zip(toks, weights)):
        for j in range(len(R)):
            b = d * len(R) + j
            n, y = int(res.n[b]), int(res.next_token[b])
            key = (n, tuple(xs[:n]) + (y,))
            got[key] = got.get(key, 0.0) + w / len(R)
    keys = set(law) | set(got)
    for k in keys:
        assert abs(law.get(k, 0.0) - got.get(k, 0.0)) < 1e-15, k


def _chi_run(rounds=1_000_000, seed=0):
    x = synth.chi_square_set(rounds=rounds)
    p = softmax64(x.meta["target_rows"])
    q = softmax64(x.meta["draft_rows"])
    return x, p, q


@pytest.fixture(scope="module")
def chi_set():
    return _chi_run()


def _law_pvalues(x, res, p, q):
    """p-values of: (i) the first emitted token vs p_0; (ii) the joint of
    (n, token emitted at position n) vs the closed form; (iii) the token at
    position k given n >= k vs p_k, for each k."""
    g, V = q.shape
    toks = x.tokens.reshape(-1, g)
    n, y = res.n.astype(np.int64), res.next_token.astype(np.int64)
    out = {}
    first = np.where(n > 0, toks[:, 0], y)
    out["first_token"] = stats.chisquare(np.bincount(first, minlength=V), p[0] * len(n)).pvalue
    pn, alpha = closed_form_nk(p, q)
    joint = np.zeros((g + 1, V))
    for k in range(g):
        joint[k] = pn[k] * residual(p[k], q[k])
    joint[g] = pn[g] * p[g]
    obs = np.bincount(n * V + y, minlength=(g + 1) * V)
    exp = joint.ravel() * len(n)
    keep = exp > 0
    # an outcome of probability 0 that occurs refutes the law outright
    out["impossible_outcomes"] = 1.0 if obs[~keep].sum() == 0 else 0.0
    out["joint_n_token"] = stats.chisquare(obs[keep], exp[keep] * obs[keep].sum() / exp[keep].sum()).pvalue
    for k in range(g + 1):
        reach = n >= k
        tok_k = np.where(n[reach] > k, toks[reach, k] if k < g else 0, y[reach])
        out["position_%d" % k] = stats.chisquare(np.bincount(tok_k, minlength=V),
                                                 p[k] * reach.sum()).pvalue
    return out


@pytest.mark.slow
def test_output_law_chi_square_1e6(chi_set):
    x, p, q = chi_set
    res = run_oracle(x)
    assert ((res.n >= 0) & (res.n <= 4)).all()  # 1 <= tokens per round <= gamma + 1
    pv = _law_pvalues(x, res, p, q)
    for name, v in pv.items():
        assert v > P_MIN, (name, v, pv)
    # acceptance rate per position vs alpha_k = sum min(p_k, q_k) = 1 - TV
    g = q.shape[0]
    _, alpha = closed_form_nk(p, q)
    for k in range(g):
        reach = res.n >= k
        acc = (res.n[reach] > k).sum()
        z = (acc - alpha[k] * reach.sum()) / np.sqrt(reach.sum() * alpha[k] * (1 - alpha[k]))
        assert abs(z) < 4.5, (k, z)
    # mean tokens per round vs sum_k prod_{j<k} alpha_j
    want = sum(np.prod(alpha[:k]) for k in range(g + 1))
    tok = res.n + 1.0
    assert abs(tok.mean() - want) < 4.5 * tok.std() / np.sqrt(len(tok))


@pytest.mark.slow
@pytest.mark.parametrize("which", [oracle.MUTANT_RESIDUAL_IS_P, oracle.MUTANT_RESIDUAL_IS_Q,
                                   oracle.MUTANT_N_PLUS_ONE])
def test_chi_square_has_power_against_planted_mistakes(chi_set, which):
    x, p, q = chi_set
    with oracle.mutant(which):
        res = run_oracle(x)
    pv = _law_pvalues(x, res, p, q)
    assert min(pv.values()) < P_MIN, pv


@pytest.mark.slow
def test_worked_example_alpha_08_gamma_4():
    g = json.loads((GOLDEN / "worked_example_tokens_per_round.json").read_text())
    law = json.loads((GOLDEN / "accepted_count_law.json").read_text())
    alpha, k = g["alpha"], g["k"]
    # two-token rows with sum min(p, q) = 0.8: p = (0.9, 0.1), q = (0.7, 0.3)
    pt, qd = np.log([0.9, 0.1]), np.log([0.7, 0.3])
    rounds = 1_000_000
    zt = np.tile(pt.astype(np.float32), (k + 1, 1))
    zd = np.tile(qd.astype(np.float32), (k, 1))
    x = synth.Inputs("worked", 2, k, "f32",
                     np.ascontiguousarray(np.broadcast_to(zt, (rounds, k + 1, 2))).reshape(-1, 2),
                     np.ascontiguousarray(np.broadcast_to(zd, (rounds, k, 2))).reshape(-1, 2),
                     (np.random.default_rng(3).random((rounds, k)) < 0.3).astype(np.int32).reshape(-1),
                     np.full(rounds, k, np.int32), np.full(rounds, 1.0, np.float32))
    res = run_oracle(x)
    assert (res.n + 1).min() >= 1 and (res.n + 1).max() <= k + 1
    exact = (1 - alpha ** (k + 1)) / (1 - alpha)
    assert abs(exact - g["exact"]) < 1e-12 and round(exact) == 3  # "roughly 3"
    tok = res.n + 1.0
    assert abs(tok.mean() - exact) < 4.5 * tok.std() / np.sqrt(rounds)
    pn = np.array(law["p_n"])
    np.testing.assert_allclose(pn, [alpha ** i - alpha ** (i + 1) for i in range(k)] + [alpha ** k])
    assert stats.chisquare(np.bincount(res.n, minlength=k + 1), pn * rounds).pvalue > P_MIN
