"""GPU parity: libspecverify (through its C ABI) against the CPU oracle on the
same seeded inputs and the same Philox stream.

Bar: accepted counts and emitted tokens are bit-exact on every sequence, with
one allowance where a decisive uniform lies within 1e-6 of its boundary (the
oracle's near-tie rule: r_i within 1e-6 relative of its accept threshold, or
u * C within 1e-6 * C of a step of the final draw's CDF). There the GPU's
outcome must still be one the oracle admits: n exact and the token inside the
oracle's window of tokens on either side of the step, or, for a near-tie
accept decision, the oracle's outcome with that one decision reversed. The
number of flagged sequences must stay within its expectation (the oracle's
per-sequence chance of a flag, summed) plus five standard deviations.
Probabilities within 1e-5 absolute; row maxima and argmax exact; runs
bit-identical run to run. Greedy sequences have no near-ties.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import pack, run_oracle, subset

pytestmark = pytest.mark.gpu

EPS24 = 2.0 ** -24


@pytest.fixture(scope="module")
def svx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_sampling_verify_amd as m
    return m


def log(*a):
    print(*a, flush=True)


def run_gpu(svx, x, r=None, u=None, seed=None, row_offset=None, max_gamma=None):
    d = svx.from_inputs(x)
    mg = x.max_gamma if max_gamma is None else max_gamma
    ws = svx.workspace_for(svx._shape_of(d["target"], d["draft"], d["gamma"], mg), "cuda")
    if r is not None:
        n, nxt = svx.specv_verify_with_uniforms(
            d["target"], d["draft"], d["draft_tokens"], d["gamma"], d["temperature"],
            torch.from_numpy(np.ascontiguousarray(r, np.float32)).cuda(),
            torch.from_numpy(np.ascontiguousarray(u, np.float32)).cuda(), max_gamma=mg, workspace=ws)
    else:
        n, nxt = svx.specv_verify(d["target"], d["draft"], d["draft_tokens"], d["gamma"],
                                  d["temperature"], max_gamma=mg,
                                  seed=x.seed if seed is None else seed,
                                  philox_row_offset=x.row_offset if row_offset is None else row_offset,
                                  workspace=ws)
    torch.cuda.synchronize()
    return n.cpu().numpy(), nxt.cpu().numpy(), svx.read_status(ws)


def flag_cap(orc):
    """The most flagged sequences the rule allows: the expected count plus
    five standard deviations (a sum of independent flags) and a few."""
    e = float(orc.near_prob[orc.n >= 0].sum())
    return e, e + 5.0 * np.sqrt(e) + 3.0


def assert_parity(name, x, got, orc):
    n, nxt = got[0], got[1]
    exact = (n == orc.n) & (nxt == orc.next_token)
    ok = orc.admits(n, nxt)
    in_window = ~exact & (n == orc.n) & (nxt >= orc.tok_lo) & (nxt <= orc.tok_hi)
    reversed_ = ~exact & ~in_window & ok
    flagged = int(orc.near_tie.sum())
    expect, cap = flag_cap(orc)
    log("[parity] %s: B=%d V=%d %s  exact=%d in_draw_window=%d reversed_accept=%d failed=%d "
        "flagged=%d (expected %.1f, cap %.1f) mean_tokens=%.4f"
        % (name, x.batch, x.vocab, x.dtype, exact.sum(), in_window.sum(), reversed_.sum(),
           (~ok).sum(), flagged, expect, cap,
           np.mean(orc.n[orc.n >= 0] + 1) if (orc.n >= 0).any() else 0.0))
    if not ok.all():
        idx = np.flatnonzero(~ok)[:10]
        detail = [(int(i), int(n[i]), int(orc.n[i]), int(nxt[i]), int(orc.next_token[i]),
                   int(orc.tok_lo[i]), int(orc.tok_hi[i]), int(orc.alt_n[i]),
                   float(orc.accept_margin[i]), float(orc.draw_margin[i])) for i in idx]
        raise AssertionError("%s: %d outcomes the oracle does not admit (b, n_gpu, n_orc, "
                             "tok_gpu, tok_orc, window_lo, window_hi, alt_n, accept_margin, "
                             "draw_margin): %s" % (name, (~ok).sum(), detail))
    assert flagged <= cap, "%s: %d flagged sequences, expected %.1f" % (name, flagged, expect)
    return int((~exact).sum())


def parity_case(svx, name, x, repeat=True):
    log("[case] %s" % name)
    got = run_gpu(svx, x)
    orc = run_oracle(x)
    assert_parity(name, x, got, orc)
    if repeat:  # run-to-run bit identity
        again = run_gpu(svx, x)
        np.testing.assert_array_equal(got[0], again[0])
        np.testing.assert_array_equal(got[1], again[1])
    return got, orc


# ---------------------------------------------------------------- Philox

def test_device_philox_matches_oracle(svx):
    rng = np.random.default_rng(9)
    ctr = rng.integers(0, 2**32, (4096, 4), dtype=np.uint64).astype(np.uint32)
    for seed in (0, 1, 2**64 - 1, 0x243F6A8885A308D3):
        dev = svx.specv_philox4x32_10(seed, torch.from_numpy(ctr.view(np.int32)).cuda())
        got = dev.cpu().numpy().view(np.uint32)
        np.testing.assert_array_equal(got, oracle.philox_blocks(seed, ctr))


# ------------------------------------------------------- row statistics

ROW_CASES = [
    ("tiny_cpu", dict(rounds=64)),
    ("t5xxl_like", dict(rounds=16)),
    ("t5xxl_like_greedy", dict(rounds=16, greedy=True)),
    ("serving_b64", dict(batch=4)),
    ("ragged_b256", dict(batch=8)),
    ("large_vocab", dict(batch=6)),
]


def make(name, **kw):
    if name.endswith("_greedy"):
        return synth.by_name(name[:-7], **kw)
    return synth.by_name(name, **kw)


@pytest.mark.parametrize("name,kw", ROW_CASES, ids=[c[0] for c in ROW_CASES])
def test_row_stats_parity(svx, name, kw):
    log("[case] row stats %s" % name)
    x = make(name, **kw)
    d = svx.from_inputs(x)
    got = svx.specv_row_stats(d["target"], d["draft"], d["gamma"], d["temperature"],
                              max_gamma=x.max_gamma)
    got = {k: v.cpu().numpy() for k, v in got.items()}
    toff, doff = x.offsets()
    Tt = np.repeat(x.temperature, x.gamma + 1)
    Td = np.repeat(x.temperature, x.gamma)
    for side, logits, T in (("target", x.target, Tt), ("draft", x.draft, Td)):
        m, s, a, ok = oracle.row_stats(logits, x.vocab, T)
        need = T > 0 if side == "draft" else np.ones_like(T, bool)
        np.testing.assert_array_equal(got[side + "_max"][need], m[need].astype(np.float32))
        np.testing.assert_array_equal(got[side + "_argmax"][need], a[need])
        samp = need & (T > 0)
        rel = np.abs(got[side + "_sum"][samp] / s[samp] - 1.0)
        log("[rowstats] %s %s rows=%d max_rel_sum_err=%.3g" % (name, side, samp.sum(),
                                                               rel.max() if rel.size else 0.0))
        assert (rel < 1e-6).all()
        if side == "draft":
            assert (got["draft_argmax"][~need] == -1).all()


SOFTMAX_CASES = [("tiny_cpu", dict(rounds=64)), ("t5xxl_like", dict(rounds=8)),
                 ("serving_b64", dict(batch=4)), ("ragged_b256", dict(batch=6)),
                 ("large_vocab", dict(batch=6))]


@pytest.mark.parametrize("name,kw", SOFTMAX_CASES, ids=[c[0] for c in SOFTMAX_CASES])
def test_softmax_rows_within_1e5(svx, name, kw):
    # every sampling target and draft row of a few sequences of each workload
    log("[case] softmax rows %s" % name)
    x = make(name, **kw)
    d = svx.from_inputs(x)
    samp = np.flatnonzero(np.repeat(x.temperature, x.gamma + 1) > 0)[:48]
    dsamp = np.flatnonzero(np.repeat(x.temperature, x.gamma) > 0)[:40]
    rows = np.concatenate([samp, -dsamp - 1]).astype(np.int64)
    p = svx.specv_softmax_rows(d["target"], d["draft"], d["gamma"], d["temperature"],
                               torch.from_numpy(rows), max_gamma=x.max_gamma).cpu().numpy()
    Tt = np.repeat(x.temperature, x.gamma + 1)
    Td = np.repeat(x.temperature, x.gamma)
    worst = 0.0
    for k, r in enumerate(rows):
        ref = oracle.softmax_row(x.target, x.vocab, r, Tt[r]) if r >= 0 else \
            oracle.softmax_row(x.draft, x.vocab, -r - 1, Td[-r - 1])
        err = np.abs(p[k] - ref).max()
        worst = max(worst, err)
        assert err < 1e-5, (name, int(r), err)
        assert abs(p[k].astype(np.float64).sum() - 1.0) < 1e-5
    log("[softmax] %s rows=%d worst_abs_err=%.3g" % (name, len(rows), worst))


# ------------------------------------------ hand cases (injected uniforms)

def uniform_row(V, support):
    z = np.full(V, -np.inf, np.float32)
    z[list(support)] = 0.0
    return z


def step(V, p_sup, q_sup, tokens, T=1.0):
    t = np.stack([uniform_row(V, s) for s in p_sup])
    d = np.stack([uniform_row(V, s) for s in q_sup]) if q_sup else np.zeros((0, V), np.float32)
    return {"target": t, "draft": d, "tokens": tokens, "T": T}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_hand_cases_exact(svx, dtype):
    log("[case] hand cases %s" % dtype)
    V = 4
    s = step(V, [range(4), range(4)], [[0, 1]], [0])
    x = pack([s] * 8, V, dtype)
    r = np.array([[0.5], [0.5 + EPS24], [0.5], [0.5 + EPS24], [EPS24], [1.0], [0.5 + EPS24],
                  [0.5 + EPS24]], np.float32)
    u = np.array([0.25, 0.5, 0.25 + EPS24, 0.5 + EPS24, 1.0, EPS24, EPS24, 1.0], np.float32)
    n, nxt, st = run_gpu(svx, x, r=r, u=u)
    assert list(n) == [1, 0, 1, 0, 1, 0, 0, 0]
    assert list(nxt) == [0, 2, 1, 3, 3, 2, 2, 3]
    assert st == 0


def test_dyadic_quadrature_matches_oracle(svx):
    log("[case] dyadic quadrature")
    import itertools
    V, g, M = 4, 2, 8
    zt = np.full((3, V), -np.inf, np.float32)
    for i, sup in enumerate([[0, 1, 2, 3], [0, 2], [1, 3]]):
        zt[i, sup] = 0
    zd = np.full((2, V), -np.inf, np.float32)
    for i, sup in enumerate([[0, 1], [0, 1, 2, 3]]):
        zd[i, sup] = 0
    grid = (np.arange(M) + 0.5) / M
    R = np.array(list(itertools.product(grid, repeat=g + 1)))
    drafts = [xs for xs in itertools.product(range(V), repeat=g) if xs[0] in (0, 1)]
    seqs = [{"target": zt, "draft": zd, "tokens": list(xs), "T": 1.0} for xs in drafts for _ in R]
    x = pack(seqs, V)
    r = np.tile(R[:, :g], (len(drafts), 1)).astype(np.float32)
    u = np.tile(R[:, g], len(drafts)).astype(np.float32)
    n, nxt, _ = run_gpu(svx, x, r=r, u=u)
    orc = run_oracle(x, r=r, u=u)
    np.testing.assert_array_equal(n, orc.n)
    np.testing.assert_array_equal(nxt, orc.next_token)


# ------------------------------------------------------- workload parity

WORKLOADS = [
    ("tiny_cpu_10000_rounds", lambda: synth.tiny_cpu(rounds=10000)),
    ("tiny_cpu_greedy", lambda: synth.tiny_cpu(rounds=10000, greedy=True)),
    ("t5xxl_like_300_rounds", lambda: synth.t5xxl_like(rounds=300)),
    ("t5xxl_like_greedy_2000 (bench launch)", lambda: synth.t5xxl_like(rounds=2000, greedy=True)),
    ("serving_b64_full", lambda: synth.serving_b64()),
    ("ragged_b256_b48", lambda: synth.ragged_b256(batch=48)),
    ("large_vocab_b24", lambda: synth.large_vocab(batch=24, identical=2)),
]


@pytest.mark.parametrize("name,fn", WORKLOADS, ids=[w[0] for w in WORKLOADS])
def test_workload_parity(svx, name, fn):
    x = fn()
    got, orc = parity_case(svx, name, x)
    assert got[2] == 0  # no data errors in generated workloads


def test_bench_launch_full_size_parity(svx):
    # The launch the benchmark times: 2000 rounds of the T5-XXL-like shape.
    x = synth.t5xxl_like(rounds=2000)
    parity_case(svx, "t5xxl_like_2000_rounds (bench launch)", x, repeat=False)


@pytest.mark.parametrize("name,fn", [("ragged_b256_full", lambda: synth.ragged_b256()),
                                     ("large_vocab_full", lambda: synth.large_vocab())])
def test_full_size_parity(svx, name, fn):
    x = fn()
    got, orc = parity_case(svx, name, x, repeat=False)
    if name.startswith("large_vocab"):
        same = x.meta["identical_sequences"]
        assert (got[0][same] == x.gamma[same]).all()  # draft == target: all accepted


# ------------------------------------------------------------ edge cases

def test_edge_shapes_and_scalar_path(svx):
    cases = [
        ("V=1001 bf16 (rows not 16B aligned: scalar path)", synth.tiny_cpu(rounds=300, vocab=1001)),
        ("V=12345 fp32 (scalar path)", synth.tiny_cpu(rounds=50, vocab=12345)),
        ("V=8", synth.tiny_cpu(rounds=2000, vocab=8)),
        ("V=1", synth.tiny_cpu(rounds=64, vocab=1)),
        ("V=40000 bf16 ragged tail", synth.ragged_b256(batch=6, vocab=40000, max_gamma=5)),
        ("B=1", synth.serving_b64(batch=1)),
    ]
    # make the 1001 case bf16
    x = cases[0][1]
    cases[0] = (cases[0][0], synth.Inputs(x.name, x.vocab, x.max_gamma, "bf16",
                                          synth.to_bf16_bits(x.target), synth.to_bf16_bits(x.draft),
                                          x.tokens, x.gamma, x.temperature))
    for name, x in cases:
        parity_case(svx, name, x, repeat=False)


def test_gamma_zero_mixed_temperatures_and_ties(svx):
    rng = np.random.default_rng(17)
    V = 3000
    seqs = []
    for b in range(40):
        g = int(rng.integers(0, 5))
        # few distinct values -> many argmax ties after bf16 rounding
        t = rng.integers(-3, 4, (g + 1, V)).astype(np.float32)
        d = t[:g] + rng.integers(-1, 2, (g, V)).astype(np.float32)
        if b % 5 == 0:
            t[:, rng.choice(V, 100, replace=False)] = -np.inf
        T = [0.0, 1.0, 0.5, 2.0][b % 4]
        toks = [int(np.argmax(d[i])) if T == 0 else int(rng.integers(0, V)) for i in range(g)]
        for i in range(g):  # keep sampled tokens off -inf draft entries
            if d[i, toks[i]] == -np.inf:
                toks[i] = int(np.argmax(d[i]))
        seqs.append({"target": t, "draft": d, "tokens": toks, "T": T})
    for dt in ("bf16", "f32"):
        x = pack(seqs, V, dt)
        x.max_gamma = 4
        x.seed, x.row_offset = 123, 456
        parity_case(svx, "gamma 0..4, T in {0, .5, 1, 2}, ties, masks (%s)" % dt, x)


def test_uniform_gamma_zero_batch(svx):
    # every gamma 0: a uniform batch with no draft rows, so pass 1 covers the
    # target rows only and its first workgroup still sets the status word;
    # each sequence emits one token drawn from p_0 (argmax when greedy)
    rng = np.random.default_rng(23)
    V = 5000
    seqs = [{"target": (rng.standard_normal((1, V)) * 2).astype(np.float32),
             "draft": np.zeros((0, V), np.float32), "tokens": [],
             "T": [1.0, 0.0, 0.7][b % 3]} for b in range(300)]
    for dt in ("bf16", "f32"):
        x = pack(seqs, V, dt)
        x.max_gamma = 0
        x.seed, x.row_offset = 9, 77
        got, _ = parity_case(svx, "uniform gamma 0, B=300 (%s)" % dt, x, repeat=False)
        assert (got[0] == 0).all() and got[2] == 0


def test_data_errors(svx):
    V = 64
    rng = np.random.default_rng(2)
    base = {"target": rng.standard_normal((3, V)).astype(np.float32),
            "draft": rng.standard_normal((2, V)).astype(np.float32), "tokens": [1, 2], "T": 1.0}
    def mod(**kw):
        s = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in base.items()}
        s.update(kw)
        return s
    t_nan = base["target"].copy(); t_nan[2, 5] = np.nan
    t_inf = base["target"].copy(); t_inf[0, 9] = np.inf
    d_nan = base["draft"].copy(); d_nan[1, 3] = np.nan
    t_all = base["target"].copy(); t_all[1, :] = -np.inf
    seqs = [base, mod(target=t_nan), mod(target=t_inf), mod(draft=d_nan), mod(target=t_all),
            mod(tokens=[1, V]), mod(tokens=[-5, 2]), mod(T=-1.0), mod(T=np.nan), mod(T=np.inf),
            mod(draft=d_nan, T=0.0), mod(target=t_nan, T=0.0), base]
    for dt in ("f32", "bf16"):
        x = pack(seqs, V, dt)
        n, nxt, st = run_gpu(svx, x)
        orc = run_oracle(x)
        np.testing.assert_array_equal(n, orc.n)
        np.testing.assert_array_equal(nxt, orc.next_token)
        assert list(n[1:10]) == [-1] * 9 and n[10] >= 0 and n[11] == -1
        assert st & svx.SPECV_DEV_SEQ_ERROR and not st & svx.SPECV_DEV_LAYOUT_ERROR


def test_layout_error_and_empty_batch(svx):
    # gammas that pass every host check but disagree with max_gamma or with the
    # row totals: only the device can see them
    for g0, g1 in ((5, 3), (3, 4)):
        x = synth.tiny_cpu(rounds=8, vocab=100)
        x.gamma[0], x.gamma[1] = g0, g1
        log("[case] layout error gamma[0:2]=(%d, %d)" % (g0, g1))
        n, nxt, st = run_gpu(svx, x)
        orc = run_oracle(x)
        assert not orc.layout_ok
        assert (n == -1).all() and (nxt == -1).all() and st & svx.SPECV_DEV_LAYOUT_ERROR
    e = svx.specv_verify(torch.zeros((0, 16), device="cuda"), None, None,
                         torch.zeros(0, dtype=torch.int32, device="cuda"),
                         torch.zeros(0, device="cuda"), max_gamma=0)
    assert e[0].numel() == 0


def ragged_case(B, V, max_gamma, seed, dtype="f32"):
    """A ragged batch of B sequences, gammas uniform in [0, max_gamma] (the
    first one at max_gamma), every fifth sequence greedy, draft rows = target
    rows + N(0, 1), draft tokens drawn from the draft rows."""
    rng = np.random.default_rng(seed)
    g = rng.integers(0, max_gamma + 1, size=B).astype(np.int32)
    g[0] = max_gamma
    T = np.where(np.arange(B) % 5 == 3, 0.0, 1.0).astype(np.float32)
    toff = np.concatenate([[0], np.cumsum(g + 1)])
    doff = np.concatenate([[0], np.cumsum(g)])
    target = (rng.standard_normal((int(toff[-1]), V)) * 2).astype(np.float32)
    seq = np.repeat(np.arange(B), g)
    trow = toff[seq] + (np.arange(int(doff[-1])) - doff[seq])
    draft = (target[trow] + rng.standard_normal((len(trow), V))).astype(np.float32)
    Ts = np.where(T[seq] > 0, T[seq], 1.0)[:, None]
    noise = np.where(T[seq][:, None] > 0, rng.gumbel(size=draft.shape), 0.0)
    tokens = np.argmax(draft / Ts + noise, axis=1).astype(np.int32)
    conv = synth.to_bf16_bits if dtype == "bf16" else (lambda a: a)
    return synth.Inputs("ragged B=%d" % B, V, max_gamma, dtype, conv(target), conv(draft), tokens,
                        g, T)


@pytest.mark.parametrize("B", [1, 63, 64, 65, 700, 1024, 1025, 2500])
def test_ragged_plan_in_pass1_and_planned(svx, B):
    # ragged batches up to 1024 sequences are planned inside pass 1 (no plan
    # launch), larger ones by their own plan launch: both against the oracle
    x = ragged_case(B, 40 if B > 100 else 333, 7, seed=B, dtype="bf16" if B % 2 else "f32")
    parity_case(svx, "ragged B=%d (%s plan)" % (B, "in-pass-1" if B <= 1024 else "launched"), x)


@pytest.mark.parametrize("B", [5, 1024, 1100])
def test_ragged_layout_errors(svx, B):
    # a gamma above max_gamma, a negative gamma, and gammas whose sum differs
    # from the row totals, all with totals the host accepts: the device sees
    # them, in pass 1's plan (B <= 1024) or in the plan launch
    base = ragged_case(B, 24, 4, seed=7 + B)
    assert base.total_draft_rows < B * base.max_gamma  # not a uniform batch
    cases = []
    g = base.gamma.copy(); i = int(np.flatnonzero(g == 4)[0]); j = int(np.flatnonzero(g > 0)[-1])
    if i != j:
        g[i], g[j] = 5, g[j] - 1          # 5 > max_gamma, totals unchanged
        cases.append(("gamma above max_gamma", g))
    g = base.gamma.copy(); i = int(np.flatnonzero(g > 1)[0])
    k = (i + 1) % B
    g[k], g[i] = -1, g[i] + g[k] + 1      # a negative gamma
    cases.append(("negative gamma", g))
    g = base.gamma.copy(); g[int(np.flatnonzero(g < 4)[0])] += 1
    cases.append(("gamma sum above the row total", g))
    for what, gam in cases:
        x = synth.Inputs(base.name, base.vocab, base.max_gamma, base.dtype, base.target, base.draft,
                         base.tokens, gam.astype(np.int32), base.temperature)
        log("[case] ragged B=%d layout error: %s" % (B, what))
        n, nxt, st = run_gpu(svx, x)
        orc = run_oracle(x)
        assert not orc.layout_ok
        assert (n == -1).all() and (nxt == -1).all() and st & svx.SPECV_DEV_LAYOUT_ERROR, what
    # and the untouched batch is fine
    n, nxt, st = run_gpu(svx, base)
    assert not st & svx.SPECV_DEV_LAYOUT_ERROR
    assert_parity("ragged B=%d" % B, base, (n, nxt), run_oracle(base))


def uniform_case(B, V, g, seed, dtype="bf16", errors=False):
    """A uniform batch (every gamma = g): T = 1, every fifth sequence greedy,
    every seventh at T = 0.7; draft rows = target rows + N(0, 1); tokens drawn
    from the draft rows. With `errors`, a few sequences carry data errors
    (NaN or +inf logits, a draft token outside [0, V), invalid
    temperatures)."""
    rng = np.random.default_rng(seed)
    T = np.ones(B, np.float32)
    T[3::5] = 0.0
    T[6::7] = 0.7
    target = (rng.standard_normal((B * (g + 1), V)) * 2).astype(np.float32)
    trow = (np.arange(B * g) // g) * (g + 1) + np.arange(B * g) % g
    draft = (target[trow] + rng.standard_normal((B * g, V))).astype(np.float32)
    Ts = np.repeat(T, g)
    noise = np.where(Ts[:, None] > 0, rng.gumbel(size=draft.shape), 0.0)
    tokens = np.argmax(draft / np.where(Ts > 0, Ts, 1.0)[:, None] + noise, axis=1).astype(np.int32)
    if errors:
        target[1 * (g + 1) + 1, 7] = np.nan
        target[2 * (g + 1) + g, 9] = np.inf      # the bonus row
        draft[4 * g + 0, 3] = np.nan
        tokens[8 * g + 1] = V
        tokens[9 * g] = -1
        T[10], T[11], T[12] = -1.0, np.nan, np.inf
        target[13 * (g + 1) + 2, :] = -np.inf    # no finite logit (sequence 13 greedy)
    conv = synth.to_bf16_bits if dtype == "bf16" else (lambda a: a)
    return synth.Inputs("uniform B=%d" % B, V, g, dtype, conv(target), conv(draft), tokens,
                        np.full(B, g, np.int32), T)


@pytest.mark.parametrize("B,V,g,dtype", [(1024, 8192, 3, "bf16"), (1100, 8193, 2, "bf16"),
                                         (1030, 4096, 5, "f32"), (1500, 5000, 1, "f32"),
                                         (2048, 20000, 0, "bf16")])
def test_large_uniform_batch_parity(svx, B, V, g, dtype):
    # uniform batches of a thousand and more sequences (no plan launch, the
    # draw in the accept step's launch): vector and scalar loads (rows not
    # 16-byte multiples), bf16 and fp32, gamma 0..5, greedy and sampling mixed
    x = uniform_case(B, V, g, seed=B + V, dtype=dtype)
    parity_case(svx, "uniform B=%d V=%d gamma=%d %s" % (B, V, g, dtype), x)


@pytest.mark.parametrize("B,V,g,dtype,errors", [
    (333, 1024, 4, "f32", True),   # 2,997 rows: the last wave's second row is past the end
    (257, 2048, 2, "bf16", True),  # one bf16 tile per row
    (64, 1020, 5, "f32", False),   # 4,080-byte rows: the last vectors of each lane masked
    (100, 4, 3, "f32", False),     # 16-byte rows: one vector per row
    (101, 8, 1, "bf16", False),    # 16-byte bf16 rows
])
def test_short_row_pass1(svx, B, V, g, dtype, errors):
    # rows of one 4 KiB tile: two rows per pass-1 wave, with greedy sequences'
    # draft rows and invalid temperatures' rows skipped (their loads go to the
    # first target row), NaN / +inf / all -inf rows and bad tokens
    x = uniform_case(B, V, g, seed=B * 7 + V, dtype=dtype, errors=errors)
    got, orc = parity_case(svx, "short rows B=%d V=%d gamma=%d %s%s" % (
        B, V, g, dtype, " errors" if errors else ""), x)
    if errors:
        assert got[2] & svx.SPECV_DEV_SEQ_ERROR


def short_rows_random_case(seed):
    """A seeded random batch of short rows (up to one 4 KiB tile, mostly
    16-byte multiples): uniform, or ragged past 1024 sequences (the plan
    launch); gamma 0..16, greedy, sampling and an occasional invalid
    temperature, masked tokens, draft tokens drawn from the draft rows."""
    rng = np.random.default_rng(50000 + seed)
    dtype = "bf16" if rng.random() < 0.5 else "f32"
    vec = 8 if dtype == "bf16" else 4
    vmax = 2048 if dtype == "bf16" else 1024
    V = (int(rng.integers(1, vmax // vec + 1)) * vec if rng.random() < 0.85
         else int(rng.integers(1, vmax + 1)))
    ragged = rng.random() < 0.25
    g = int(rng.integers(0, 17))
    bmax = max(1, min(3000, 12_000_000 // max(1, (2 * g + 1) * V)))
    B = int(rng.integers(1025, 1400)) if ragged and bmax >= 1025 else int(rng.integers(1, bmax + 1))
    gam = rng.integers(0, g + 1, size=B).astype(np.int32) if ragged else np.full(B, g, np.int32)
    gam[0] = g
    T = np.where(rng.random(B) < 0.2, 0.0, rng.uniform(0.3, 2.0, B)).astype(np.float32)
    if rng.random() < 0.2:
        T[rng.integers(0, B)] = -1.0
    toff = np.concatenate([[0], np.cumsum(gam + 1)])
    doff = np.concatenate([[0], np.cumsum(gam)])
    target = (rng.standard_normal((int(toff[-1]), V)) * float(rng.choice([0.5, 2.0, 4.0]))).astype(np.float32)
    seq = np.repeat(np.arange(B), gam)
    trow = toff[seq] + (np.arange(int(doff[-1])) - doff[seq])
    draft = (target[trow] + rng.standard_normal((len(trow), V)) * float(rng.choice([0.1, 1.0]))).astype(np.float32)
    if V > 4 and rng.random() < 0.3:
        cols = rng.choice(V, size=V // 4, replace=False)
        target[:, cols] = -np.inf
        draft[:, cols[: len(cols) // 2]] = -np.inf
    Ts = np.where(T[seq] > 0, T[seq], 1.0)[:, None]
    z = np.where(np.isfinite(draft), draft / Ts, -np.inf)
    noise = np.where(T[seq][:, None] > 0, rng.gumbel(size=draft.shape), 0.0)
    tokens = np.argmax(z + noise, axis=1).astype(np.int32)
    conv = synth.to_bf16_bits if dtype == "bf16" else (lambda a: a)
    return synth.Inputs("short rows random %d" % seed, V, g, dtype, conv(target), conv(draft), tokens,
                        gam, T)


@pytest.mark.parametrize("seed", range(8))
def test_short_rows_random_lenient(svx, seed):
    # the lossy step on the random short-row batches (each lenience function)
    x = short_rows_random_case(100 + seed)
    kind, eps = [("lin", 0.5), ("sq", 0.3), ("exp", 0.2), ("lin", 0.05)][seed % 4]
    log("[case] short rows random %d lenient %s %g (V=%d %s B=%d)" % (100 + seed, kind, eps, x.vocab,
                                                                     x.dtype, x.batch))
    got = run_gpu_lenient(svx, x, kind, eps)
    orc = run_oracle(x, lenience=kind, epsilon=eps)
    assert_parity("short rows random %d lenient %s %g" % (100 + seed, kind, eps), x, got, orc)


@pytest.mark.parametrize("seed", range(32))
def test_short_rows_random(svx, seed):
    # short rows at random shapes: pass 1 two rows per wave, pass 2 one wave
    # per sequence (weights left in LDS for the draw where V <= 1024)
    x = short_rows_random_case(seed)
    parity_case(svx, "short rows random %d (V=%d %s B=%d gamma<=%d %s)" % (
        seed, x.vocab, x.dtype, x.batch, x.max_gamma,
        "ragged" if (x.gamma != x.gamma[0]).any() else "uniform"), x, repeat=False)


@pytest.mark.parametrize("V,g,dtype,K", [(32128, 5, "bf16", 16), (1000, 4, "f32", 64),
                                         (256000, 8, "f32", 4)])
def test_logits_past_4_gib(svx, V, g, dtype, K):
    # byte offsets past 32 bits: a uniform batch just long enough that the
    # last K sequences' target and draft rows start beyond 4 GiB (5-10 GB of
    # logits on the device). Those K hold random rows (every fifth greedy)
    # and are checked against the oracle at their own Philox rows; the others
    # hold zero logits (p = q uniform: every draft accepted, the token drawn
    # from p) and are checked for that.
    row_bytes = V * (2 if dtype == "bf16" else 4)
    b0 = 2**32 // (g * row_bytes) + 1
    B = b0 + K
    assert b0 * g * row_bytes > 2**32
    xs = uniform_case(K, V, g, seed=V + K, dtype=dtype)
    d = svx.from_inputs(xs)
    el = torch.int16 if dtype == "bf16" else torch.float32
    log("[case] logits past 4 GiB: V=%d gamma=%d %s B=%d (%.1f GB), random sequences %d.." % (
        V, g, dtype, B, B * (2 * g + 1) * row_bytes / 1e9, b0))
    target = torch.zeros((B * (g + 1), V), dtype=el, device="cuda")
    draft = torch.zeros((B * g, V), dtype=el, device="cuda")
    target[b0 * (g + 1):] = d["target"]
    draft[b0 * g:] = d["draft"]
    tokens = torch.zeros(B * g, dtype=torch.int32, device="cuda")
    tokens[b0 * g:] = d["draft_tokens"]
    gamma = torch.full((B,), g, dtype=torch.int32, device="cuda")
    temp = torch.ones(B, dtype=torch.float32, device="cuda")
    temp[b0:] = d["temperature"]
    ws = svx.workspace_for(svx._shape_of(target, draft, gamma, g), "cuda")
    P = 12345
    n, nxt = svx.specv_verify(target, draft, tokens, gamma, temp, max_gamma=g, seed=xs.seed,
                              philox_row_offset=P, workspace=ws)
    torch.cuda.synchronize()
    n, nxt, st = n.cpu().numpy(), nxt.cpu().numpy(), svx.read_status(ws)
    # the diagnostics on the same rows: the last K * g positions against the
    # oracle, the zero rows' alpha = 1 and entropy = ln V
    dg = svx.specv_position_diagnostics(target, draft, gamma, temp, 16, max_gamma=g)
    torch.cuda.synchronize()
    dg = {name: t.cpu().numpy() for name, t in dg.items()}
    del target, draft
    torch.cuda.empty_cache()
    assert st == 0
    assert (n[:b0] == g).all() and (nxt[:b0] >= 0).all() and (nxt[:b0] < V).all()
    orc = run_oracle(xs, row_offset=P + b0)
    assert_parity("past 4 GiB V=%d %s" % (V, dtype), xs, (n[b0:], nxt[b0:], st), orc)
    want = oracle.position_diagnostics(xs.target, xs.draft, xs.gamma, xs.temperature, vocab=V,
                                       top_k=16)
    q0 = b0 * g
    nan = np.isnan(want.alpha)
    np.testing.assert_array_equal(np.isnan(dg["alpha"][q0:]), nan)
    assert np.abs(dg["alpha"][q0:][~nan] - want.alpha[~nan]).max(initial=0) <= DIAG_ALPHA_TOL
    assert np.abs(dg["entropy"][q0:][~nan] - want.entropy[~nan]).max(initial=0) <= DIAG_ENTROPY_TOL
    np.testing.assert_array_equal(dg["topk_index"][q0:], want.topk_index)
    assert np.abs(dg["alpha"][:q0] - 1.0).max() <= DIAG_ALPHA_TOL
    assert np.abs(dg["entropy"][:q0] - np.log(V)).max() <= DIAG_ENTROPY_TOL


def test_concurrent_streams(svx):
    # two streams (default priority), each with its own inputs and workspace
    # (a T5-XXL-like batch and a batch of one-tile fp32 rows), calls enqueued
    # alternately: every call returns what the same call returns alone, so
    # the library keeps no state between calls but the caller's workspace
    xa = synth.t5xxl_like(rounds=64)
    xb = uniform_case(300, 1000, 4, seed=3, dtype="f32")
    ref = [run_gpu(svx, xa), run_gpu(svx, xb)]
    log("[case] concurrent streams: B=%d V=%d and B=%d V=%d" % (xa.batch, xa.vocab, xb.batch, xb.vocab))
    calls = []
    for x in (xa, xb):
        d = svx.from_inputs(x)
        ws = svx.workspace_for(svx._shape_of(d["target"], d["draft"], d["gamma"], x.max_gamma), "cuda")
        calls.append((x, d, ws, torch.cuda.Stream()))
    torch.cuda.synchronize()
    outs = []
    for i in range(8):
        for k, (x, d, ws, st) in enumerate(calls):
            with torch.cuda.stream(st):
                n, nxt = svx.specv_verify(d["target"], d["draft"], d["draft_tokens"], d["gamma"],
                                          d["temperature"], max_gamma=x.max_gamma, seed=x.seed,
                                          philox_row_offset=x.row_offset, workspace=ws, stream=st)
            outs.append((k, n, nxt))
    torch.cuda.synchronize()
    for k, n, nxt in outs:
        np.testing.assert_array_equal(n.cpu().numpy(), ref[k][0])
        np.testing.assert_array_equal(nxt.cpu().numpy(), ref[k][1])


BF16_LOWEST = -3.3895313892515355e38  # the most negative finite bf16 (0xff7f)


def range_case(kind, dtype, seed, B=48, V=3000, g=4):
    """Logits at the ends of the floating-point range (uniform batch, every
    fourth sequence greedy, V = 3000: several pass-1 tiles per row):
    - "lowest_mask": a random half of each sequence's vocabulary masked with
      the dtype's most negative finite value instead of -inf (what
      torch.finfo(dtype).min masking produces), the same tokens in its
      target and draft rows;
    - "minus_1e30_mask": the same with -1e30;
    - "huge": logits of magnitude about 1e12 (nearly one-hot rows);
    - "offset": logits + 1e9 (quantised to multiples of 64 in fp32: ties);
    - "tiny_T": T = 1e-30 for the sampling sequences (nearly one-hot);
    - "huge_T": T = 3e38 (nearly uniform; log2(e)/T is an fp32 subnormal);
    - "denormal_T": T = 1e-40, where log2(e)/T overflows fp32: outside the
      stated domain, a data error on both sides.
    Draft tokens are drawn from the draft rows, so masked tokens are never
    drafted."""
    rng = np.random.default_rng(seed)
    T = np.where(np.arange(B) % 4 == 3, 0.0, np.where(np.arange(B) % 4 == 1, 0.7, 1.0)).astype(np.float32)
    rows_t = B * (g + 1)
    target = (rng.standard_normal((rows_t, V)) * 2).astype(np.float32)
    trow = (np.arange(B * g) // g) * (g + 1) + np.arange(B * g) % g
    draft = (target[trow] + rng.standard_normal((B * g, V))).astype(np.float32)
    if kind in ("lowest_mask", "minus_1e30_mask"):
        low = {"lowest_mask": BF16_LOWEST if dtype == "bf16" else np.finfo(np.float32).min,
               "minus_1e30_mask": -1e30}[kind]
        mask = rng.random((B, V)) < 0.5
        target[mask[np.arange(rows_t) // (g + 1)]] = low
        draft[mask[np.arange(B * g) // g]] = low
    elif kind == "huge":
        target *= np.float32(1e12)
        draft *= np.float32(1e12)
    elif kind == "offset":
        target += np.float32(1e9)
        draft += np.float32(1e9)
    elif kind == "tiny_T":
        T = np.where(T > 0, np.float32(1e-30), T).astype(np.float32)
    elif kind == "huge_T":
        T = np.where(T > 0, np.float32(3e38), T).astype(np.float32)
    elif kind == "denormal_T":  # log2(e)/T overflows fp32: outside the domain
        T = np.where(T > 0, np.float32(1e-40), T).astype(np.float32)
    Ts = np.repeat(T, g).astype(np.float64)
    Ts = np.where(Ts < 1e-38, 0.0, Ts)  # drafting at an invalid T: argmax
    z = draft.astype(np.float64) / np.where(Ts > 0, Ts, 1.0)[:, None]
    noise = np.where(Ts[:, None] > 0, rng.gumbel(size=draft.shape), 0.0)
    tokens = np.argmax(z + noise, axis=1).astype(np.int32)
    conv = synth.to_bf16_bits if dtype == "bf16" else (lambda a: a)
    return synth.Inputs("range %s" % kind, V, g, dtype, conv(target), conv(draft), tokens,
                        np.full(B, g, np.int32), T)


@pytest.mark.parametrize("kind", ["lowest_mask", "minus_1e30_mask", "huge", "offset", "tiny_T",
                                  "huge_T", "denormal_T"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_extreme_logit_ranges(svx, kind, dtype):
    # the softmax of a row at any finite logits and temperature: masks with
    # the most negative finite value, logits of magnitude 1e12, a large common
    # offset, T = 1e-30 and T = 3e38 all give the oracle's outcomes, with no
    # sequence reported as a data error; T = 1e-40 fails every sampling
    # sequence on both sides
    x = range_case(kind, dtype, seed=len(kind) * 7 + (dtype == "bf16"))
    got, orc = parity_case(svx, "range %s %s" % (kind, dtype), x)
    if kind == "denormal_T":
        sampling = x.temperature > 0
        assert (orc.n[sampling] == -1).all() and (orc.n[~sampling] >= 0).all()
        assert got[2] & svx.SPECV_DEV_SEQ_ERROR
    else:
        assert (orc.n >= 0).all() and (got[0] >= 0).all() and got[2] == 0


@pytest.mark.parametrize("B,V,g,dtype", [(8, 262144, 3, "f32"), (8, 262145, 3, "bf16"),
                                         (512, 270000, 0, "bf16")])
def test_draw_scan_paths(svx, B, V, g, dtype):
    # the draw's scans over the sub-block masses (1024 elements each): held
    # in registers up to 256 sub-blocks (V <= 262144), read from memory past
    # that; with the draw in its own launch (few sequences) and in the mass
    # launch (one workgroup per sequence)
    x = uniform_case(B, V, g, seed=V + g, dtype=dtype)
    parity_case(svx, "draw scan B=%d V=%d gamma=%d %s" % (B, V, g, dtype), x)


def test_large_uniform_batch_errors(svx):
    x = uniform_case(1100, 8192, 3, seed=5, errors=True)
    n, nxt, st = run_gpu(svx, x)
    orc = run_oracle(x)
    np.testing.assert_array_equal(n[:20], orc.n[:20])
    assert list(n[[1, 2, 4, 8, 9, 10, 11, 12, 13]]) == [-1] * 9
    assert st & svx.SPECV_DEV_SEQ_ERROR and not st & svx.SPECV_DEV_LAYOUT_ERROR
    assert_parity("uniform batch with data errors", x, (n, nxt), orc)
    # gammas that keep the row totals but differ from max_gamma: a layout
    # error that pass 1's first workgroup finds
    gam = x.gamma.copy()
    gam[700], gam[900] = 4, 2
    y = synth.Inputs(x.name, x.vocab, x.max_gamma, x.dtype, x.target, x.draft, x.tokens, gam,
                     x.temperature)
    n, nxt, st = run_gpu(svx, y)
    assert not run_oracle(y).layout_ok
    assert (n == -1).all() and (nxt == -1).all() and st == svx.SPECV_DEV_LAYOUT_ERROR
    # and a clean batch after it in the same workspace shape
    clean = uniform_case(1100, 8192, 3, seed=6)
    got, _ = parity_case(svx, "uniform batch after a layout error", clean)
    assert run_gpu(svx, clean)[2] == 0


@pytest.mark.parametrize("case", ["uniform", "ragged in pass 1", "ragged planned"])
def test_long_rows_capture_and_data_errors(svx, case):
    # long rows (48 KiB or more per pass-1 chunk, many tiles per chunk) with
    # each draft token's logit recorded by the pass-1 wave whose chunk holds
    # it: uniform, ragged with the plan inside pass 1 and ragged with the
    # plan launch (its token table), with data errors on the uniform batch
    # (tokens outside [0, V), NaN/+inf logits, invalid temperatures)
    if case == "uniform":
        x = uniform_case(16, 65536, 3, seed=21, errors=True)
    elif case == "ragged in pass 1":
        x = ragged_case(40, 65536, 5, seed=22, dtype="bf16")
    else:
        x = ragged_case(1100, 49152, 3, seed=23, dtype="bf16")
    got, orc = parity_case(svx, "long rows, %s (B=%d V=%d)" % (case, x.batch, x.vocab), x)
    if case == "uniform":
        assert list(got[0][[1, 2, 4, 8, 9, 10, 11, 12, 13]]) == [-1] * 9
        assert got[2] & svx.SPECV_DEV_SEQ_ERROR


# ------------------------------------------------- statistics on the GPU

@pytest.mark.parametrize("rounds", [1_000_000])
def test_gpu_output_law_chi_square(svx, rounds):
    from scipy import stats
    log("[case] chi-square V=8, %d rounds on the GPU" % rounds)
    x = synth.chi_square_set(rounds=rounds)
    n, nxt, _ = run_gpu(svx, x)
    p = torch.softmax(torch.from_numpy(x.meta["target_rows"].astype(np.float64)), -1).numpy()
    toks = x.tokens.reshape(-1, 4)
    first = np.where(n > 0, toks[:, 0], nxt)
    pv = stats.chisquare(np.bincount(first, minlength=8), p[0] * rounds).pvalue
    log("[chi] first-token p-value %.4g" % pv)
    assert pv > 1e-4
    orc = run_oracle(x)
    assert_parity("chi-square set", x, (n, nxt), orc)


# --------------------------------------------------- lossy verification

def run_gpu_lenient(svx, x, kind, eps, r=None, u=None):
    d = svx.from_inputs(x)
    ws = svx.workspace_for(svx._shape_of(d["target"], d["draft"], d["gamma"], x.max_gamma), "cuda")
    rt = None if r is None else torch.from_numpy(np.ascontiguousarray(r, np.float32)).cuda()
    ut = None if u is None else torch.from_numpy(np.ascontiguousarray(u, np.float32)).cuda()
    n, nxt = svx.specv_verify_lenient(d["target"], d["draft"], d["draft_tokens"], d["gamma"],
                                      d["temperature"], kind, eps, max_gamma=x.max_gamma,
                                      seed=x.seed, philox_row_offset=x.row_offset, r=rt, u=ut,
                                      workspace=ws)
    torch.cuda.synchronize()
    return n.cpu().numpy(), nxt.cpu().numpy(), svx.read_status(ws)


LENIENT_CASES = [("lin", 0.5), ("lin", 0.05), ("sq", 0.7), ("sq", 0.1), ("exp", 0.5),
                 ("exp", 0.05)]


@pytest.mark.parametrize("kind,eps", LENIENT_CASES, ids=["%s-%g" % c for c in LENIENT_CASES])
def test_lenient_parity_t5xxl_like(svx, kind, eps):
    # bf16, V = 32128: several pass-1 chunks per row
    x = synth.t5xxl_like(rounds=96)
    log("[case] lenient %s eps=%g t5xxl_like B=%d" % (kind, eps, x.batch))
    got = run_gpu_lenient(svx, x, kind, eps)
    orc = run_oracle(x, lenience=kind, epsilon=eps)
    assert got[2] == 0
    assert_parity("lenient %s %g" % (kind, eps), x, got, orc)


def test_lenient_bench_launch_full_size(svx):
    # the launch the lossy benchmark times: 2000 rounds of the T5-XXL-like
    # shape with f_sq and eps = 0.5
    x = synth.t5xxl_like(rounds=2000)
    log("[case] lenient sq eps=0.5 t5xxl_like B=%d (bench launch)" % x.batch)
    got = run_gpu_lenient(svx, x, "sq", 0.5)
    orc = run_oracle(x, lenience="sq", epsilon=0.5)
    assert got[2] == 0
    assert_parity("lenient sq 0.5 bench launch", x, got, orc)


def test_lenient_parity_mixed_greedy_fp32(svx):
    # fp32, odd sequences greedy (lenience must not touch them), V = 256000
    x = synth.large_vocab(batch=6)
    log("[case] lenient sq 0.3 large_vocab B=%d" % x.batch)
    got = run_gpu_lenient(svx, x, "sq", 0.3)
    orc = run_oracle(x, lenience="sq", epsilon=0.3)
    assert_parity("lenient sq 0.3 large_vocab", x, got, orc)
    base = run_gpu(svx, x)
    greedy = x.temperature == 0
    np.testing.assert_array_equal(got[0][greedy], base[0][greedy])
    np.testing.assert_array_equal(got[1][greedy], base[1][greedy])


@pytest.mark.parametrize("kind", ["lowest_mask", "huge", "offset", "tiny_T", "huge_T"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_lenient_extreme_logit_ranges(svx, kind, dtype):
    # the lossy acceptance reads the same max-relative probabilities as the
    # lossless one: at the ends of the range it still gives the oracle's
    # outcomes, with no sequence reported as a data error
    x = range_case(kind, dtype, seed=len(kind) * 13 + (dtype == "bf16"))
    log("[case] lenient sq 0.3 range %s %s B=%d" % (kind, dtype, x.batch))
    got = run_gpu_lenient(svx, x, "sq", 0.3)
    orc = run_oracle(x, lenience="sq", epsilon=0.3)
    assert got[2] == 0 and (orc.n >= 0).all()
    assert_parity("lenient sq 0.3 range %s %s" % (kind, dtype), x, got, orc)


@pytest.mark.parametrize("kind", ["none", "lin", "sq", "exp"])
def test_lenient_eps_one_equals_lossless(svx, kind):
    x = synth.tiny_cpu(rounds=512)
    log("[case] lenient %s eps=1 tiny_cpu" % kind)
    got = run_gpu_lenient(svx, x, kind, 1.0)
    base = run_gpu(svx, x)
    np.testing.assert_array_equal(got[0], base[0])
    np.testing.assert_array_equal(got[1], base[1])


def test_lenient_injected_uniforms_and_monotone(svx):
    x = synth.tiny_cpu(rounds=512, vocab=64, gamma=6, gen_seed=5)
    rng = np.random.default_rng(21)
    r = ((rng.integers(0, 2**24, (x.batch, x.max_gamma)) + 1) * EPS24).astype(np.float32)
    u = ((rng.integers(0, 2**24, x.batch) + 1) * EPS24).astype(np.float32)
    log("[case] lenient injected uniforms tiny_cpu V=64")
    prev = None
    for eps in [1.0, 0.6, 0.2, 0.02]:
        got = run_gpu_lenient(svx, x, "lin", eps, r=r, u=u)
        orc = run_oracle(x, r=r, u=u, lenience="lin", epsilon=eps)
        assert_parity("lenient lin %g injected" % eps, x, got, orc)
        if prev is not None:
            assert (got[0] >= prev).all()
        prev = got[0]


def test_lenient_argument_errors(svx):
    x = synth.tiny_cpu(rounds=4)
    for kind, eps in [("lin", 0.0), ("sq", -0.5), ("exp", 1.5), ("lin", float("nan")), (7, 0.5)]:
        with pytest.raises(svx.SpecvError):
            run_gpu_lenient(svx, x, kind, eps)


# ------------------------------------------------ per-position diagnostics

# alpha and entropy are float64 sums of fp32 terms (each within a few ulp):
# |error(alpha)| <= ~1e-6; the entropy ln S - ln2 * A / S carries the fp32
# term error times ln S - H <= ln V, so 1e-5 (nats) bounds it at V <= 256000.
DIAG_ALPHA_TOL = 2e-6
DIAG_ENTROPY_TOL = 1e-5
DIAG_PROB_TOL = 1e-5


def run_gpu_diag(svx, x, k):
    d = svx.from_inputs(x)
    out = svx.specv_position_diagnostics(d["target"], d["draft"], d["gamma"], d["temperature"], k,
                                         max_gamma=x.max_gamma)
    torch.cuda.synchronize()
    return {name: t.cpu().numpy() for name, t in out.items()}


def assert_diag_parity(name, x, k):
    log("[case] diagnostics %s k=%d B=%d V=%d %s" % (name, k, x.batch, x.vocab, x.dtype))
    got = run_gpu_diag(svx_mod(), x, k)
    want = oracle.position_diagnostics(x.target, x.draft, x.gamma, x.temperature, vocab=x.vocab,
                                       top_k=k)
    nan = np.isnan(want.alpha)
    np.testing.assert_array_equal(np.isnan(got["alpha"]), nan)
    np.testing.assert_array_equal(np.isnan(got["entropy"]), np.isnan(want.entropy))
    ea = np.abs(got["alpha"][~nan] - want.alpha[~nan])
    ee = np.abs(got["entropy"][~nan] - want.entropy[~nan])
    log("[parity] diagnostics %s: positions=%d max|d alpha|=%.3g max|d entropy|=%.3g"
        % (name, len(nan), ea.max(initial=0), ee.max(initial=0)))
    assert ea.max(initial=0) <= DIAG_ALPHA_TOL and ee.max(initial=0) <= DIAG_ENTROPY_TOL
    np.testing.assert_array_equal(got["topk_index"], want.topk_index)
    ok = ~np.isnan(want.topk_prob)
    np.testing.assert_array_equal(np.isnan(got["topk_prob"]), ~ok)
    assert np.abs(got["topk_prob"][ok] - want.topk_prob[ok]).max(initial=0) <= DIAG_PROB_TOL
    return got, want


def svx_mod():
    import speculative_sampling_verify_amd as m
    return m


DIAG_CASES = [
    ("tiny_cpu", dict(rounds=200), 16),              # fp32, V = 1000, one chunk
    ("t5xxl_like", dict(rounds=48), 16),             # bf16, V = 32128, bf16 ties
    ("t5xxl_like_greedy", dict(rounds=32, greedy=True), 8),
    ("serving_b64", dict(batch=6), 64),              # T = 0.7, K at its maximum
    ("ragged_b256", dict(batch=10), 1),              # ragged gammas, 10 chunks
    ("large_vocab", dict(batch=8), 10),              # fp32, V = 256000, odd greedy, p == q rows
    # long merged lists: 5 chunks x 64 (the 8-slot merge), 11 chunks x 64 (16 slots)
    ("ragged_b256", dict(batch=4), 64),
    ("large_vocab", dict(batch=4), 64),
]


@pytest.mark.parametrize("name,kw,k", DIAG_CASES, ids=["%s-k%d" % (c[0], c[2]) for c in DIAG_CASES])
def test_diagnostics_parity(svx, name, kw, k):
    assert_diag_parity(name, make(name, **kw), k)


def test_diagnostics_bench_launch_full_size(svx):
    # the launch the diagnostics benchmark times: 2000 rounds of the T5-XXL-like
    # shape (10,000 draft positions), top-16
    assert_diag_parity("t5xxl_like_2000_rounds (bench launch)", synth.t5xxl_like(rounds=2000), 16)


def test_diagnostics_edges(svx):
    rng = np.random.default_rng(8)
    # odd V (scalar loads), masked tails, ties, a NaN row, T = 0 and k = 0 / k = V
    V = 13
    t = np.round(rng.standard_normal((4, V)) * 2).astype(np.float32)  # many equal logits
    dr = np.round(rng.standard_normal((3, V)) * 2).astype(np.float32)
    dr[1, 7:] = -np.inf
    bad = t.copy()
    bad[0, 2] = np.nan
    seqs = [{"target": t, "draft": dr, "tokens": [0, 1, 2], "T": 1.0},
            {"target": t[:2], "draft": dr[1:2], "tokens": [0], "T": 0.0},
            {"target": bad[:3], "draft": dr[:2], "tokens": [3, 4], "T": 0.5},
            {"target": t[:1], "draft": dr[:0], "tokens": [], "T": 1.0}]
    for dtype in ("f32", "bf16"):
        x = pack(seqs, V, dtype)
        for k in (0, 1, V):
            assert_diag_parity("edges %s" % dtype, x, k)


def test_diagnostics_heavy_ties(svx):
    # bf16 logits on an integer grid (thousands of equal values per row) and
    # an all-equal row: the top-64 boundary falls inside runs of ties, which
    # rank by index
    rng = np.random.default_rng(12)
    V, g = 32128, 3
    seqs = []
    for b in range(4):
        t = np.round(rng.standard_normal((g + 1, V)) * 1.5).astype(np.float32)
        d = np.round(rng.standard_normal((g, V)) * 1.5).astype(np.float32)
        if b == 3:
            d[1] = 0.0
        seqs.append({"target": t, "draft": d, "tokens": [0] * g, "T": 1.0 if b % 2 == 0 else 0.0})
    x = pack(seqs, V, "bf16")
    for k in (64, 7):
        assert_diag_parity("heavy ties", x, k)


@pytest.mark.parametrize("kind", ["lowest_mask", "minus_1e30_mask", "huge", "tiny_T"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_diagnostics_extreme_ranges(svx, kind, dtype):
    # alpha, entropy and top-16 at the ends of the range: masks with the most
    # negative finite value (their q is 0 and adds nothing to the entropy),
    # logits of magnitude 1e12 and T = 1e-30 (one-hot rows)
    x = range_case(kind, dtype, seed=len(kind) * 11 + (dtype == "bf16"), B=16)
    assert_diag_parity("range %s %s" % (kind, dtype), x, 16)


def test_diagnostics_argument_errors(svx):
    x = synth.tiny_cpu(rounds=4, vocab=32)
    for k in (-1, 33, 65):
        with pytest.raises(svx.SpecvError):
            run_gpu_diag(svx, x, k)


def test_max_gamma_63(svx):
    # gamma = 63: the accept step's wave has one lane per target row (64)
    x = synth.tiny_cpu(rounds=96, vocab=512, gamma=63, gen_seed=41)
    parity_case(svx, "gamma=63 uniform", x, repeat=False)
    # ragged 0 / 63 mix, and sequences whose draft rows equal their target
    # rows (every draft accepted: n = 63, the token drawn from row 63)
    rng = np.random.default_rng(42)
    V, seqs = 256, []
    for b in range(24):
        g = 63 if b % 3 else 0
        t = rng.standard_normal((g + 1, V)).astype(np.float32) * 2
        same = b % 3 == 1
        d = t[:g].copy() if same else (t[:g] + rng.standard_normal((g, V)).astype(np.float32))
        toks = [int(np.argmax(d[i] + rng.gumbel(size=V))) for i in range(g)]
        seqs.append({"target": t, "draft": d, "tokens": toks, "T": 1.0})
    x = pack(seqs, V, "bf16")
    got, orc = parity_case(svx, "gamma 0/63 ragged", x, repeat=False)
    assert (orc.n[1::3] == 63).all() and (got[0][1::3] == 63).all()


def random_case(seed):
    """A seeded random shape: V (16-byte aligned or not), dtype, batch,
    ragged gammas up to 20, greedy and sampling temperatures, masked tokens
    (-inf) in some rows, draft tokens drawn from the draft rows."""
    rng = np.random.default_rng(1000 + seed)
    V = int(rng.choice([1, 2, 7, 63, 64, 513, 1000, 2049, 4096, 8191, 16384, 33333, 65536]))
    dtype = "bf16" if rng.random() < 0.5 else "f32"
    B = int(rng.integers(1, 40))
    mg = int(rng.integers(0, 21))
    seqs = []
    for b in range(B):
        g = int(rng.integers(0, mg + 1))
        scale = float(rng.choice([0.5, 2.0, 4.0]))
        t = (rng.standard_normal((g + 1, V)) * scale).astype(np.float32)
        d = (t[:g] + rng.standard_normal((g, V)) * float(rng.choice([0.1, 1.0, 3.0]))).astype(np.float32)
        if V > 4 and rng.random() < 0.3:
            cols = rng.choice(V, size=V // 4, replace=False)
            t[:, cols] = -np.inf
            d[:, cols[: len(cols) // 2]] = -np.inf
        T = 0.0 if rng.random() < 0.25 else float(rng.uniform(0.3, 2.0))
        toks = []
        for i in range(g):
            z = d[i].astype(np.float64) / (T if T > 0 else 1.0)
            z = np.where(np.isfinite(z), z, -np.inf)
            toks.append(int(np.argmax(z + rng.gumbel(size=V))))
        seqs.append({"target": t, "draft": d, "tokens": toks, "T": T})
    return pack(seqs, V, dtype)


@pytest.mark.parametrize("seed", range(96))
def test_random_shapes_parity(svx, seed):
    x = random_case(seed)
    parity_case(svx, "random %d (V=%d %s B=%d max_gamma=%d)" % (seed, x.vocab, x.dtype, x.batch,
                                                               x.max_gamma), x, repeat=False)


@pytest.mark.parametrize("seed", range(32))
def test_diagnostics_random_shapes(svx, seed):
    # the random shapes above (ragged, masked, mixed greedy) with a random top-k
    x = random_case(seed)
    if x.total_draft_rows == 0:
        pytest.skip("no draft positions")
    k = int(np.random.default_rng(seed).integers(0, min(64, x.vocab) + 1))
    assert_diag_parity("random %d" % seed, x, k)


@pytest.mark.parametrize("seed", range(32))
def test_lenient_random_shapes(svx, seed):
    # the random shapes above with a random lenience function and epsilon
    x = random_case(seed)
    rng = np.random.default_rng(7 * seed + 3)
    kind = ["lin", "sq", "exp"][int(rng.integers(0, 3))]
    eps = float(rng.choice([1.0, 0.9, 0.5, 0.2, 0.05, 0.01]))
    got = run_gpu_lenient(svx, x, kind, eps)
    orc = run_oracle(x, lenience=kind, epsilon=eps)
    assert_parity("lenient random %d %s %g" % (seed, kind, eps), x, got, orc)
