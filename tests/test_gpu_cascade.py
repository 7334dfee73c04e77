"""GPU parity of CS Drafting's vertical cascade over bigram tables
(specv_cascade_bigram, through the C ABI) against the oracle's cascade on
the same tables, start tokens, temperatures, lenience and Philox stream.

Bar: generated tokens and the target review's accepted counts are identical
up to the first round in which the oracle saw a near-tie (drafting, the
intermediate review or the target review); the GPU cascade's own output law
is tested against the target Markov chain with a lenient intermediate
review.
"""
import numpy as np
import pytest
import torch
from scipy import stats

import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def svx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_sampling_verify_amd as m
    return m


def log(*a):
    print(*a, flush=True)


def bf16(a):
    import synth
    return synth.to_bf16_bits(np.asarray(a, np.float32))


def tables(V, seed, s_mid=0.6, s_small=1.4, scale=1.5):
    rng = np.random.default_rng(seed)
    t = (rng.standard_normal((V, V)) * scale).astype(np.float32)
    m = (t + rng.standard_normal((V, V)) * s_mid).astype(np.float32)
    s = (t + rng.standard_normal((V, V)) * s_small).astype(np.float32)
    return t, m, s


def run_gpu(svx, tabs, T, start, **kw):
    def tens(a):
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()
    out = svx.specv_cascade_bigram(*[tens(t) for t in tabs], tens(np.asarray(T, np.float32)),
                                   tens(np.asarray(start, np.int32)), **kw)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def assert_cascade_parity(name, svx, tabs, T, start, **kw):
    V = tabs[0].shape[0]
    log("[case] cascade %s B=%d V=%d %s" % (name, len(start), V, kw))
    gkw = dict(kw)
    gkw["philox_row_offset"] = gkw.pop("row_offset", 0)
    got = run_gpu(svx, tabs, T, start, **gkw)
    want = oracle.cascade_bigram(*tabs, T, start, **kw)
    rounds, k1, k2 = kw["rounds"], kw["k1"], kw["k2"]
    diverged = 0
    for b in range(len(start)):
        f = int(want.first_near[b])
        np.testing.assert_array_equal(got["accepted"][b, :f], want.accepted[b, :f], err_msg=str(b))
        if want.length[b] < 0:
            assert got["length"][b] == -1
            continue
        upto = int((want.accepted[b, :f] + 1).sum())
        np.testing.assert_array_equal(got["tokens"][b, :upto], want.tokens[b, :upto], err_msg=str(b))
        if f == rounds:
            assert got["length"][b] == want.length[b]
        else:
            diverged += 1
    # draws per sequence and round: k1 inner rounds of k2 drafts and one
    # inner draw, and the target review's draw; each lands within 1e-6 of
    # one of V boundaries with probability about 2e-6 V
    expect = min(1.0, 2e-6 * V * rounds * (k1 * (k2 + 1) + 1))
    log("[parity] cascade %s: sequences=%d with a near-tie=%d (expected share %.3f)"
        % (name, len(start), diverged, expect))
    assert diverged <= 2 * expect * len(start) + 4
    return got, want


def test_cascade_parity_fp32_lenient(svx):
    tabs = tables(1000, 1)
    B = 128
    start = np.random.default_rng(2).integers(0, 1000, B)
    assert_cascade_parity("fp32 sq 0.5", svx, tabs, np.ones(B, np.float32), start, k1=4, k2=2,
                          rounds=4, lenience="sq", epsilon=0.5, seed=5)


def test_cascade_parity_bf16_mixed_greedy(svx):
    tabs = [bf16(t) for t in tables(2048, 3, scale=2.0)]
    B = 96
    T = np.where(np.arange(B) % 3 == 0, 0.0, 0.8).astype(np.float32)
    start = np.random.default_rng(4).integers(0, 2048, B)
    assert_cascade_parity("bf16 exp 0.3", svx, tabs, T, start, k1=3, k2=3, rounds=3,
                          lenience="exp", epsilon=0.3, seed=7, row_offset=100)


def test_cascade_parity_lossless_no_inner_drafts_and_bad_starts(svx):
    # k2 = 0: every inner round is one draw from the intermediate model
    tabs = tables(300, 5)
    B = 64
    start = np.random.default_rng(6).integers(0, 300, B).astype(np.int32)
    start[7] = 300
    got, _ = assert_cascade_parity("fp32 k2=0", svx, tabs, np.full(B, 1.2, np.float32), start,
                                   k1=3, k2=0, rounds=3)
    assert got["length"][7] == -1


def test_cascade_parity_inner_drafts_past_k1(svx):
    # k2 > k1: one inner round drafts past the k1 tokens the target reviews
    tabs = [bf16(t) for t in tables(700, 14)]
    B = 80
    T = np.where(np.arange(B) % 5 == 0, 0.0, 1.1).astype(np.float32)
    start = np.random.default_rng(15).integers(0, 700, B)
    assert_cascade_parity("bf16 k1=2 k2=5 sq 0.4", svx, tabs, T, start, k1=2, k2=5, rounds=3,
                          lenience="sq", epsilon=0.4, seed=17)


BF16_LOWEST = -3.3895313892515355e38  # the most negative finite bf16 (0xff7f)


@pytest.mark.parametrize("kind", ["lowest_mask", "tiny_T"])
def test_cascade_parity_extreme_ranges(svx, kind):
    # the three tables mask half the vocabulary with the most negative finite
    # bf16 (never generated), or T = 1e-30 (every draw one-hot)
    V, B = 2048, 64
    tabs = list(tables(V, 41, scale=2.0))
    rng = np.random.default_rng(42)
    T = np.where(np.arange(B) % 4 == 0, 0.0, 0.9).astype(np.float32)
    ok = np.arange(V)
    if kind == "lowest_mask":
        cols = rng.random(V) < 0.5
        for t in tabs:
            t[:, cols] = BF16_LOWEST
        ok = np.flatnonzero(~cols)
    else:
        T = np.where(T > 0, np.float32(1e-30), T).astype(np.float32)
    got, want = assert_cascade_parity(kind, svx, [bf16(t) for t in tabs], T, rng.choice(ok, B),
                                      k1=3, k2=2, rounds=3, lenience="sq", epsilon=0.5, seed=9)
    assert (want.length > 0).all() and (got["length"] > 0).all()
    if kind == "lowest_mask":
        assert np.isin(got["tokens"][got["tokens"] >= 0], ok).all()


def test_cascade_gpu_target_law(svx):
    tabs = tables(5, 0)
    B, c = 400_000, 2
    got = run_gpu(svx, tabs, np.ones(B, np.float32), np.full(B, c, np.int32), k1=3, k2=2,
                  rounds=3, lenience="sq", epsilon=0.5, seed=9)
    assert (got["length"] >= 3).all()
    P = torch.softmax(torch.from_numpy(tabs[0].astype(np.float64)), dim=-1).numpy()
    y = got["tokens"][:, :3].astype(np.int64)
    obs = np.bincount((y[:, 0] * 5 + y[:, 1]) * 5 + y[:, 2], minlength=125)
    exp = np.einsum("a,ab,bc->abc", P[c], P, P).reshape(-1) * B
    pv = stats.chisquare(obs, exp).pvalue
    log("[law] cascade GPU joint of 3 tokens (sq 0.5 inner): p = %.4g" % pv)
    assert pv > 1e-4


def test_cascade_parity_scalar_rows(svx):
    # V = 999 (bf16): rows are not 16-byte multiples, so every kernel of the
    # cascade takes its scalar path
    tabs = [bf16(t) for t in tables(999, 8)]
    B = 48
    start = np.random.default_rng(9).integers(0, 999, B)
    assert_cascade_parity("bf16 V=999 lin 0.4", svx, tabs, np.full(B, 0.9, np.float32), start,
                          k1=3, k2=2, rounds=3, lenience="lin", epsilon=0.4, seed=12)


def test_cascade_parity_streamed_rows(svx):
    # V = 9000: rows longer than the 8192 elements a workgroup holds in
    # registers, so drafting and the target review's row builder take their
    # one-wave streaming kernels
    tabs = [bf16(t) for t in tables(9000, 10)]
    B = 32
    T = np.where(np.arange(B) % 4 == 0, 0.0, 1.0).astype(np.float32)
    start = np.random.default_rng(11).integers(0, 9000, B)
    assert_cascade_parity("bf16 V=9000 sq 0.5", svx, tabs, T, start, k1=3, k2=2, rounds=2,
                          lenience="sq", epsilon=0.5, seed=13)


def random_cascade_case(seed):
    """A seeded random cascade problem: V (aligned or not, up to past the
    8192 elements a workgroup holds), dtype, batch, k1 0..6, k2 0..4, rounds,
    lenience and epsilon, greedy and sampling temperatures with an occasional
    NaN one, and an occasional start token outside [0, V)."""
    rng = np.random.default_rng(7000 + seed)
    V = int(rng.choice([1, 2, 7, 64, 100, 999, 1024, 2048, 8192, 8200,
                        int(rng.integers(2, 2000))]))
    B = int(rng.integers(1, 64 if V <= 2048 else 16))
    tabs = tables(V, 8000 + seed, s_mid=float(rng.choice([0.2, 0.6, 1.5])),
                  s_small=float(rng.choice([0.5, 1.4, 3.0])), scale=float(rng.choice([0.7, 1.5, 2.5])))
    if rng.random() < 0.5:
        tabs = [bf16(t) for t in tabs]
    T = np.where(rng.random(B) < 0.3, 0.0, rng.uniform(0.3, 2.0, B)).astype(np.float32)
    T[rng.random(B) < 0.03] = np.nan
    start = rng.integers(0, V, B).astype(np.int32)
    bad = rng.random(B) < 0.03
    start[bad] = np.where(rng.random(int(bad.sum())) < 0.5, -1, V)
    kind = ["none", "lin", "sq", "exp"][int(rng.integers(0, 4))]
    eps = 1.0 if kind == "none" else float(rng.choice([1.0, 0.7, 0.3, 0.05]))
    kw = dict(k1=int(rng.integers(0, 7)), k2=int(rng.integers(0, 5)), rounds=int(rng.integers(1, 4)),
              lenience=kind, epsilon=eps, seed=int(rng.integers(0, 2**63)),
              row_offset=int(rng.integers(0, 2**40)))
    return tabs, T, start, kw


@pytest.mark.parametrize("seed", range(12))
def test_cascade_random_shapes(svx, seed):
    tabs, T, start, kw = random_cascade_case(seed)
    got, _ = assert_cascade_parity("random %d %s" % (seed, "bf16" if tabs[0].dtype == np.uint16
                                                     else "fp32"), svx, tabs, T, start, **kw)
    failed = np.isnan(T) | (start < 0) | (start >= tabs[0].shape[0])
    assert (got["length"][failed] == -1).all()


def test_cascade_bench_launch_full_size(svx):
    # the launch the cascade benchmark times: the benchmark's three bigram
    # tables (V = 8192, bf16), 2048 sequences, k1 = 5, k2 = 3, 8 rounds, f_sq
    # with eps = 0.5 at the intermediate review, T = 1
    import synth
    tabs = synth.bigram_tables(8192, small=True)
    B = 2048
    assert_cascade_parity("bench launch", svx, [tabs.target, tabs.draft, tabs.small],
                          np.ones(B, np.float32), tabs.start(B), k1=5, k2=3, rounds=8,
                          lenience="sq", epsilon=0.5, seed=0)
