"""GPU parity of the multi-round bigram decode loop (specv_decode_bigram,
through the C ABI) against the oracle's loop on the same tables, start
tokens, temperatures and Philox stream.

Bar: generated tokens and per-round accepted counts are identical up to the
first round in which the oracle saw a near-tie (a decisive uniform within
1e-6 relative of its threshold, in drafting or in verification); from there
a sequence may follow another path, and such sequences are counted. The
GPU's own output law is also tested against the target Markov chain.
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


def to_bf16_bits(a):
    import synth
    return synth.to_bf16_bits(np.asarray(a, np.float32))


def tables(V, seed, sigma=0.7, scale=1.5):
    rng = np.random.default_rng(seed)
    t = (rng.standard_normal((V, V)) * scale).astype(np.float32)
    d = (t + rng.standard_normal((V, V)) * sigma).astype(np.float32)
    return t, d


def run_gpu(svx, t, d, T, start, gamma, rounds, seed=0, row_offset=0):
    dev = "cuda"
    def tens(a):
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)
    out = svx.specv_decode_bigram(tens(t), tens(d), tens(np.asarray(T, np.float32)),
                                  tens(np.asarray(start, np.int32)), gamma=gamma, rounds=rounds,
                                  seed=seed, philox_row_offset=row_offset)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def assert_decode_parity(name, svx, t, d, T, start, gamma, rounds, seed=0, row_offset=0):
    log("[case] decode %s B=%d V=%d gamma=%d rounds=%d" % (name, len(start), t.shape[0], gamma,
                                                          rounds))
    got = run_gpu(svx, t, d, T, start, gamma, rounds, seed, row_offset)
    want = oracle.decode_bigram(t, d, T, start, gamma=gamma, rounds=rounds, seed=seed,
                                row_offset=row_offset)
    B = len(start)
    diverged = 0
    for b in range(B):
        f = int(want.first_near[b])
        np.testing.assert_array_equal(got["accepted"][b, :f], want.accepted[b, :f], err_msg=str(b))
        if want.length[b] < 0:
            assert got["length"][b] == -1
            continue
        upto = int((want.accepted[b, :f] + 1).sum())
        np.testing.assert_array_equal(got["tokens"][b, :upto], want.tokens[b, :upto],
                                      err_msg=str(b))
        if f == rounds:
            assert got["length"][b] == want.length[b]
            np.testing.assert_array_equal(got["tokens"][b], want.tokens[b])
        else:
            diverged += 1
    log("[parity] decode %s: sequences=%d with a near-tie=%d mean tokens/round=%.4f"
        % (name, B, diverged, float(np.mean(got["accepted"][got["accepted"] >= 0] + 1))))
    # a uniform falls within 1e-6 (relative) of one of the V boundaries of an
    # inverse CDF with probability about 2e-6 * V per draw; with up to
    # rounds * (gamma + 1) draws per sequence that bounds the expected share of
    # sequences with a near-tie; twice that share plus a few is the sanity cap
    expect = min(1.0, 2e-6 * t.shape[0] * rounds * (gamma + 1))
    assert diverged <= 2 * expect * B + 4, (diverged, expect)
    return got, want


def test_decode_parity_fp32(svx):
    t, d = tables(1000, 1)
    B = 256
    rng = np.random.default_rng(2)
    assert_decode_parity("fp32 V=1000", svx, t, d, np.ones(B, np.float32),
                         rng.integers(0, 1000, B), gamma=4, rounds=6, seed=11)


def test_decode_parity_bf16_mixed_greedy(svx):
    t, d = tables(4096, 3, sigma=1.0, scale=2.0)
    B = 128
    T = np.where(np.arange(B) % 2 == 0, 0.8, 0.0).astype(np.float32)
    rng = np.random.default_rng(4)
    assert_decode_parity("bf16 V=4096", svx, to_bf16_bits(t), to_bf16_bits(d), T,
                         rng.integers(0, 4096, B), gamma=5, rounds=5, seed=3, row_offset=1000)


def test_decode_parity_odd_vocab_and_bad_starts(svx):
    # V = 999: rows are not 16-byte multiples (scalar gather and verify paths)
    t, d = tables(999, 5)
    B = 64
    start = np.random.default_rng(6).integers(0, 999, B).astype(np.int32)
    start[3], start[10] = -1, 999
    got, _ = assert_decode_parity("bf16 V=999", svx, to_bf16_bits(t), to_bf16_bits(d),
                                  np.full(B, 1.3, np.float32), start, gamma=3, rounds=4)
    assert got["length"][3] == -1 and got["length"][10] == -1


def test_decode_parity_streamed_rows(svx):
    # V = 9000: rows longer than the 8192 elements a drafting workgroup holds in
    # registers, so each sequence is drafted by one wave that streams its row
    t, d = tables(9000, 8)
    B = 48
    rng = np.random.default_rng(9)
    T = np.where(np.arange(B) % 3 == 0, 0.0, 0.9).astype(np.float32)
    assert_decode_parity("bf16 V=9000", svx, to_bf16_bits(t), to_bf16_bits(d), T,
                         rng.integers(0, 9000, B), gamma=4, rounds=3, seed=21)


BF16_LOWEST = -3.3895313892515355e38  # the most negative finite bf16 (0xff7f)


@pytest.mark.parametrize("kind,dtype", [("lowest_mask", "bf16"), ("lowest_mask", "f32"),
                                        ("tiny_T", "bf16")])
def test_decode_parity_extreme_ranges(svx, kind, dtype):
    # tables whose rows mask half the vocabulary with the dtype's most
    # negative finite value (those tokens are never generated), or T = 1e-30
    # (drafting and verification one-hot at the row maxima)
    V, B = 2048, 64
    t, d = tables(V, 31, sigma=1.0, scale=2.0)
    rng = np.random.default_rng(32)
    T = np.where(np.arange(B) % 4 == 0, 0.0, 1.0).astype(np.float32)
    ok = np.arange(V)
    if kind == "lowest_mask":
        cols = rng.random(V) < 0.5
        low = BF16_LOWEST if dtype == "bf16" else np.finfo(np.float32).min
        t[:, cols] = low
        d[:, cols] = low
        ok = np.flatnonzero(~cols)
    else:
        T = np.where(T > 0, np.float32(1e-30), T).astype(np.float32)
    conv = to_bf16_bits if dtype == "bf16" else (lambda a: a)
    got, want = assert_decode_parity("%s %s" % (kind, dtype), svx, conv(t), conv(d), T,
                                     rng.choice(ok, B), gamma=4, rounds=4, seed=33)
    assert (want.length > 0).all() and (got["length"] > 0).all()
    if kind == "lowest_mask":
        assert np.isin(got["tokens"][got["tokens"] >= 0], ok).all()


def test_decode_gpu_sequence_law(svx):
    # the GPU loop's own output: joint of the first three tokens vs the chain
    t, d = tables(5, 0)
    B, c = 400_000, 2
    got = run_gpu(svx, t, d, np.ones(B, np.float32), np.full(B, c, np.int32), 3, 3, seed=7)
    P = torch.softmax(torch.from_numpy(t.astype(np.float64)), dim=-1).numpy()
    y = got["tokens"][:, :3].astype(np.int64)
    assert (got["length"] >= 3).all()
    obs = np.bincount((y[:, 0] * 5 + y[:, 1]) * 5 + y[:, 2], minlength=125)
    exp = np.einsum("a,ab,bc->abc", P[c], P, P).reshape(-1) * B
    pv = stats.chisquare(obs, exp).pvalue
    log("[law] decode GPU joint of 3 tokens: p = %.4g" % pv)
    assert pv > 1e-4


def random_decode_case(seed):
    """A seeded random decode problem: V (aligned or not, from 1 up to past
    the 8192 elements a drafting workgroup holds), dtype, batch, gamma 0..8,
    rounds, greedy and sampling temperatures with an occasional NaN one, and
    an occasional start token outside [0, V)."""
    rng = np.random.default_rng(5000 + seed)
    V = int(rng.choice([1, 2, 5, 63, 64, 65, 255, 1000, 2048, 2050, 8192, 8200,
                        int(rng.integers(2, 2500))]))
    B = int(rng.integers(1, 80 if V <= 2500 else 24))
    gamma = int(rng.integers(0, 9))
    rounds = int(rng.integers(1, 5))
    t, d = tables(V, 6000 + seed, sigma=float(rng.choice([0.1, 0.7, 2.0])),
                  scale=float(rng.choice([0.5, 1.5, 3.0])))
    if rng.random() < 0.5:
        t, d = to_bf16_bits(t), to_bf16_bits(d)
    T = np.where(rng.random(B) < 0.3, 0.0, rng.uniform(0.3, 2.0, B)).astype(np.float32)
    T[rng.random(B) < 0.03] = np.nan
    start = rng.integers(0, V, B).astype(np.int32)
    bad = rng.random(B) < 0.03
    start[bad] = np.where(rng.random(int(bad.sum())) < 0.5, -1, V)
    return t, d, T, start, gamma, rounds, int(rng.integers(0, 2**63)), int(rng.integers(0, 2**40))


@pytest.mark.parametrize("seed", range(16))
def test_decode_random_shapes(svx, seed):
    t, d, T, start, gamma, rounds, s, off = random_decode_case(seed)
    got, want = assert_decode_parity("random %d %s" % (seed, "bf16" if t.dtype == np.uint16 else
                                                       "fp32"), svx, t, d, T, start, gamma,
                                     rounds, seed=s, row_offset=off)
    failed = np.isnan(T) | (start < 0) | (start >= t.shape[0])
    assert (got["length"][failed] == -1).all()


def test_decode_bench_launch_full_size(svx):
    # the launch the decode benchmark times: the benchmark's bigram tables
    # (V = 8192, bf16), 2048 sequences, gamma = 5, 8 rounds, T = 1
    import synth
    tabs = synth.bigram_tables(8192)
    B = 2048
    assert_decode_parity("bench launch", svx, tabs.target, tabs.draft, np.ones(B, np.float32),
                         tabs.start(B), gamma=5, rounds=8, seed=0)
