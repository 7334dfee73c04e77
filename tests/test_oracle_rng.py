"""Pins of the oracle's random numbers.

Philox4x32-10 (Salmon et al., SC'11) is pinned against an independent
implementation: rocRAND's philox4x32_10 engine, built for the host from the
installed ROCm headers and driven through its public seed/subsequence/offset
interface (subsequence feeds counter words 2-3, offset/4 feeds words 0-1).
The uniform conversion U(w) = ((w >> 8) + 1) * 2^-24 is a reading of "U(0, 1)"
in DistillSpec Algorithm A.1 (step 6) and in the Leviathan et al. summary;
it is pinned exhaustively over its 2^24 outputs.
"""
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

import oracle

ROCRAND_PROBE = r"""
#include <rocrand/rocrand_kernel.h>
#include <cstdio>
#include <cstdlib>
int main(int argc, char** argv) {
  FILE* f = fopen(argv[1], "r");
  unsigned long long seed; unsigned c0, c1, c2, c3;
  while (fscanf(f, "%llu %u %u %u %u", &seed, &c0, &c1, &c2, &c3) == 5) {
    unsigned long long sub = (unsigned long long)c2 | ((unsigned long long)c3 << 32);
    unsigned long long off = ((unsigned long long)c0 | ((unsigned long long)c1 << 32)) * 4ull;
    rocrand_device::philox4x32_10_engine e(seed, sub, off);
    uint4 r = e.next4();
    printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def rocrand_probe(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not shutil.which(hipcc) and not __import__("os").path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND host probe")
    d = tmp_path_factory.mktemp("rocrand")
    src = d / "probe.hip"
    src.write_text(ROCRAND_PROBE)
    exe = d / "probe"
    subprocess.run([hipcc, "-O1", "--offload-arch=gfx950", str(src), "-o", str(exe)], check=True,
                   capture_output=True)
    return exe, d


def test_philox_matches_rocrand(rocrand_probe):
    exe, d = rocrand_probe
    rng = np.random.default_rng(1234)
    n = 2000
    seeds = rng.integers(0, 2**63, n, dtype=np.uint64)
    seeds[:3] = [0, 2**64 - 1, 0x243F6A8885A308D3]
    ctr = rng.integers(0, 2**32, (n, 4), dtype=np.uint64).astype(np.uint32)
    ctr[:, 1] &= 0x3FFFFFFF  # keep offset = 4 * (c0 | c1 << 32) inside 64 bits
    ctr[0] = [0, 0, 0, 0]
    ctr[1] = [0xFFFFFFFF, 0x3FFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF]
    inp = d / "in.txt"
    inp.write_text("".join("%d %d %d %d %d\n" % (int(s), *map(int, c)) for s, c in zip(seeds, ctr)))
    out = subprocess.run([str(exe), str(inp)], check=True, capture_output=True, text=True).stdout
    ref = np.array([[int(x) for x in line.split()] for line in out.strip().splitlines()], np.uint64)
    got = np.stack([oracle.philox_blocks(int(s), c[None, :])[0] for s, c in zip(seeds, ctr)])
    np.testing.assert_array_equal(got.astype(np.uint64), ref)


def test_philox_words_uniform():
    # 2^20 blocks of consecutive counters: each of the 4 output words' top
    # byte is uniform over 256 bins (chi-square, 255 dof).
    k = 1 << 20
    ctr = np.zeros((k, 4), np.uint32)
    ctr[:, 0] = np.arange(k, dtype=np.uint32)
    ctr[:, 2] = 7
    w = oracle.philox_blocks(42, ctr)
    for j in range(4):
        counts = np.bincount((w[:, j] >> 24).astype(np.int64), minlength=256)
        p = stats.chisquare(counts).pvalue
        assert p > 1e-4, (j, p)


def test_philox_counter_sensitivity():
    # Every counter word and both key halves change the block.
    base = oracle.philox_blocks(5, np.zeros((1, 4), np.uint32))[0]
    for j in range(4):
        c = np.zeros((1, 4), np.uint32)
        c[0, j] = 1
        assert not np.array_equal(oracle.philox_blocks(5, c)[0], base)
    assert not np.array_equal(oracle.philox_blocks(5 + (1 << 32), np.zeros((1, 4), np.uint32))[0], base)


def test_uniform24_exhaustive():
    k = np.arange(1 << 24, dtype=np.uint32)
    low = np.random.default_rng(0).integers(0, 256, k.size, dtype=np.uint32)
    u = oracle.uniform24((k << np.uint32(8)) | low)
    np.testing.assert_array_equal(u, (k.astype(np.float64) + 1.0) / 2.0**24)
    assert u.min() > 0.0 and u.max() == 1.0
    # exact in fp32: the kernel and the oracle see the same value
    np.testing.assert_array_equal(u.astype(np.float32).astype(np.float64), u)
