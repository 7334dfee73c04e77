"""The calibration kernels through the C ABI: the copy behind the
memory-counter scale factors and the bandwidth figures, and the read probe
(pass 1's access pattern, read only). Both must move exactly the bytes they
are given: the copy reproduces its source, and the probe's per-wave XOR
checksums equal the ones computed on the host from its documented tiling
(wave 2s + h of 64 KiB segment s reads the 4 KiB tiles h, h + 2, ..., h + 14).
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def svx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_sampling_verify_amd as m
    return m


@pytest.mark.parametrize("nbytes", [48, 3 * 65536 + 48, 4096 * 65536])
def test_copy_bytes_exact(svx, nbytes):
    # whole 64 KiB segments take the tiled copy, a shorter tail the grid-stride one
    print("[case] copy %d bytes" % nbytes, flush=True)
    rng = np.random.default_rng(1)
    src = rng.integers(0, 256, nbytes, dtype=np.uint8)
    s = torch.from_numpy(src).cuda()
    d = torch.zeros_like(s)
    svx.specv_copy_bytes(d, s)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(d.cpu().numpy(), src)


@pytest.mark.parametrize("segments", [1, 7, 4096])
def test_read_probe_checksums(svx, segments):
    print("[case] read probe, %d segments" % segments, flush=True)
    rng = np.random.default_rng(segments)
    words = rng.integers(0, 2 ** 32, segments * 16384, dtype=np.uint64).astype(np.uint32)
    s = torch.from_numpy(words.view(np.int32)).cuda()
    sink = svx.specv_read_bytes(s)
    torch.cuda.synchronize()
    tiles = words.reshape(segments, 16, 1024)  # 4 KiB tiles of 1024 dwords
    want = np.empty((segments, 2), np.uint32)
    for h in (0, 1):
        want[:, h] = np.bitwise_xor.reduce(tiles[:, h::2, :].reshape(segments, -1), axis=1)
    np.testing.assert_array_equal(sink.cpu().numpy().view(np.uint32), want.reshape(-1))
