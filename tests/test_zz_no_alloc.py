"""specv_verify_noalloc, the entry point for callers that cannot allocate
(HIP graph capture, tight serving loops, harnesses that forbid hipMalloc),
called through the C ABI and checked against specv_verify: the same kernels
on the library's static scratch instead of a caller workspace, so outcomes
and status words must agree bit for bit, over calls in a row on the shared
array (the second call smaller than the first)."""
import numpy as np
import pytest
import torch

import synth
from helpers import pack

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def svx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_sampling_verify_amd as m
    return m


def both(svx, x):
    d = svx.from_inputs(x)
    ws = svx.workspace_for(svx._shape_of(d["target"], d["draft"], d["gamma"], x.max_gamma), "cuda")
    ref = svx.specv_verify(d["target"], d["draft"], d["draft_tokens"], d["gamma"], d["temperature"],
                           max_gamma=x.max_gamma, seed=x.seed, philox_row_offset=x.row_offset,
                           workspace=ws)
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    got = svx.specv_verify_noalloc(d["target"], d["draft"], d["draft_tokens"], d["gamma"],
                                   d["temperature"], max_gamma=x.max_gamma, seed=x.seed,
                                   philox_row_offset=x.row_offset, out_status=status)
    torch.cuda.synchronize()
    return ([t.cpu().numpy() for t in ref], svx.read_status(ws),
            [t.cpu().numpy() for t in got], int(status.item()))


def check(name, svx, x):
    (rn, rt), rs, (n, t), s = both(svx, x)
    print("[noalloc] %s: B=%d V=%d %s status=%d" % (name, x.batch, x.vocab, x.dtype, s), flush=True)
    np.testing.assert_array_equal(n, rn)
    np.testing.assert_array_equal(t, rt)
    assert s == rs
    return n, t, s


def test_noalloc_equals_verify_on_calls_in_a_row(svx):
    # a uniform batch (no plan launch), then a smaller ragged one (plan launch),
    # then the first again: each call's outcome matches specv_verify's
    a = synth.t5xxl_like(rounds=400)
    b = synth.ragged_b256(batch=24)
    assert b.total_target_rows * b.vocab * 2 < a.total_target_rows * a.vocab * 2 * 2
    check("t5xxl_like 400 rounds", svx, a)
    check("ragged 24 sequences", svx, b)
    check("t5xxl_like 400 rounds, again", svx, a)


def test_noalloc_smaller_second_call_and_status(svx):
    # fp32 large vocab with greedy rows, then a small batch with data errors:
    # the status word of the second call is its own (no bits left over)
    check("large_vocab 12 sequences", svx, synth.large_vocab(batch=12))
    V = 64
    rng = np.random.default_rng(4)
    t = rng.standard_normal((3, V)).astype(np.float32)
    dr = rng.standard_normal((2, V)).astype(np.float32)
    bad = t.copy()
    bad[1, 5] = np.nan
    seqs = [{"target": t, "draft": dr, "tokens": [1, 2], "T": 1.0},
            {"target": bad, "draft": dr, "tokens": [1, 2], "T": 1.0},
            {"target": t, "draft": dr, "tokens": [3, 4], "T": 0.0}]
    n, _, s = check("small batch with a NaN row", svx, pack(seqs, V))
    assert n[1] == -1 and n[0] >= 0 and n[2] >= 0
    assert s == svx.SPECV_DEV_SEQ_ERROR
    check("t5xxl_like 8 rounds", svx, synth.t5xxl_like(rounds=8))


def test_noalloc_short_rows(svx):
    # rows of one tile (two per pass-1 wave) and one-wave draws from the
    # weights in LDS, sampling and then greedy, the second call smaller
    check("tiny_cpu 3000 rounds", svx, synth.tiny_cpu(rounds=3000))
    check("tiny_cpu 500 rounds greedy", svx, synth.tiny_cpu(rounds=500, greedy=True))


def test_noalloc_rejects_shapes_beyond_its_scratch(svx):
    # 2^20 sequences of gamma 7 need far more than the static scratch: the call
    # is refused before anything is enqueued (no tensor is read)
    B, g, V = 1 << 20, 7, 2
    shape = svx.make_shape(B, V, g, svx.SPECV_F32, B * (g + 1), B * g)
    assert svx.specv_workspace_bytes(shape) > svx.SPECV_NOALLOC_SCRATCH_BYTES
    import ctypes
    fake = ctypes.c_void_p(0x100000)
    st = svx._lib.specv_verify_noalloc(ctypes.byref(shape), fake, fake, fake, fake, fake, 0, 0, fake,
                                       fake, None, None)
    assert st == svx.SPECV_ERR_SCRATCH_LIMIT
    assert "scratch" in svx.specv_status_string(st)


def test_noalloc_empty_batch(svx):
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    n, t = svx.specv_verify_noalloc(torch.zeros((0, 16), device="cuda"), None, None,
                                    torch.zeros(0, dtype=torch.int32, device="cuda"),
                                    torch.zeros(0, device="cuda"), max_gamma=0, out_status=status)
    torch.cuda.synchronize()
    assert n.numel() == 0 and t.numel() == 0 and int(status.item()) == 0
