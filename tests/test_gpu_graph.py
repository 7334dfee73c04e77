"""The verify step under HIP graph capture (through the C ABI): the call only
enqueues kernels on the caller's stream and allocates nothing, so a captured
graph replays it. Each replay, with new inputs copied into the captured
buffers and eager work and synchronisations in between, must give what an
eager call on the same inputs gives, bit for bit.
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def svx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_sampling_verify_amd as m
    return m


@pytest.mark.parametrize("name", ["t5xxl_like", "ragged_b256"])
def test_graph_replays_match_eager(svx, name):
    print("[case] graph capture %s" % name, flush=True)
    x0 = synth.t5xxl_like(rounds=64) if name == "t5xxl_like" else synth.ragged_b256(batch=12)
    base = svx.from_inputs(x0)
    # four input sets with one layout: the logits rolled along the vocabulary
    # (bf16 bit patterns move as they are), the draft tokens moved with them,
    # and the temperatures changed
    V = x0.vocab
    dev = []
    for i in range(4):
        sh = 7919 * i
        dev.append({"target": torch.roll(base["target"], sh, dims=1).contiguous(),
                    "draft": torch.roll(base["draft"], sh, dims=1).contiguous(),
                    "draft_tokens": ((base["draft_tokens"].long() + sh) % V).to(torch.int32),
                    "gamma": base["gamma"].clone(),
                    "temperature": base["temperature"] * (1.0 + 0.25 * i)})
    static = {k: v.clone() for k, v in base.items()}
    shape = svx._shape_of(static["target"], static["draft"], static["gamma"], x0.max_gamma)
    ws = svx.workspace_for(shape, "cuda")
    out_n = torch.empty(x0.batch, dtype=torch.int32, device="cuda")
    out_next = torch.empty_like(out_n)

    def call(inp, n, nxt, w, stream=None):
        svx.specv_verify(inp["target"], inp["draft"], inp["draft_tokens"], inp["gamma"],
                         inp["temperature"], max_gamma=x0.max_gamma, seed=x0.seed,
                         philox_row_offset=x0.row_offset, out_n=n, out_next=nxt, workspace=w,
                         stream=stream)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(static, out_n, out_next, ws, s)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(static, out_n, out_next, ws, s)
    torch.cuda.synchronize()

    ws_e = svx.workspace_for(shape, "cuda")
    for rep in range(3):
        for i, d in enumerate(dev):
            for k in static:
                static[k].copy_(d[k])
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = (out_n.cpu().numpy().copy(), out_next.cpu().numpy().copy())
            en = torch.empty_like(out_n)
            ex = torch.empty_like(out_n)
            call(d, en, ex, ws_e)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(got[0], en.cpu().numpy(), err_msg="replay %d set %d" % (rep, i))
            np.testing.assert_array_equal(got[1], ex.cpu().numpy(), err_msg="replay %d set %d" % (rep, i))
            assert svx.read_status(ws) == svx.read_status(ws_e)
    print("[graph] %s: 12 replays equal to eager calls" % name, flush=True)
