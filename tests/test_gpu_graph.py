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


def _replay_check(name, capture, eager, inputs, static):
    """Capture capture() on a side stream, then for every input set copy it
    into the static buffers, replay, and compare the outputs with eager()
    on the same set (three passes over the sets, eager work and
    synchronisations in between)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        capture(s)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        out = capture(s)
    torch.cuda.synchronize()
    n = 0
    for rep in range(3):
        for i, d in enumerate(inputs):
            for k in static:
                static[k].copy_(d[k])
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = {k: v.cpu().numpy().copy() for k, v in out.items()}
            want = eager(d)
            torch.cuda.synchronize()
            for k in got:
                np.testing.assert_array_equal(got[k], want[k].cpu().numpy(),
                                              err_msg="%s replay %d set %d" % (k, rep, i))
            n += 1
    print("[graph] %s: %d replays equal to eager calls" % (name, n), flush=True)


def test_graph_decode_loop(svx):
    # a whole multi-round decode call (drafting, gather, verify, append per
    # round) captured once; new start tokens and temperatures per replay
    print("[case] graph capture decode loop", flush=True)
    V, B, g, R = 1000, 64, 4, 3
    rng = np.random.default_rng(3)
    t = synth.to_bf16_bits((rng.standard_normal((V, V)) * 1.5).astype(np.float32))
    d = synth.to_bf16_bits((synth.bf16_bits_to_f32(t) + rng.standard_normal((V, V))).astype(np.float32))
    tt = torch.from_numpy(t.view(np.int16)).cuda()
    dt = torch.from_numpy(d.view(np.int16)).cuda()
    inputs = [{"T": torch.from_numpy(np.where(np.arange(B) % 3 == 0, 0.0, 0.6 + 0.3 * i)
                                      .astype(np.float32)).cuda(),
               "start": torch.from_numpy(rng.integers(0, V, B).astype(np.int32)).cuda()}
              for i in range(3)]
    static = {k: v.clone() for k, v in inputs[0].items()}
    shape = svx.SpecvDecodeShape(B, V, g, R, svx.SPECV_BF16)
    ws = torch.empty(svx.specv_decode_workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    out = {"tokens": torch.empty((B, R * (g + 1)), dtype=torch.int32, device="cuda"),
           "length": torch.empty(B, dtype=torch.int32, device="cuda"),
           "accepted": torch.empty((B, R), dtype=torch.int32, device="cuda")}

    def capture(stream):
        return svx.specv_decode_bigram(tt, dt, static["T"], static["start"], gamma=g, rounds=R,
                                       seed=5, out=out, workspace=ws, stream=stream)

    def eager(inp):
        return svx.specv_decode_bigram(tt, dt, inp["T"], inp["start"], gamma=g, rounds=R, seed=5)

    _replay_check("decode loop", capture, eager, inputs, static)


def test_graph_diagnostics(svx):
    print("[case] graph capture diagnostics", flush=True)
    x0 = synth.t5xxl_like(rounds=24)
    base = svx.from_inputs(x0)
    inputs = [{"target": torch.roll(base["target"], 7919 * i, dims=1).contiguous(),
               "draft": torch.roll(base["draft"], 7919 * i, dims=1).contiguous(),
               "temperature": base["temperature"] * (1.0 + 0.25 * i)} for i in range(3)]
    static = {k: v.clone() for k, v in inputs[0].items()}
    k = 16
    shape = svx._shape_of(static["target"], static["draft"], base["gamma"], x0.max_gamma)
    ws = torch.empty(svx.specv_diagnostics_workspace_bytes(shape, k), dtype=torch.uint8,
                     device="cuda")
    td = x0.total_draft_rows
    out = {"alpha": torch.empty(td, dtype=torch.float64, device="cuda"),
           "entropy": torch.empty(td, dtype=torch.float64, device="cuda"),
           "topk_index": torch.empty((td, k), dtype=torch.int32, device="cuda"),
           "topk_prob": torch.empty((td, k), dtype=torch.float64, device="cuda")}

    def capture(stream):
        return svx.specv_position_diagnostics(static["target"], static["draft"], base["gamma"],
                                              static["temperature"], k, max_gamma=x0.max_gamma,
                                              out=out, workspace=ws, stream=stream)

    def eager(inp):
        return svx.specv_position_diagnostics(inp["target"], inp["draft"], base["gamma"],
                                              inp["temperature"], k, max_gamma=x0.max_gamma)

    _replay_check("diagnostics", capture, eager, inputs, static)


def test_graph_cascade(svx):
    # a whole vertical-cascade call (inner drafting and lenient reviews, the
    # target review's row builder and lossless review) captured once
    print("[case] graph capture cascade", flush=True)
    V, B = 700, 48
    rng = np.random.default_rng(4)
    t = (rng.standard_normal((V, V)) * 1.5).astype(np.float32)
    tabs = [torch.from_numpy(synth.to_bf16_bits(a).view(np.int16)).cuda()
            for a in (t, t + rng.standard_normal((V, V)).astype(np.float32) * 0.6,
                      t + rng.standard_normal((V, V)).astype(np.float32) * 1.4)]
    inputs = [{"T": torch.from_numpy(np.where(np.arange(B) % 4 == 0, 0.0, 0.7 + 0.3 * i)
                                      .astype(np.float32)).cuda(),
               "start": torch.from_numpy(rng.integers(0, V, B).astype(np.int32)).cuda()}
              for i in range(3)]
    static = {k: v.clone() for k, v in inputs[0].items()}
    k1, k2, R = 3, 2, 2
    shape = svx.SpecvCascadeShape(B, V, k1, k2, R, svx.SPECV_BF16)
    ws = torch.empty(svx.specv_cascade_workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    out = {"tokens": torch.empty((B, R * (k1 + 1)), dtype=torch.int32, device="cuda"),
           "length": torch.empty(B, dtype=torch.int32, device="cuda"),
           "accepted": torch.empty((B, R), dtype=torch.int32, device="cuda")}
    kw = dict(k1=k1, k2=k2, rounds=R, lenience="sq", epsilon=0.5, seed=9)

    def capture(stream):
        return svx.specv_cascade_bigram(*tabs, static["T"], static["start"], out=out,
                                        workspace=ws, stream=stream, **kw)

    def eager(inp):
        return svx.specv_cascade_bigram(*tabs, inp["T"], inp["start"], **kw)

    _replay_check("cascade", capture, eager, inputs, static)
