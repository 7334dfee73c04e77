"""Stage events through the C ABI (specv_verify_profiled and the events
argument of the other entry points): recording them changes no output, every
recorded pair gives a non-negative time, slots left NULL are skipped, and a
stage that shares another's launch (the plan of a uniform batch, the draw when
one workgroup holds a sequence's pass-2 waves) has its pair recorded back to
back. Each stage is timed on the caller's stream.
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


def verify_args(x):
    return dict(max_gamma=x.max_gamma, seed=x.seed, philox_row_offset=x.row_offset)


@pytest.mark.parametrize("name", ["t5xxl_like", "ragged_b256"])
def test_profiled_verify_matches_and_times_stages(svx, name):
    print("[case] profiled verify %s" % name, flush=True)
    x = synth.t5xxl_like(rounds=600) if name == "t5xxl_like" else synth.ragged_b256(batch=16)
    d = svx.from_inputs(x)
    n0, t0 = svx.specv_verify(d["target"], d["draft"], d["draft_tokens"], d["gamma"],
                              d["temperature"], **verify_args(x))
    ev = svx.StageEvents()
    n1, t1 = svx.specv_verify_profiled(d["target"], d["draft"], d["draft_tokens"], d["gamma"],
                                       d["temperature"], ev, **verify_args(x))
    torch.cuda.synchronize()
    assert torch.equal(n0, n1) and torch.equal(t0, t1)
    ms = {s: ev.elapsed_ms(i) for i, s in enumerate(svx.STAGES)}
    print("[events] %s: %s" % (name, {k: round(v, 4) for k, v in ms.items()}), flush=True)
    assert all(v >= 0.0 for v in ms.values())
    assert ms["row_stats"] > 0.0 and ms["accept_and_mass"] > 0.0
    if name == "t5xxl_like":
        # uniform batch: no plan launch; 600 sequences with V = 32128: the draw
        # shares the pass-2 launch. Back-to-back pairs time next to nothing.
        assert ms["plan"] < 0.2 * ms["row_stats"] and ms["draw"] < 0.2 * ms["row_stats"]
    # only some slots recorded: the others are NULL and skipped
    ev1 = svx.StageEvents(stages=(svx.STAGES.index("row_stats"),))
    n2, t2 = svx.specv_verify_profiled(d["target"], d["draft"], d["draft_tokens"], d["gamma"],
                                       d["temperature"], ev1, **verify_args(x))
    torch.cuda.synchronize()
    assert torch.equal(n0, n2) and torch.equal(t0, t2)
    assert ev1.elapsed_ms(svx.STAGES.index("row_stats")) > 0.0


def test_events_change_no_output_elsewhere(svx):
    print("[case] events on decode, cascade, diagnostics", flush=True)
    V, B = 600, 40
    rng = np.random.default_rng(12)
    t = (rng.standard_normal((V, V)) * 1.5).astype(np.float32)
    tabs = [torch.from_numpy(synth.to_bf16_bits(a).view(np.int16)).cuda()
            for a in (t, t + rng.standard_normal((V, V)).astype(np.float32) * 0.6,
                      t + rng.standard_normal((V, V)).astype(np.float32) * 1.4)]
    T = torch.from_numpy(np.where(np.arange(B) % 3 == 0, 0.0, 0.9).astype(np.float32)).cuda()
    start = torch.from_numpy(rng.integers(0, V, B).astype(np.int32)).cuda()
    a = svx.specv_decode_bigram(tabs[0], tabs[1], T, start, gamma=4, rounds=3, seed=2)
    b = svx.specv_decode_bigram(tabs[0], tabs[1], T, start, gamma=4, rounds=3, seed=2,
                                events=svx.StageEvents())
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k
    kw = dict(k1=3, k2=2, rounds=2, lenience="lin", epsilon=0.5, seed=3)
    a = svx.specv_cascade_bigram(*tabs, T, start, **kw)
    b = svx.specv_cascade_bigram(*tabs, T, start, events=svx.StageEvents(), **kw)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k
    x = synth.t5xxl_like(rounds=12)
    d = svx.from_inputs(x)
    a = svx.specv_position_diagnostics(d["target"], d["draft"], d["gamma"], d["temperature"], 16,
                                       max_gamma=x.max_gamma)
    ev = svx.StageEvents()
    b = svx.specv_position_diagnostics(d["target"], d["draft"], d["gamma"], d["temperature"], 16,
                                       max_gamma=x.max_gamma, events=ev)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k
    assert all(ev.elapsed_ms(i) >= 0.0 for i in range(len(svx.STAGES)))
