"""The C ABI without a GPU: every declared symbol is exported, and argument
errors are reported before anything is enqueued (no HIP call is made on these
paths, so they run on a CPU-only host)."""
import ctypes
import re
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "specverify.h"

svx = pytest.importorskip("speculative_sampling_verify_amd",
                          reason="libspecverify.so not built (run __graft_entry__.build())")
OK, INVALID, WORKSPACE = 0, 1, 2
FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: validation fails first


def declared():
    text = HEADER.read_text()
    return sorted(set(re.findall(r"\b(specv_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared()
    assert "specv_verify" in names and "specv_workspace_bytes" in names
    out = subprocess.run(["nm", "-D", "--defined-only", str(svx.LIBRARY)], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (specv_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert set(svx.EXPORTED) == set(names)


def shape(B=4, V=1000, g=3, dt=1, tt=None, td=None):
    td = B * g if td is None else td
    tt = td + B if tt is None else tt
    return svx.make_shape(B, V, g, dt, tt, td)


def test_noalloc_scratch_limit_before_any_hip_call():
    # the no-allocation entry point refuses a shape whose workspace exceeds its
    # static scratch before it looks anything up (no GPU needed)
    B, g = 1 << 20, 7
    big = svx.make_shape(B, 2, g, 0, B * (g + 1), B * g)
    assert svx.specv_workspace_bytes(big) > svx.SPECV_NOALLOC_SCRATCH_BYTES
    st = svx._lib.specv_verify_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0, FAKE,
                                       FAKE, None, None)
    assert st == 5
    bad = svx.make_shape(4, 0, 1, 0, 8, 4)  # V = 0
    assert svx._lib.specv_verify_noalloc(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0, FAKE,
                                         FAKE, None, None) == INVALID


def test_workspace_bytes():
    assert svx.specv_workspace_bytes(shape()) >= 256
    assert svx.specv_workspace_bytes(shape(B=0, td=0)) >= 256
    for bad in [shape(tt=5), shape(g=64, td=4), shape(V=0), shape(dt=7), shape(td=13, tt=17),
                svx.make_shape(-1, 10, 1, 0, 0, 0)]:
        assert svx.specv_workspace_bytes(bad) == 0
    a = svx.specv_workspace_bytes(shape(B=64, V=128256, g=7))
    b = svx.specv_workspace_bytes(shape(B=128, V=128256, g=7))
    assert 0 < a < b
    # row totals: at most 2^29 target rows (launch grids), rows * V at most 2^40
    B = (1 << 29) // 8
    assert svx.specv_workspace_bytes(shape(B=B, V=1, g=7)) > 0
    assert svx.specv_workspace_bytes(shape(B=B + 1, V=1, g=7)) == 0
    assert svx.specv_workspace_bytes(shape(B=1 << 20, V=1 << 20, g=0)) > 0
    assert svx.specv_workspace_bytes(shape(B=(1 << 20) + 1, V=1 << 20, g=0)) == 0
    assert svx.specv_decode_workspace_bytes(svx.SpecvDecodeShape(B + 1, 2, 7, 1, 1)) == 0
    assert svx.specv_cascade_workspace_bytes(svx.SpecvCascadeShape(B + 1, 2, 7, 1, 1, 1)) == 0


def call_verify(shp, ws=FAKE, ws_bytes=1 << 30, target=FAKE, draft=FAKE, out=FAKE):
    lib = svx._lib
    return lib.specv_verify(ctypes.byref(shp), target, draft, FAKE, FAKE, FAKE, 0, 0, out, out,
                            ws, ws_bytes, None)


def test_verify_argument_errors():
    lib = svx._lib
    assert lib.specv_verify(None, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0, FAKE, FAKE, FAKE, 1 << 30,
                            None) == INVALID
    assert call_verify(shape(tt=5)) == INVALID
    assert call_verify(shape(g=64, td=4)) == INVALID
    assert call_verify(shape(), target=None) == INVALID
    assert call_verify(shape(), draft=None) == INVALID
    assert call_verify(shape(), out=None) == INVALID
    assert call_verify(shape(), target=ctypes.c_void_p(0x100001)) == INVALID  # misaligned bf16
    assert call_verify(shape(), ws=None) == WORKSPACE
    assert call_verify(shape(), ws_bytes=100) == WORKSPACE
    assert call_verify(shape(), ws=ctypes.c_void_p(0x100010)) == WORKSPACE  # not 256-aligned
    assert call_verify(shape(B=0, td=0)) == OK  # nothing to do, nothing enqueued


def test_other_entry_points_validate():
    lib = svx._lib
    assert lib.specv_philox4x32_10(0, FAKE, FAKE, -1, None) == INVALID
    assert lib.specv_philox4x32_10(0, None, None, 0, None) == OK
    assert lib.specv_copy_bytes(FAKE, FAKE, 15, None) == INVALID
    assert lib.specv_copy_bytes(FAKE, FAKE, 0, None) == OK
    assert lib.specv_read_bytes(FAKE, 65536 + 16, FAKE, None) == INVALID  # not whole segments
    assert lib.specv_read_bytes(None, 65536, FAKE, None) == INVALID
    assert lib.specv_read_bytes(FAKE, 65536, None, None) == INVALID
    assert lib.specv_read_bytes(None, 0, None, None) == OK
    shp = shape()
    assert lib.specv_softmax_rows(ctypes.byref(shp), FAKE, FAKE, FAKE, FAKE, FAKE, -1, FAKE, FAKE,
                                  1 << 30, None) == INVALID
    assert lib.specv_row_stats(ctypes.byref(shp), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE,
                               FAKE, FAKE, FAKE, 1 << 30, None) == INVALID
    assert lib.specv_verify_with_uniforms(ctypes.byref(shp), FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                          FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == INVALID


def test_status_strings():
    for code in range(5):
        assert svx.specv_status_string(code)
    assert svx.specv_status_string(99) == "unknown status"


def shape_valid(B, V, mg, dt, tt, td):
    """The documented shape rules of specverify.h."""
    return (B >= 0 and V >= 1 and 0 <= mg <= 63 and dt in (0, 1) and td >= 0 and tt >= 0
            and tt == td + B and td <= B * mg and tt <= (1 << 29) and tt * V <= (1 << 40))


def test_shape_rules_property():
    # random descriptors, extremes included: the workspace query is nonzero exactly
    # for the shapes the header allows, and the verify call rejects every other one
    # before anything is enqueued (the fake pointers are never touched)
    hyp = pytest.importorskip("hypothesis")
    st = pytest.importorskip("hypothesis.strategies")
    i32 = st.one_of(st.integers(-3, 70), st.integers(-(1 << 31), (1 << 31) - 1))
    i64 = st.one_of(st.integers(-3, 300), st.integers(0, 1 << 41), st.integers(-(1 << 63), (1 << 63) - 1))

    @hyp.settings(max_examples=3000, deadline=None, derandomize=True)
    @hyp.given(B=i32, V=i32, mg=i32, dt=st.integers(-2, 3), td=i64, extra=st.integers(-2, 2),
               exact=st.booleans())
    def check(B, V, mg, dt, td, extra, exact):
        tt = td + B if exact else td + B + extra
        tt = max(-(1 << 63), min(tt, (1 << 63) - 1))
        shp = svx.make_shape(B, V, mg, dt, tt, td)
        n = svx.specv_workspace_bytes(shp)
        if shape_valid(B, V, mg, dt, tt, td):
            assert n >= 256
        else:
            assert n == 0
            assert call_verify(shp) == INVALID

    check()


def test_decode_and_cascade_shape_rules_property():
    hyp = pytest.importorskip("hypothesis")
    st = pytest.importorskip("hypothesis.strategies")
    i32 = st.one_of(st.integers(-3, 70), st.integers(-(1 << 31), (1 << 31) - 1))

    @hyp.settings(max_examples=2000, deadline=None, derandomize=True)
    @hyp.given(B=i32, V=i32, g=i32, k2=i32, R=i32, dt=st.integers(-1, 2))
    def check(B, V, g, k2, R, dt):
        nd = svx.specv_decode_workspace_bytes(svx.SpecvDecodeShape(B, V, g, R, dt))
        ok = (B >= 0 and V >= 1 and 0 <= g <= 63 and R >= 0 and dt in (0, 1) and V * V <= (1 << 40)
              and B * R * (g + 1) <= (1 << 40) and B * (g + 1) <= (1 << 29)
              and B * (g + 1) * V <= (1 << 40))
        assert (nd > 0) == ok, (B, V, g, R, dt, nd)
        nc = svx.specv_cascade_workspace_bytes(svx.SpecvCascadeShape(B, V, g, k2, R, dt))
        okc = (B >= 0 and V >= 1 and 0 <= g <= 63 and 0 <= k2 <= 63 and R >= 0 and dt in (0, 1)
               and V * V <= (1 << 40) and B * R * (g + 1) <= (1 << 40)
               and max(B * (g + 1), B * (k2 + 1)) <= (1 << 29)
               and max(B * (g + 1), B * (k2 + 1)) * V <= (1 << 40))
        assert (nc > 0) == okc, (B, V, g, k2, R, dt, nc)

    check()
