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
