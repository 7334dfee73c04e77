"""Python binding of libspecverify (the speculative-sampling verify step on MI355X).

Argument marshalling only: every step of the verify path runs in the HIP
kernels of ``libspecverify.so``; torch provides device memory and the stream.
Function names follow the C ABI in ``include/specverify.h``. If the library
is not built, importing this package raises instead of falling back.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

import torch

_HERE = Path(__file__).resolve().parent
LIBRARY = _HERE / "libspecverify.so"

SPECV_F32, SPECV_BF16 = 0, 1
SPECV_MAX_GAMMA = 63
SPECV_DEV_SEQ_ERROR = 1
SPECV_DEV_LAYOUT_ERROR = 2
SPECV_ERR_SCRATCH_LIMIT = 5
SPECV_NOALLOC_SCRATCH_BYTES = 16 << 20
STAGES = ("plan", "row_stats", "accept_and_mass", "draw")
LENIENCE = {"none": 0, "lin": 1, "sq": 2, "exp": 3}

if not LIBRARY.exists():
    raise ImportError("libspecverify.so is not built (run __graft_entry__.build() or "
                      "python -m speculative_sampling_verify_amd.build)")

_lib = ctypes.CDLL(str(LIBRARY))


class SpecvShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("max_gamma", ctypes.c_int32), ("dtype", ctypes.c_int),
                ("total_target_rows", ctypes.c_int64), ("total_draft_rows", ctypes.c_int64)]


class SpecvDecodeShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("vocab", ctypes.c_int32), ("gamma", ctypes.c_int32),
                ("rounds", ctypes.c_int32), ("dtype", ctypes.c_int)]


class SpecvCascadeShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("vocab", ctypes.c_int32), ("k1", ctypes.c_int32),
                ("k2", ctypes.c_int32), ("rounds", ctypes.c_int32), ("dtype", ctypes.c_int)]


_P = ctypes.c_void_p
_SHP = ctypes.POINTER(SpecvShape)
_DSHP = ctypes.POINTER(SpecvDecodeShape)
_u64, _i64, _sz = ctypes.c_uint64, ctypes.c_int64, ctypes.c_size_t
_lib.specv_workspace_bytes.restype = _sz
_lib.specv_workspace_bytes.argtypes = [_SHP]
_lib.specv_verify.restype = ctypes.c_int
_lib.specv_verify.argtypes = [_SHP, _P, _P, _P, _P, _P, _u64, _u64, _P, _P, _P, _sz, _P]
_lib.specv_verify_noalloc.restype = ctypes.c_int
_lib.specv_verify_noalloc.argtypes = [_SHP, _P, _P, _P, _P, _P, _u64, _u64, _P, _P, _P, _P]
_lib.specv_verify_profiled.restype = ctypes.c_int
_lib.specv_verify_profiled.argtypes = [_SHP, _P, _P, _P, _P, _P, _u64, _u64, _P, _P, _P, _sz, _P, _P]
_lib.specv_verify_with_uniforms.restype = ctypes.c_int
_lib.specv_verify_with_uniforms.argtypes = [_SHP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _sz, _P]
_lib.specv_verify_lenient.restype = ctypes.c_int
_lib.specv_verify_lenient.argtypes = [_SHP, _P, _P, _P, _P, _P, ctypes.c_int, ctypes.c_float, _u64,
                                      _u64, _P, _P, _P, _P, _P, _sz, _P, _P]
_lib.specv_diagnostics_workspace_bytes.restype = _sz
_lib.specv_diagnostics_workspace_bytes.argtypes = [_SHP, ctypes.c_int32]
_lib.specv_position_diagnostics.restype = ctypes.c_int
_lib.specv_position_diagnostics.argtypes = [_SHP, _P, _P, _P, _P, ctypes.c_int32, _P, _P, _P, _P, _P,
                                            _sz, _P, _P]
_lib.specv_decode_workspace_bytes.restype = _sz
_lib.specv_decode_workspace_bytes.argtypes = [_DSHP]
_lib.specv_decode_bigram.restype = ctypes.c_int
_lib.specv_decode_bigram.argtypes = [_DSHP, _P, _P, _P, _P, _u64, _u64, _P, _P, _P, _P, _sz, _P, _P]
_CSHP = ctypes.POINTER(SpecvCascadeShape)
_lib.specv_cascade_workspace_bytes.restype = _sz
_lib.specv_cascade_workspace_bytes.argtypes = [_CSHP]
_lib.specv_cascade_bigram.restype = ctypes.c_int
_lib.specv_cascade_bigram.argtypes = [_CSHP, _P, _P, _P, _P, _P, ctypes.c_int, ctypes.c_float, _u64,
                                      _u64, _P, _P, _P, _P, _sz, _P, _P]
_lib.specv_row_stats.restype = ctypes.c_int
_lib.specv_row_stats.argtypes = [_SHP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _sz, _P]
_lib.specv_softmax_rows.restype = ctypes.c_int
_lib.specv_softmax_rows.argtypes = [_SHP, _P, _P, _P, _P, _P, _i64, _P, _P, _sz, _P]
_lib.specv_philox4x32_10.restype = ctypes.c_int
_lib.specv_philox4x32_10.argtypes = [_u64, _P, _P, _i64, _P]
_lib.specv_copy_bytes.restype = ctypes.c_int
_lib.specv_copy_bytes.argtypes = [_P, _P, _sz, _P]
_lib.specv_read_bytes.restype = ctypes.c_int
_lib.specv_read_bytes.argtypes = [_P, _sz, _P, _P]
_lib.specv_status_string.restype = ctypes.c_char_p
_lib.specv_status_string.argtypes = [ctypes.c_int]

EXPORTED = ("specv_workspace_bytes", "specv_verify", "specv_verify_noalloc", "specv_verify_profiled",
            "specv_verify_with_uniforms", "specv_verify_lenient",
            "specv_diagnostics_workspace_bytes", "specv_position_diagnostics",
            "specv_decode_workspace_bytes", "specv_decode_bigram",
            "specv_cascade_workspace_bytes", "specv_cascade_bigram", "specv_row_stats", "specv_softmax_rows",
            "specv_philox4x32_10", "specv_copy_bytes", "specv_read_bytes", "specv_status_string")


class SpecvError(RuntimeError):
    pass


def specv_status_string(status: int) -> str:
    return _lib.specv_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != 0:
        raise SpecvError("%s: %s (status %d)" % (what, specv_status_string(status), status))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return SPECV_BF16
    if t.dtype == torch.float32:
        return SPECV_F32
    raise TypeError("logits must be bfloat16 (or its 16-bit pattern) or float32, got %s" % t.dtype)


def make_shape(batch, vocab, max_gamma, dtype, total_target_rows, total_draft_rows) -> SpecvShape:
    return SpecvShape(int(batch), int(vocab), int(max_gamma), int(dtype), int(total_target_rows),
                      int(total_draft_rows))


def specv_workspace_bytes(shape: SpecvShape) -> int:
    return int(_lib.specv_workspace_bytes(ctypes.byref(shape)))


def _shape_of(target, draft, gamma, max_gamma) -> SpecvShape:
    if target.dim() != 2:
        raise ValueError("target logits must be [rows, V]")
    V = target.shape[1]
    td = draft.shape[0] if draft is not None and draft.dim() == 2 else 0
    return make_shape(gamma.shape[0], V, max_gamma, _dtype_code(target), target.shape[0], td)


def _check_tensors(device, **tensors):
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda or t.device != device:
            raise ValueError("%s must be on %s" % (name, device))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)


def workspace_for(shape: SpecvShape, device) -> torch.Tensor:
    n = specv_workspace_bytes(shape)
    if n == 0:
        raise SpecvError("invalid shape")
    return torch.empty(n, dtype=torch.uint8, device=device)


def read_status(workspace: torch.Tensor) -> int:
    """Device status word (valid after the stream has finished the call)."""
    return int(workspace[:4].view(torch.int32).item())


def _common(target, draft, tokens, gamma, temperature, max_gamma, out_n, out_next, workspace):
    device = target.device
    gamma = gamma if gamma.dtype == torch.int32 else gamma.to(torch.int32)
    if draft is None:
        draft = target[:0]
    if tokens is None:
        tokens = torch.empty(0, dtype=torch.int32, device=device)
    if max_gamma is None:
        max_gamma = int(gamma.max().item()) if gamma.numel() else 0
    shape = _shape_of(target, draft, gamma, max_gamma)
    if out_n is None:
        out_n = torch.empty(gamma.shape[0], dtype=torch.int32, device=device)
    if out_next is None:
        out_next = torch.empty(gamma.shape[0], dtype=torch.int32, device=device)
    if workspace is None:
        workspace = workspace_for(shape, device)
    _check_tensors(device, target=target, draft=draft, tokens=tokens, gamma=gamma,
                   temperature=temperature, out_n=out_n, out_next=out_next, workspace=workspace)
    return shape, draft, tokens, gamma, out_n, out_next, workspace


def specv_verify(target, draft, draft_tokens, gamma, temperature, *, max_gamma=None, seed=0,
                 philox_row_offset=0, out_n=None, out_next=None, workspace=None, stream=None):
    """Verify step for a packed batch; returns (n_accepted, next_token), int32 [B]."""
    shape, draft, draft_tokens, gamma, out_n, out_next, workspace = _common(
        target, draft, draft_tokens, gamma, temperature, max_gamma, out_n, out_next, workspace)
    st = _lib.specv_verify(ctypes.byref(shape), _ptr(target), _ptr(draft), _ptr(draft_tokens),
                           _ptr(gamma), _ptr(temperature), int(seed), int(philox_row_offset),
                           _ptr(out_n), _ptr(out_next), _ptr(workspace), workspace.numel(),
                           _stream(stream, target.device))
    _check(st, "specv_verify")
    return out_n, out_next


def specv_verify_noalloc(target, draft, draft_tokens, gamma, temperature, *, max_gamma=None,
                         seed=0, philox_row_offset=0, out_n=None, out_next=None, out_status=None,
                         stream=None):
    """specv_verify with the library's static scratch instead of a workspace
    (allocates nothing itself when the outputs are given); ``out_status`` is
    an optional int32 [1] device tensor receiving the status word."""
    device = target.device
    gamma = gamma if gamma.dtype == torch.int32 else gamma.to(torch.int32)
    if draft is None:
        draft = target[:0]
    if draft_tokens is None:
        draft_tokens = torch.empty(0, dtype=torch.int32, device=device)
    if max_gamma is None:
        max_gamma = int(gamma.max().item()) if gamma.numel() else 0
    shape = _shape_of(target, draft, gamma, max_gamma)
    if out_n is None:
        out_n = torch.empty(gamma.shape[0], dtype=torch.int32, device=device)
    if out_next is None:
        out_next = torch.empty(gamma.shape[0], dtype=torch.int32, device=device)
    _check_tensors(device, target=target, draft=draft, tokens=draft_tokens, gamma=gamma,
                   temperature=temperature, out_n=out_n, out_next=out_next, out_status=out_status)
    st = _lib.specv_verify_noalloc(ctypes.byref(shape), _ptr(target), _ptr(draft),
                                   _ptr(draft_tokens), _ptr(gamma), _ptr(temperature), int(seed),
                                   int(philox_row_offset), _ptr(out_n), _ptr(out_next),
                                   _ptr(out_status), _stream(stream, device))
    _check(st, "specv_verify_noalloc")
    return out_n, out_next


def specv_verify_profiled(target, draft, draft_tokens, gamma, temperature, events, *,
                          max_gamma=None, seed=0, philox_row_offset=0, out_n=None, out_next=None,
                          workspace=None, stream=None):
    """specv_verify recording events[2s] / events[2s+1] around stage s."""
    shape, draft, draft_tokens, gamma, out_n, out_next, workspace = _common(
        target, draft, draft_tokens, gamma, temperature, max_gamma, out_n, out_next, workspace)
    st = _lib.specv_verify_profiled(ctypes.byref(shape), _ptr(target), _ptr(draft),
                                    _ptr(draft_tokens), _ptr(gamma), _ptr(temperature), int(seed),
                                    int(philox_row_offset), _ptr(out_n), _ptr(out_next),
                                    _ptr(workspace), workspace.numel(),
                                    _stream(stream, target.device),
                                    ctypes.cast(events.array, ctypes.c_void_p))
    _check(st, "specv_verify_profiled")
    return out_n, out_next


def specv_verify_with_uniforms(target, draft, draft_tokens, gamma, temperature, r, u, *,
                               max_gamma=None, out_n=None, out_next=None, workspace=None,
                               stream=None):
    """Verify step with injected uniforms r [B, max_gamma] and u [B] (float32)."""
    shape, draft, draft_tokens, gamma, out_n, out_next, workspace = _common(
        target, draft, draft_tokens, gamma, temperature, max_gamma, out_n, out_next, workspace)
    _check_tensors(target.device, r=r, u=u)
    st = _lib.specv_verify_with_uniforms(ctypes.byref(shape), _ptr(target), _ptr(draft),
                                         _ptr(draft_tokens), _ptr(gamma), _ptr(temperature),
                                         _ptr(r), _ptr(u), _ptr(out_n), _ptr(out_next),
                                         _ptr(workspace), workspace.numel(),
                                         _stream(stream, target.device))
    _check(st, "specv_verify_with_uniforms")
    return out_n, out_next


def specv_verify_lenient(target, draft, draft_tokens, gamma, temperature, lenience, epsilon, *,
                         max_gamma=None, seed=0, philox_row_offset=0, r=None, u=None, out_n=None,
                         out_next=None, workspace=None, stream=None, events=None):
    """Lossy verify step: threshold f(p, epsilon)/q with lenience "none",
    "lin" (p/eps), "sq" (p/eps^2) or "exp" (p^eps). Uniforms from Philox
    unless r [B, max_gamma] and u [B] are given; ``events`` is an optional
    StageEvents."""
    shape, draft, draft_tokens, gamma, out_n, out_next, workspace = _common(
        target, draft, draft_tokens, gamma, temperature, max_gamma, out_n, out_next, workspace)
    _check_tensors(target.device, r=r, u=u)
    kind = LENIENCE[lenience] if isinstance(lenience, str) else int(lenience)
    st = _lib.specv_verify_lenient(ctypes.byref(shape), _ptr(target), _ptr(draft),
                                   _ptr(draft_tokens), _ptr(gamma), _ptr(temperature), kind,
                                   float(epsilon), int(seed), int(philox_row_offset), _ptr(r),
                                   _ptr(u), _ptr(out_n), _ptr(out_next), _ptr(workspace),
                                   workspace.numel(), _stream(stream, target.device),
                                   None if events is None else
                                   ctypes.cast(events.array, ctypes.c_void_p))
    _check(st, "specv_verify_lenient")
    return out_n, out_next


def specv_diagnostics_workspace_bytes(shape: SpecvShape, top_k: int) -> int:
    return int(_lib.specv_diagnostics_workspace_bytes(ctypes.byref(shape), int(top_k)))


def specv_position_diagnostics(target, draft, gamma, temperature, top_k, *, max_gamma=None,
                               out=None, workspace=None, stream=None, events=None):
    """Per draft position (packed draft-row order): alpha = sum min(p, q),
    draft entropy (nats), and the top_k most probable draft tokens with
    their probabilities. Returns a dict of device tensors."""
    shape, draft, _, gamma, _, _, _ = _common(target, draft, None, gamma, temperature, max_gamma,
                                              None, None, torch.empty(0, device=target.device))
    dev = target.device
    k = int(top_k)
    if workspace is None:
        n = specv_diagnostics_workspace_bytes(shape, k)
        if n == 0:
            raise SpecvError("invalid shape or top_k")
        workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    td = shape.total_draft_rows
    if out is None:
        out = {"alpha": torch.empty(td, dtype=torch.float64, device=dev),
               "entropy": torch.empty(td, dtype=torch.float64, device=dev),
               "topk_index": torch.empty((td, k), dtype=torch.int32, device=dev),
               "topk_prob": torch.empty((td, k), dtype=torch.float64, device=dev)}
    _check_tensors(dev, workspace=workspace, **out)
    st = _lib.specv_position_diagnostics(ctypes.byref(shape), _ptr(target), _ptr(draft),
                                         _ptr(gamma), _ptr(temperature), k, _ptr(out["alpha"]),
                                         _ptr(out["entropy"]), _ptr(out["topk_index"]),
                                         _ptr(out["topk_prob"]), _ptr(workspace),
                                         workspace.numel(), _stream(stream, dev),
                                         None if events is None else
                                         ctypes.cast(events.array, ctypes.c_void_p))
    _check(st, "specv_position_diagnostics")
    return out


def specv_decode_workspace_bytes(shape: SpecvDecodeShape) -> int:
    return int(_lib.specv_decode_workspace_bytes(ctypes.byref(shape)))


def specv_decode_bigram(target_table, draft_table, temperature, start_token, *, gamma, rounds,
                        seed=0, philox_row_offset=0, out=None, workspace=None, stream=None,
                        events=None):
    """Multi-round speculative decoding with bigram tables [V, V] (row = the
    previous token). Returns a dict of device tensors: tokens [B, rounds *
    (gamma + 1)], length [B], accepted [B, rounds]."""
    if target_table.dim() != 2 or target_table.shape != draft_table.shape or \
            target_table.shape[0] != target_table.shape[1]:
        raise ValueError("tables must be [V, V] and alike")
    dev = target_table.device
    start_token = start_token if start_token.dtype == torch.int32 else start_token.to(torch.int32)
    B = start_token.shape[0]
    shape = SpecvDecodeShape(int(B), int(target_table.shape[0]), int(gamma), int(rounds),
                             _dtype_code(target_table))
    if _dtype_code(draft_table) != shape.dtype:
        raise TypeError("tables must share a dtype")
    if workspace is None:
        n = specv_decode_workspace_bytes(shape)
        if n == 0:
            raise SpecvError("invalid decode shape")
        workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    if out is None:
        out = {"tokens": torch.empty((B, rounds * (gamma + 1)), dtype=torch.int32, device=dev),
               "length": torch.empty(B, dtype=torch.int32, device=dev),
               "accepted": torch.empty((B, rounds), dtype=torch.int32, device=dev)}
    _check_tensors(dev, target_table=target_table, draft_table=draft_table,
                   temperature=temperature, start_token=start_token, workspace=workspace, **out)
    st = _lib.specv_decode_bigram(ctypes.byref(shape), _ptr(target_table), _ptr(draft_table),
                                  _ptr(temperature), _ptr(start_token), int(seed),
                                  int(philox_row_offset), _ptr(out["tokens"]), _ptr(out["length"]),
                                  _ptr(out["accepted"]), _ptr(workspace), workspace.numel(),
                                  _stream(stream, dev),
                                  None if events is None else
                                  ctypes.cast(events.array, ctypes.c_void_p))
    _check(st, "specv_decode_bigram")
    return out


def specv_cascade_workspace_bytes(shape: SpecvCascadeShape) -> int:
    return int(_lib.specv_cascade_workspace_bytes(ctypes.byref(shape)))


def specv_cascade_bigram(target_table, mid_table, small_table, temperature, start_token, *, k1,
                         k2, rounds, lenience="none", epsilon=1.0, seed=0, philox_row_offset=0,
                         out=None, workspace=None, stream=None, events=None):
    """CS Drafting's vertical cascade over bigram tables [V, V]; returns a
    dict of device tensors: tokens [B, rounds * (k1 + 1)], length [B],
    accepted [B, rounds] (the target review's n)."""
    tabs = (target_table, mid_table, small_table)
    if any(t.dim() != 2 or t.shape != target_table.shape for t in tabs) or \
            target_table.shape[0] != target_table.shape[1]:
        raise ValueError("tables must be [V, V] and alike")
    dt = _dtype_code(target_table)
    if any(_dtype_code(t) != dt for t in tabs):
        raise TypeError("tables must share a dtype")
    dev = target_table.device
    start_token = start_token if start_token.dtype == torch.int32 else start_token.to(torch.int32)
    B = start_token.shape[0]
    shape = SpecvCascadeShape(int(B), int(target_table.shape[0]), int(k1), int(k2), int(rounds),
                              dt)
    if workspace is None:
        n = specv_cascade_workspace_bytes(shape)
        if n == 0:
            raise SpecvError("invalid cascade shape")
        workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    if out is None:
        out = {"tokens": torch.empty((B, rounds * (k1 + 1)), dtype=torch.int32, device=dev),
               "length": torch.empty(B, dtype=torch.int32, device=dev),
               "accepted": torch.empty((B, rounds), dtype=torch.int32, device=dev)}
    _check_tensors(dev, target_table=target_table, mid_table=mid_table, small_table=small_table,
                   temperature=temperature, start_token=start_token, workspace=workspace, **out)
    kind = LENIENCE[lenience] if isinstance(lenience, str) else int(lenience)
    st = _lib.specv_cascade_bigram(ctypes.byref(shape), _ptr(target_table), _ptr(mid_table),
                                   _ptr(small_table), _ptr(temperature), _ptr(start_token), kind,
                                   float(epsilon), int(seed), int(philox_row_offset),
                                   _ptr(out["tokens"]), _ptr(out["length"]), _ptr(out["accepted"]),
                                   _ptr(workspace), workspace.numel(), _stream(stream, dev),
                                   None if events is None else
                                   ctypes.cast(events.array, ctypes.c_void_p))
    _check(st, "specv_cascade_bigram")
    return out


def specv_row_stats(target, draft, gamma, temperature, *, max_gamma=None, workspace=None,
                    stream=None):
    """Merged per-row (max, sum exp((z-m)/T), argmax) of target and draft rows."""
    shape, draft, _, gamma, _, _, workspace = _common(target, draft, None, gamma, temperature,
                                                     max_gamma, None, None, workspace)
    dev = target.device
    tt, td = shape.total_target_rows, shape.total_draft_rows
    out = {"target_max": torch.empty(tt, dtype=torch.float32, device=dev),
           "target_sum": torch.empty(tt, dtype=torch.float64, device=dev),
           "target_argmax": torch.empty(tt, dtype=torch.int32, device=dev),
           "draft_max": torch.empty(td, dtype=torch.float32, device=dev),
           "draft_sum": torch.empty(td, dtype=torch.float64, device=dev),
           "draft_argmax": torch.empty(td, dtype=torch.int32, device=dev)}
    st = _lib.specv_row_stats(ctypes.byref(shape), _ptr(target), _ptr(draft), _ptr(gamma),
                              _ptr(temperature), _ptr(out["target_max"]), _ptr(out["target_sum"]),
                              _ptr(out["target_argmax"]), _ptr(out["draft_max"]),
                              _ptr(out["draft_sum"]), _ptr(out["draft_argmax"]), _ptr(workspace),
                              workspace.numel(), _stream(stream, dev))
    _check(st, "specv_row_stats")
    return out


def specv_softmax_rows(target, draft, gamma, temperature, rows, *, max_gamma=None, workspace=None,
                       stream=None):
    """Probabilities of selected rows (rows[k] >= 0: target row, < 0: draft row -rows[k]-1)."""
    shape, draft, _, gamma, _, _, workspace = _common(target, draft, None, gamma, temperature,
                                                     max_gamma, None, None, workspace)
    dev = target.device
    rows = rows.to(device=dev, dtype=torch.int64).contiguous()
    out = torch.empty((rows.numel(), shape.vocab), dtype=torch.float32, device=dev)
    st = _lib.specv_softmax_rows(ctypes.byref(shape), _ptr(target), _ptr(draft), _ptr(gamma),
                                 _ptr(temperature), _ptr(rows), rows.numel(), _ptr(out),
                                 _ptr(workspace), workspace.numel(), _stream(stream, dev))
    _check(st, "specv_softmax_rows")
    return out


def specv_philox4x32_10(seed, counters, stream=None):
    """Device Philox4x32-10 blocks for counters [k, 4] (uint32 values in int32/int64)."""
    ctr = counters.to(torch.int32).contiguous()
    out = torch.empty_like(ctr)
    st = _lib.specv_philox4x32_10(int(seed), _ptr(ctr), _ptr(out), ctr.shape[0],
                                  _stream(stream, ctr.device))
    _check(st, "specv_philox4x32_10")
    return out


def specv_copy_bytes(dst, src, stream=None):
    n = src.numel() * src.element_size()
    st = _lib.specv_copy_bytes(_ptr(dst), _ptr(src), n, _stream(stream, src.device))
    _check(st, "specv_copy_bytes")


def specv_read_bytes(src, sink=None, stream=None):
    """Read-only stream of src (a multiple of 64 KiB) with pass 1's access
    pattern; returns the per-wave XOR checksums (int32, bytes / 32768)."""
    n = src.numel() * src.element_size()
    if sink is None:
        sink = torch.empty(n // 32768, dtype=torch.int32, device=src.device)
    st = _lib.specv_read_bytes(_ptr(src), n, _ptr(sink), _stream(stream, src.device))
    _check(st, "specv_read_bytes")
    return sink


# hipEventDisableSystemFence: the event only timestamps; recording it does not
# write back and invalidate the caches as a system-scope fence would (on a
# multi-XCD part that fence costs about as much as a small kernel).
HIP_EVENT_TIMING_ONLY = 0x20000000


class StageEvents:
    """2 * len(STAGES) HIP event slots for specv_verify_profiled (created
    through the HIP runtime as timing-only events). Only the stages listed get
    events; the other slots stay NULL and are not recorded."""

    _hip = None

    def __init__(self, stages=None):
        if StageEvents._hip is None:
            h = ctypes.CDLL("libamdhip64.so")
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                              ctypes.c_void_p]
            h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
            h.hipEventDestroy.argtypes = [ctypes.c_void_p]
            StageEvents._hip = h
        n = 2 * len(STAGES)
        self.array = (ctypes.c_void_p * n)()
        wanted = range(len(STAGES)) if stages is None else stages
        for i in [2 * st + h for st in wanted for h in (0, 1)]:
            ev = ctypes.c_void_p()
            if StageEvents._hip.hipEventCreateWithFlags(ctypes.byref(ev), HIP_EVENT_TIMING_ONLY) != 0:
                raise SpecvError("hipEventCreateWithFlags failed")
            self.array[i] = ev

    def elapsed_ms(self, stage: int) -> float:
        ms = ctypes.c_float()
        h = StageEvents._hip
        h.hipEventSynchronize(self.array[2 * stage + 1])
        if h.hipEventElapsedTime(ctypes.byref(ms), self.array[2 * stage], self.array[2 * stage + 1]) != 0:
            raise SpecvError("hipEventElapsedTime failed")
        return float(ms.value)

    def __del__(self):
        # type(self), not the module global, which may already be gone at
        # interpreter shutdown
        h = getattr(type(self), "_hip", None)
        if h is not None:
            for ev in self.array:
                if ev:
                    h.hipEventDestroy(ev)


def from_inputs(x, device="cuda"):
    """Device tensors of a synth.Inputs-like object (numpy arrays): bf16 logits
    travel as their 16-bit patterns."""
    def dev(a, dt=None):
        t = torch.from_numpy(a.view("int16") if a.dtype.name == "uint16" else a)
        return t.to(device=device, dtype=dt) if dt is not None else t.to(device)
    return dict(target=dev(x.target), draft=dev(x.draft), draft_tokens=dev(x.tokens),
                gamma=dev(x.gamma), temperature=dev(x.temperature))
