"""ctypes wrapper around the CPU oracle (oracle/specv_oracle.c).

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package. The HIP library and
its Python binding never import it and never fall back to it.

Every function takes numpy arrays in the packed layout of the verify step:
target logits ``[sum(gamma_b + 1), V]``, draft logits ``[sum(gamma_b), V]``
(bf16 stored as uint16 bit patterns, or float32), draft tokens
``[sum(gamma_b)]`` int32, ``gamma[B]`` int32, ``temperature[B]`` float32.
"""
import ctypes
import os
from dataclasses import dataclass
from pathlib import Path

import numpy as np

from . import build as _build

F32, BF16 = 0, 1
NEAR_TIE = 1e-6

MUTANT_NONE = 0
MUTANT_RESIDUAL_IS_P = 1
MUTANT_RESIDUAL_IS_Q = 2
MUTANT_N_PLUS_ONE = 3
MUTANT_LENIENCE_TIMES = 4

# lenience functions f(p, eps) of lossy decoding (DistillSpec section 4, the
# paragraph on lossy SD; Algorithm A.1 thresholds)
LENIENCE_NONE, LENIENCE_LIN, LENIENCE_SQ, LENIENCE_EXP = 0, 1, 2, 3
LENIENCE = {"none": LENIENCE_NONE, "lin": LENIENCE_LIN, "sq": LENIENCE_SQ, "exp": LENIENCE_EXP}

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not _build.LIBRARY.exists():
        _build.build()
    lib = ctypes.CDLL(str(_build.LIBRARY))
    P = ctypes.c_void_p
    i64, u64 = ctypes.c_int64, ctypes.c_uint64
    lib.oracle_verify.restype = ctypes.c_int
    lib.oracle_verify.argtypes = [i64, i64, i64, ctypes.c_int, i64, i64, P, P, P, P, P,
                                  u64, u64, ctypes.c_int, ctypes.c_float,
                                  P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_int]
    lib.oracle_position_diagnostics.restype = ctypes.c_int
    lib.oracle_position_diagnostics.argtypes = [i64, i64, ctypes.c_int, i64, i64, P, P, P, P, i64,
                                                P, P, P, P]
    lib.oracle_decode_bigram.restype = ctypes.c_int
    lib.oracle_decode_bigram.argtypes = [i64, i64, i64, i64, ctypes.c_int, P, P, P, P, u64, u64,
                                         P, P, P, P, ctypes.c_int]
    lib.oracle_cascade_bigram.restype = ctypes.c_int
    lib.oracle_cascade_bigram.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int, P, P, P, P, P,
                                          ctypes.c_int, ctypes.c_float, u64, u64, ctypes.c_int,
                                          P, P, P, P, ctypes.c_int]
    lib.oracle_row_stats.restype = None
    lib.oracle_row_stats.argtypes = [P, ctypes.c_int, i64, i64, P, P, P, P, P]
    lib.oracle_softmax_row.restype = None
    lib.oracle_softmax_row.argtypes = [P, ctypes.c_int, i64, i64, ctypes.c_float, P]
    lib.oracle_philox_blocks.restype = None
    lib.oracle_philox_blocks.argtypes = [u64, P, P, i64]
    lib.oracle_uniform24.restype = ctypes.c_double
    lib.oracle_uniform24.argtypes = [ctypes.c_uint32]
    lib.oracle_uniform24_many.restype = None
    lib.oracle_uniform24_many.argtypes = [P, P, i64]
    lib.oracle_decode_bf16.restype = None
    lib.oracle_decode_bf16.argtypes = [P, P, i64]
    lib.oracle_set_mutant.restype = None
    lib.oracle_set_mutant.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    raise TypeError("logits must be uint16 (bf16 bits) or float32, got %s" % a.dtype)


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(n, 16))


@dataclass
class VerifyResult:
    n: np.ndarray          # [B] int32 accepted counts, -1 on a data error
    next_token: np.ndarray  # [B] int32 emitted token, -1 on a data error
    margin: np.ndarray     # [B] float64 smallest relative decision margin
    near_tie: np.ndarray   # [B] bool, margin < 1e-6
    ratio: np.ndarray      # [B, max_gamma] float64 f(p_i(x_i))/q_i(x_i) (NaN if not reached)
    resmass: np.ndarray    # [B] float64 total weight of the final draw (NaN if greedy)
    layout_ok: bool
    # the accept margin (smallest |r_i - ratio_i| / ratio_i over the decisive
    # positions) and the draw margin (distance of u * C to the nearer end of
    # the drawn token's CDF interval, over C), each +inf where there is none
    accept_margin: np.ndarray = None
    draw_margin: np.ndarray = None
    # tokens whose CDF interval meets [u C - 1e-6 C, u C + 1e-6 C]: the
    # outcomes a computation with rounding below 1e-6 of C can reach (only
    # next_token when the draw is not a near-tie)
    tok_lo: np.ndarray = None
    tok_hi: np.ndarray = None
    # the outcome with the first near-tie accept decision reversed: n and its
    # token window; alt_n = -2 where no accept decision is a near-tie
    alt_n: np.ndarray = None
    alt_lo: np.ndarray = None
    alt_hi: np.ndarray = None
    # the chance, over the uniforms, that a decisive one lands within its
    # window (given the rows and the n reached): the expected share of
    # sequences the rule flags
    near_prob: np.ndarray = None

    def admits(self, n, tok):
        """Per sequence: (n, tok) is the oracle's outcome up to the near-tie
        rule -- n exact and tok inside the draw window, or the outcome on the
        other side of the first near-tie accept decision."""
        n = np.asarray(n)
        tok = np.asarray(tok)
        primary = (n == self.n) & (tok >= self.tok_lo) & (tok <= self.tok_hi)
        alt = (self.alt_n >= 0) & (n == self.alt_n) & (tok >= self.alt_lo) & (tok <= self.alt_hi)
        return primary | alt


def verify(target, draft, tokens, gamma, temperature, *, vocab, max_gamma, seed=0,
           row_offset=0, r=None, u=None, lenience="none", epsilon=1.0,
           nthreads=None) -> VerifyResult:
    """Run the oracle over every sequence. ``r`` ([B, max_gamma] float32) and
    ``u`` ([B] float32) inject the uniforms instead of drawing them from
    Philox4x32-10. ``lenience`` ("none", "lin", "sq", "exp") and ``epsilon``
    (a float32 in (0, 1]) select the threshold f(p, eps)/q of lossy
    decoding."""
    lib = _load()
    gamma = np.ascontiguousarray(gamma, dtype=np.int32)
    B = int(gamma.shape[0])
    target = np.ascontiguousarray(target)
    draft = np.ascontiguousarray(draft)
    if draft.size and draft.dtype != target.dtype:
        raise TypeError("target and draft logits must share a dtype")
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    temperature = np.ascontiguousarray(temperature, dtype=np.float32)
    tt = target.size // vocab
    td = draft.size // vocab if vocab else 0
    out_n = np.empty(B, np.int32)
    out_next = np.empty(B, np.int32)
    margin = np.empty(B, np.float64)
    near = np.empty(B, np.uint8)
    ratio = np.full((B, max(max_gamma, 1)), np.nan, np.float64)
    resmass = np.full(B, np.nan, np.float64)
    am = np.empty(B, np.float64)
    dm = np.empty(B, np.float64)
    win = np.empty((B, 5), np.int32)
    nprob = np.empty(B, np.float64)
    if r is not None:
        r = np.ascontiguousarray(r, dtype=np.float32).reshape(B, max_gamma)
    if u is not None:
        u = np.ascontiguousarray(u, dtype=np.float32).reshape(B)
    code = lib.oracle_verify(B, vocab, max_gamma, _dtype_code(target), tt, td, _ptr(target),
                             _ptr(draft), _ptr(tokens), _ptr(gamma), _ptr(temperature),
                             int(seed), int(row_offset), LENIENCE[lenience],
                             float(np.float32(epsilon)), _ptr(r), _ptr(u), _ptr(out_n),
                             _ptr(out_next), _ptr(margin), _ptr(near), _ptr(ratio),
                             _ptr(resmass), _ptr(am), _ptr(dm), _ptr(win), _ptr(nprob),
                             int(nthreads or default_threads()))
    return VerifyResult(out_n, out_next, margin, near.astype(bool),
                        ratio[:, :max_gamma], resmass, code == 0, am, dm,
                        win[:, 0].copy(), win[:, 1].copy(), win[:, 2].copy(), win[:, 3].copy(),
                        win[:, 4].copy(), nprob)


@dataclass
class Diagnostics:
    alpha: np.ndarray        # [draft rows] float64 sum_v min(p_v, q_v)
    entropy: np.ndarray      # [draft rows] float64 -sum_v q_v ln q_v
    topk_index: np.ndarray   # [draft rows, k] int32, most probable first
    topk_prob: np.ndarray    # [draft rows, k] float64 q of those tokens


def position_diagnostics(target, draft, gamma, temperature, *, vocab, top_k) -> Diagnostics:
    """Per draft position: acceptance probability alpha = sum min(p, q),
    draft entropy and the top-k draft tokens (packed draft-row order)."""
    lib = _load()
    gamma = np.ascontiguousarray(gamma, dtype=np.int32)
    target = np.ascontiguousarray(target)
    draft = np.ascontiguousarray(draft)
    temperature = np.ascontiguousarray(temperature, dtype=np.float32)
    tt, td = target.size // vocab, draft.size // vocab
    k = int(top_k)
    alpha, ent = np.empty(td, np.float64), np.empty(td, np.float64)
    idx, prob = np.empty((td, k), np.int32), np.empty((td, k), np.float64)
    code = lib.oracle_position_diagnostics(gamma.shape[0], vocab, _dtype_code(target), tt, td,
                                           _ptr(target), _ptr(draft), _ptr(gamma),
                                           _ptr(temperature), k, _ptr(alpha), _ptr(ent), _ptr(idx),
                                           _ptr(prob))
    if code != 0:
        raise ValueError("gammas and row totals disagree")
    return Diagnostics(alpha, ent, idx, prob)


@dataclass
class DecodeResult:
    tokens: np.ndarray      # [B, rounds * (gamma + 1)] int32 generated tokens
    length: np.ndarray      # [B] int32 tokens generated (-1 after a failed round)
    accepted: np.ndarray    # [B, rounds] int32 n of each round (-1 after a failure)
    first_near: np.ndarray  # [B] int32 first round with a near-tie (rounds if none)


def decode_bigram(target_table, draft_table, temperature, start, *, gamma, rounds, seed=0,
                  row_offset=0, nthreads=None) -> DecodeResult:
    """Multi-round speculative decoding with bigram tables [V, V] (row = the
    previous token), every sequence drafting gamma tokens per round."""
    lib = _load()
    ttab = np.ascontiguousarray(target_table)
    dtab = np.ascontiguousarray(draft_table)
    if ttab.dtype != dtab.dtype or ttab.shape != dtab.shape or ttab.shape[0] != ttab.shape[1]:
        raise ValueError("tables must be [V, V] of one dtype")
    V = ttab.shape[0]
    temperature = np.ascontiguousarray(temperature, dtype=np.float32)
    start = np.ascontiguousarray(start, dtype=np.int32)
    B = start.shape[0]
    cap = rounds * (gamma + 1)
    tokens = np.full((B, cap), -1, np.int32)
    length = np.empty(B, np.int32)
    accepted = np.empty((B, rounds), np.int32)
    first_near = np.empty(B, np.int32)
    lib.oracle_decode_bigram(B, V, gamma, rounds, _dtype_code(ttab), _ptr(ttab), _ptr(dtab),
                             _ptr(temperature), _ptr(start), int(seed), int(row_offset),
                             _ptr(tokens), _ptr(length), _ptr(accepted), _ptr(first_near),
                             int(nthreads or default_threads()))
    return DecodeResult(tokens, length, accepted, first_near)


def cascade_bigram(target_table, mid_table, small_table, temperature, start, *, k1, k2, rounds,
                   lenience="none", epsilon=1.0, seed=0, row_offset=0, mutant_q_is_p1=False,
                   nthreads=None) -> DecodeResult:
    """CS Drafting's vertical cascade with bigram tables: the smallest table
    drafts k2 tokens per inner round for the intermediate one (reviewed with
    the given lenience) until k1 tokens are drafted; the target reviews them
    without lenience."""
    lib = _load()
    tabs = [np.ascontiguousarray(t) for t in (target_table, mid_table, small_table)]
    if len({(t.dtype, t.shape) for t in tabs}) != 1 or tabs[0].shape[0] != tabs[0].shape[1]:
        raise ValueError("tables must be [V, V] of one dtype")
    V = tabs[0].shape[0]
    temperature = np.ascontiguousarray(temperature, dtype=np.float32)
    start = np.ascontiguousarray(start, dtype=np.int32)
    B = start.shape[0]
    cap = rounds * (k1 + 1)
    tokens = np.full((B, cap), -1, np.int32)
    length = np.empty(B, np.int32)
    accepted = np.empty((B, rounds), np.int32)
    first_near = np.empty(B, np.int32)
    lib.oracle_cascade_bigram(B, V, k1, k2, rounds, _dtype_code(tabs[0]), _ptr(tabs[0]),
                              _ptr(tabs[1]), _ptr(tabs[2]), _ptr(temperature), _ptr(start),
                              LENIENCE[lenience], float(np.float32(epsilon)), int(seed),
                              int(row_offset), int(bool(mutant_q_is_p1)), _ptr(tokens),
                              _ptr(length), _ptr(accepted), _ptr(first_near),
                              int(nthreads or default_threads()))
    return DecodeResult(tokens, length, accepted, first_near)


def row_stats(logits, vocab, temperature_per_row):
    """(m, S, argmax, valid) per row; S is NaN where the row's T is 0."""
    lib = _load()
    logits = np.ascontiguousarray(logits)
    rows = logits.size // vocab
    T = np.ascontiguousarray(temperature_per_row, dtype=np.float32).reshape(rows)
    m = np.empty(rows, np.float64)
    s = np.empty(rows, np.float64)
    a = np.empty(rows, np.int32)
    ok = np.empty(rows, np.uint8)
    lib.oracle_row_stats(_ptr(logits), _dtype_code(logits), rows, vocab, _ptr(T), _ptr(m),
                         _ptr(s), _ptr(a), _ptr(ok))
    return m, s, a, ok.astype(bool)


def softmax_row(logits, vocab, row, T):
    lib = _load()
    logits = np.ascontiguousarray(logits)
    out = np.empty(vocab, np.float64)
    lib.oracle_softmax_row(_ptr(logits), _dtype_code(logits), vocab, int(row), float(T),
                           _ptr(out))
    return out


def philox_blocks(seed, counters):
    """Philox4x32-10 blocks for counters [k, 4] uint32 -> [k, 4] uint32."""
    lib = _load()
    ctr = np.ascontiguousarray(counters, dtype=np.uint32).reshape(-1, 4)
    out = np.empty_like(ctr)
    lib.oracle_philox_blocks(int(seed), _ptr(ctr), _ptr(out), ctr.shape[0])
    return out


def uniform24(words):
    """U(w) = ((w >> 8) + 1) * 2^-24 for every 32-bit word."""
    lib = _load()
    w = np.ascontiguousarray(words, dtype=np.uint32).ravel()
    out = np.empty(w.shape, np.float64)
    lib.oracle_uniform24_many(_ptr(w), _ptr(out), w.size)
    return out


def decode_bf16(bits):
    lib = _load()
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, np.float64)
    lib.oracle_decode_bf16(_ptr(bits), _ptr(out), bits.size)
    return out


class mutant:
    """Context manager that plants one known mistake in the oracle (negative
    controls for the statistical tests)."""

    def __init__(self, which: int):
        self.which = which

    def __enter__(self):
        _load().oracle_set_mutant(self.which)
        return self

    def __exit__(self, *exc):
        _load().oracle_set_mutant(MUTANT_NONE)
        return False
