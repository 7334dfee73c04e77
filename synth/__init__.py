"""Seeded synthetic inputs for the speculative-sampling verify step.

This module serves both the HIP path (tests, benchmark) and the CPU oracle. It
holds none of the verify step's arithmetic: it draws logits, rounds them to
bf16, and samples draft tokens from the draft rows by the Gumbel-max rule
(argmax of z/T plus Gumbel noise), which is an exact sampler for the
temperature softmax that needs no softmax, ratio or CDF.

Workloads, each shaped after a setting on the pages:
  1 tiny_cpu        B sequences (default 10,000 rounds), gamma=4, V=1000, fp32;
                    target ~ N(0, 2^2), draft = target + N(0, 0.5^2); T=1 (or 0).
  2 t5xxl_like      gamma=5, V=32128 (the T5 vocabulary size used by DistillSpec),
                    bf16; target ~ N(0, 3^2) with 20 distinct tokens per target
                    row raised by 8; draft = target + N(0, 1); T=1 (or 0).
                    Rounds are independent sequences batched into one call.
  3 serving_b64     B=64, gamma=7, V=128256, bf16; target = 2 * Gumbel(0, 1);
                    draft = 0.8 * target + N(0, 1.5^2); T=0.7.
  4 ragged_b256     B=256, gamma_b ~ U{1..16} (dynamic speculation lookahead, as
                    in DISCO), V=152064, bf16; target ~ N(0, 2.5^2); draft =
                    target + N(0, sigma_b^2), sigma_b ~ U[0.2, 3.0]; T=1.
  5 large_vocab     B=128, gamma=8, V=256000, fp32; target ~ N(0, 2^2); draft =
                    target + N(0, 0.8^2); odd sequences greedy (T=0), even ones
                    T=1; 6 of the even sequences have draft rows bit-identical
                    to their target rows (the all-accept path).
  chi               V=8, gamma=4, fp32, one fixed set of rows (workload 1's
                    recipe) shared by every round, fresh draft tokens per round.

Generator: numpy PCG64 streams keyed by SeedSequence((workload seed, sequence,
...)), so every sequence is reproducible on its own and rows are generated in
parallel threads. Later rounds of a workload (`first` / `round_index`) use the
streams of later global sequence numbers: fresh logits and draft tokens. Storage: fp32 values are rounded to bf16 with
round-to-nearest-even where the workload is bf16.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

WORKLOADS = ("tiny_cpu", "t5xxl_like", "serving_b64", "ragged_b256", "large_vocab")


@dataclass
class Inputs:
    name: str
    vocab: int
    max_gamma: int
    dtype: str                 # "bf16" (uint16 bit patterns) or "f32"
    target: np.ndarray         # [sum(gamma_b + 1), V]
    draft: np.ndarray          # [sum(gamma_b), V]
    tokens: np.ndarray         # [sum(gamma_b)] int32
    gamma: np.ndarray          # [B] int32
    temperature: np.ndarray    # [B] float32
    seed: int = 0              # verify (Philox) seed
    row_offset: int = 0        # Philox row of sequence 0
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.gamma.shape[0])

    @property
    def total_target_rows(self) -> int:
        return int(self.target.shape[0])

    @property
    def total_draft_rows(self) -> int:
        return int(self.draft.shape[0])

    @property
    def bytes_per_logit(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def offsets(self):
        g = self.gamma.astype(np.int64)
        toff = np.concatenate([[0], np.cumsum(g + 1)])
        doff = np.concatenate([[0], np.cumsum(g)])
        return toff, doff

    def pass1_bytes(self) -> int:
        """Bytes the first pass must read: every target row, plus the draft
        rows of sampling sequences (greedy sequences never read draft rows)."""
        g = self.gamma.astype(np.int64)
        sampling = self.temperature > 0
        rows = int(np.sum(g + 1) + np.sum(g[sampling]))
        return rows * self.vocab * self.bytes_per_logit

    def diagnostics_bytes(self) -> dict:
        """Bytes the per-position diagnostics must read: pass 1 reads every
        target and draft row; pass 2 reads each position's draft row and, for
        sampling sequences, its target row."""
        g = self.gamma.astype(np.int64)
        sampling = self.temperature > 0
        row = self.vocab * self.bytes_per_logit
        pass1 = int(np.sum(g + 1) + np.sum(g)) * row
        pass2 = int(np.sum(g) + np.sum(g[sampling])) * row
        return {"pass1": pass1, "pass2": pass2}


def _threads() -> int:
    return max(1, min(os.cpu_count() or 1, 16))


def _rng(*keys: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in keys])))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (h.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _stored(x32: np.ndarray, dtype: str) -> np.ndarray:
    return to_bf16_bits(x32) if dtype == "bf16" else x32.astype(np.float32)


def _as_f64(stored: np.ndarray, dtype: str) -> np.ndarray:
    return (bf16_bits_to_f32(stored) if dtype == "bf16" else stored).astype(np.float64)


def gumbel_max_token(stored_row: np.ndarray, dtype: str, T: float, rng: np.random.Generator) -> int:
    """One draft token from the stored draft row at temperature T: argmax of
    z/T + Gumbel noise (T > 0), or argmax z, lowest index on ties (T == 0)."""
    z = _as_f64(stored_row, dtype)
    if T == 0.0:
        return int(np.argmax(z))
    u = (rng.integers(0, 1 << 52, z.shape[0]) + 0.5) / float(1 << 52)
    return int(np.argmax(z / float(T) - np.log(-np.log(u))))


def gumbel_max_tokens(stored_rows: np.ndarray, dtype: str, T: float,
                      rng: np.random.Generator) -> np.ndarray:
    """gumbel_max_token for every row of a [g, V] block, one noise draw per row."""
    z = _as_f64(stored_rows, dtype)
    if T == 0.0:
        return np.argmax(z, axis=1).astype(np.int32)
    u = (rng.integers(0, 1 << 52, z.shape) + 0.5) / float(1 << 52)
    return np.argmax(z / float(T) - np.log(-np.log(u)), axis=1).astype(np.int32)


def _open_uniform(rng, n):
    return (rng.integers(0, 1 << 52, n) + 0.5) / float(1 << 52)


def _assemble(name, V, max_gamma, dtype, gammas, temps, row_fn, gen_seed, meta=None,
              first: int = 0) -> Inputs:
    """Allocate the packed layout and fill sequence b's rows with
    row_fn(b, rng) -> (target_f32 [g+1, V], draft_f32 [g, V], same_rows).
    Sequence b draws from the streams of global sequence first + b, so a
    batch that starts at `first` holds fresh sequences (a later round)."""
    gammas = np.asarray(gammas, dtype=np.int32)
    temps = np.asarray(temps, dtype=np.float32)
    B = gammas.shape[0]
    toff = np.concatenate([[0], np.cumsum(gammas.astype(np.int64) + 1)])
    doff = np.concatenate([[0], np.cumsum(gammas.astype(np.int64))])
    sdt = np.uint16 if dtype == "bf16" else np.float32
    target = np.empty((int(toff[-1]), V), sdt)
    draft = np.empty((int(doff[-1]), V), sdt)
    tokens = np.empty(int(doff[-1]), np.int32)

    def fill(b):
        rng = _rng(gen_seed, first + b)
        t32, d32, same = row_fn(b, rng)
        g = int(gammas[b])
        target[toff[b]:toff[b + 1]] = _stored(t32, dtype)
        if same:
            draft[doff[b]:doff[b + 1]] = target[toff[b]:toff[b] + g]
        else:
            draft[doff[b]:doff[b + 1]] = _stored(d32, dtype)
        if g:
            tokens[doff[b]:doff[b + 1]] = gumbel_max_tokens(draft[doff[b]:doff[b + 1]], dtype,
                                                            float(temps[b]),
                                                            _rng(gen_seed, first + b, 1 << 20))

    def fill_range(lo_hi):
        for b in range(*lo_hi):
            fill(b)

    # Tasks of at least ~4M logits each keep thread hand-off overhead small.
    per_seq = max(1, int((2 * np.mean(gammas) + 1) * V)) if B else 1
    step = max(1, min(B, (1 << 22) // per_seq))
    ranges = [(lo, min(B, lo + step)) for lo in range(0, B, step)]
    if len(ranges) == 1:
        fill_range(ranges[0])
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill_range, ranges))
    return Inputs(name, V, max_gamma, dtype, target, draft, tokens, gammas, temps,
                  meta=dict(meta or {}, first=first))


def tiny_cpu(rounds: int = 10000, greedy: bool = False, vocab: int = 1000, gamma: int = 4,
             gen_seed: int = 1) -> Inputs:
    def rows(b, rng):
        t = (rng.standard_normal((gamma + 1, vocab)) * 2.0).astype(np.float32)
        d = (t[:gamma] + rng.standard_normal((gamma, vocab)) * 0.5).astype(np.float32)
        return t, d, False
    T = 0.0 if greedy else 1.0
    return _assemble("tiny_cpu", vocab, gamma, "f32", [gamma] * rounds, [T] * rounds, rows,
                     gen_seed, {"greedy": greedy})


def t5xxl_like(rounds: int = 2000, greedy: bool = False, vocab: int = 32128, gamma: int = 5,
               gen_seed: int = 2, first: int = 0) -> Inputs:
    def rows(b, rng):
        t = (rng.standard_normal((gamma + 1, vocab), dtype=np.float32) * 3.0)
        for i in range(gamma + 1):
            t[i, rng.choice(vocab, 20, replace=False)] += 8.0
        d = t[:gamma] + rng.standard_normal((gamma, vocab), dtype=np.float32)
        return t, d, False
    T = 0.0 if greedy else 1.0
    return _assemble("t5xxl_like", vocab, gamma, "bf16", [gamma] * rounds, [T] * rounds, rows,
                     gen_seed, {"greedy": greedy}, first)


def serving_b64(batch: int = 64, vocab: int = 128256, gamma: int = 7, gen_seed: int = 3,
                round_index: int = 0) -> Inputs:
    def rows(b, rng):
        t = (-2.0 * np.log(-np.log(_open_uniform(rng, (gamma + 1) * vocab)))).astype(np.float32)
        t = t.reshape(gamma + 1, vocab)
        d = 0.8 * t[:gamma] + rng.standard_normal((gamma, vocab), dtype=np.float32) * 1.5
        return t, d.astype(np.float32), False
    return _assemble("serving_b64", vocab, gamma, "bf16", [gamma] * batch, [0.7] * batch, rows,
                     gen_seed, None, round_index * batch)


def _batch_rng(gen_seed: int, round_index: int) -> np.random.Generator:
    # per-batch draws (gammas, spreads, which sequences repeat their rows);
    # round 0 keeps the original stream
    return _rng(gen_seed, 1 << 30) if round_index == 0 else _rng(gen_seed, 1 << 30, round_index)


def ragged_b256(batch: int = 256, vocab: int = 152064, max_gamma: int = 16,
                gen_seed: int = 4, round_index: int = 0) -> Inputs:
    brng = _batch_rng(gen_seed, round_index)
    gammas = brng.integers(1, max_gamma + 1, batch).astype(np.int32)
    sigmas = brng.uniform(0.2, 3.0, batch)

    def rows(b, rng):
        g = int(gammas[b])
        t = rng.standard_normal((g + 1, vocab), dtype=np.float32) * 2.5
        d = t[:g] + rng.standard_normal((g, vocab), dtype=np.float32) * np.float32(sigmas[b])
        return t, d, False
    return _assemble("ragged_b256", vocab, max_gamma, "bf16", gammas, [1.0] * batch, rows, gen_seed,
                     {"sigma": sigmas}, round_index * batch)


def large_vocab(batch: int = 128, vocab: int = 256000, gamma: int = 8, gen_seed: int = 5,
                identical: int | None = None, round_index: int = 0) -> Inputs:
    temps = np.where(np.arange(batch) % 2 == 1, 0.0, 1.0).astype(np.float32)
    evens = np.arange(0, batch, 2)
    k = int(round(0.05 * batch)) if identical is None else identical
    same = set(int(x) for x in _batch_rng(gen_seed, round_index).choice(evens, min(k, len(evens)),
                                                                         replace=False))

    def rows(b, rng):
        t = rng.standard_normal((gamma + 1, vocab), dtype=np.float32) * 2.0
        if b in same:
            return t, None, True
        d = t[:gamma] + rng.standard_normal((gamma, vocab), dtype=np.float32) * 0.8
        return t, d, False
    return _assemble("large_vocab", vocab, gamma, "f32", [gamma] * batch, temps, rows, gen_seed,
                     {"identical_sequences": sorted(same)}, round_index * batch)


def chi_square_set(rounds: int = 1_000_000, vocab: int = 8, gamma: int = 4, gen_seed: int = 11,
                   draft_sigma: float = 0.5, T: float = 1.0) -> Inputs:
    """One fixed set of rows (target N(0, 2^2), draft = target + N(0, draft_sigma^2))
    shared by every round, with fresh draft tokens per round. Rows are stored
    fp32, replicated per round in the packed layout."""
    rng = _rng(gen_seed, 0)
    t = (rng.standard_normal((gamma + 1, vocab)) * 2.0).astype(np.float32)
    d = (t[:gamma] + rng.standard_normal((gamma, vocab)) * draft_sigma).astype(np.float32)
    target = np.ascontiguousarray(np.broadcast_to(t, (rounds, gamma + 1, vocab))).reshape(-1, vocab)
    draft = np.ascontiguousarray(np.broadcast_to(d, (rounds, gamma, vocab))).reshape(-1, vocab)
    # Fresh tokens: Gumbel-max per (round, position), vectorised over rounds.
    trng = _rng(gen_seed, 1)
    tokens = np.empty((rounds, gamma), np.int32)
    dz = d.astype(np.float64) / T
    for i in range(gamma):
        u = _open_uniform(trng, rounds * vocab).reshape(rounds, vocab)
        tokens[:, i] = np.argmax(dz[i][None, :] - np.log(-np.log(u)), axis=1)
    return Inputs("chi", vocab, gamma, "f32", target, draft, tokens.reshape(-1),
                  np.full(rounds, gamma, np.int32), np.full(rounds, T, np.float32),
                  meta={"target_rows": t, "draft_rows": d})


def subset(x: Inputs, seqs) -> Inputs:
    """The packed inputs of sequences `seqs` (in order) of x: slicing only.
    Note that a sequence keeps its Philox row only where its index is
    unchanged (the row is row_offset + its position in the batch)."""
    toff, doff = x.offsets()
    t = np.concatenate([x.target[toff[b]:toff[b + 1]] for b in seqs])
    d = [x.draft[doff[b]:doff[b + 1]] for b in seqs]
    d = np.concatenate(d) if sum(len(a) for a in d) else x.draft[:0]
    k = [x.tokens[doff[b]:doff[b + 1]] for b in seqs]
    k = np.concatenate(k) if sum(len(a) for a in k) else x.tokens[:0]
    return Inputs(x.name, x.vocab, x.max_gamma, x.dtype, t, d, k, x.gamma[seqs].copy(),
                  x.temperature[seqs].copy(), x.seed, x.row_offset, dict(x.meta))


@dataclass
class BigramTables:
    """Bigram "models": row s of each [V, V] table holds the logits of the
    next token after token s (bf16 bit patterns). `small` is a second, weaker
    drafter for cascades (None unless asked for)."""
    target: np.ndarray
    draft: np.ndarray
    seed: int
    small: np.ndarray = None

    def start(self, n: int) -> np.ndarray:
        return _rng(self.seed, 99).integers(0, self.target.shape[0], n).astype(np.int32)


def bigram_tables(vocab: int = 8192, gen_seed: int = 6, small: bool = False) -> BigramTables:
    """The T5-XXL-like row recipe per table row: target logits N(0, 3^2)
    with 20 uniformly chosen entries raised by 8, draft = target + N(0, 1);
    the small drafter (cascades) = target + N(0, 2^2)."""
    rng = _rng(gen_seed, 0)
    t = rng.standard_normal((vocab, vocab), dtype=np.float32) * 3.0
    rows = np.repeat(np.arange(vocab), 20)
    t[rows, rng.integers(0, vocab, vocab * 20)] += 8.0
    d = t + rng.standard_normal((vocab, vocab), dtype=np.float32)
    s = None
    if small:
        s = to_bf16_bits(t + rng.standard_normal((vocab, vocab), dtype=np.float32) * 2.0)
    return BigramTables(to_bf16_bits(t), to_bf16_bits(d), gen_seed, s)


def by_name(name: str, **kw) -> Inputs:
    return {"tiny_cpu": tiny_cpu, "t5xxl_like": t5xxl_like, "serving_b64": serving_b64,
            "ragged_b256": ragged_b256, "large_vocab": large_vocab, "chi": chi_square_set}[name](**kw)
