// kernels.hpp -- the verify step's kernels for gfx950.
//
// The step (DistillSpec, Appendix A.3, Algorithm A.1, lenience 1) runs as:
//   k0_plan        offsets of the packed ragged rows, row -> sequence maps,
//                  layout validation; initialises the status word. Launched
//                  only for ragged batches of more than 1024 sequences: a
//                  uniform batch (every gamma equal) has arithmetic offsets,
//                  and k1's first workgroup checks its gammas; a smaller
//                  ragged batch is planned by k1's first workgroup, and each
//                  pass-1 wave finds its row's sequence with a wave scan.
//   k1_row_stats   pass 1, the HBM-bound hot loop: every needed logit row is
//                  streamed once with 16-byte non-temporal loads; each wave
//                  owns one (row, chunk) and keeps (max, sum of 2^((z - max) k),
//                  argmax) in registers, reduced across the wave by shuffles;
//                  the wave whose chunk holds a row's draft token also
//                  records that logit for the accept step.
//   k1_short_rows  pass 1 for rows of one 4 KiB tile (uniform and plan-launch
//                  batches): two rows per wave, the second row's tile in
//                  flight while the first is reduced; the same statistics.
//   k3_accept_mass the accept step (one wave per sequence, one lane per draft
//                  position: merge the chunk statistics, p_i(x_i) and
//                  q_i(x_i) from the recorded logits, r_i from Philox, first
//                  rejection by ballot; greedy sequences finish here) fused
//                  with pass 2 over the one selected row pair of each
//                  sampling sequence: weight mass max(0, p - q) or p per
//                  1024-element sub-block.
//   k4_draw        one wave per sampling sequence picks the sub-block that
//                  holds u * total and a wave prefix scan inside it finds the
//                  token (inverse CDF in index order).
//   k3_accept_mass_draw  both of the last two in one launch when a sequence's
//                  pass-2 waves fit one workgroup (a barrier, not a kernel
//                  boundary, orders the masses before the draw); with one
//                  wave and one sub-block per sequence the draw walks the
//                  weights that wave left in LDS.
#pragma once

#include <type_traits>

#include "device.hpp"

namespace specv {

// Statistics of one (row, chunk): s = sum over the chunk's elements of
// 2^(fl32(fl32(z - ref_logit(m)) k)) (sampling rows) or 0/NaN (greedy rows, NaN
// flags a NaN/+inf logit); m = max; arg = lowest index attaining m. The
// verify step needs no argmax of a sampling row: there, arg of the chunk
// that holds the row's draft token carries that logit's fp32 bits instead,
// and the other chunks' arg is not written.
struct RowPart {
  double s;
  float m;
  int32_t arg;
};

// What the final draw of one sampling sequence needs (written by the accept step).
enum : int32_t { kModeNone = 0, kModeResidual = 1, kModeBonus = 2 };
// Lenience functions f(p, eps) of the acceptance threshold f(p, eps)/q
// (DistillSpec section 4, lossy SD paragraph; Algorithm A.1 thresholds).
enum : int32_t { kLenNone = 0, kLenLin = 1, kLenSq = 2, kLenExp = 3 };
struct Select {
  int32_t mode;
  int32_t n;
  int64_t trow;  // target row (packed index) of the draw
  int64_t drow;  // draft row for the residual, else -1
  float k;       // log2(e) / T
  float refT, refD;  // reference logits (row maxima) of the selected rows
  int32_t pad;
  double sT, sD;
  double u;
};

// Per-row temperature scale written by k0_plan: k = log2(e)/T_b > 0 for a
// sampling sequence, 0 for a greedy one, -1 for an invalid temperature.
struct PlanArgs {
  const int32_t* gamma;
  const float* temperature;
  int64_t* toff;
  int64_t* doff;
  float* tk;
  float* dk;
  int32_t* dseq;  // optional: the sequence of each draft row
  int32_t* ttok;  // optional: for each target row, the packed index of its
                  // draft token (-1 for a sequence's last row)
  uint32_t* status;
  int64_t total_t, total_d;
  int32_t B, max_gamma;
};

// One workgroup of 1024 threads: thread t owns a contiguous run of sequences.
// Writes the packed row offsets, the per-row temperature scale, and the
// status word (layout error or 0). Runs of up to kPlanKeep sequences per
// thread stay in registers between the scan and the writes.
constexpr int kPlanKeep = 4;

__global__ __launch_bounds__(1024) void k0_plan(PlanArgs a) {
  __shared__ int64_t sh_t[16], sh_d[16];
  __shared__ int sh_bad[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (a.B + 1023) / 1024;
  const int lo = min(a.B, tid * per), hi = min(a.B, lo + per);
  int32_t keep_g[kPlanKeep];
  float keep_k[kPlanKeep];
  int64_t st = 0, sd = 0;
  int bad = 0;
  for (int b = lo; b < hi; ++b) {
    const int32_t g = a.gamma[b];
    const float T = a.temperature[b];
    bad |= (g < 0 || g > a.max_gamma);
    const int64_t gg = g < 0 ? 0 : g;
    st += gg + 1;
    sd += gg;
    if (b - lo < kPlanKeep) {
      keep_g[b - lo] = g;
      keep_k[b - lo] = seq_scale(T);
    }
  }
  // workgroup exclusive scan of (st, sd): waves, then the 16 wave totals
  int64_t it = st, id = sd;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t ot = __shfl_up(it, off, 64), od = __shfl_up(id, off, 64);
    if (lane >= off) { it += ot; id += od; }
  }
  const int wbad = __any(bad) ? 1 : 0;
  if (lane == 63) { sh_t[wave] = it; sh_d[wave] = id; sh_bad[wave] = wbad; }
  __syncthreads();
  int64_t wt = 0, wd = 0, tot_t = 0, tot_d = 0;
  int anybad = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    if (w < wave) { wt += sh_t[w]; wd += sh_d[w]; }
    tot_t += sh_t[w];
    tot_d += sh_d[w];
    anybad |= sh_bad[w];
  }
  if (tid == 0) {
    const bool layout_bad = anybad || tot_t != a.total_t || tot_d != a.total_d;
    a.status[0] = layout_bad ? kLayoutError : 0u;
  }
  int64_t t = wt + it - st, d = wd + id - sd;
  for (int b = lo; b < hi; ++b) {
    int32_t g;
    float kk;
    if (b - lo < kPlanKeep) {
      g = keep_g[b - lo];
      kk = keep_k[b - lo];
    } else {
      g = a.gamma[b];
      const float T = a.temperature[b];
      kk = seq_scale(T);
    }
    const int64_t gg = g < 0 ? 0 : g;
    a.toff[b] = t;
    a.doff[b] = d;
    const int64_t tend = min(t + gg + 1, a.total_t), dend = min(d + gg, a.total_d);
    for (int64_t j = t; j < tend; ++j) a.tk[j] = kk;
    for (int64_t j = d; j < dend; ++j) a.dk[j] = kk;
    if (a.dseq)
      for (int64_t j = d; j < dend; ++j) a.dseq[j] = b;
    if (a.ttok)
      for (int64_t j = t; j < tend; ++j) a.ttok[j] = (j - t < gg) ? (int32_t)(d + (j - t)) : -1;
    t += gg + 1;
    d += gg;
  }
  if (tid == 1023) {
    a.toff[a.B] = tot_t;
    a.doff[a.B] = tot_d;
  }
}

struct RowStatsArgs {
  const void* target;
  const void* draft;
  const float* tk;
  const float* dk;
  RowPart* tparts;
  RowPart* dparts;
  const uint32_t* status;
  int64_t total_t, total_d, V;
  int32_t B, chunks;
  int32_t all_drafts;  // also read the draft rows of greedy sequences
  int32_t bar_k;       // > 0: write the bar_k-th largest lane maximum of each
  float* bar;          //      draft (row, chunk) to bar[row * chunks + chunk]
  int32_t uniform_g;   // >= 0: uniform batch with this gamma (row scales from
  const float* temperature;  // temperature[row / (gamma (+1))], tk/dk unused)
  const int32_t* gamma;  // non-null (uniform batch): workgroup 0 also does the
  uint32_t* status_out;  // plan's check (every gamma == uniform_g) and sets the status word
  // inline_plan (a ragged batch of at most kInlinePlanMax sequences, gamma
  // non-null, uniform_g < 0): no plan launch. Workgroup 0 writes the packed
  // row offsets toff/doff [B + 1] and the status word; every wave finds its
  // row's sequence with a wave scan of the gammas (tk/dk unused).
  int32_t inline_plan, max_gamma;
  int64_t* toff;
  int64_t* doff;
  // tokens non-null (the verify step, no argmax of sampling rows): each
  // sampling row that has a draft token x records its logit z[x] (the accept
  // step's ratio needs it) as it passes: the wave whose chunk holds x writes
  // the float's bits to the arg field of its partial, which sampling rows do
  // not otherwise use; the other chunks leave that field as it was. The token
  // of target row j comes from arithmetic (uniform batch), the wave's own scan
  // (inline plan) or ttok[j] (the plan launch's table).
  const int32_t* tokens;
  const int32_t* ttok;
};

// A 4-byte load from a wave-uniform, 4-byte-aligned address through the
// scalar data cache (constant address space): the value lands in a scalar
// register, so a wave can hold it across its chunk loop at no cost in vector
// registers. Read-only data only.
__device__ __forceinline__ uintptr_t uniform_address(uintptr_t addr) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)addr >> 32));
  return ((uintptr_t)hi << 32) | lo;
}
__device__ __forceinline__ uint32_t scalar_load_u32(uintptr_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(4))) uint32_t*>(uniform_address(addr));
}
__device__ __forceinline__ float scalar_load_f32(const float* p) {
  return __uint_as_float(scalar_load_u32(reinterpret_cast<uintptr_t>(p)));
}

constexpr int kInlinePlanMax = 1024;      // largest ragged batch planned inside pass 1
constexpr int kInlinePlanRun = kInlinePlanMax / kWave;  // sequences per lane in its scans

// Workgroup-wide exclusive scan of one int64 per thread (kBlock threads);
// returns the exclusive prefix and the total in *total.
__device__ __forceinline__ int64_t block_exclusive_scan(int64_t v, int64_t* total) {
  __shared__ int64_t wsum[kWavesPerBlock];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  int64_t incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int64_t o = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int64_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kWavesPerBlock; ++w) {
    before += (w < wave) ? wsum[w] : 0;
    all += wsum[w];
  }
  *total = all;
  return before + incl - v;
}

// The plan of a ragged batch of B <= kInlinePlanMax sequences, by workgroup 0
// of pass 1 (every thread of it takes this branch): thread t owns sequences
// [t P, t P + P), P = ceil(B / kBlock). Writes the packed row offsets
// toff/doff (with the totals at index B) and the status word: layout error
// when a gamma lies outside [0, max_gamma] or the totals differ from the
// shape's, the same rule and offsets as k0_plan.
__device__ void inline_plan_wg0(const RowStatsArgs& a) {
  constexpr int R = kInlinePlanMax / kBlock;
  const int per = (a.B + kBlock - 1) / kBlock;
  const int lo = (int)threadIdx.x * per;
  int32_t g[R];
  int64_t st = 0, sd = 0;
  bool bad = false;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int b = lo + i;
    g[i] = (i < per && b < a.B) ? a.gamma[b] : 0;
    bad |= (i < per && b < a.B) && (g[i] < 0 || g[i] > a.max_gamma);
    const int64_t gg = g[i] < 0 ? 0 : g[i];
    if (i < per && b < a.B) {
      st += gg + 1;
      sd += gg;
    }
  }
  int64_t tot_t, tot_d;
  int64_t t = block_exclusive_scan(st, &tot_t);
  __syncthreads();  // the scan's LDS is reused by the second scan
  int64_t d = block_exclusive_scan(sd, &tot_d);
  bad = __syncthreads_or(bad);
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int b = lo + i;
    if (i < per && b < a.B) {
      const int64_t gg = g[i] < 0 ? 0 : g[i];
      a.toff[b] = t;
      a.doff[b] = d;
      t += gg + 1;
      d += gg;
    }
  }
  if (threadIdx.x == 0) {
    a.toff[a.B] = tot_t;
    a.doff[a.B] = tot_d;
    const bool layout_bad = bad || tot_t != a.total_t || tot_d != a.total_d;
    a.status_out[0] = layout_bad ? kLayoutError : 0u;
  }
}

// The sequence that owns packed target row j (draft row j with `draft`) of a
// ragged batch of B <= kInlinePlanMax sequences, by one wave: lane l counts
// the rows of sequences [l P, l P + P), P = ceil(B / 64), a wave scan of the
// counts finds the lane whose run holds row j, and that run is walked with
// v_readlane. The counts follow k0_plan (a negative gamma counts as 0);
// gammas are also capped at max_gamma here, which changes no valid batch and
// keeps the sums small. Also reports the sequence's first row and its row
// count. A row past the total (only in a batch with a layout error, which
// the accept step reports) maps to the last sequence, with first row -1.
__device__ __forceinline__ int32_t row_sequence(const RowStatsArgs& a, int64_t j, bool draft,
                                                int lane, int64_t* first_row, int32_t* n_rows) {
  constexpr int R = kInlinePlanRun;
  const int per = (a.B + kWave - 1) / kWave;
  const int lo = lane * per;
  int32_t c[R];
  int32_t sum = 0;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int b = lo + i;
    int32_t g = (i < per && b < a.B) ? a.gamma[b] : -1;
    g = g < 0 ? 0 : (g > a.max_gamma ? a.max_gamma : g);
    c[i] = (i < per && b < a.B) ? g + (draft ? 0 : 1) : 0;
    sum += c[i];
  }
  int32_t incl = sum;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int32_t o = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += o;
  }
  const uint64_t m = ballot((int64_t)incl > j);
  if (!m) {
    *first_row = -1;
    *n_rows = 0;
    return a.B - 1;
  }
  const int L = first_lane(m);
  int64_t cum = __builtin_amdgcn_readlane(incl - sum, L);
  int found = -1;
  int64_t start = 0;
  int32_t cnt = 0;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int32_t ci = __builtin_amdgcn_readlane(c[i], L);
    if (found < 0 && cum + ci > j) {
      found = i;
      start = cum;
      cnt = ci;
    }
    cum += ci;
  }
  *first_row = start;
  *n_rows = cnt;
  return L * per + found;
}

// Pass-1 loop over one (row, chunk), double-buffered: the loads of tile it+1
// are in flight while tile it is processed. A row is cut into tiles of EPI
// elements; chunk c of a row with C chunks is the tiles t = c, c + C, c + 2C,
// ..., so the C waves of a row read neighbouring tiles at about the same time
// (DRAM locality of the concurrently active waves). Within a lane, element
// indices grow with the iteration. `a` holds tile c on entry (the caller
// issues it before its metadata lookups).
//
// Sampling rows: online (max, sum). Per element: widen, max (v_max3), one fma
// and one v_exp_f32 into a pairwise sum; the per-lane running sum is float64,
// rescaled only when the lane's maximum grows. Greedy rows: max, argmax and
// a NaN/+inf check only. For the argmax (greedy rows, or WITH_ARG) a lane
// remembers the iteration where its maximum last grew and re-reads that one
// tile at the end.
template <int DT, bool VEC>
__device__ __forceinline__ void load_tile(const void* row, int64_t V, int64_t t, int lane,
                                          typename Tile<DT, VEC>::Raw& r) {
  using TL = Tile<DT, VEC>;
  const int64_t e0 = t * TL::EPI;
  if (e0 + TL::EPI <= V) TL::template load_raw<false>(row, e0, V, 0, lane, r);
  else TL::template load_raw<true>(row, e0, V, 0, lane, r);
}

//
// With STORE, every tile is also written to `dst` (a row of the same length)
// as it is processed: a producer that writes the rows computes their
// statistics in the same pass.
//
// With cap >= 0 (Tile::capture_code of one element of the chunk), the lane
// that holds that element stores its logit's fp32 bits to *cap_dst after the
// loop. Every tile takes its candidate dword with a uniform-index register
// move and keeps it when the tile is the element's: no branch in the loop (a
// branch there made the compiler drain the tile in flight at each back edge).
//
// With ONE, `a` is the row's only tile (n_iter == 1, chunks == 1) and the
// argmax reads it from the registers instead of loading it again: the same
// values, so the same result.
template <int DT, bool VEC, bool SAMPLING, bool WITH_ARG, bool STORE = false, bool ONE = false>
__device__ __forceinline__ RowPart chunk_pass(const void* row, int64_t V, int c, int chunks,
                                              int n_iter, float k, int lane,
                                              typename Tile<DT, VEC>::Raw& a, float& lane_max,
                                              void* dst = nullptr, int32_t cap = -1,
                                              uint32_t* cap_dst = nullptr) {
  using TL = Tile<DT, VEC>;
  using Raw = typename TL::Raw;
  constexpr int NE = TL::NE;
  constexpr bool ARG = WITH_ARG || !SAMPLING;
  float m = ninf();
  double s = 0.0;
  bool bad = false;
  int best = -1;
  uint32_t capv = 0u;
  auto process = [&](const Raw& raw, int it) {
    if constexpr (STORE) TL::store_raw(dst, ((int64_t)c + (int64_t)it * chunks) * TL::EPI, V, 0, lane, raw);
    if constexpr (SAMPLING && !WITH_ARG && !STORE) {
      static_assert(TL::RD == 16, "the capture indexes 16 raw dwords");
      typedef uint32_t v16 __attribute__((ext_vector_type(16)));
      v16 vv;
#pragma unroll
      for (int q = 0; q < 16; ++q) vv[q] = raw.d[q];
      const uint32_t w = vv[(cap >> 7) & 15];
      capv = ((cap >> 11) == it) ? w : capv;
    }
    float z[NE];
    TL::widen(raw, z);
    const float g = tile_max(z);
    if constexpr (ARG) best = (g > m) ? it : best;
    if constexpr (SAMPLING) {
      const float mn = fmaxf(m, g);
      const float sc = rescale32(m, mn, k);
      const float ref = ref_logit(mn);
      float e[NE];
#pragma unroll
      for (int j = 0; j < NE; ++j) e[j] = exp2_hw(term_exp(z[j], ref, k));
      const float acc = tree_sum(e);
      s = __builtin_fma(s, (double)sc, (double)acc);
      m = mn;
    } else {
#pragma unroll
      for (int j = 0; j < NE; ++j) bad |= !(z[j] < pinf());
      m = fmaxf(m, g);
    }
  };
  auto tile_of = [&](int it) { return (int64_t)c + (int64_t)it * chunks; };
  Raw b;
  int it = 0;
  if constexpr (ONE) {
    process(a, 0);
  } else if constexpr (DT == kBF16) {
    // Only a chunk's last tile can be partial (it is the row's last tile).
    // This loop loads full tiles only, with no branch around the loads: each
    // step issues one tile and then works on the one before it, so the
    // compiler's wait before that work leaves the new tile in flight (a load
    // under a branch makes it wait for every load). The last one to three
    // tiles take the loop below. For fp32 tiles the extra live tile costs
    // occupancy (7 -> 5 waves per SIMD) and the plain loop is faster.
    for (; it + 3 < n_iter; it += 2) {
      TL::template load_raw<false>(row, tile_of(it + 1) * TL::EPI, V, 0, lane, b);
      process(a, it);
      TL::template load_raw<false>(row, tile_of(it + 2) * TL::EPI, V, 0, lane, a);
      process(b, it + 1);
    }
  }
  if constexpr (!ONE) {
    for (; it < n_iter; it += 2) {
      if (it + 1 < n_iter) load_tile<DT, VEC>(row, V, tile_of(it + 1), lane, b);
      process(a, it);
      if (it + 1 >= n_iter) break;
      if (it + 2 < n_iter) load_tile<DT, VEC>(row, V, tile_of(it + 2), lane, a);
      process(b, it + 1);
    }
  }
  lane_max = m;
  if constexpr (SAMPLING && !WITH_ARG && !STORE) {
    if (cap >= 0 && lane == (cap & 63)) *cap_dst = TL::bits_of(capv, cap);
  }
  // wave merge: maximum first, then one rescale per lane and a float64 sum
  const float M = wave_max(m);
  double S;
  if constexpr (SAMPLING) {
    const double f = (m == ninf()) ? 0.0 : exp2(((double)m - (double)ref_logit(M)) * (double)k);
    S = wave_sum(s * f);
  } else {
    S = (ballot(bad) != 0) ? __builtin_nan("") : 0.0;
  }
  int arg = INT32_MAX;
  if constexpr (ARG) {
    if (best >= 0 && m == M) {
      const int64_t e0 = tile_of(best) * TL::EPI;
      float z[NE];
      if constexpr (ONE) TL::widen(a, z);
      else TL::template load<true>(row, e0, V, 0, lane, z);
#pragma unroll
      for (int j = NE - 1; j >= 0; --j)
        if (z[j] == m) arg = (int)TL::index(e0, 0, lane, j);
    }
    arg = wave_min(arg);
  }
  return RowPart{S, M, arg};
}

template <int DT, bool VEC, bool WITH_ARG>
__global__ __launch_bounds__(kBlock) void k1_row_stats(RowStatsArgs a) {
  using TL = Tile<DT, VEC>;
  if (a.inline_plan && blockIdx.x == 0) {
    // A ragged batch's plan, in this launch (offsets read after it ends).
    inline_plan_wg0(a);
  } else if (a.gamma && blockIdx.x == 0) {
    // The uniform batch's plan, in this launch: offsets and row scales are
    // arithmetic, so only the gammas are checked and the status word is set
    // (read after this launch ends). The whole workgroup takes this branch
    // before any of its waves can return.
    bool bad = false;
    for (int64_t b = threadIdx.x; b < a.B; b += blockDim.x) bad |= a.gamma[b] != a.uniform_g;
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) a.status_out[0] = bad ? kLayoutError : 0u;
  }
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t item = wave_uniform((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  const int64_t rows = a.total_t + a.total_d;
  if (item >= rows * a.chunks) return;
  const int64_t r = item / a.chunks;
  const int c = (int)(item - r * a.chunks);
  const bool is_draft = r >= a.total_t;
  const int64_t j = is_draft ? r - a.total_t : r;
  constexpr int64_t esz = (DT == kBF16) ? 2 : 4;
  const void* row = static_cast<const char*>(is_draft ? a.draft : a.target) + j * a.V * esz;
  const int64_t tiles = (a.V + TL::EPI - 1) / TL::EPI;  // >= chunks
  const int n_iter = (int)((tiles - c + a.chunks - 1) / a.chunks);
  // Target rows are always read: tile c is in flight while the row's scale
  // and the status word are looked up. Draft rows are read only for sampling
  // sequences, so their scale comes first.
  // With the plan inside this launch the scale takes two dependent loads
  // (the gammas, then T_b): the first tile of a draft row is then requested
  // before them too, at the cost of one unneeded tile per (row, chunk) of a
  // greedy sequence.
  typename TL::Raw first;
  float k;
  // The row's draft token (packed index; -1 for a sequence's last target
  // row), for the capture of its logit below. Scalar loads: the token and the
  // temperature come from wave-uniform addresses.
  int64_t tok = -1;
  if (is_draft && !a.inline_plan) {
    tok = j;
    k = (a.uniform_g >= 0) ? seq_scale(scalar_load_f32(a.temperature + j / a.uniform_g))
                           : scalar_load_f32(a.dk + j);
    // greedy (or invalid) sequence: the verify step needs no draft row
    if (!(k > 0.f) && !(a.all_drafts && k == 0.f)) return;
    load_tile<DT, VEC>(row, a.V, c, lane, first);
  } else {
    load_tile<DT, VEC>(row, a.V, c, lane, first);
    if (a.inline_plan) {
      int64_t first_row;
      int32_t n_rows;
      const int32_t sb = row_sequence(a, j, is_draft, lane, &first_row, &n_rows);
      // target row i of sequence sb: its token is draft row doff + i, with
      // doff = (the sequence's first target row) - sb; none for the last row
      if (is_draft) tok = j;
      else if (first_row >= 0 && j - first_row < n_rows - 1) tok = (first_row - sb) + (j - first_row);
      k = seq_scale(scalar_load_f32(a.temperature + sb));
    } else if (a.uniform_g >= 0) {  // a target row (draft rows: inline plan only)
      const int64_t sb = j / (a.uniform_g + 1), i = j - sb * (a.uniform_g + 1);
      tok = (i < a.uniform_g) ? sb * a.uniform_g + i : -1;
      k = seq_scale(scalar_load_f32(a.temperature + sb));
    } else {
      if (a.ttok) tok = (int32_t)scalar_load_u32(reinterpret_cast<uintptr_t>(a.ttok + j));
      k = scalar_load_f32(a.tk + j);
    }
    if (is_draft) {
      if (!(k > 0.f) && !(a.all_drafts && k == 0.f)) return;
    } else if (!(k >= 0.f)) {
      return;  // invalid temperature: the accept step fails the sequence
    }
  }
  // The draft token's logit for the accept step: the wave whose chunk holds
  // token x takes it from the tile in its registers (capture code below). A
  // token outside [0, V) is recorded nowhere: the accept step fails that
  // sequence without looking for it.
  int32_t cap = -1;
  if constexpr (!WITH_ARG) {
    if (a.tokens && k > 0.f && tok >= 0 && tok < a.total_d) {
      const int32_t x = (int32_t)scalar_load_u32(reinterpret_cast<uintptr_t>(a.tokens + tok));
      if (x >= 0 && (int64_t)x < a.V) {
        const int64_t t = x / TL::EPI;
        if (t % a.chunks == c) cap = TL::capture_code((int)(t / a.chunks), (int)(x - t * TL::EPI));
      }
    }
  }
  // a uniform batch reads only arithmetic offsets, and a batch planned in
  // this launch only its gammas: their rows are computed whatever the gammas
  // hold, and the accept step reports a layout error
  if (!a.gamma && (a.status[0] & kLayoutError)) return;
  // outputs addressed before the chunk loop: fewer scalar registers live
  // across it (the kernel is at the scalar register limit)
  RowPart* const dst = (is_draft ? a.dparts : a.tparts) + j * a.chunks + c;
  float* const bar_dst = (is_draft && a.bar_k > 0) ? a.bar + j * a.chunks + c : nullptr;
  const int32_t bar_k = a.bar_k;
  RowPart out;
  float lm;
  const bool capturing = !WITH_ARG && a.tokens && k > 0.f;
  if (k > 0.f)
    out = chunk_pass<DT, VEC, true, WITH_ARG>(row, a.V, c, a.chunks, n_iter, k, lane, first, lm, nullptr,
                                              cap, reinterpret_cast<uint32_t*>(&dst->arg));
  else
    out = chunk_pass<DT, VEC, false, true>(row, a.V, c, a.chunks, n_iter, 0.f, lane, first, lm);
  if (lane == 0) {
    if (capturing) {  // the arg field is the capture's
      dst->s = out.s;
      dst->m = out.m;
    } else {
      *dst = out;
    }
  }
  if (bar_dst) {
    // The bar_k-th largest of the lanes' maxima: a logit of the chunk with
    // at least bar_k logits of the chunk at or above it (-inf when fewer
    // lanes hold a logit), for the top-k selection of the diagnostics.
    int rank = 0;
#pragma unroll
    for (int l = 0; l < kWave; ++l) {
      const float o = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(lm), l));
      rank += (o > lm || (o == lm && l < lane)) ? 1 : 0;
    }
    if (rank == bar_k - 1) *bar_dst = lm;
  }
}

// Pass 1 for rows of one tile (vector path, V <= EPI, so one chunk per row)
// in a uniform or planned batch, without the diagnostics' extras: each wave
// takes R consecutive rows (target rows, then draft rows, numbered as
// k1_row_stats numbers them) and keeps the next row's tile in flight while it
// works on the current one (with one such row per wave, a wave would have
// nothing of its own in flight during its reductions). A row that is not
// read (the draft row of a greedy sequence, a row with an invalid
// temperature, one past the last row) loads the first target row's tile
// instead, so that no load sits under a branch, and writes nothing. Each row
// gets the statistics k1_row_stats gives it, bit for bit: the same
// chunk_pass on the same tile.
template <int DT, int R>
__global__ __launch_bounds__(kBlock) void k1_short_rows(RowStatsArgs a) {
  static_assert(R >= 2 && R % 2 == 0, "rows per wave: a positive even number");
  using TL = Tile<DT, true>;
  using Raw = typename TL::Raw;
  if (a.gamma && blockIdx.x == 0) {
    // the uniform batch's check of its gammas, as in k1_row_stats
    bool bad = false;
    for (int64_t b = threadIdx.x; b < a.B; b += blockDim.x) bad |= a.gamma[b] != a.uniform_g;
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) a.status_out[0] = bad ? kLayoutError : 0u;
  }
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t r0 = wave_uniform(((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6)) * R);
  const int64_t rows = a.total_t + a.total_d;
  if (r0 >= rows) return;
  if (!a.gamma && (a.status[0] & kLayoutError)) return;
  constexpr int64_t esz = (DT == kBF16) ? 2 : 4;
  struct Row {
    const void* row;
    RowPart* dst;  // nullptr: the row is not read
    float k;
    int32_t cap;
  };
  // The row's logits, scale and capture code, found as k1_row_stats finds
  // them (scalar loads only).
  auto row_of = [&](int64_t r) {
    Row w{a.target, nullptr, 0.f, -1};
    if (r >= rows) return w;
    const bool is_draft = r >= a.total_t;
    const int64_t j = is_draft ? r - a.total_t : r;
    int64_t tok = -1;
    float k;
    if (a.uniform_g >= 0) {
      int64_t sb;
      if (is_draft) {
        sb = j / a.uniform_g;
        tok = j;
      } else {
        sb = j / (a.uniform_g + 1);
        const int64_t i = j - sb * (a.uniform_g + 1);
        tok = (i < a.uniform_g) ? sb * a.uniform_g + i : -1;
      }
      k = seq_scale(scalar_load_f32(a.temperature + sb));
    } else if (is_draft) {
      tok = j;
      k = scalar_load_f32(a.dk + j);
    } else {
      if (a.ttok) tok = (int32_t)scalar_load_u32(reinterpret_cast<uintptr_t>(a.ttok + j));
      k = scalar_load_f32(a.tk + j);
    }
    // greedy or invalid sequences need no draft row; an invalid temperature
    // needs no target row either (the accept step fails the sequence)
    const bool read = is_draft ? (k > 0.f || (a.all_drafts && k == 0.f)) : (k >= 0.f);
    if (!read) return w;
    w.row = static_cast<const char*>(is_draft ? a.draft : a.target) + j * a.V * esz;
    w.dst = (is_draft ? a.dparts : a.tparts) + j;
    w.k = k;
    if (a.tokens && k > 0.f && tok >= 0 && tok < a.total_d) {
      const int32_t x = (int32_t)scalar_load_u32(reinterpret_cast<uintptr_t>(a.tokens + tok));
      if (x >= 0 && (int64_t)x < a.V) w.cap = TL::capture_code(0, x);
    }
    return w;
  };
  auto work = [&](const Row& w, Raw& t) {
    if (!w.dst) {
      // Unused tile: its loads are waited for here all the same. A path that
      // left them outstanding made the compiler wait, after the join, for
      // the next row's tile too before it reused these registers.
#pragma unroll
      for (int q = 0; q < TL::RD; ++q) asm volatile("" ::"v"(t.d[q]));
      return;
    }
    RowPart out;
    float lm;
    const bool sampling = w.k > 0.f;
    if (sampling)
      out = chunk_pass<DT, true, true, false, false, true>(w.row, a.V, 0, 1, 1, w.k, lane, t, lm, nullptr,
                                                           w.cap, reinterpret_cast<uint32_t*>(&w.dst->arg));
    else
      out = chunk_pass<DT, true, false, true, false, true>(w.row, a.V, 0, 1, 1, 0.f, lane, t, lm);
    if (lane == 0) {
      if (sampling && a.tokens) {  // the arg field is the capture's
        w.dst->s = out.s;
        w.dst->m = out.m;
      } else {
        *w.dst = out;
      }
    }
  };
  Raw ta, tb;
  Row wa = row_of(r0);
  TL::load_only_tile(wa.row, a.V, lane, ta);
#pragma unroll
  for (int i = 0; i < R; i += 2) {
    const Row wb = row_of(r0 + i + 1);
    TL::load_only_tile(wb.row, a.V, lane, tb);
    work(wa, ta);
    if (i + 2 < R) {
      wa = row_of(r0 + i + 2);
      TL::load_only_tile(wa.row, a.V, lane, ta);
    }
    work(wb, tb);
  }
}

// Per-row merge of the chunk statistics.
struct RowStat {
  double s;    // sum of 2^(fl32(fl32(z - ref) k)) over the row (sampling), 0/NaN (greedy)
  float m;     // row max
  float ref;   // ref_logit(m)
  int32_t arg; // lowest index attaining m
  bool valid;  // no NaN/+inf and at least one finite logit
};

// The first four chunk partials of a row (padding past `chunks`), loaded on
// their own so that a caller can issue them early.
__device__ __forceinline__ void load_parts4(const RowPart* p, int chunks, RowPart (&q)[4]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) q[u] = (u < chunks) ? p[u] : RowPart{0.0, ninf(), INT32_MAX};
}

// Merge of a row's chunk partials, the first four given. With cx >= 0, *cap
// also receives the arg field of chunk cx (the logit bits that pass 1
// recorded there) as the loop passes it.
__device__ __forceinline__ RowStat merge_row_from(const RowPart (&q0)[4], const RowPart* p,
                                                  int chunks, float k, bool sampling, int cx = -1,
                                                  uint32_t* cap = nullptr) {
  // Chunks in order, four loads in flight at a time: a running maximum (the
  // lowest index attaining it gives the argmax), the running sum moved onto
  // the new maximum's reference when it grows, and each group's terms moved
  // onto the group's maximum. The factors come from v_exp_f32 (within 1 ulp);
  // the chunk that holds the maximum gets exactly 1, so the error only
  // touches the other chunks' share of the sum, as in the in-chunk rescales.
  float M = ninf();
  double S = 0.0;
  int32_t arg = INT32_MAX;
  for (int c0 = 0; c0 < chunks; c0 += 4) {
    RowPart q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      q[u] = (c0 == 0) ? q0[u] : (c0 + u < chunks) ? p[c0 + u] : RowPart{0.0, ninf(), INT32_MAX};
    if (cx >= 0) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (c0 + u == cx) *cap = (uint32_t)q[u].arg;
    }
    float mg = M;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      // chunks interleave tiles: on equal maxima keep the lowest index
      if (q[u].m > mg) arg = q[u].arg;
      else if (q[u].m == mg) arg = min(arg, q[u].arg);
      mg = fmaxf(mg, q[u].m);
    }
    if (sampling) {
      double add = 0.0;
#pragma unroll
      for (int u = 0; u < 4; ++u) add += q[u].s * (double)rescale32(q[u].m, mg, k);
      S = S * (double)rescale32(M, mg, k) + add;
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) S += q[u].s;
    }
    M = mg;
  }
  RowStat st;
  st.s = S;
  st.m = M;
  st.ref = ref_logit(M);
  st.arg = arg;
  st.valid = (M > ninf()) && (M < pinf()) && !__builtin_isnan(S);
  return st;
}

__device__ __forceinline__ RowStat merge_row(const RowPart* p, int chunks, float k, bool sampling) {
  RowPart q0[4];
  load_parts4(p, chunks, q0);
  return merge_row_from(q0, p, chunks, k, sampling);
}

struct AcceptArgs {
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const int32_t* gamma;
  const float* temperature;
  const int64_t* toff;
  const int64_t* doff;
  const RowPart* tparts;
  const RowPart* dparts;
  uint32_t* status;
  Select* sel;
  int32_t* out_n;
  int32_t* out_next;
  const float* inj_r;
  const float* inj_u;
  uint64_t seed, row_offset;
  int64_t V;
  int32_t B, max_gamma, chunks;
  int32_t lenience;  // kLen*; kLenNone is the lossless step
  float eps;         // lenience parameter in (0, 1)
  int32_t uniform_g;  // >= 0: uniform batch with this gamma (offsets arithmetic)
  // > 0: pass 1 recorded each draft token's logit in the partial of the
  // chunk that holds it, with tiles of 1 << cap_shift elements; 0: the
  // accept step reads the logits from the rows
  int32_t cap_shift;
};

// f(p, eps): p / eps, p / eps^2 or p^eps, in float64 (f(p, 1) = p; the host
// passes kLenNone for eps = 1).
__device__ __forceinline__ double lenient(double p, int32_t kind, float eps) {
  const double e = (double)eps;
  if (kind == kLenLin) return p / e;
  if (kind == kLenSq) return p / (e * e);
  if (kind == kLenExp) return pow(p, e);
  return p;
}

// The accept step of one sequence, by one wave; lane i owns draft position i
// and target row i. Returns the selection for the final draw (kModeNone for
// greedy and failed sequences, which are finished here). With `write` the
// wave also stores n (and the token of a greedy or failed sequence), the
// selection, and the status bit of a data error.
template <int DT>
__device__ Select accept_sequence(const AcceptArgs& a, int64_t b, int lane, bool write) {
  Select s{};
  s.mode = kModeNone;
  auto finish = [&](int n, int next, bool error) {
    if (write && lane == 0) {
      a.out_n[b] = n;
      a.out_next[b] = next;
      a.sel[b] = s;
      if (error) atomicOr(a.status, kSeqError);
    }
    return s;
  };
  // Independent loads first, so that they are in flight together. In a
  // uniform batch gamma and the offsets are known without any load, so the
  // chunk partials and the draft tokens are requested with the metadata (all
  // addresses stay inside the packed arrays whatever the data holds).
  const bool uni = a.uniform_g >= 0;
  const uint32_t status = a.status[0];
  const int g = uni ? a.uniform_g : a.gamma[b];
  const float T = a.temperature[b];
  const int64_t t0 = uni ? b * (a.uniform_g + 1) : a.toff[b];
  const int64_t d0 = uni ? b * a.uniform_g : a.doff[b];
  RowPart tq[4], dq[4];
  int x = 0;
  if (uni) {
    if (lane <= g) load_parts4(a.tparts + (t0 + lane) * a.chunks, a.chunks, tq);
    if (lane < g) {
      x = a.tokens[d0 + lane];
      load_parts4(a.dparts + (d0 + lane) * a.chunks, a.chunks, dq);
    }
  }
  if (status & kLayoutError) return finish(-1, -1, false);
  const bool greedy = (T == 0.f);
  const bool sampling = sampling_temperature(T);
  if (!greedy && !sampling) return finish(-1, -1, true);
  const float k = sampling ? temp_scale(T) : 0.f;
  if (!uni) {  // a valid layout: the offsets address the packed arrays
    if (lane <= g) load_parts4(a.tparts + (t0 + lane) * a.chunks, a.chunks, tq);
    if (lane < g) {
      x = a.tokens[d0 + lane];
      if (sampling) load_parts4(a.dparts + (d0 + lane) * a.chunks, a.chunks, dq);
    }
  }
  // the chunk whose partial holds x's logit, where pass 1 recorded it
  const bool captured = a.cap_shift > 0;
  int cx = -1;
  if (captured && sampling && lane < g && x >= 0 && (int64_t)x < a.V) cx = (x >> a.cap_shift) % a.chunks;
  uint32_t zTb = 0u, zDb = 0u;
  RowStat st_t{}, st_d{};
  bool bad = false;
  if (lane <= g) {
    st_t = merge_row_from(tq, a.tparts + (t0 + lane) * a.chunks, a.chunks, k, sampling, cx, &zTb);
    bad |= !st_t.valid;
  }
  if (lane < g) {
    bad |= (x < 0) || ((int64_t)x >= a.V);
    if (sampling) {
      st_d = merge_row_from(dq, a.dparts + (d0 + lane) * a.chunks, a.chunks, k, true, cx, &zDb);
      bad |= !st_d.valid;
    }
  }
  if (ballot(bad) != 0) return finish(-1, -1, true);

  if (greedy) {
    const uint64_t rej = ballot(lane < g && x != st_t.arg);
    const int n = rej ? first_lane(rej) : g;
    return finish(n, __shfl(st_t.arg, n, kWave), false);
  }

  // Sampling: block (row, i) of Philox gives r_i (word 0) and the uniform of
  // a final draw at position i (word 1).
  const uint64_t prow = a.row_offset + (uint64_t)b;
  double r = 0.0, u = 0.0;
  if (lane <= g) {
    const PhiloxBlock w = philox4x32_10(a.seed, (uint32_t)prow, (uint32_t)(prow >> 32), (uint32_t)lane, 0u);
    if (lane < g) r = a.inj_r ? (double)a.inj_r[b * a.max_gamma + lane] : (double)uniform24(w.w0);
    u = a.inj_u ? (double)a.inj_u[b] : (double)uniform24(w.w1);
  }
  bool rej = false;
  if (lane < g) {
    float zT, zD;
    if (captured) {
      zT = __uint_as_float(zTb);
      zD = __uint_as_float(zDb);
    } else {
      zT = load_logit<DT>(a.target, (t0 + lane) * a.V + x);
      zD = load_logit<DT>(a.draft, (d0 + lane) * a.V + x);
    }
    const double p = exp2(((double)zT - (double)st_t.ref) * (double)k) / st_t.s;
    const double q = exp2(((double)zD - (double)st_d.ref) * (double)k) / st_d.s;
    const double ratio = (q == 0.0) ? (double)pinf() : lenient(p, a.lenience, a.eps) / q;
    rej = r > ratio;
  }
  const uint64_t mask = ballot(rej);
  const int n = mask ? first_lane(mask) : g;
  s.mode = (n < g) ? kModeResidual : kModeBonus;
  s.n = n;
  s.trow = t0 + n;
  s.drow = (n < g) ? d0 + n : -1;
  s.k = k;
  s.refT = __shfl(st_t.ref, n, kWave);
  s.refD = __shfl(st_d.ref, n, kWave);
  s.pad = 0;
  s.sT = __shfl(st_t.s, n, kWave);
  s.sD = __shfl(st_d.s, n, kWave);
  s.u = __shfl(u, n, kWave);
  if (write && lane == 0) {
    a.out_n[b] = n;
    a.sel[b] = s;
  }
  return s;
}

// The selection is the same in every lane after the accept step's shuffles;
// v_readfirstlane moves it to scalar registers for the passes that follow.
__device__ __forceinline__ double uniform_f64(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ float uniform_f32(float v) {
  return __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(v)));
}
__device__ __forceinline__ Select uniform_select(const Select& s) {
  Select u;
  u.mode = __builtin_amdgcn_readfirstlane(s.mode);
  u.n = __builtin_amdgcn_readfirstlane(s.n);
  u.trow = wave_uniform(s.trow);
  u.drow = wave_uniform(s.drow);
  u.k = uniform_f32(s.k);
  u.refT = uniform_f32(s.refT);
  u.refD = uniform_f32(s.refD);
  u.pad = 0;
  u.sT = uniform_f64(s.sT);
  u.sD = uniform_f64(s.sD);
  u.u = uniform_f64(s.u);
  return u;
}

// Weight of one token in the final draw: max(0, p - q) or p, in fp32. Two
// forms of p = 2^((z - M) k) / S (M the row maximum), equal to fp32
// rounding:
//   exact (any logits): 2^(fl32(fl32(z - M) k)) * fl32(1/S);
//   FMA, where |fl32(M k)| < 2^24 (every realistic row): 2^(fl32(z k - r)) * c
//     with r = fl32(M k) and c = fl32(2^-e / S), e = M k - r exactly (one
//     fma): the terms' common factor 2^e (|e| <= 1 there) is divided out.
// The form is chosen once per sequence (weights_fma: both rows of a
// residual) and serves both the masses and the draw's walk, so they agree
// bit for bit. With log2(1/S) folded into the exponent instead, a likely
// token's exponent sits near -log2 S, where fp32 resolves only about 2^-19:
// ten times the error of the product form.
template <bool FMA>
struct Weights {
  float k, aT, aD, cT, cD;  // aT = M (exact form) or r (FMA form); cT the multiplier
  bool residual;
  __device__ __forceinline__ float operator()(float zT, float zD) const {
    const float pT = exp2_hw(FMA ? __builtin_fmaf(zT, k, -aT) : term_exp(zT, aT, k)) * cT;
    if (!residual) return pT;
    const float pD = exp2_hw(FMA ? __builtin_fmaf(zD, k, -aD) : term_exp(zD, aD, k)) * cD;
    return fmaxf(pT - pD, 0.f);
  }
};

__device__ __forceinline__ bool residual_weights(const Select& s, bool force_bonus) {
  return (s.mode == kModeResidual) && !force_bonus;
}

__device__ __forceinline__ bool weights_fma(const Select& s, bool force_bonus) {
  constexpr float kLim = 16777216.f;  // 2^24: |M k - fl32(M k)| <= 1 below it
  return fabsf(s.refT * s.k) < kLim && (!residual_weights(s, force_bonus) || fabsf(s.refD * s.k) < kLim);
}

template <bool FMA>
__device__ __forceinline__ Weights<FMA> make_weights(const Select& s, bool force_bonus) {
  Weights<FMA> w;
  w.k = s.k;
  w.residual = residual_weights(s, force_bonus);
  if constexpr (FMA) {
    w.aT = s.refT * s.k;
    w.aD = s.refD * s.k;
    const float eT = __builtin_fmaf(s.refT, s.k, -w.aT), eD = __builtin_fmaf(s.refD, s.k, -w.aD);
    w.cT = (float)((double)exp2_hw(-eT) / s.sT);
    w.cD = (float)((double)exp2_hw(-eD) / s.sD);
  } else {
    w.aT = s.refT;
    w.aD = s.refD;
    w.cT = (float)(1.0 / s.sT);
    w.cD = (float)(1.0 / s.sD);
  }
  return w;
}

constexpr int kSub = 1024;  // elements per sub-block of the final draw

struct DrawArgs {
  const void* target;
  const void* draft;
  const Select* sel;
  double* sub;        // [B, nsub] weight mass of each 1024-element sub-block
  int32_t* out_next;
  int64_t V;
  int32_t B, chunks3, nsub;
  // k3_accept_mass_draw with one wave and one sub-block per sequence: the
  // launch's LDS also holds the wave's weights (16 bytes after the mass)
  int32_t weights_in_lds;
};

// Wave-level inclusive scan of a sequence's sub-block masses in passes of 64
// entries with a carry. t < 0: returns -1 and the total (the inclusive prefix
// through the last entry; entries past nsub add exact zeros). t >= 0: returns
// the first entry whose inclusive prefix reaches t and its exclusive prefix
// in *base. Both modes make the same additions in the same order, so any
// t <= total finds an entry.
__device__ int64_t wave_scan_subs(const double* sub, int64_t nsub, double t, int lane, double* base,
                                  double* total) {
  double carry = 0.0;
  for (int64_t p = 0; p < nsub; p += kWave) {
    const int64_t i = p + lane;
    const double v = (i < nsub) ? sub[i] : 0.0;
    const double incl = wave_inclusive_scan(v, lane) + carry;
    const double prev = __shfl_up(incl, 1, kWave);
    const double excl = (lane == 0) ? carry : prev;
    if (t >= 0.0) {
      const uint64_t m = ballot(i < nsub && incl >= t);
      if (m) {
        const int L = first_lane(m);
        if (base) *base = __shfl(excl, L, kWave);
        return p + L;
      }
    }
    carry = __shfl(incl, kWave - 1, kWave);
  }
  if (total) *total = carry;
  return -1;
}

// The same scan over masses held in registers: lane l holds entries l,
// l + 64, ... of at most kSubRegs passes (nsub <= 64 kSubRegs), requested all
// at once, so the draw waits for them once instead of once per 64-entry pass
// of each of its two scans. One sweep keeps every pass's prefixes; they are
// the same additions in the same order as wave_scan_subs, so the total and
// the located entry have the same bits.
constexpr int kSubRegs = 4;

__device__ __forceinline__ bool subs_fit_regs(int64_t nsub) { return nsub <= (int64_t)kWave * kSubRegs; }

__device__ __forceinline__ void load_subs(const double* sub, int64_t nsub, int lane, double (&v)[kSubRegs]) {
#pragma unroll
  for (int q = 0; q < kSubRegs; ++q) {
    const int64_t i = (int64_t)q * kWave + lane;
    v[q] = (i < nsub) ? sub[i] : 0.0;
  }
}

struct SubPrefix {
  double incl[kSubRegs], excl[kSubRegs];
  double total;
};

__device__ __forceinline__ void scan_subs_regs(const double (&v)[kSubRegs], int64_t nsub, int lane,
                                               SubPrefix& P) {
  double carry = 0.0;
#pragma unroll
  for (int q = 0; q < kSubRegs; ++q) {
    P.incl[q] = 0.0;
    P.excl[q] = 0.0;
    if ((int64_t)q * kWave < nsub) {
      P.incl[q] = wave_inclusive_scan(v[q], lane) + carry;
      const double prev = __shfl_up(P.incl[q], 1, kWave);
      P.excl[q] = (lane == 0) ? carry : prev;
      carry = __shfl(P.incl[q], kWave - 1, kWave);
    }
  }
  P.total = carry;
}

// The first entry whose inclusive prefix reaches t, and its exclusive prefix.
__device__ __forceinline__ int64_t find_sub_regs(const SubPrefix& P, int64_t nsub, double t, int lane,
                                                 double* base) {
#pragma unroll
  for (int q = 0; q < kSubRegs; ++q) {
    const int64_t i = (int64_t)q * kWave + lane;
    if ((int64_t)q * kWave < nsub) {
      const uint64_t m = ballot(i < nsub && P.incl[q] >= t);
      if (m) {
        const int L = first_lane(m);
        *base = __shfl(P.excl[q], L, kWave);
        return (int64_t)q * kWave + L;
      }
    }
  }
  return -1;
}

// Sixteen consecutive logits [lo, lo + 16) of a row as fp32 (slots at or past
// V read -inf). Vector path: lo is a multiple of 16 elements and rows are
// 16-byte aligned, so a lane's run is 2 (bf16) or 4 (fp32) aligned 16-byte
// vectors, each entirely inside or entirely past the row.
template <int DT, bool VEC>
__device__ __forceinline__ void load16(const void* row, int64_t lo, int64_t V, float (&z)[16]) {
  if constexpr (VEC) {
    constexpr int VE = (DT == kBF16) ? 8 : 4;
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const char*>(row) + lo * (DT == kBF16 ? 2 : 4));
#pragma unroll
    for (int u = 0; u < 16 / VE; ++u) {
      u32x4 q = (lo + u * VE < V) ? p[u] : u32x4{0xff800000u, 0xff800000u, 0xff800000u, 0xff800000u};
      if constexpr (DT == kBF16) {
        if (!(lo + u * VE < V)) q = u32x4{0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};
        z[u * 8 + 0] = bf16_lo(q.x); z[u * 8 + 1] = bf16_hi(q.x);
        z[u * 8 + 2] = bf16_lo(q.y); z[u * 8 + 3] = bf16_hi(q.y);
        z[u * 8 + 4] = bf16_lo(q.z); z[u * 8 + 5] = bf16_hi(q.z);
        z[u * 8 + 6] = bf16_lo(q.w); z[u * 8 + 7] = bf16_hi(q.w);
      } else {
        z[u * 4 + 0] = __uint_as_float(q.x); z[u * 4 + 1] = __uint_as_float(q.y);
        z[u * 4 + 2] = __uint_as_float(q.z); z[u * 4 + 3] = __uint_as_float(q.w);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) z[j] = (lo + j < V) ? load_logit<DT>(row, lo + j) : ninf();
  }
}

// Inverse-CDF walk over sub-blocks [sb0, sb1) of the selected row, starting
// from prefix `carry`: lane l owns elements [sb*1024 + 16 l, +16) in index
// order; a wave inclusive scan of the lane sums finds the lane whose run
// reaches t, and that lane walks its 16 weights. Returns the token, or -1 if
// t is not reached (with t < 0: always), the final prefix in *total and the
// last element of positive weight in *last.
//
// `weights(sb, lo, w)` gives the lane's sixteen weights of sub-block sb,
// elements [lo, lo + 16): from the rows (wave_draw) or from where the masses'
// pass left them (wave_draw_from).
template <class SRC>
__device__ int wave_draw_src(const SRC& weights, int64_t sb0, int64_t sb1, double carry, double t,
                             int lane, double* total, int64_t* last) {
  int64_t lastpos = -1;
  for (int64_t sb = sb0; sb < sb1; ++sb) {
    const int64_t lo = sb * kSub + (int64_t)lane * 16;
    float w[16];
    weights(sb, lo, w);
    // positions within the lane's run are kept as 0..15 (not as 64-bit
    // element indices): it halves the registers the walk needs
    double ls = 0.0;
    int lastj = -1;  // last slot of positive weight in this lane's run
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      lastj = (w[j] > 0.f) ? j : lastj;
      ls += (double)w[j];
    }
    if (lastj >= 0) lastpos = lo + lastj;
    const double incl = wave_inclusive_scan(ls, lane) + carry;
    const double prev = __shfl_up(incl, 1, kWave);
    const double excl = (lane == 0) ? carry : prev;
    if (t >= 0.0) {
      const uint64_t m = ballot(incl >= t);
      if (m) {
        // Lane L's run reaches t: every lane walks L's sixteen weights, read
        // with v_readlane (wave-uniform values, so the walk's float64
        // conversions are not the ones of the lane sum above and those die
        // there instead of staying live across the scan).
        const int L = first_lane(m);
        double cum = __shfl(excl, L, kWave);
        int tj = -1;  // first slot of positive weight whose prefix reaches t
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float wl = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(w[j]), L));
          cum += (double)wl;
          tj = (tj < 0 && wl > 0.f && t <= cum) ? j : tj;
        }
        // rounding: stay inside the run that reached t (its last positive slot)
        if (tj < 0) tj = __builtin_amdgcn_readlane(lastj, L);
        return (tj >= 0) ? (int)(sb * kSub + (int64_t)L * 16 + tj) : -1;
      }
    }
    carry = __shfl(incl, kWave - 1, kWave);
  }
  if (total) *total = carry;
  if (last) {
    long long lp = lastpos;
#pragma unroll
    for (int off = kWave / 2; off >= 1; off >>= 1) lp = max(lp, (long long)__shfl_xor(lp, off, kWave));
    *last = lp;
  }
  return -1;
}

// The walk with the weights formed from the selected rows.
template <int DT, bool VEC, class WT>
__device__ int wave_draw(const void* trow, const void* drow, const WT& W, int64_t V,
                         int64_t sb0, int64_t sb1, double carry, double t, int lane,
                         double* total, int64_t* last) {
  auto from_rows = [&](int64_t, int64_t lo, float (&w)[16]) {
    float zt[16], zd[16];
    load16<DT, VEC>(trow, lo, V, zt);
    if (W.residual) load16<DT, VEC>(drow, lo, V, zd);
#pragma unroll
    for (int j = 0; j < 16; ++j) w[j] = W(zt[j], W.residual ? zd[j] : 0.f);
  };
  return wave_draw_src(from_rows, sb0, sb1, carry, t, lane, total, last);
}

// The walk over sub-block 0 with the weights the masses' pass stored in LDS
// at their element indices (`wl[e]` = the weight of element e < kSub): the
// same values wave_draw would form again from the rows.
__device__ __forceinline__ int wave_draw_from(const float* wl, double carry, double t, int lane,
                                              int64_t* last) {
  auto from_lds = [&](int64_t, int64_t lo, float (&w)[16]) {
    const float4* p = reinterpret_cast<const float4*>(wl + lo);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float4 q = p[u];
      w[4 * u + 0] = q.x;
      w[4 * u + 1] = q.y;
      w[4 * u + 2] = q.z;
      w[4 * u + 3] = q.w;
    }
  };
  return wave_draw_src(from_lds, 0, 1, carry, t, lane, nullptr, last);
}

// The final draw of one sequence by one wave: picks the sub-block that holds
// u * total from the pass-2 masses `sub` (global or LDS), then walks that
// sub-block. Where subs_fit_regs(nsub), `v` holds the masses as load_subs
// leaves them (the caller requests them early) and the scans run on it.
template <int DT, bool VEC>
__device__ int draw_token(const DrawArgs& a, const double* sub, const double (&v)[kSubRegs],
                          const Select& s, int lane, const float* wl = nullptr) {
  constexpr int64_t esz = (DT == kBF16) ? 2 : 4;
  const void* trow = static_cast<const char*>(a.target) + s.trow * a.V * esz;
  const void* drow = (s.mode == kModeResidual) ? static_cast<const char*>(a.draft) + s.drow * a.V * esz : nullptr;
  const bool regs = subs_fit_regs(a.nsub);
  SubPrefix P;
  double total = 0.0;
  if (regs) {
    scan_subs_regs(v, a.nsub, lane, P);
    total = P.total;
  } else {
    wave_scan_subs(sub, a.nsub, -1.0, lane, nullptr, &total);
  }
  int token = -1;
  if (total > 0.0) {
    const double t = s.u * total;  // u in (0, 1]: t <= total
    double base = 0.0;
    const int64_t sb = regs ? find_sub_regs(P, a.nsub, t, lane, &base)
                            : wave_scan_subs(sub, a.nsub, t, lane, &base, nullptr);
    auto walk = [&](auto fma) {
      const Weights<decltype(fma)::value> W = make_weights<decltype(fma)::value>(s, false);
      int tok = -1;
      int64_t last = -1;
      // wl (one sub-block): the residual weights the masses' pass left in LDS
      if (sb >= 0) {
        tok = wl ? wave_draw_from(wl, base, t, lane, &last)
                 : wave_draw<DT, VEC>(trow, drow, W, a.V, sb, sb + 1, base, t, lane, nullptr, &last);
        if (tok < 0) tok = (int)last;
      }
      for (int64_t q = a.nsub - 1; tok < 0 && q >= 0; --q) {
        // rounding left t past every prefix: the last token of positive weight
        if (!(sub[q] > 0.0)) continue;
        if (wl) wave_draw_from(wl, 0.0, -1.0, lane, &last);
        else wave_draw<DT, VEC>(trow, drow, W, a.V, q, q + 1, 0.0, -1.0, lane, nullptr, &last);
        tok = (int)last;
      }
      return tok;
    };
    token = weights_fma(s, false) ? walk(std::true_type{}) : walk(std::false_type{});
  } else {
    // The residual has no mass in fp32 (p_n == q_n to rounding): draw from p_n.
    auto walk = [&](auto fma) {
      const Weights<decltype(fma)::value> W = make_weights<decltype(fma)::value>(s, true);
      double tot = 0.0;
      int64_t last = -1;
      wave_draw<DT, VEC>(trow, nullptr, W, a.V, 0, a.nsub, 0.0, -1.0, lane, &tot, &last);
      const int tok = wave_draw<DT, VEC>(trow, nullptr, W, a.V, 0, a.nsub, 0.0, s.u * tot, lane,
                                         nullptr, nullptr);
      return (tok < 0) ? (int)last : tok;
    };
    token = weights_fma(s, true) ? walk(std::true_type{}) : walk(std::false_type{});
  }
  return token;
}

// Accept step and pass 2 in one launch: wave (b, c) first runs the accept
// step of sequence b (every wave of b computes the same, wave c == 0 stores
// it), then, for a sampling sequence, the weight mass max(0, p - q) (or p)
// of chunk c of the selected row pair, written per 1024-element sub-block so
// that the draw only has to scan one sub-block. A tile (EPI = 1024 or 2048
// elements) holds one or two sub-blocks: in the bf16 vector tile, slots
// 0..15 of every lane lie in the first 1024 elements.
// Pass 2 over chunk c of the selected row pair of one sequence: the weight
// mass of every 1024-element sub-block of the chunk, stored to out[sub-block]
// (global memory or LDS).
//
// With wsave (a row of one sub-block), the weights of sub-block 0 are also
// stored there at their element indices, for the draw's walk.
template <int DT, bool VEC, bool FMA>
__device__ __forceinline__ void chunk_masses_w(const DrawArgs& a, const Select& s, int c, int lane,
                                               double* out, float* wsave) {
  using TL = Tile<DT, VEC>;
  constexpr int NE = TL::NE;
  constexpr int SUBS = TL::EPI / kSub;  // sub-blocks per tile (1 or 2)
  constexpr int PER = NE / SUBS;        // slots per lane per sub-block
  const Weights<FMA> W = make_weights<FMA>(s, false);
  constexpr int64_t esz = (DT == kBF16) ? 2 : 4;
  const void* trow = static_cast<const char*>(a.target) + s.trow * a.V * esz;
  const void* drow = W.residual ? static_cast<const char*>(a.draft) + s.drow * a.V * esz : nullptr;
  // the row's tiles interleaved over the sequence's pass-2 waves (wave c
  // takes tiles c, c + chunks3, ...), so neighbouring waves read neighbouring
  // tiles at about the same time, as in pass 1
  const int64_t tiles = (a.V + TL::EPI - 1) / TL::EPI;
  typename TL::Raw rt, rd;
  float w[NE];
  for (int64_t t = c; t < tiles; t += a.chunks3) {
    const int64_t e0 = t * TL::EPI;
    if (e0 + TL::EPI <= a.V) {
      TL::template load_raw<false>(trow, e0, a.V, 0, lane, rt);
      if (W.residual) TL::template load_raw<false>(drow, e0, a.V, 0, lane, rd);
    } else {
      TL::template load_raw<true>(trow, e0, a.V, 0, lane, rt);
      if (W.residual) TL::template load_raw<true>(drow, e0, a.V, 0, lane, rd);
    }
    if constexpr (VEC && DT == kBF16) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        w[2 * q] = W(bf16_lo(rt.d[q]), W.residual ? bf16_lo(rd.d[q]) : 0.f);
        w[2 * q + 1] = W(bf16_hi(rt.d[q]), W.residual ? bf16_hi(rd.d[q]) : 0.f);
      }
    } else {
#pragma unroll
      for (int q = 0; q < NE; ++q)
        w[q] = W(__uint_as_float(rt.d[q]), W.residual ? __uint_as_float(rd.d[q]) : 0.f);
    }
    if (wsave && e0 == 0) {
#pragma unroll
      for (int j = 0; j < PER; ++j) wsave[TL::index(0, 0, lane, j)] = w[j];
    }
#pragma unroll
    for (int h = 0; h < SUBS; ++h) {
      float part[PER];
#pragma unroll
      for (int j = 0; j < PER; ++j) part[j] = w[h * PER + j];
      const double m = wave_sum((double)tree_sum(part));
      const int64_t sb = e0 / kSub + h;
      if (lane == 0 && sb < a.nsub) out[sb] = m;
    }
  }
}

// The weights' form is the same for the whole sequence (weights_fma).
template <int DT, bool VEC>
__device__ __forceinline__ void chunk_masses(const DrawArgs& a, const Select& s, int c, int lane,
                                             double* out, float* wsave = nullptr) {
  if (weights_fma(s, false)) chunk_masses_w<DT, VEC, true>(a, s, c, lane, out, wsave);
  else chunk_masses_w<DT, VEC, false>(a, s, c, lane, out, wsave);
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void k3_accept_mass(AcceptArgs acc, DrawArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t item = wave_uniform((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  if (item >= (int64_t)a.B * a.chunks3) return;
  const int64_t b = item / a.chunks3;
  const int c = (int)(item - b * a.chunks3);
  const Select s = uniform_select(accept_sequence<DT>(acc, b, lane, c == 0));
  if (s.mode == kModeNone) return;
  chunk_masses<DT, VEC>(a, s, c, lane, a.sub + b * a.nsub);
}

// The final draw: one wave per sampling sequence, in its own launch (the
// kernel boundary orders every pass-2 store before the draw's reads).
template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void k4_draw(DrawArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t b = wave_uniform((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  if (b >= a.B) return;
  // the masses are requested with the selection, before its mode is known
  double v[kSubRegs];
  if (subs_fit_regs(a.nsub)) load_subs(a.sub + b * a.nsub, a.nsub, lane, v);
  const Select s = a.sel[b];
  if (s.mode == kModeNone) return;
  const int token = draw_token<DT, VEC>(a, a.sub + b * a.nsub, v, s, lane);
  if (lane == 0) a.out_next[b] = token;
}

// Accept step, pass 2 and the final draw in one launch, one workgroup per
// sequence with one wave per pass-2 chunk (blockDim = 64 * chunks3, at most
// 1024). Wave 0 runs the accept step and, with several waves, leaves the
// selection in LDS for the others (a few sequences' workgroups are alone on
// their compute units, where copies of the accept step in every wave would
// share the SIMDs); every wave takes the masses of its chunk into LDS, and
// after the workgroup barrier wave 0 draws from them: the barrier replaces
// the kernel boundary of the two-launch form, and the arithmetic is the
// same, so both forms give the same bits. Every wave reaches both barriers:
// nothing returns before them.
template <int DT, bool VEC>
__global__ __launch_bounds__(1024) void k3_accept_mass_draw(AcceptArgs acc, DrawArgs a) {
  extern __shared__ double sub_lds[];  // [nsub] masses of the sequence's sub-blocks
  __shared__ Select sel_lds;
  const int lane = threadIdx.x & (kWave - 1);
  const int c = (int)(threadIdx.x >> 6);
  const int64_t b = blockIdx.x;
  Select s;
  if (blockDim.x == kWave) {
    s = uniform_select(accept_sequence<DT>(acc, b, lane, true));
  } else {
    if (c == 0) {
      const Select s0 = accept_sequence<DT>(acc, b, lane, true);
      if (lane == 0) sel_lds = s0;
    }
    __syncthreads();
    s = uniform_select(sel_lds);
  }
  const bool active = s.mode != kModeNone;
  // one wave and one sub-block: the wave keeps its weights in LDS (after the
  // mass, 16 bytes on) and the draw walks them instead of forming them again
  // from the rows
  float* const wl = a.weights_in_lds ? reinterpret_cast<float*>(sub_lds + 2) : nullptr;
  if (active) chunk_masses<DT, VEC>(a, s, c, lane, sub_lds, wl);
  __syncthreads();
  if (active && c == 0) {
    double v[kSubRegs];
    if (subs_fit_regs(a.nsub)) load_subs(sub_lds, a.nsub, lane, v);
    const int token = draw_token<DT, VEC>(a, sub_lds, v, s, lane, wl);
    if (lane == 0) a.out_next[b] = token;
  }
}

// ----------------------------- test exports --------------------------------

struct MergeArgs {
  const RowPart* tparts;
  const RowPart* dparts;
  const float* tk;
  const float* dk;
  const uint32_t* status;
  float* out_tm;
  double* out_ts;
  int32_t* out_ta;
  float* out_dm;
  double* out_ds;
  int32_t* out_da;
  int64_t total_t, total_d;
  int32_t B, chunks;
};

// One thread per row: merged (m, sum of exp((z - m)/T), argmax).
__global__ __launch_bounds__(kBlock) void k_merge_rows(MergeArgs a) {
  const int64_t r = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (r >= a.total_t + a.total_d) return;
  const bool is_draft = r >= a.total_t;
  const int64_t j = is_draft ? r - a.total_t : r;
  float* om = is_draft ? a.out_dm : a.out_tm;
  double* os = is_draft ? a.out_ds : a.out_ts;
  int32_t* oa = is_draft ? a.out_da : a.out_ta;
  if (a.status[0] & kLayoutError) {
    om[j] = __builtin_nanf("");
    os[j] = __builtin_nan("");
    oa[j] = -1;
    return;
  }
  const float kk = is_draft ? a.dk[j] : a.tk[j];
  const bool sampling = kk > 0.f;
  if ((is_draft && !sampling) || !(kk >= 0.f)) {
    om[j] = __builtin_nanf("");
    os[j] = __builtin_nan("");
    oa[j] = -1;
    return;
  }
  const float k = sampling ? kk : 0.f;
  const RowStat st = merge_row((is_draft ? a.dparts : a.tparts) + j * a.chunks, a.chunks, k, sampling);
  om[j] = st.m;
  // the sum is taken relative to m: sum 2^((z - m) k)
  os[j] = sampling ? (st.valid ? st.s : __builtin_nan("")) : (st.valid ? 0.0 : __builtin_nan(""));
  oa[j] = st.arg;
}

struct ProbArgs {
  const void* target;
  const void* draft;
  const RowPart* tparts;
  const RowPart* dparts;
  const float* tk;
  const float* dk;
  const int64_t* rows;
  float* out;
  int64_t V, n_rows, total_t, total_d;
  int32_t B, chunks;
};

// grid (element chunks of 2048, rows): p_v = 2^(fl32(fl32(z - m) k)) *
// fl32(1/S), the same arithmetic as the final draw's weights.
template <int DT>
__global__ __launch_bounds__(kBlock) void k_softmax_rows(ProbArgs a) {
  const int64_t k_row = blockIdx.y;
  if (k_row >= a.n_rows) return;
  const int64_t sel = a.rows[k_row];
  const bool is_draft = sel < 0;
  const int64_t j = is_draft ? -sel - 1 : sel;
  if (j >= (is_draft ? a.total_d : a.total_t)) {  // no such row: NaN row
    for (int q = threadIdx.x; q < 2048; q += kBlock) {
      const int64_t v = (int64_t)blockIdx.x * 2048 + q;
      if (v < a.V) a.out[k_row * a.V + v] = __builtin_nanf("");
    }
    return;
  }
  const float k = is_draft ? a.dk[j] : a.tk[j];
  const RowStat st = merge_row((is_draft ? a.dparts : a.tparts) + j * a.chunks, a.chunks, k, true);
  Select s{};
  s.mode = kModeBonus;
  s.k = k;
  s.refT = st.ref;
  s.sT = st.s;
  constexpr int64_t esz = (DT == kBF16) ? 2 : 4;
  const void* row = static_cast<const char*>(is_draft ? a.draft : a.target) + j * a.V * esz;
  const int64_t v0 = (int64_t)blockIdx.x * 2048;
  auto fill = [&](auto fma) {
    const Weights<decltype(fma)::value> W = make_weights<decltype(fma)::value>(s, true);
    for (int q = threadIdx.x; q < 2048; q += kBlock) {
      const int64_t v = v0 + q;
      if (v < a.V) a.out[k_row * a.V + v] = W(load_logit<DT>(row, v), 0.f);
    }
  };
  if (weights_fma(s, true)) fill(std::true_type{});
  else fill(std::false_type{});
}

__global__ __launch_bounds__(kBlock) void k_philox(uint64_t seed, const uint32_t* ctr,
                                                   uint32_t* out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i >= n) return;
  const PhiloxBlock w = philox4x32_10(seed, ctr[4 * i], ctr[4 * i + 1], ctr[4 * i + 2], ctr[4 * i + 3]);
  out[4 * i] = w.w0;
  out[4 * i + 1] = w.w1;
  out[4 * i + 2] = w.w2;
  out[4 * i + 3] = w.w3;
}

// Read-only stream with pass 1's access pattern, for the read bandwidth the
// part reaches with it: 64 KiB segments, each read by two sibling waves that
// take alternate 4 KiB tiles with 16-byte non-temporal loads, the next tile
// issued before the previous one is folded; every dword is XOR-folded into
// one word per wave (so the loads are not dead).
constexpr int64_t kProbeSegBytes = 65536;

__global__ __launch_bounds__(kBlock) void k_read_probe(const u32x4* src, int64_t segments,
                                                       uint32_t* sink) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t item = wave_uniform((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  if (item >= 2 * segments) return;
  const u32x4* p = src + (item >> 1) * (kProbeSegBytes / 16);
  const int sib = (int)(item & 1);
  constexpr int kTiles = (int)(kProbeSegBytes / 4096 / 2);  // 8 per wave
  auto load = [&](int t, u32x4 (&r)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      r[u] = __builtin_nontemporal_load(p + (int64_t)(sib + 2 * t) * 256 + u * kWave + lane);
  };
  uint32_t acc = 0u;
  auto fold = [&](const u32x4 (&r)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= r[u].x ^ r[u].y ^ r[u].z ^ r[u].w;
  };
  u32x4 a[4], b[4];
  load(0, a);
  for (int t = 0; t + 3 < kTiles; t += 2) {
    load(t + 1, b);
    fold(a);
    load(t + 2, a);
    fold(b);
  }
  load(kTiles - 1, b);
  fold(a);
  fold(b);
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off, kWave);
  if (lane == 0) sink[item] = acc;
}

// Copy with the same pattern: each 64 KiB segment moved by two sibling waves
// on alternate 4 KiB tiles, the next tile's non-temporal loads issued before
// the previous tile's non-temporal stores (6.2 TB/s of read plus write on
// this part, where a grid-stride copy reaches 5.4).
__global__ __launch_bounds__(kBlock) void k_copy_tiled(u32x4* dst, const u32x4* src,
                                                       int64_t segments) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t item = wave_uniform((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  if (item >= 2 * segments) return;
  const int64_t base = (item >> 1) * (kProbeSegBytes / 16);
  const int sib = (int)(item & 1);
  constexpr int kTiles = (int)(kProbeSegBytes / 4096 / 2);  // 8 per wave
  auto at = [&](int t, int u) { return base + (int64_t)(sib + 2 * t) * 256 + u * kWave + lane; };
  auto load = [&](int t, u32x4 (&r)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) r[u] = __builtin_nontemporal_load(src + at(t, u));
  };
  auto store = [&](int t, const u32x4 (&r)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(r[u], dst + at(t, u));
  };
  u32x4 a[4], b[4];
  load(0, a);
  for (int t = 0; t + 3 < kTiles; t += 2) {
    load(t + 1, b);
    store(t, a);
    load(t + 2, a);
    store(t + 1, b);
  }
  load(kTiles - 1, b);
  store(kTiles - 2, a);
  store(kTiles - 1, b);
}

// Grid-stride copy, for a tail shorter than a segment.
__global__ __launch_bounds__(kBlock) void k_copy(u32x4* dst, const u32x4* src, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n16; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace specv
