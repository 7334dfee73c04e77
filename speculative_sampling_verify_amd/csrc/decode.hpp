// decode.hpp -- multi-round speculative decoding with bigram "models" (gfx950).
//
// The step of DistillSpec Algorithm A.1 repeated over rounds, with models
// that are bigram tables: the logits of the next token after token s are row
// s of a [V, V] table (one for the target, one for the draft). One round:
//   k_dec_draft_wg  (V <= 8192; else k_dec_draft, one wave per sequence)
//                 a workgroup per sequence drafts gamma tokens autoregressively
//                 from softmax(draft row / T) by inverse CDF in index order
//                 (u = word 0 of Philox(seed; row, i, 1)), or by argmax when
//                 T = 0, and records which table row feeds each packed row;
//   k_dec_gather_stats  copies those table rows into the packed layout of
//                 the verify step (what a model's output layer would write)
//                 and forms the verify step's pass-1 statistics of each row
//                 as it writes it (as an output layer's epilogue could);
//   the rest of the verify step (accept + pass 2 + draw);
//   k_dec_append  appends the n accepted drafts and the drawn token.
// Within a lane the drafting scan holds 16 consecutive elements, so lane
// order is index order and the walk follows the index-order CDF.
#pragma once

#include "kernels.hpp"

namespace specv {

struct DecodeArgs {
  const void* ttab;          // [V, V] target bigram logits
  const void* dtab;          // [V, V] draft bigram logits
  const float* temperature;  // [B]
  const int32_t* start;      // [B]
  int32_t* cur;              // [B] last token of each sequence
  int32_t* drafts;           // [B * gamma] this round's draft tokens (packed)
  int32_t* trow_src;         // [B * (gamma + 1)] table row of each packed target row
  int32_t* drow_src;         // [B * gamma] table row of each packed draft row
  int32_t* gam;              // [B] gamma of every sequence (verify input)
  int32_t* len;              // [B] tokens generated so far
  int32_t* fail;             // [B] 1 once a round failed
  const int32_t* vn;         // [B] verify output n
  const int32_t* vnext;      // [B] verify output token
  int32_t* out_tokens;       // [B, cap]
  int32_t* out_length;       // [B]
  int32_t* out_accepted;     // [B, rounds]
  uint64_t seed, row_base;   // Philox row of sequence b this round: row_base + b
  int64_t V, cap;
  int32_t B, gamma, rounds, round;
};

constexpr int kDecPL = 16;               // consecutive elements per lane per tile
constexpr int kDecTE = kWave * kDecPL;   // elements per drafting tile

__global__ __launch_bounds__(kBlock) void k_dec_init(DecodeArgs a) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t b = t; b < a.B; b += stride) {
    const int32_t s = a.start[b];
    const bool bad = s < 0 || (int64_t)s >= a.V;
    a.cur[b] = bad ? 0 : s;
    a.fail[b] = bad ? 1 : 0;
    a.len[b] = 0;
    a.gam[b] = a.gamma;
  }
  for (int64_t e = t; e < (int64_t)a.B * a.cap; e += stride) a.out_tokens[e] = -1;
}

// The lane's 16 consecutive elements of the drafting tile at e0 (-inf past
// V): four or two 16-byte loads when rows are 16-byte aligned, else scalar.
template <int DT, bool VEC>
__device__ __forceinline__ void dec_load(const void* row, int64_t V, int64_t e0, int lane,
                                         float (&z)[kDecPL]) {
  const int64_t base = e0 + (int64_t)lane * kDecPL;
  if constexpr (VEC) {
    constexpr int VE = (DT == kBF16) ? 8 : 4;  // elements per 16 bytes
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const char*>(row) +
                                                    base * (DT == kBF16 ? 2 : 4));
#pragma unroll
    for (int v = 0; v < kDecPL / VE; ++v) {
      // V * element size is a multiple of 16 here, so a vector is all in or all out
      u32x4 q = {0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};
      if (DT != kBF16) q = u32x4{0xff800000u, 0xff800000u, 0xff800000u, 0xff800000u};
      if (base + v * VE < V) q = p[v];
      if constexpr (DT == kBF16) {
        z[v * 8 + 0] = bf16_lo(q.x); z[v * 8 + 1] = bf16_hi(q.x);
        z[v * 8 + 2] = bf16_lo(q.y); z[v * 8 + 3] = bf16_hi(q.y);
        z[v * 8 + 4] = bf16_lo(q.z); z[v * 8 + 5] = bf16_hi(q.z);
        z[v * 8 + 6] = bf16_lo(q.w); z[v * 8 + 7] = bf16_hi(q.w);
      } else {
        z[v * 4 + 0] = __uint_as_float(q.x); z[v * 4 + 1] = __uint_as_float(q.y);
        z[v * 4 + 2] = __uint_as_float(q.z); z[v * 4 + 3] = __uint_as_float(q.w);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < kDecPL; ++j) z[j] = (base + j < V) ? load_logit<DT>(row, base + j) : ninf();
  }
}

// Drafting tiles whose loads are issued together. One wave drafts one
// sequence and the launch has only B waves (a few per SIMD), so registers are
// not what limits it: a row of up to kDecBatch tiles (8192 elements) is read
// once, with all its loads in flight together, and stays in registers for the
// CDF walk.
constexpr int kDecBatch = 8;

// One draw from softmax(row * k) (k = log2(e)/T), or the argmax for k == 0.
// Pass 1: per-lane online (max, sum of 2^((z - max) k)) over the row, merged
// across the wave (fp64 sum). Pass 2 walks the tiles in order: a tile's
// per-lane fp32 tree sums are scanned in fp64 across the wave; the first
// tile whose running total reaches u * S holds the token, the first lane
// whose prefix reaches it, and that lane's first element.
template <int DT, bool VEC>
__device__ int dec_sample_row(const void* row, int64_t V, float k, double u, int lane) {
  const int64_t n_tiles = (V + kDecTE - 1) / kDecTE;
  const bool resident = n_tiles <= kDecBatch;  // one batch: pass 2 reuses the registers
  float z[kDecBatch][kDecPL];
  auto load_batch = [&](int64_t t0) {
#pragma unroll
    for (int b = 0; b < kDecBatch; ++b) {
      if (t0 + b < n_tiles) dec_load<DT, VEC>(row, V, (t0 + b) * kDecTE, lane, z[b]);
      else {
#pragma unroll
        for (int j = 0; j < kDecPL; ++j) z[b][j] = ninf();
      }
    }
  };
  float m = ninf();
  double s = 0.0;
  int64_t arg = INT32_MAX;
  for (int64_t t0 = 0; t0 < n_tiles; t0 += kDecBatch) {
    load_batch(t0);
#pragma unroll
    for (int b = 0; b < kDecBatch; ++b) {
      const float g = tile_max(z[b]);
      if (k == 0.f) {
#pragma unroll
        for (int j = 0; j < kDecPL; ++j)
          if (z[b][j] > m) {
            m = z[b][j];
            arg = (t0 + b) * kDecTE + (int64_t)lane * kDecPL + j;
          }
      } else if (g > ninf()) {
        const float mn = fmaxf(m, g);
        const float sc = rescale32(m, mn, k);
        const float ref = ref_logit(mn);
        float e[kDecPL];
#pragma unroll
        for (int j = 0; j < kDecPL; ++j) e[j] = exp2_hw(term_exp(z[b][j], ref, k));
        s = __builtin_fma(s, (double)sc, (double)tree_sum(e));
        m = mn;
      }
    }
  }
  const float M = wave_max(m);
  if (k == 0.f) {
    const int best = wave_min((m == M && arg < INT32_MAX) ? (int)arg : INT32_MAX);
    return best == INT32_MAX ? 0 : best;
  }
  const float refM = ref_logit(M);
  const double S = wave_sum((m == ninf()) ? 0.0 : s * exp2(((double)m - (double)refM) * (double)k));
  const double target = u * S;
  double C = 0.0;
  for (int64_t t0 = 0; t0 < n_tiles; t0 += kDecBatch) {
    if (!resident) load_batch(t0);
#pragma unroll
    for (int b = 0; b < kDecBatch; ++b) {
      if (t0 + b >= n_tiles) break;
      float w[kDecPL], tw[kDecPL];
#pragma unroll
      for (int j = 0; j < kDecPL; ++j) {
        w[j] = exp2_hw(term_exp(z[b][j], refM, k));
        tw[j] = w[j];
      }
      const float ls = tree_sum(tw);
      const double incl = wave_inclusive_scan((double)ls, lane);
      const double tot = __shfl(incl, kWave - 1, kWave);
      if (C + tot >= target || t0 + b + 1 >= n_tiles) {
        const uint64_t hit = ballot(C + incl >= target);
        const uint64_t pos = ballot(ls > 0.f);
        if (hit == 0 && pos == 0) return 0;  // no mass at all (unusable row)
        const int L = hit ? first_lane(hit) : 63 - __builtin_clzll(pos);
        double ex = __shfl_up(incl, 1, kWave);
        if (lane == 0) ex = 0.0;
        int tok = -1;
        if (lane == L) {
          double c = C + ex;
          int last = -1;
#pragma unroll
          for (int j = 0; j < kDecPL; ++j) {
            if (w[j] > 0.f) last = j;
            c += (double)w[j];
            if (tok < 0 && w[j] > 0.f && c >= target) tok = j;
          }
          if (tok < 0) tok = last < 0 ? 0 : last;
          tok = (int)((t0 + b) * kDecTE + (int64_t)lane * kDecPL + tok);
        }
        return __shfl(tok, L, kWave);
      }
      C += tot;
    }
  }
  return 0;
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void k_dec_draft(DecodeArgs a) {
  constexpr int64_t esz = (DT == kBF16) ? 2 : 4;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t b = wave_uniform((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  if (b >= a.B) return;
  const float T = a.temperature[b];
  const bool sampling = sampling_temperature(T);
  const bool greedy = T == 0.f;
  const float k = sampling ? temp_scale(T) : 0.f;
  const uint64_t prow = a.row_base + (uint64_t)b;
  int32_t prev = a.cur[b];
  for (int i = 0; i <= a.gamma; ++i) {
    if (lane == 0) a.trow_src[b * (a.gamma + 1) + i] = prev;
    if (i == a.gamma) break;
    if (lane == 0) a.drow_src[b * a.gamma + i] = prev;
    int x = 0;  // an invalid temperature drafts token 0; the verify step fails the sequence
    if (sampling || greedy) {
      double u = 0.0;
      if (sampling) {
        const PhiloxBlock w = philox4x32_10(a.seed, (uint32_t)prow, (uint32_t)(prow >> 32),
                                            (uint32_t)i, 1u);
        u = (double)uniform24(w.w0);
      }
      const void* row = static_cast<const char*>(a.dtab) + (int64_t)prev * a.V * esz;
      x = dec_sample_row<DT, VEC>(row, a.V, k, u, lane);
      if (x < 0 || (int64_t)x >= a.V) x = 0;
    }
    if (lane == 0) a.drafts[b * a.gamma + i] = x;
    prev = x;
  }
}

// Drafting by a workgroup of kDecWaves waves per sequence, for rows of at
// most kDecWaves * kDecTPW tiles (8192 elements): wave w holds the tiles
// [w tpw, (w + 1) tpw) of the row in registers (tpw = ceil(tiles / waves)),
// so a drafted token costs one row load and three LDS exchanges:
//   1. each wave's maximum (and its lowest index attaining it); greedy
//      sequences take the row's argmax from these and stop here;
//   2. weights 2^(fl32(fl32(z - M) k)) against the row maximum M, per-lane fp32
//      tree sums per tile, a wave inclusive scan per tile (fp64) whose last
//      lane is the tile's mass, and the wave's segment mass (its tiles'
//      masses added in order); S = the segment masses added in wave order;
//   3. the first wave whose running total reaches u * S walks its tiles and
//      lanes in index order (the same additions, so the total is reached)
//      and publishes the token.
// The LDS slots alternate between two sets by token parity: a set is
// rewritten two tokens later, after every wave has passed the barriers of
// the token in between, so no wave can still be reading it.
#ifndef SPECV_DEC_WAVES
#define SPECV_DEC_WAVES 4
#endif
constexpr int kDecWaves = SPECV_DEC_WAVES;
constexpr int kDecTPW = 8 / kDecWaves;
constexpr int64_t kDecResident = (int64_t)kDecWaves * kDecTPW * kDecTE;

struct DecLds {
  float m[2][kDecWaves];
  int32_t arg[2][kDecWaves];
  double seg[2][kDecWaves];
  int32_t x[2];
};

template <int DT, bool VEC>
__device__ int wg_sample_row(const void* row, int64_t V, float k, double u, int lane, int w,
                             int par, DecLds& sh) {
  const int64_t n_tiles = (V + kDecTE - 1) / kDecTE;
  const int64_t tpw = (n_tiles + kDecWaves - 1) / kDecWaves;
  const int64_t t_lo = (int64_t)w * tpw;
  float z[kDecTPW][kDecPL];
#pragma unroll
  for (int t = 0; t < kDecTPW; ++t) {
    if (t < tpw && t_lo + t < n_tiles) dec_load<DT, VEC>(row, V, (t_lo + t) * kDecTE, lane, z[t]);
    else {
#pragma unroll
      for (int j = 0; j < kDecPL; ++j) z[t][j] = ninf();
    }
  }
  // 1. maxima; within a lane the index grows with t, then j
  float m = ninf();
  int arg = INT32_MAX;
#pragma unroll
  for (int t = 0; t < kDecTPW; ++t)
#pragma unroll
    for (int j = 0; j < kDecPL; ++j)
      if (z[t][j] > m) {
        m = z[t][j];
        arg = (int)((t_lo + t) * kDecTE + (int64_t)lane * kDecPL + j);
      }
  const float Mw = wave_max(m);
  const int aw = wave_min((m == Mw && m > ninf()) ? arg : INT32_MAX);
  if (lane == 0) {
    sh.m[par][w] = Mw;
    sh.arg[par][w] = aw;
  }
  __syncthreads();
  float M = ninf();
#pragma unroll
  for (int q = 0; q < kDecWaves; ++q) M = fmaxf(M, sh.m[par][q]);
  if (k == 0.f) {
    int best = INT32_MAX;
#pragma unroll
    for (int q = 0; q < kDecWaves; ++q)
      if (sh.m[par][q] == M) best = min(best, sh.arg[par][q]);
    return best == INT32_MAX ? 0 : best;
  }
  // 2. weights, tile scans and segment masses
  const float refM = ref_logit(M);
  float ls[kDecTPW];
  double incl[kDecTPW];
  double seg = 0.0;
#pragma unroll
  for (int t = 0; t < kDecTPW; ++t) {
    float tw[kDecPL];
#pragma unroll
    for (int j = 0; j < kDecPL; ++j) {
      z[t][j] = exp2_hw(term_exp(z[t][j], refM, k));  // the weight, in place
      tw[j] = z[t][j];
    }
    ls[t] = tree_sum(tw);
    incl[t] = wave_inclusive_scan((double)ls[t], lane);
    seg += __shfl(incl[t], kWave - 1, kWave);
  }
  if (lane == 0) sh.seg[par][w] = seg;
  __syncthreads();
  double S = 0.0, Cw = 0.0;
  int hw = -1;
#pragma unroll
  for (int q = 0; q < kDecWaves; ++q) {
    if (q == w) Cw = S;
    S += sh.seg[par][q];
  }
  const double target = u * S;
  {
    double C = 0.0;
#pragma unroll
    for (int q = 0; q < kDecWaves; ++q) {
      if (hw < 0 && sh.seg[par][q] > 0.0 && C + sh.seg[par][q] >= target) hw = q;
      C += sh.seg[par][q];
    }
  }
  // 3. the walk in the wave that holds the target: its first tile whose
  // running total reaches it, else (rounding: the segment mass was added as
  // one number) its last tile of positive mass, then the lane and the slot
  // likewise
  if (w == hw) {
    int tsel = -1, tlast = -1;
    double Csel = 0.0, Clast = 0.0, C = Cw;
#pragma unroll
    for (int t = 0; t < kDecTPW; ++t) {
      const double tot = __shfl(incl[t], kWave - 1, kWave);
      if (tot > 0.0) {
        if (tsel < 0 && C + tot >= target) {
          tsel = t;
          Csel = C;
        }
        tlast = t;
        Clast = C;
      }
      C += tot;
    }
    if (tsel < 0) {
      tsel = tlast;
      Csel = Clast;
    }
    int tok = 0;
#pragma unroll
    for (int t = 0; t < kDecTPW; ++t) {
      if (t != tsel) continue;
      const uint64_t hit = ballot(Csel + incl[t] >= target);
      const uint64_t pos = ballot(ls[t] > 0.f);
      const int L = hit ? first_lane(hit) : 63 - __builtin_clzll(pos);
      double ex = __shfl_up(incl[t], 1, kWave);
      if (lane == 0) ex = 0.0;
      int tl = -1;
      if (lane == L) {
        double c = Csel + ex;
        int lastj = -1;
#pragma unroll
        for (int j = 0; j < kDecPL; ++j) {
          if (z[t][j] > 0.f) lastj = j;
          c += (double)z[t][j];
          if (tl < 0 && z[t][j] > 0.f && c >= target) tl = j;
        }
        if (tl < 0) tl = lastj < 0 ? 0 : lastj;
        tl = (int)((t_lo + t) * kDecTE + (int64_t)lane * kDecPL + tl);
      }
      tok = __shfl(tl, L, kWave);
    }
    if (lane == 0) sh.x[par] = tok;
  }
  __syncthreads();
  return (hw < 0) ? 0 : sh.x[par];  // no mass at all (unusable row): token 0
}

// One workgroup of kDecWaves waves per sequence (grid = B workgroups). Every
// wave runs the same loop and reaches every barrier: gamma, the temperature
// and the drafted tokens are the same in all of them.
template <int DT, bool VEC>
__global__ __launch_bounds__(kDecWaves * kWave) void k_dec_draft_wg(DecodeArgs a) {
  constexpr int64_t esz = (DT == kBF16) ? 2 : 4;
  __shared__ DecLds sh;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = (int)(threadIdx.x >> 6);
  const int64_t b = blockIdx.x;
  const float T = a.temperature[b];
  const bool sampling = sampling_temperature(T);
  const bool greedy = T == 0.f;
  const float k = sampling ? temp_scale(T) : 0.f;
  const uint64_t prow = a.row_base + (uint64_t)b;
  const bool lead = (threadIdx.x == 0);
  int32_t prev = a.cur[b];
  for (int i = 0; i <= a.gamma; ++i) {
    if (lead) a.trow_src[b * (a.gamma + 1) + i] = prev;
    if (i == a.gamma) break;
    if (lead) a.drow_src[b * a.gamma + i] = prev;
    int x = 0;  // an invalid temperature drafts token 0; the verify step fails the sequence
    if (sampling || greedy) {
      double u = 0.0;
      if (sampling) {
        const PhiloxBlock pw = philox4x32_10(a.seed, (uint32_t)prow, (uint32_t)(prow >> 32),
                                             (uint32_t)i, 1u);
        u = (double)uniform24(pw.w0);
      }
      const void* row = static_cast<const char*>(a.dtab) + (int64_t)prev * a.V * esz;
      x = wg_sample_row<DT, VEC>(row, a.V, k, u, lane, w, i & 1, sh);
      if (x < 0 || (int64_t)x >= a.V) x = 0;
    }
    if (lead) a.drafts[b * a.gamma + i] = x;
    prev = x;
  }
}

// Where the rows of one round come from and go to: packed target rows
// [0, n_t) and draft rows [0, n_d), row r copied from table row *_src[r].
struct GatherArgs {
  const void* ttab;
  const void* dtab;
  const int32_t* trow_src;
  const int32_t* drow_src;
  void* tdst;
  void* ddst;
  int64_t row_bytes, n_t, n_d;
};

// The gather with the verify step's pass 1 folded in: one wave per (packed
// row, pass-1 chunk), the chunk's tiles as k1_row_stats takes them, each tile
// stored to the packed row while its statistics are formed (chunk_pass with
// STORE), so the verify step starts at the accept step. The partials are
// those k1_row_stats would write from the packed rows, bit for bit. Rows
// without statistics (draft rows of greedy sequences, invalid temperatures)
// are only copied. The batch is uniform (gamma for every sequence): the first
// workgroup also checks the gammas and sets the status word, as pass 1 does.
template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void k_dec_gather_stats(GatherArgs g, RowStatsArgs a) {
  using TL = Tile<DT, VEC>;
  if (a.gamma && blockIdx.x == 0) {
    bool bad = false;
    for (int64_t b = threadIdx.x; b < a.B; b += blockDim.x) bad |= a.gamma[b] != a.uniform_g;
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) a.status_out[0] = bad ? kLayoutError : 0u;
  }
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t item = wave_uniform((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  if (item >= (a.total_t + a.total_d) * a.chunks) return;
  const int64_t r = item / a.chunks;
  const int c = (int)(item - r * a.chunks);
  const bool is_draft = r >= a.total_t;
  const int64_t j = is_draft ? r - a.total_t : r;
  const int64_t src_row = is_draft ? g.drow_src[j] : g.trow_src[j];
  const void* src = static_cast<const char*>(is_draft ? g.dtab : g.ttab) + src_row * g.row_bytes;
  void* dst = static_cast<char*>(is_draft ? g.ddst : g.tdst) + j * g.row_bytes;
  const int64_t tiles = (a.V + TL::EPI - 1) / TL::EPI;
  const int n_iter = (int)((tiles - c + a.chunks - 1) / a.chunks);
  typename TL::Raw first;
  load_tile<DT, VEC>(src, a.V, c, lane, first);
  const int64_t seq = is_draft ? j / a.uniform_g : j / (a.uniform_g + 1);
  const float k = seq_scale(a.temperature[seq]);
  const bool stats = is_draft ? (k > 0.f) : (k >= 0.f);
  if (!stats) {
    // copy only: the verify step reads no statistics of this row
    for (int it = 0; it < n_iter; ++it) {
      const int64_t t = (int64_t)c + (int64_t)it * a.chunks;
      if (it > 0) load_tile<DT, VEC>(src, a.V, t, lane, first);
      TL::store_raw(dst, t * TL::EPI, a.V, 0, lane, first);
    }
    return;
  }
  RowPart out;
  float lm;
  if (k > 0.f)
    out = chunk_pass<DT, VEC, true, false, true>(src, a.V, c, a.chunks, n_iter, k, lane, first, lm, dst);
  else
    out = chunk_pass<DT, VEC, false, true, true>(src, a.V, c, a.chunks, n_iter, 0.f, lane, first, lm, dst);
  if (lane == 0) (is_draft ? a.dparts : a.tparts)[j * a.chunks + c] = out;
}

__global__ __launch_bounds__(kBlock) void k_dec_append(DecodeArgs a) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= a.B) return;
  int32_t* acc = a.out_accepted + b * a.rounds + a.round;
  const int32_t n = a.vn[b];
  if (a.fail[b] || n < 0) {
    a.fail[b] = 1;
    *acc = -1;
    return;
  }
  const int32_t nx = a.vnext[b];
  int32_t* out = a.out_tokens + b * a.cap + a.len[b];
  for (int32_t i = 0; i < n; ++i) out[i] = a.drafts[b * a.gamma + i];
  out[n] = nx;
  a.len[b] += n + 1;
  a.cur[b] = nx;
  *acc = n;
}

__global__ __launch_bounds__(kBlock) void k_dec_finish(DecodeArgs a) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= a.B) return;
  a.out_length[b] = a.fail[b] ? -1 : a.len[b];
}

}  // namespace specv
