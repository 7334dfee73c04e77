// decode.hpp -- multi-round speculative decoding with bigram "models" (gfx950).
//
// The step of DistillSpec Algorithm A.1 repeated over rounds, with models
// that are bigram tables: the logits of the next token after token s are row
// s of a [V, V] table (one for the target, one for the draft). One round:
//   k_dec_draft   one wave per sequence drafts gamma tokens autoregressively
//                 from softmax(draft row / T) by inverse CDF in index order
//                 (u = word 0 of Philox(seed; row, i, 1)), or by argmax when
//                 T = 0, and records which table row feeds each packed row;
//   k_dec_gather  copies those table rows into the packed layout of the
//                 verify step (what a model's output layer would write);
//   the verify step (plan, pass 1, accept + pass 2, draw);
//   k_dec_append  appends the n accepted drafts and the drawn token.
// Within a lane the drafting scan holds 16 consecutive elements, so lane
// order is index order and the running sums follow the index-order CDF: a
// tile's per-lane fp32 tree sums are scanned across the wave in float64,
// and the tile totals are added in tile order; the same code gives the total
// S and the walk that finds the first cumulative sum >= u * S.
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

template <int DT>
__device__ __forceinline__ float dec_elem(const void* row, int64_t V, int64_t e) {
  return e < V ? load_logit<DT>(row, e) : ninf();
}

// One draw from softmax(row * k) (k = log2(e)/T), or the argmax for k == 0.
template <int DT>
__device__ int dec_sample_row(const void* row, int64_t V, float k, double u, int lane) {
  float m = ninf();
  int64_t arg = INT32_MAX;
  for (int64_t e0 = 0; e0 < V; e0 += kDecTE) {
#pragma unroll
    for (int j = 0; j < kDecPL; ++j) {
      const int64_t e = e0 + (int64_t)lane * kDecPL + j;
      const float z = dec_elem<DT>(row, V, e);
      if (z > m) {
        m = z;
        arg = e;
      }
    }
  }
  const float M = wave_max(m);
  if (k == 0.f) {
    const int best = wave_min((m == M && arg < INT32_MAX) ? (int)arg : INT32_MAX);
    return best == INT32_MAX ? 0 : best;
  }
  const float rk = ref_point(M, k);
  auto tile_scan = [&](int64_t e0, float (&w)[kDecPL], float& ls) {
#pragma unroll
    for (int j = 0; j < kDecPL; ++j)
      w[j] = exp2_hw(__builtin_fmaf(dec_elem<DT>(row, V, e0 + (int64_t)lane * kDecPL + j), k, -rk));
    float t[kDecPL];
#pragma unroll
    for (int j = 0; j < kDecPL; ++j) t[j] = w[j];
    ls = tree_sum(t);
    return wave_inclusive_scan((double)ls, lane);
  };
  double S = 0.0;
  for (int64_t e0 = 0; e0 < V; e0 += kDecTE) {
    float w[kDecPL], ls;
    const double incl = tile_scan(e0, w, ls);
    S += __shfl(incl, kWave - 1, kWave);
  }
  const double target = u * S;
  double C = 0.0;
  for (int64_t e0 = 0; e0 < V; e0 += kDecTE) {
    float w[kDecPL], ls;
    const double incl = tile_scan(e0, w, ls);
    const double tot = __shfl(incl, kWave - 1, kWave);
    if (C + tot >= target || e0 + kDecTE >= V) {
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
        if (tok < 0) tok = last;
        tok = (int)(e0 + (int64_t)lane * kDecPL + (tok < 0 ? 0 : tok));
      }
      return __shfl(tok, L, kWave);
    }
    C += tot;
  }
  return 0;
}

template <int DT>
__global__ __launch_bounds__(kBlock) void k_dec_draft(DecodeArgs a) {
  constexpr int64_t esz = (DT == kBF16) ? 2 : 4;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t b = wave_uniform((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  if (b >= a.B) return;
  const float T = a.temperature[b];
  const bool sampling = T > 0.f && T < pinf();
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
      x = dec_sample_row<DT>(row, a.V, k, u, lane);
      if (x < 0 || (int64_t)x >= a.V) x = 0;
    }
    if (lane == 0) a.drafts[b * a.gamma + i] = x;
    prev = x;
  }
}

// Copies table rows into the packed verify layout: one wave per (packed row,
// 16 KiB piece). Rows [0, n_t) are target rows, then n_d draft rows.
struct GatherArgs {
  const void* ttab;
  const void* dtab;
  const int32_t* trow_src;
  const int32_t* drow_src;
  void* tdst;
  void* ddst;
  int64_t row_bytes, n_t, n_d;
  int32_t pieces;  // per row
};

constexpr int64_t kGatherPiece = 16384;

template <bool VEC>
__global__ __launch_bounds__(kBlock) void k_dec_gather(GatherArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t item = wave_uniform((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  if (item >= (a.n_t + a.n_d) * a.pieces) return;
  const int64_t r = item / a.pieces;
  const int64_t p = item - r * a.pieces;
  const bool tgt = r < a.n_t;
  const int64_t src_row = tgt ? a.trow_src[r] : a.drow_src[r - a.n_t];
  const char* src = static_cast<const char*>(tgt ? a.ttab : a.dtab) + src_row * a.row_bytes;
  char* dst = static_cast<char*>(tgt ? a.tdst : a.ddst) + (tgt ? r : r - a.n_t) * a.row_bytes;
  const int64_t b0 = p * kGatherPiece;
  const int64_t b1 = min(a.row_bytes, b0 + kGatherPiece);
  if constexpr (VEC) {
    for (int64_t o = b0 + (int64_t)lane * 16; o < b1; o += kWave * 16)
      *reinterpret_cast<u32x4*>(dst + o) = *reinterpret_cast<const u32x4*>(src + o);
  } else {
    for (int64_t o = b0 + (int64_t)lane * 2; o < b1; o += kWave * 2)
      *reinterpret_cast<uint16_t*>(dst + o) = *reinterpret_cast<const uint16_t*>(src + o);
  }
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
