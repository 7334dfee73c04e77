// kernels.hpp -- the verify step's kernels for gfx950.
//
// The step (DistillSpec, Appendix A.3, Algorithm A.1, lenience 1) runs as:
//   k0_plan        offsets of the packed ragged rows, row -> sequence maps,
//                  layout validation; initialises the status word.
//   k1_row_stats   pass 1, the HBM-bound hot loop: every needed logit row is
//                  streamed once with 16-byte non-temporal loads; each wave
//                  owns one (row, chunk) and keeps (max, sum of 2^(z k - rk),
//                  argmax) in registers, reduced across the wave by shuffles.
//   k2_accept      one wave per sequence, one lane per draft position: merges
//                  the chunk statistics, gathers p_i(x_i) and q_i(x_i), draws
//                  r_i from Philox, and takes the first rejection by ballot.
//                  Greedy sequences finish here (argmax match).
//   k3_mass        pass 2 over the one selected row pair of each sampling
//                  sequence: weight mass max(0, p - q) (or p) per chunk.
//   k3_draw        one workgroup per sampling sequence: picks the chunk that
//                  holds u * total, then an LDS-assisted workgroup prefix scan
//                  inside it finds the token (inverse CDF in index order).
#pragma once

#include "device.hpp"

namespace specv {

// Statistics of one (row, chunk): s = sum over the chunk of
// 2^(fl32(z k - ref_point(m, k))) (sampling rows) or 0/NaN (greedy rows, NaN
// flags a NaN/+inf logit); m = max; arg = lowest index attaining m.
struct RowPart {
  double s;
  float m;
  int32_t arg;
};

// What the final draw of one sampling sequence needs (written by k2_accept).
enum : int32_t { kModeNone = 0, kModeResidual = 1, kModeBonus = 2 };
struct Select {
  int32_t mode;
  int32_t n;
  int64_t trow;  // target row (packed index) of the draw
  int64_t drow;  // draft row for the residual, else -1
  float k;       // log2(e) / T
  float rkT, rkD;
  int32_t pad;
  double sT, sD;
  double u;
};

struct PlanArgs {
  const int32_t* gamma;
  int64_t* toff;
  int64_t* doff;
  int32_t* tmap;
  int32_t* dmap;
  uint32_t* status;
  int64_t total_t, total_d;
  int32_t B, max_gamma;
};

// One workgroup of 1024 threads: thread t owns a contiguous run of sequences.
__global__ __launch_bounds__(1024) void k0_plan(PlanArgs a) {
  __shared__ int64_t sh_t[16], sh_d[16];
  __shared__ int sh_bad[16];
  __shared__ int64_t sh_tot_t, sh_tot_d;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (a.B + 1023) / 1024;
  const int lo = min(a.B, tid * per), hi = min(a.B, lo + per);
  int64_t st = 0, sd = 0;
  int bad = 0;
  for (int b = lo; b < hi; ++b) {
    const int32_t g = a.gamma[b];
    bad |= (g < 0 || g > a.max_gamma);
    const int64_t gg = g < 0 ? 0 : g;
    st += gg + 1;
    sd += gg;
  }
  // workgroup exclusive scan of (st, sd)
  int64_t it = st, id = sd;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t ot = __shfl_up(it, off, 64), od = __shfl_up(id, off, 64);
    if (lane >= off) { it += ot; id += od; }
  }
  const int wbad = __any(bad) ? 1 : 0;
  if (lane == 63) { sh_t[wave] = it; sh_d[wave] = id; sh_bad[wave] = wbad; }
  __syncthreads();
  if (tid == 0) {
    int64_t ct = 0, cd = 0;
    int ab = 0;
    for (int w = 0; w < 16; ++w) {
      const int64_t t = sh_t[w], d = sh_d[w];
      sh_t[w] = ct; sh_d[w] = cd;
      ct += t; cd += d; ab |= sh_bad[w];
    }
    sh_tot_t = ct; sh_tot_d = cd;
    const bool layout_bad = ab || ct != a.total_t || cd != a.total_d;
    a.status[0] = layout_bad ? kLayoutError : 0u;
  }
  __syncthreads();
  int64_t t = sh_t[wave] + it - st, d = sh_d[wave] + id - sd;
  for (int b = lo; b < hi; ++b) {
    const int32_t g = a.gamma[b];
    const int64_t gg = g < 0 ? 0 : g;
    a.toff[b] = t;
    a.doff[b] = d;
    const int64_t tend = min(t + gg + 1, a.total_t), dend = min(d + gg, a.total_d);
    for (int64_t j = t; j < tend; ++j) a.tmap[j] = b;
    for (int64_t j = d; j < dend; ++j) a.dmap[j] = b;
    t += gg + 1;
    d += gg;
  }
  if (tid == 1023) {
    a.toff[a.B] = sh_tot_t;
    a.doff[a.B] = sh_tot_d;
  }
}

struct RowStatsArgs {
  const void* target;
  const void* draft;
  const float* temperature;
  const int32_t* tmap;
  const int32_t* dmap;
  RowPart* tparts;
  RowPart* dparts;
  const uint32_t* status;
  int64_t total_t, total_d, V;
  int32_t B, chunks, chunk_elems;
};

// Online (max, sum) over one chunk for a sampling row. Per element: widen,
// max, one fma and one v_exp_f32 into a pairwise sum; the running sum is
// float64 and is rescaled only when the lane's maximum grows.
template <int DT, bool VEC>
__device__ __forceinline__ RowPart chunk_stats_sampling(const void* row, int64_t e0, int64_t e1,
                                                        float k, int lane) {
  using TL = Tile<DT, VEC>;
  constexpr int NE = TL::NE;
  const int64_t n = e1 - e0;
  const int n_full = (int)(n / TL::EPI), n_iter = (int)((n + TL::EPI - 1) / TL::EPI);
  float m = ninf(), rk = 0.f;
  double s = 0.0;
  int best = -1;
  float z[NE];
  auto step = [&](int it) {
    const float g = tile_max(z);
    if (g > m) best = it;
    const float mn = fmaxf(m, g);
    const float rkn = ref_point(mn, k);
    const float sc = (m == ninf()) ? 0.f : exp2_hw(rk - rkn);
    float e[NE];
#pragma unroll
    for (int j = 0; j < NE; ++j) e[j] = exp2_hw(__builtin_fmaf(z[j], k, -rkn));
    const float acc = tree_sum(e);
    s = __builtin_fma(s, (double)sc, (double)acc);
    m = mn;
    rk = rkn;
  };
  for (int it = 0; it < n_full; ++it) {
    TL::template load<false>(row, e0, e1, it, lane, z);
    step(it);
  }
  if (n_full < n_iter) {
    TL::template load<true>(row, e0, e1, n_full, lane, z);
    step(n_full);
  }
  // the lane's lowest index attaining m: re-read the one tile where m appeared
  int arg = INT32_MAX;
  if (best >= 0) {
    TL::template load<true>(row, e0, e1, best, lane, z);
#pragma unroll
    for (int j = NE - 1; j >= 0; --j)
      if (z[j] == m) arg = (int)TL::index(e0, best, lane, j);
  }
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off, kWave);
    const double s2 = __shfl_xor(s, off, kWave);
    const int a2 = __shfl_xor(arg, off, kWave);
    const float mn = fmaxf(m, m2);
    s = s * rescale64(m, mn, k) + s2 * rescale64(m2, mn, k);
    arg = (m2 > m) ? a2 : ((m2 == m) ? min(arg, a2) : arg);
    m = mn;
  }
  return RowPart{s, m, arg};
}

// Max and argmax only (greedy rows); s = NaN if any logit is NaN or +inf.
template <int DT, bool VEC>
__device__ __forceinline__ RowPart chunk_stats_greedy(const void* row, int64_t e0, int64_t e1,
                                                      int lane) {
  using TL = Tile<DT, VEC>;
  constexpr int NE = TL::NE;
  const int64_t n = e1 - e0;
  const int n_full = (int)(n / TL::EPI), n_iter = (int)((n + TL::EPI - 1) / TL::EPI);
  float m = ninf();
  int best = -1;
  bool bad = false;
  float z[NE];
  auto step = [&](int it) {
    const float g = tile_max(z);
#pragma unroll
    for (int j = 0; j < NE; ++j) bad |= !(z[j] < pinf());
    if (g > m) best = it;
    m = fmaxf(m, g);
  };
  for (int it = 0; it < n_full; ++it) {
    TL::template load<false>(row, e0, e1, it, lane, z);
    step(it);
  }
  if (n_full < n_iter) {
    TL::template load<true>(row, e0, e1, n_full, lane, z);
    step(n_full);
  }
  int arg = INT32_MAX;
  if (best >= 0) {
    TL::template load<true>(row, e0, e1, best, lane, z);
#pragma unroll
    for (int j = NE - 1; j >= 0; --j)
      if (z[j] == m) arg = (int)TL::index(e0, best, lane, j);
  }
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off, kWave);
    const int a2 = __shfl_xor(arg, off, kWave);
    arg = (m2 > m) ? a2 : ((m2 == m) ? min(arg, a2) : arg);
    m = fmaxf(m, m2);
  }
  const bool any_bad = ballot(bad) != 0;
  return RowPart{any_bad ? __builtin_nan("") : 0.0, m, arg};
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void k1_row_stats(RowStatsArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t item = wave_uniform((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  const int64_t rows = a.total_t + a.total_d;
  if (item >= rows * a.chunks) return;
  if (a.status[0] & kLayoutError) return;
  const int64_t r = item / a.chunks;
  const int c = (int)(item - r * a.chunks);
  const bool is_draft = r >= a.total_t;
  const int64_t j = is_draft ? r - a.total_t : r;
  int b = is_draft ? a.dmap[j] : a.tmap[j];
  b = min(max(b, 0), a.B - 1);
  const float T = a.temperature[b];
  const bool sampling = T > 0.f && T < pinf();
  if (is_draft && !sampling) return;  // greedy sequences never read draft rows
  constexpr int64_t esz = (DT == kBF16) ? 2 : 4;
  const void* row = static_cast<const char*>(is_draft ? a.draft : a.target) + j * a.V * esz;
  const int64_t e0 = (int64_t)c * a.chunk_elems;
  const int64_t e1 = min(a.V, e0 + a.chunk_elems);
  RowPart out;
  if (sampling)
    out = chunk_stats_sampling<DT, VEC>(row, e0, e1, temp_scale(T), lane);
  else
    out = chunk_stats_greedy<DT, VEC>(row, e0, e1, lane);
  if (lane == 0) (is_draft ? a.dparts : a.tparts)[j * a.chunks + c] = out;
}

// Per-row merge of the chunk statistics.
struct RowStat {
  double s;    // sum of 2^(fl32(z k - rk)) over the row (sampling), 0/NaN (greedy)
  float m;     // row max
  float rk;    // ref_point(m, k)
  int32_t arg; // lowest index attaining m
  bool valid;  // no NaN/+inf and at least one finite logit
};

__device__ __forceinline__ RowStat merge_row(const RowPart* p, int chunks, float k, bool sampling) {
  float M = ninf();
  for (int c = 0; c < chunks; ++c) M = fmaxf(M, p[c].m);
  int32_t arg = INT32_MAX;
  double S = 0.0;
  for (int c = 0; c < chunks; ++c) {
    const RowPart q = p[c];
    if (q.m == M && arg == INT32_MAX) arg = q.arg;
    S += sampling ? q.s * rescale64(q.m, M, k) : q.s;
  }
  RowStat st;
  st.s = S;
  st.m = M;
  st.rk = ref_point(M, k);
  st.arg = arg;
  st.valid = (M > ninf()) && (M < pinf()) && !__builtin_isnan(S);
  return st;
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
};

// One wave per sequence; lane i owns draft position i and target row i.
template <int DT>
__global__ __launch_bounds__(kBlock) void k2_accept(AcceptArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t b = wave_uniform((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  if (b >= a.B) return;
  Select* sel = a.sel + b;
  auto fail = [&]() {
    if (lane == 0) {
      a.out_n[b] = -1;
      a.out_next[b] = -1;
      sel->mode = kModeNone;
      atomicOr(a.status, kSeqError);
    }
  };
  if (a.status[0] & kLayoutError) {
    if (lane == 0) {
      a.out_n[b] = -1;
      a.out_next[b] = -1;
      sel->mode = kModeNone;
    }
    return;
  }
  const int g = a.gamma[b];
  const float T = a.temperature[b];
  const bool greedy = (T == 0.f);
  const bool sampling = (T > 0.f) && (T < pinf());
  if (!greedy && !sampling) { fail(); return; }
  const int64_t t0 = a.toff[b], d0 = a.doff[b];
  const float k = sampling ? temp_scale(T) : 0.f;
  RowStat st_t{}, st_d{};
  int x = 0;
  bool bad = false;
  if (lane <= g) {
    st_t = merge_row(a.tparts + (t0 + lane) * a.chunks, a.chunks, k, sampling);
    bad |= !st_t.valid;
  }
  if (lane < g) {
    x = a.tokens[d0 + lane];
    bad |= (x < 0) || ((int64_t)x >= a.V);
    if (sampling) {
      st_d = merge_row(a.dparts + (d0 + lane) * a.chunks, a.chunks, k, true);
      bad |= !st_d.valid;
    }
  }
  if (ballot(bad) != 0) { fail(); return; }

  if (greedy) {
    const uint64_t rej = ballot(lane < g && x != st_t.arg);
    const int n = rej ? first_lane(rej) : g;
    const int next = __shfl(st_t.arg, n, kWave);
    if (lane == 0) {
      a.out_n[b] = n;
      a.out_next[b] = next;
      sel->mode = kModeNone;
    }
    return;
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
    const float zT = load_logit<DT>(a.target, (t0 + lane) * a.V + x);
    const float zD = load_logit<DT>(a.draft, (d0 + lane) * a.V + x);
    const double p = exp2((double)zT * (double)k - (double)st_t.rk) / st_t.s;
    const double q = exp2((double)zD * (double)k - (double)st_d.rk) / st_d.s;
    const double ratio = (q == 0.0) ? (double)pinf() : p / q;
    rej = r > ratio;
  }
  const uint64_t mask = ballot(rej);
  const int n = mask ? first_lane(mask) : g;
  const double un = __shfl(u, n, kWave);
  const float rkT = __shfl(st_t.rk, n, kWave);
  const double sT = __shfl(st_t.s, n, kWave);
  const float rkD = __shfl(st_d.rk, n, kWave);
  const double sD = __shfl(st_d.s, n, kWave);
  if (lane == 0) {
    Select s;
    s.mode = (n < g) ? kModeResidual : kModeBonus;
    s.n = n;
    s.trow = t0 + n;
    s.drow = (n < g) ? d0 + n : -1;
    s.k = k;
    s.rkT = rkT;
    s.rkD = rkD;
    s.pad = 0;
    s.sT = sT;
    s.sD = sD;
    s.u = un;
    *sel = s;
    a.out_n[b] = n;
  }
}

// Weight of one token in the final draw: max(0, p - q) or p, in fp32.
struct Weights {
  float k, rkT, rkD, iT, iD;
  bool residual;
  __device__ __forceinline__ float operator()(float zT, float zD) const {
    const float pT = exp2_hw(__builtin_fmaf(zT, k, -rkT)) * iT;
    if (!residual) return pT;
    const float pD = exp2_hw(__builtin_fmaf(zD, k, -rkD)) * iD;
    return fmaxf(pT - pD, 0.f);
  }
};

__device__ __forceinline__ Weights make_weights(const Select& s, bool force_bonus) {
  Weights w;
  w.k = s.k;
  w.rkT = s.rkT;
  w.rkD = s.rkD;
  w.iT = (float)(1.0 / s.sT);
  w.iD = (float)(1.0 / s.sD);
  w.residual = (s.mode == kModeResidual) && !force_bonus;
  return w;
}

struct DrawArgs {
  const void* target;
  const void* draft;
  const Select* sel;
  double* mass;       // [B, chunks3]
  int32_t* out_next;
  int64_t V;
  int32_t B, chunks3, chunk3_elems;
};

// Pass 2: weight mass of one chunk of the selected row pair.
template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void k3_mass(DrawArgs a) {
  using TL = Tile<DT, VEC>;
  constexpr int NE = TL::NE;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t item = wave_uniform((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  if (item >= (int64_t)a.B * a.chunks3) return;
  const int64_t b = item / a.chunks3;
  const int c = (int)(item - b * a.chunks3);
  const Select s = a.sel[b];
  if (s.mode == kModeNone) return;
  const Weights W = make_weights(s, false);
  constexpr int64_t esz = (DT == kBF16) ? 2 : 4;
  const void* trow = static_cast<const char*>(a.target) + s.trow * a.V * esz;
  const void* drow = W.residual ? static_cast<const char*>(a.draft) + s.drow * a.V * esz : nullptr;
  const int64_t e0 = (int64_t)c * a.chunk3_elems, e1 = min(a.V, e0 + a.chunk3_elems);
  const int64_t n = max((int64_t)0, e1 - e0);
  const int n_full = (int)(n / TL::EPI), n_iter = (int)((n + TL::EPI - 1) / TL::EPI);
  double acc = 0.0;
  float zt[NE], zd[NE], w[NE];
  for (int it = 0; it < n_iter; ++it) {
    if (it < n_full) {
      TL::template load<false>(trow, e0, e1, it, lane, zt);
      if (W.residual) TL::template load<false>(drow, e0, e1, it, lane, zd);
    } else {
      TL::template load<true>(trow, e0, e1, it, lane, zt);
      if (W.residual) TL::template load<true>(drow, e0, e1, it, lane, zd);
    }
#pragma unroll
    for (int j = 0; j < NE; ++j) w[j] = W(zt[j], W.residual ? zd[j] : 0.f);
    acc += (double)tree_sum(w);
  }
  acc = wave_sum(acc);
  if (lane == 0) a.mass[item] = acc;
}

// Inverse-CDF search inside [lo, hi) of the selected row: the smallest v with
// t <= base + sum_{lo <= v' <= v} w_v'. Every thread owns 8 consecutive
// elements per step; a workgroup inclusive scan (wave shuffles + LDS across
// waves) locates the owning thread, which walks its 8 elements. Returns -1 if
// rounding leaves t above the range's total (caller falls back).
template <int DT>
__device__ int block_draw(const void* trow, const void* drow, const Weights& W, int64_t lo,
                          int64_t hi, double base, double t, double* total_out,
                          int64_t* last_pos_out) {
  __shared__ double sh_wave[kWavesPerBlock];
  __shared__ int sh_found[kWavesPerBlock];
  __shared__ int sh_tok;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int64_t last_pos = -1;
  int token = -1;
  for (int64_t e = lo; e < hi; e += (int64_t)kBlock * 8) {
    const int64_t my = e + (int64_t)tid * 8;
    float w[8];
    double ts = 0.0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t v = my + j;
      float wv = 0.f;
      if (v < hi) {
        const float zT = load_logit<DT>(trow, v);
        const float zD = W.residual ? load_logit<DT>(drow, v) : 0.f;
        wv = W(zT, zD);
      }
      w[j] = wv;
      if (wv > 0.f) last_pos = v;
      ts += (double)wv;
    }
    double incl = wave_inclusive_scan(ts, lane);
    if (lane == 63) sh_wave[wave] = incl;
    __syncthreads();
    double wbase = 0.0, step_total = 0.0;
    for (int q = 0; q < kWavesPerBlock; ++q) {
      if (q < wave) wbase += sh_wave[q];
      step_total += sh_wave[q];
    }
    incl += wbase;
    const double excl = incl - ts;
    const uint64_t m = ballot(base + incl >= t);
    if (lane == 0) sh_found[wave] = m ? first_lane(m) : 64;
    if (tid == 0) sh_tok = -1;
    __syncthreads();
    int owner = -1;
    for (int q = 0; q < kWavesPerBlock; ++q)
      if (sh_found[q] < 64) { owner = q * 64 + sh_found[q]; break; }
    if (owner >= 0) {
      if (tid == owner) {
        double c = base + excl;
        int tok = -1;
        int64_t lastpos_here = -1;
        for (int j = 0; j < 8; ++j) {
          c += (double)w[j];
          if (w[j] > 0.f) lastpos_here = my + j;
          if (t <= c && tok < 0 && w[j] > 0.f) tok = (int)(my + j);
        }
        if (tok < 0) tok = (int)lastpos_here;  // rounding: stay inside the owning run
        sh_tok = tok;
      }
      __syncthreads();
      token = sh_tok;
      break;
    }
    base += step_total;
    __syncthreads();
  }
  // block-wide last positive element (rounding fallback of the caller)
  __shared__ long long sh_last[kWavesPerBlock];
  long long lp = last_pos;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) lp = max(lp, (long long)__shfl_xor(lp, off, 64));
  if (lane == 0) sh_last[wave] = lp;
  __syncthreads();
  long long best = -1;
  for (int q = 0; q < kWavesPerBlock; ++q) best = max(best, sh_last[q]);
  if (last_pos_out) *last_pos_out = best;
  if (total_out) *total_out = base;
  __syncthreads();
  return token;
}

template <int DT>
__global__ __launch_bounds__(kBlock) void k3_draw(DrawArgs a) {
  const int64_t b = blockIdx.x;
  if (b >= a.B) return;
  const Select s = a.sel[b];
  if (s.mode == kModeNone) return;
  __shared__ double sh_base, sh_t;
  __shared__ int sh_chunk;
  const double* mass = a.mass + b * a.chunks3;
  if (threadIdx.x == 0) {
    double tot = 0.0;
    for (int c = 0; c < a.chunks3; ++c) tot += mass[c];
    int chunk = -1;
    double base = 0.0, t = 0.0;
    if (tot > 0.0) {
      t = s.u * tot;
      double cum = 0.0;
      int lastnz = -1;
      for (int c = 0; c < a.chunks3; ++c) {
        if (mass[c] > 0.0) lastnz = c;
        if (t <= cum + mass[c] && mass[c] > 0.0) { chunk = c; break; }
        cum += mass[c];
      }
      if (chunk < 0) {  // rounding: t above the last prefix
        chunk = lastnz;
        cum = 0.0;
        for (int c = 0; c < chunk; ++c) cum += mass[c];
      }
      base = cum;
    }
    sh_chunk = chunk;
    sh_base = base;
    sh_t = t;
  }
  __syncthreads();
  constexpr int64_t esz = (DT == kBF16) ? 2 : 4;
  const void* trow = static_cast<const char*>(a.target) + s.trow * a.V * esz;
  const void* drow = (s.mode == kModeResidual) ? static_cast<const char*>(a.draft) + s.drow * a.V * esz : nullptr;
  int token;
  if (sh_chunk >= 0) {
    const Weights W = make_weights(s, false);
    const int64_t lo = (int64_t)sh_chunk * a.chunk3_elems, hi = min(a.V, lo + a.chunk3_elems);
    int64_t last_pos = -1;
    token = block_draw<DT>(trow, drow, W, lo, hi, sh_base, sh_t, nullptr, &last_pos);
    if (token < 0) token = (int)last_pos;
  } else {
    // The residual has no mass in fp32 (p_n == q_n to rounding): draw from p_n.
    const Weights W = make_weights(s, true);
    double total = 0.0;
    int64_t last_pos = -1;
    block_draw<DT>(trow, nullptr, W, 0, a.V, 0.0, __builtin_huge_val(), &total, &last_pos);
    token = block_draw<DT>(trow, nullptr, W, 0, a.V, 0.0, s.u * total, nullptr, &last_pos);
    if (token < 0) token = (int)last_pos;
  }
  if (threadIdx.x == 0) a.out_next[b] = token;
}

// ----------------------------- test exports --------------------------------

struct MergeArgs {
  const RowPart* tparts;
  const RowPart* dparts;
  const int32_t* tmap;
  const int32_t* dmap;
  const float* temperature;
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
  const int b = min(max(is_draft ? a.dmap[j] : a.tmap[j], 0), a.B - 1);
  const float T = a.temperature[b];
  const bool sampling = T > 0.f && T < pinf();
  if (is_draft && !sampling) {
    om[j] = __builtin_nanf("");
    os[j] = __builtin_nan("");
    oa[j] = -1;
    return;
  }
  const float k = sampling ? temp_scale(T) : 0.f;
  const RowStat st = merge_row((is_draft ? a.dparts : a.tparts) + j * a.chunks, a.chunks, k, sampling);
  om[j] = st.m;
  // re-reference the sum from fl32(m k) to m k exactly: sum 2^((z - m) k)
  os[j] = sampling ? (st.valid ? st.s * exp2((double)st.rk - (double)st.m * (double)k) : __builtin_nan(""))
                   : (st.valid ? 0.0 : __builtin_nan(""));
  oa[j] = st.arg;
}

struct ProbArgs {
  const void* target;
  const void* draft;
  const RowPart* tparts;
  const RowPart* dparts;
  const int32_t* tmap;
  const int32_t* dmap;
  const float* temperature;
  const int64_t* rows;
  float* out;
  int64_t V, n_rows, total_t, total_d;
  int32_t B, chunks;
};

// grid (element chunks of 2048, rows): p_v = 2^(fl32(z k - rk)) * fl32(1/S),
// the same arithmetic as the final draw's weights.
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
  const int b = min(max(is_draft ? a.dmap[j] : a.tmap[j], 0), a.B - 1);
  const float T = a.temperature[b];
  const float k = temp_scale(T);
  const RowStat st = merge_row((is_draft ? a.dparts : a.tparts) + j * a.chunks, a.chunks, k, true);
  Select s{};
  s.mode = kModeBonus;
  s.k = k;
  s.rkT = st.rk;
  s.sT = st.s;
  const Weights W = make_weights(s, true);
  constexpr int64_t esz = (DT == kBF16) ? 2 : 4;
  const void* row = static_cast<const char*>(is_draft ? a.draft : a.target) + j * a.V * esz;
  const int64_t v0 = (int64_t)blockIdx.x * 2048;
  for (int q = threadIdx.x; q < 2048; q += kBlock) {
    const int64_t v = v0 + q;
    if (v < a.V) a.out[k_row * a.V + v] = W(load_logit<DT>(row, v), 0.f);
  }
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

__global__ __launch_bounds__(kBlock) void k_copy(u32x4* dst, const u32x4* src, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n16; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace specv
