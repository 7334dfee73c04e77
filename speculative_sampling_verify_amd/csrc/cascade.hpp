// cascade.hpp -- CS Drafting's vertical cascade with bigram "models" (gfx950).
//
// Three bigram tables: the target, an intermediate drafter m1 and the
// smallest drafter m2 ("Cascade Speculative Drafting for Even Faster LLM
// Inference", sections 3.1 and 3.4). An outer round builds a draft of k1
// tokens for the target from inner rounds: m2 drafts k2 tokens (the decode
// loop's drafting kernel), m1 reviews them with a lenience (the verify
// step's lenient accept), and the n accepted tokens plus the drawn one join
// the draft. The target then reviews the first k1 draft tokens without
// lenience, against the law each draft token was drawn from:
//   from an inner position i < k2: Q = min(q2, f(p1)) + (1 - beta) *
//     norm(max(0, p1 - q2)), beta = sum_v min(q2(v), f(p1(v)));
//   from the inner bonus position: Q = p1 (the m1 row itself serves).
// k_cas_outer_rows_wg (V <= 8192; else k_cas_outer_rows) writes the target
// review's fp32 rows: the target table rows, and draft rows fl32(T ln Q) so
// that softmax(row / T) = Q.
#pragma once

#include "decode.hpp"

namespace specv {

struct CascadeArgs {
  const void* ttab;
  const void* m1tab;
  const void* m2tab;
  const float* temperature;
  int32_t* cur;      // [B] last token of each sequence
  int32_t* icur;     // [B] last token of context + partial draft (inner drafting start)
  int32_t* fail;     // [B]
  int32_t* dlen;     // [B] draft tokens so far this outer round
  int32_t* dtok;     // [B, dcap] draft tokens
  int32_t* dprev;    // [B, dcap] the token before each (the row its law comes from)
  int32_t* dbonus;   // [B, dcap] 1 if it came from an inner bonus position
  const int32_t* itok;  // [B, k2] inner drafts
  const int32_t* ipr;   // [B, k2 + 1] inner prev per slot (the m1 row of each)
  const int32_t* vn;    // [B] review outputs
  const int32_t* vnext;
  float* otpack;        // [B (k1 + 1), V] target review: target rows (fp32)
  float* odpack;        // [B k1, V] target review: draft rows fT ln Q (fp32)
  int32_t* otok;        // [B k1] target review: draft tokens
  int32_t lenience;
  float eps;
  int64_t V, dcap;
  int32_t B, k1, k2;
};

__global__ __launch_bounds__(kBlock) void k_cas_round_init(CascadeArgs a) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= a.B) return;
  a.dlen[b] = 0;
  a.icur[b] = a.cur[b];
}

// After an inner review: the n accepted drafts and the drawn token join the
// draft of every sequence whose draft is not complete yet.
__global__ __launch_bounds__(kBlock) void k_cas_inner_append(CascadeArgs a) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= a.B) return;
  int32_t d = a.dlen[b];
  if (d >= a.k1) return;  // complete: this round's result is not used
  const int32_t n = a.vn[b];
  int32_t* tok = a.dtok + b * a.dcap;
  int32_t* prv = a.dprev + b * a.dcap;
  int32_t* bon = a.dbonus + b * a.dcap;
  if (n < 0) {
    // the sequence failed: pad with token 0 so that every row the target
    // review addresses exists
    a.fail[b] = 1;
    for (; d < a.k1; ++d) {
      tok[d] = 0;
      prv[d] = 0;
      bon[d] = 0;
    }
    a.dlen[b] = a.k1;
    return;
  }
  for (int32_t i = 0; i <= n; ++i) {
    tok[d + i] = (i < n) ? a.itok[b * a.k2 + i] : a.vnext[b];
    prv[d + i] = a.ipr[b * (a.k2 + 1) + i];
    bon[d + i] = (i == a.k2) ? 1 : 0;
  }
  a.dlen[b] = d + n + 1;
  a.icur[b] = tok[d + n];
}

// Eight consecutive elements at v0 (-inf past V): one 16-byte load for bf16,
// two for fp32, when rows are 16-byte multiples and aligned; else scalar.
template <int DT, bool VEC>
__device__ __forceinline__ void cas_load8(const void* row, int64_t V, int64_t v0, float (&z)[8]) {
  if constexpr (VEC) {
    // V is a multiple of the vector width here: a vector is all in or all out
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const char*>(row) +
                                                    v0 * (DT == kBF16 ? 2 : 4));
    if constexpr (DT == kBF16) {
      u32x4 q = {0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};
      if (v0 < V) q = p[0];
      z[0] = bf16_lo(q.x); z[1] = bf16_hi(q.x); z[2] = bf16_lo(q.y); z[3] = bf16_hi(q.y);
      z[4] = bf16_lo(q.z); z[5] = bf16_hi(q.z); z[6] = bf16_lo(q.w); z[7] = bf16_hi(q.w);
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4 q = {0xff800000u, 0xff800000u, 0xff800000u, 0xff800000u};
        if (v0 + 4 * h < V) q = p[h];
        z[4 * h + 0] = __uint_as_float(q.x); z[4 * h + 1] = __uint_as_float(q.y);
        z[4 * h + 2] = __uint_as_float(q.z); z[4 * h + 3] = __uint_as_float(q.w);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) z[j] = (v0 + j < V) ? load_logit<DT>(row, v0 + j) : ninf();
  }
}

// The same eight elements as raw 32-bit words: bf16 pairs (element 2w in the
// low half of word w) or fp32 values. The workgroup row builder holds its
// rows this way (half the registers for bf16) and widens them in each pass.
template <int DT>
struct CasRaw {
  static constexpr int W = (DT == kBF16) ? 4 : 8;
  uint32_t w[W];
  __device__ __forceinline__ float operator[](int j) const {
    if constexpr (DT == kBF16) return (j & 1) ? bf16_hi(w[j / 2]) : bf16_lo(w[j / 2]);
    else return __uint_as_float(w[j]);
  }
};

template <int DT, bool VEC>
__device__ __forceinline__ void cas_load8_raw(const void* row, int64_t V, int64_t v0, CasRaw<DT>& r) {
  if constexpr (VEC && DT == kBF16) {
    u32x4 q = {0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};
    if (v0 < V) q = *reinterpret_cast<const u32x4*>(static_cast<const char*>(row) + v0 * 2);
    r.w[0] = q.x; r.w[1] = q.y; r.w[2] = q.z; r.w[3] = q.w;
  } else {
    float z[8];
    cas_load8<DT, VEC>(row, V, v0, z);
#pragma unroll
    for (int q = 0; q < CasRaw<DT>::W; ++q) {
      if constexpr (DT == kBF16)
        r.w[q] = (__float_as_uint(z[2 * q + 1]) & 0xffff0000u) | (__float_as_uint(z[2 * q]) >> 16);
      else
        r.w[q] = __float_as_uint(z[q]);
    }
  }
}

// Empty asm statements that the compiler must assume change the words, so
// that a pass widens and exponentiates them again instead of keeping an
// earlier pass's values alive (several times the registers).
template <int DT>
__device__ __forceinline__ void cas_opaque(CasRaw<DT>& r) {
#pragma unroll
  for (int u = 0; u < CasRaw<DT>::W; ++u) asm volatile("" : "+v"(r.w[u]));
}

template <bool VEC>
__device__ __forceinline__ void cas_store8(float* row, int64_t V, int64_t v0, const float (&z)[8]) {
  if constexpr (VEC) {
    if (v0 >= V) return;
    f32x4* p = reinterpret_cast<f32x4*>(row + v0);
    p[0] = f32x4{z[0], z[1], z[2], z[3]};
    if (v0 + 4 < V) p[1] = f32x4{z[4], z[5], z[6], z[7]};
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (v0 + j < V) row[v0 + j] = z[j];
  }
}

// T ln Q in fp32: v_log_f32 (log2, within about 1 ulp) times T ln 2. A
// subnormal Q is scaled by 2^64 first (the hardware logarithm flushes
// subnormal inputs); Q <= 0 gives -inf.
__device__ __forceinline__ float t_ln32(float Q, float T_ln2) {
  if (!(Q > 0.f)) return ninf();
  const float l = (Q < 1.17549435e-38f) ? __builtin_amdgcn_logf(Q * 0x1p64f) - 64.f
                                        : __builtin_amdgcn_logf(Q);
  return T_ln2 * l;
}

// f(p, eps) in fp32 for the row builder: p / eps and p / eps^2 as products
// with the reciprocal, p^eps = 2^(eps log2 p) on the transcendental unit.
__device__ __forceinline__ float lenient32(float p, int32_t kind, float eps, float inv) {
  if (kind == kLenLin || kind == kLenSq) return p * inv;
  if (kind == kLenExp) return (p > 0.f) ? exp2_hw(eps * __builtin_amdgcn_logf(p)) : 0.f;
  return p;
}

// One wave per (sequence, position i <= k1): the target row of position i
// and, for i < k1, the draft row fl32(T ln Q). Eight consecutive elements per
// lane per step; Q's row statistics in one online (max, sum) pass, then a
// pass for beta and the residual mass and a pass that writes the row.
template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void k_cas_outer_rows(CascadeArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t item = wave_uniform((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  if (item >= (int64_t)a.B * (a.k1 + 1)) return;
  const int64_t b = item / (a.k1 + 1);
  const int i = (int)(item - b * (a.k1 + 1));
  const int64_t V = a.V;
  constexpr int64_t kStep = kWave * 8;
  const int32_t prev = (i == 0) ? a.cur[b] : a.dtok[b * a.dcap + i - 1];
  constexpr int64_t esz = (DT == kBF16) ? 2 : 4;
  {
    const void* src = static_cast<const char*>(a.ttab) + (int64_t)prev * V * esz;
    float* dst = a.otpack + (b * (a.k1 + 1) + i) * V;
    for (int64_t v0 = (int64_t)lane * 8; v0 < V; v0 += kStep) {
      float z[8];
      cas_load8<DT, VEC>(src, V, v0, z);
      cas_store8<VEC>(dst, V, v0, z);
    }
  }
  if (i == a.k1) return;
  if (lane == 0) a.otok[b * a.k1 + i] = a.dtok[b * a.dcap + i];
  float* out = a.odpack + (b * a.k1 + i) * V;
  const float T = a.temperature[b];
  const bool sampling = sampling_temperature(T);
  if (!sampling || a.fail[b]) {
    const float zero[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int64_t v0 = (int64_t)lane * 8; v0 < V; v0 += kStep) cas_store8<VEC>(out, V, v0, zero);
    return;  // not read (greedy or failed)
  }
  const int32_t pv = a.dprev[b * a.dcap + i];
  const void* r1 = static_cast<const char*>(a.m1tab) + (int64_t)pv * V * esz;
  if (a.dbonus[b * a.dcap + i]) {  // Q = p1: the m1 row itself
    for (int64_t v0 = (int64_t)lane * 8; v0 < V; v0 += kStep) {
      float z[8];
      cas_load8<DT, VEC>(r1, V, v0, z);
      cas_store8<VEC>(out, V, v0, z);
    }
    return;
  }
  const void* r2 = static_cast<const char*>(a.m2tab) + (int64_t)pv * V * esz;
  const float k = temp_scale(T);
  // pass 1: per-lane online max and sum of 2^((z - max) k) for both rows
  float m1 = ninf(), m2 = ninf();
  double s1 = 0.0, s2 = 0.0;
  auto online = [&](const float (&z)[8], float& m, double& s) {
    const float g = tile_max(z);
    if (!(g > ninf())) return;
    const float mn = fmaxf(m, g);
    const float sc = rescale32(m, mn, k);
    const float ref = ref_logit(mn);
    float e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = exp2_hw(term_exp(z[j], ref, k));
    s = __builtin_fma(s, (double)sc, (double)tree_sum(e));
    m = mn;
  };
  for (int64_t v0 = (int64_t)lane * 8; v0 < V; v0 += kStep) {
    float z1[8], z2[8];
    cas_load8<DT, VEC>(r1, V, v0, z1);
    cas_load8<DT, VEC>(r2, V, v0, z2);
    online(z1, m1, s1);
    online(z2, m2, s2);
  }
  const float M1 = wave_max(m1), M2 = wave_max(m2);
  const float R1 = ref_logit(M1), R2 = ref_logit(M2);
  const double S1 = wave_sum((m1 == ninf()) ? 0.0 : s1 * exp2(((double)m1 - (double)R1) * (double)k));
  const double S2 = wave_sum((m2 == ninf()) ? 0.0 : s2 * exp2(((double)m2 - (double)R2) * (double)k));
  // Passes 2 and 3 work per element in fp32 (p1 and q2 come from fp32
  // terms already) and add in fp64 per lane: the rows are fp32, and the
  // error stays near 1e-7 relative.
  const float i1 = (float)(1.0 / S1), i2 = (float)(1.0 / S2);
  const float inv = (a.lenience == kLenLin) ? (float)(1.0 / (double)a.eps)
                    : (a.lenience == kLenSq) ? (float)(1.0 / ((double)a.eps * (double)a.eps)) : 1.f;
  auto probs = [&](float z1, float z2, float& p1, float& q2) {
    p1 = exp2_hw(term_exp(z1, R1, k)) * i1;
    q2 = exp2_hw(term_exp(z2, R2, k)) * i2;
  };
  // pass 2: beta = sum min(q2, f(p1)) and the residual mass sum max(0, p1 - q2)
  double beta = 0.0, rmass = 0.0;
  for (int64_t v0 = (int64_t)lane * 8; v0 < V; v0 += kStep) {
    float z1[8], z2[8], bb[8], rr[8];
    cas_load8<DT, VEC>(r1, V, v0, z1);
    cas_load8<DT, VEC>(r2, V, v0, z2);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float p1, q2;
      probs(z1[j], z2[j], p1, q2);
      bb[j] = fminf(q2, lenient32(p1, a.lenience, a.eps, inv));
      rr[j] = fmaxf(p1 - q2, 0.f);
    }
    beta += (double)tree_sum(bb);
    rmass += (double)tree_sum(rr);
  }
  beta = wave_sum(beta);
  rmass = wave_sum(rmass);
  const float c = (rmass > 0.0) ? (float)((1.0 - beta) / rmass) : 0.f;
  const float T_ln2 = (float)((double)T * 0.69314718055994530942);
  // pass 3: Q and the row fl32(T ln Q)
  for (int64_t v0 = (int64_t)lane * 8; v0 < V; v0 += kStep) {
    float z1[8], z2[8], o[8];
    cas_load8<DT, VEC>(r1, V, v0, z1);
    cas_load8<DT, VEC>(r2, V, v0, z2);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float p1, q2;
      probs(z1[j], z2[j], p1, q2);
      const float Q = fminf(q2, lenient32(p1, a.lenience, a.eps, inv)) + c * fmaxf(p1 - q2, 0.f);
      o[j] = t_ln32(Q, T_ln2);
    }
    cas_store8<VEC>(out, V, v0, o);
  }
}

// The same rows by a workgroup of kCasWaves waves per (sequence, position),
// for V <= kCasResident: wave w holds the 512-element steps w, w + W, ... of
// both drafter rows in registers, so each row is read once and each weight
// formed once; the passes exchange per-wave results through LDS:
//   1. the rows' maxima M1, M2;
//   2. the weights 2^(fl32(fl32(z - M) k)) in place, and S1, S2 (per-lane fp32
//      tree sums of eight, fp64 lane and wave sums, the waves added in order);
//   3. beta and the residual mass from p1 = t1 fl32(1/S1), q2 = t2 fl32(1/S2);
// then each wave writes its steps of fl32(T ln Q). Every early return depends
// only on (sequence, position) and comes before the first barrier.
constexpr int kCasWaves = 4;
constexpr int kCasSteps = 4;
constexpr int64_t kCasResident = (int64_t)kCasWaves * kCasSteps * kWave * 8;

struct CasLds {
  float m1[kCasWaves], m2[kCasWaves];
  double s1[kCasWaves], s2[kCasWaves], beta[kCasWaves], rmass[kCasWaves];
};

template <int DT, bool VEC, int32_t KIND>
__global__ __launch_bounds__(kCasWaves * kWave) void k_cas_outer_rows_wg(CascadeArgs a) {
  __shared__ CasLds sh;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = (int)(threadIdx.x >> 6);
  const int64_t item = blockIdx.x;
  const int64_t b = item / (a.k1 + 1);
  const int i = (int)(item - b * (a.k1 + 1));
  const int64_t V = a.V;
  constexpr int64_t kStep = kWave * 8;
  const int64_t n_steps = (V + kStep - 1) / kStep;
  constexpr int64_t esz = (DT == kBF16) ? 2 : 4;
  const int32_t prev = (i == 0) ? a.cur[b] : a.dtok[b * a.dcap + i - 1];
  auto copy_row = [&](const void* src, float* dst) {
    for (int64_t st = w; st < n_steps; st += kCasWaves) {
      float z[8];
      cas_load8<DT, VEC>(src, V, st * kStep + (int64_t)lane * 8, z);
      cas_store8<VEC>(dst, V, st * kStep + (int64_t)lane * 8, z);
    }
  };
  copy_row(static_cast<const char*>(a.ttab) + (int64_t)prev * V * esz,
           a.otpack + (b * (a.k1 + 1) + i) * V);
  if (i == a.k1) return;
  if (threadIdx.x == 0) a.otok[b * a.k1 + i] = a.dtok[b * a.dcap + i];
  float* out = a.odpack + (b * a.k1 + i) * V;
  const float T = a.temperature[b];
  const bool sampling = sampling_temperature(T);
  if (!sampling || a.fail[b]) {
    const float zero[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int64_t st = w; st < n_steps; st += kCasWaves)
      cas_store8<VEC>(out, V, st * kStep + (int64_t)lane * 8, zero);
    return;  // not read (greedy or failed)
  }
  const int32_t pv = a.dprev[b * a.dcap + i];
  const void* r1 = static_cast<const char*>(a.m1tab) + (int64_t)pv * V * esz;
  if (a.dbonus[b * a.dcap + i]) {  // Q = p1: the m1 row itself
    copy_row(r1, out);
    return;
  }
  const void* r2 = static_cast<const char*>(a.m2tab) + (int64_t)pv * V * esz;
  const float k = temp_scale(T);
  CasRaw<DT> z1[kCasSteps], z2[kCasSteps];
#pragma unroll
  for (int q = 0; q < kCasSteps; ++q) {
    const int64_t st = w + (int64_t)q * kCasWaves;
    if (st < n_steps) {
      cas_load8_raw<DT, VEC>(r1, V, st * kStep + (int64_t)lane * 8, z1[q]);
      cas_load8_raw<DT, VEC>(r2, V, st * kStep + (int64_t)lane * 8, z2[q]);
    } else {
#pragma unroll
      for (int u = 0; u < CasRaw<DT>::W; ++u)
        z1[q].w[u] = z2[q].w[u] = (DT == kBF16) ? 0xff80ff80u : 0xff800000u;
    }
  }
  // 1. maxima
  float m1 = ninf(), m2 = ninf();
#pragma unroll
  for (int q = 0; q < kCasSteps; ++q)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      m1 = fmaxf(m1, z1[q][j]);
      m2 = fmaxf(m2, z2[q][j]);
    }
  m1 = wave_max(m1);
  m2 = wave_max(m2);
  if (lane == 0) {
    sh.m1[w] = m1;
    sh.m2[w] = m2;
  }
  __syncthreads();
  float M1 = ninf(), M2 = ninf();
#pragma unroll
  for (int q = 0; q < kCasWaves; ++q) {
    M1 = fmaxf(M1, sh.m1[q]);
    M2 = fmaxf(M2, sh.m2[q]);
  }
  const float R1 = ref_logit(M1), R2 = ref_logit(M2);
  // The weights 2^(fl32(fl32(z - R) k)) of step q, formed the same way in each
  // pass (so with the same values); one step's weights are live at a time.
  auto weights = [&](int q, float (&e1)[8], float (&e2)[8]) {
    cas_opaque(z1[q]);
    cas_opaque(z2[q]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      e1[j] = exp2_hw(term_exp(z1[q][j], R1, k));
      e2[j] = exp2_hw(term_exp(z2[q][j], R2, k));
    }
  };
  // 2. the row sums
  double s1 = 0.0, s2 = 0.0;
#pragma unroll
  for (int q = 0; q < kCasSteps; ++q) {
    float e1[8], e2[8];
    weights(q, e1, e2);
    s1 += (double)tree_sum(e1);
    s2 += (double)tree_sum(e2);
    __builtin_amdgcn_sched_barrier(0);
  }
  s1 = wave_sum(s1);
  s2 = wave_sum(s2);
  if (lane == 0) {
    sh.s1[w] = s1;
    sh.s2[w] = s2;
  }
  __syncthreads();
  double S1 = 0.0, S2 = 0.0;
#pragma unroll
  for (int q = 0; q < kCasWaves; ++q) {
    S1 += sh.s1[q];
    S2 += sh.s2[q];
  }
  const float i1 = (float)(1.0 / S1), i2 = (float)(1.0 / S2);
  const float inv = (a.lenience == kLenLin) ? (float)(1.0 / (double)a.eps)
                    : (a.lenience == kLenSq) ? (float)(1.0 / ((double)a.eps * (double)a.eps)) : 1.f;
  const float T_ln2 = (float)((double)T * 0.69314718055994530942);
  // 3. beta and the residual mass, then the row fl32(T ln Q). The lenience
  // kind (a.lenience) is the template's KIND, so each kind's arithmetic
  // gets a register allocation of its own.
  {
    double beta = 0.0, rmass = 0.0;
#pragma unroll
    for (int q = 0; q < kCasSteps; ++q) {
      float e1[8], e2[8], bb[8], rr[8];
      weights(q, e1, e2);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p1 = e1[j] * i1, q2 = e2[j] * i2;
        bb[j] = fminf(q2, lenient32(p1, KIND, a.eps, inv));
        rr[j] = fmaxf(p1 - q2, 0.f);
      }
      beta += (double)tree_sum(bb);
      rmass += (double)tree_sum(rr);
      __builtin_amdgcn_sched_barrier(0);
    }
    beta = wave_sum(beta);
    rmass = wave_sum(rmass);
    if (lane == 0) {
      sh.beta[w] = beta;
      sh.rmass[w] = rmass;
    }
    __syncthreads();
    double B = 0.0, Rm = 0.0;
#pragma unroll
    for (int q = 0; q < kCasWaves; ++q) {
      B += sh.beta[q];
      Rm += sh.rmass[q];
    }
    const float c = (Rm > 0.0) ? (float)((1.0 - B) / Rm) : 0.f;
#pragma unroll
    for (int q = 0; q < kCasSteps; ++q) {
      const int64_t st = w + (int64_t)q * kCasWaves;
      if (st >= n_steps) break;
      float e1[8], e2[8], o[8];
      weights(q, e1, e2);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p1 = e1[j] * i1, q2 = e2[j] * i2;
        const float Q = fminf(q2, lenient32(p1, KIND, a.eps, inv)) + c * fmaxf(p1 - q2, 0.f);
        o[j] = t_ln32(Q, T_ln2);
      }
      cas_store8<VEC>(out, V, st * kStep + (int64_t)lane * 8, o);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

}  // namespace specv
