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
// k_cas_outer_rows writes the target review's fp32 rows: the target table
// rows, and draft rows fl32(T ln Q) so that softmax(row / T) = Q.
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

// One wave per (sequence, position i <= k1): the target row of position i
// and, for i < k1, the draft row fl32(T ln Q).
template <int DT>
__global__ __launch_bounds__(kBlock) void k_cas_outer_rows(CascadeArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t item = wave_uniform((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  if (item >= (int64_t)a.B * (a.k1 + 1)) return;
  const int64_t b = item / (a.k1 + 1);
  const int i = (int)(item - b * (a.k1 + 1));
  const int64_t V = a.V;
  const int32_t prev = (i == 0) ? a.cur[b] : a.dtok[b * a.dcap + i - 1];
  constexpr int64_t esz = (DT == kBF16) ? 2 : 4;
  {
    const void* src = static_cast<const char*>(a.ttab) + (int64_t)prev * V * esz;
    float* dst = a.otpack + (b * (a.k1 + 1) + i) * V;
    for (int64_t v = lane; v < V; v += kWave) dst[v] = load_logit<DT>(src, v);
  }
  if (i == a.k1) return;
  if (lane == 0) a.otok[b * a.k1 + i] = a.dtok[b * a.dcap + i];
  float* out = a.odpack + (b * a.k1 + i) * V;
  const float T = a.temperature[b];
  const bool sampling = T > 0.f && T < pinf();
  if (!sampling || a.fail[b]) {
    for (int64_t v = lane; v < V; v += kWave) out[v] = 0.f;  // not read (greedy or failed)
    return;
  }
  const int32_t pv = a.dprev[b * a.dcap + i];
  const void* r1 = static_cast<const char*>(a.m1tab) + (int64_t)pv * V * esz;
  if (a.dbonus[b * a.dcap + i]) {
    for (int64_t v = lane; v < V; v += kWave) out[v] = load_logit<DT>(r1, v);  // Q = p1
    return;
  }
  const void* r2 = static_cast<const char*>(a.m2tab) + (int64_t)pv * V * esz;
  const float k = temp_scale(T);
  float m1 = ninf(), m2 = ninf();
  for (int64_t v = lane; v < V; v += kWave) {
    m1 = fmaxf(m1, load_logit<DT>(r1, v));
    m2 = fmaxf(m2, load_logit<DT>(r2, v));
  }
  const float rk1 = ref_point(wave_max(m1), k), rk2 = ref_point(wave_max(m2), k);
  double s1 = 0.0, s2 = 0.0;
  for (int64_t v = lane; v < V; v += kWave) {
    s1 += (double)exp2_hw(__builtin_fmaf(load_logit<DT>(r1, v), k, -rk1));
    s2 += (double)exp2_hw(__builtin_fmaf(load_logit<DT>(r2, v), k, -rk2));
  }
  const double S1 = wave_sum(s1), S2 = wave_sum(s2);
  auto probs = [&](int64_t v, double& p1, double& q2) {
    p1 = (double)exp2_hw(__builtin_fmaf(load_logit<DT>(r1, v), k, -rk1)) / S1;
    q2 = (double)exp2_hw(__builtin_fmaf(load_logit<DT>(r2, v), k, -rk2)) / S2;
  };
  double beta = 0.0, rmass = 0.0;
  for (int64_t v = lane; v < V; v += kWave) {
    double p1, q2;
    probs(v, p1, q2);
    beta += fmin(q2, lenient(p1, a.lenience, a.eps));
    rmass += fmax(p1 - q2, 0.0);
  }
  beta = wave_sum(beta);
  rmass = wave_sum(rmass);
  for (int64_t v = lane; v < V; v += kWave) {
    double p1, q2;
    probs(v, p1, q2);
    double Q = fmin(q2, lenient(p1, a.lenience, a.eps));
    const double d = p1 - q2;
    if (rmass > 0.0 && d > 0.0) Q += (1.0 - beta) * d / rmass;
    out[v] = (Q > 0.0) ? (float)((double)T * log(Q)) : ninf();
  }
}

}  // namespace specv
