// diagnostics.hpp -- per-position diagnostics of a packed batch (gfx950).
//
// For draft position i of sequence b (packed draft row j, target row j + b):
//   alpha   = sum_v min(p_v, q_v), the acceptance probability of a token
//             drafted from q (DistillSpec section 3; 1 - alpha is the total
//             variation distance of its section 4);
//   entropy = -sum_v q_v ln q_v, and top-k of q: the Ent and Top_k features
//             of DISCO's stopping classifier (DISCO section 3, Eq. 2).
// Pass 1 is k1_row_stats (row max, sum, argmax), run over every draft row.
// Pass 2 (k5_diag_pass) gives one wave to each (position, chunk) -- the same
// interleaved tiles as pass 1 -- and accumulates per element, in fp32 terms
// and fp64 lane sums:
//   min(t^T_v / S^T, t^D_v / S^D),   t^D_v,   t^D_v * e^D_v,
// with t = 2^e, e = fl32(fl32(z - M) k) exactly as in pass 1 (M the row's
// maximum). Since
// q_v = t^D_v / S and ln q_v = e^D_v ln 2 - ln S,
//   entropy = ln S - ln 2 * (sum_v t^D_v e^D_v) / S,   S = sum_v t^D_v.
// Top-k: q is monotone in the logit, so the list is selected on raw logits,
// exactly (larger logit first, equal logits lower index first, as the
// argmax does). Each wave appends the keys of its chunk that can still reach
// the best K to a small LDS buffer and cuts the buffer back to the best K by
// rank counting whenever it fills; the cut also raises the bar that a key
// must clear. The first bar is the K-th largest lane maximum of the chunk,
// taken in pass 1. A tile's group of 8 slots is scanned only when some
// lane's maximum over the group reaches the bar.
// k6_diag_merge (one wave per position) sums the chunks' partials and merges
// their lists; probabilities of the selected tokens are 2^((z - M) k) / S in
// float64, as the accept step computes p(x) and q(x).
#pragma once

#include <type_traits>

#include "kernels.hpp"

namespace specv {

constexpr int kMaxTopK = 64;

struct DiagPart {
  double alpha;  // sum min(p, q) over the chunk
  double s;      // sum t^D
  double a;      // sum t^D e^D
};

struct DiagArgs {
  const void* target;
  const void* draft;
  const float* dk;      // per draft row: log2(e)/T, 0 greedy, -1 invalid T
  const int32_t* dseq;  // per draft row: its sequence
  const float* bar;     // [total_d * chunks]: K-th largest lane maximum (pass 1)
  const RowPart* tparts;
  const RowPart* dparts;
  const uint32_t* status;
  DiagPart* parts;      // [total_d * chunks]
  float* topz;          // [total_d * chunks * K]
  int32_t* topi;        // [total_d * chunks * K]
  double* out_alpha;    // [total_d]
  double* out_entropy;  // [total_d]
  int32_t* out_index;   // [total_d * K]
  double* out_prob;     // [total_d * K]
  int64_t total_d, V;
  int32_t chunks, K;
  int32_t uniform_g;          // >= 0: uniform batch with this gamma; draft row j
  const float* temperature;   // belongs to sequence j / gamma (dk, dseq unused)
};

// Sequence and temperature scale of draft row j: arithmetic in a uniform
// batch, else from the plan's per-row arrays.
__device__ __forceinline__ int64_t diag_seq(const DiagArgs& a, int64_t j) {
  return (a.uniform_g > 0) ? j / a.uniform_g : (int64_t)a.dseq[j];
}
__device__ __forceinline__ float diag_scale(const DiagArgs& a, int64_t j, int64_t b) {
  return (a.uniform_g > 0) ? seq_scale(a.temperature[b]) : a.dk[j];
}

// Ranking keys: larger logit first, equal logits lower index first, as one
// unsigned 64-bit number (order-preserving float bits above the complemented
// index). -0 is folded onto +0 first, since the two compare equal. NaN never
// reaches a key (rows holding one are rejected before).
__device__ __forceinline__ uint64_t rank_key(float z, int32_t idx) {
  const uint32_t b = __float_as_uint(z + 0.f);
  const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)o << 32) | (uint32_t)~(uint32_t)idx;
}
__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t o = (uint32_t)(key >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
__device__ __forceinline__ int32_t key_index(uint64_t key) { return (int32_t)~(uint32_t)key; }

__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// A wave's candidate buffer in LDS: a slot's candidates (at most one per
// lane) are appended, and the buffer is cut back to the best K as soon as it
// holds more than max(2K, 64) keys, so it never exceeds kDiagCap. Scans go
// in groups of kDiagGroup slots.
constexpr int kDiagGroup = 8;
constexpr int kDiagCap = 2 * kMaxTopK + kWave;
constexpr int kDiagSlots = kDiagCap / kWave;

// rank[s] += number of the keys buf[0..n) above mine[s], for s < ns: eight
// broadcast reads in flight per step (the buffer is 16-byte aligned and read
// past n up to the next multiple of 8 only within its capacity, which is a
// multiple of 8; keys past n are skipped).
template <int SLOTS>
__device__ __forceinline__ void count_above(const uint64_t* buf, int n, int ns,
                                            const uint64_t (&mine)[SLOTS], int (&rank)[SLOTS]) {
  typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
  const u64x2* v = reinterpret_cast<const u64x2*>(buf);
  for (int e = 0; e < n; e += 8) {
    u64x2 o[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) o[u] = v[e / 2 + u];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint64_t key = (u & 1) ? o[u / 2].y : o[u / 2].x;
      const bool live = e + u < n;
#pragma unroll
      for (int s = 0; s < SLOTS; ++s)
        if (s < ns) rank[s] += (live && key > mine[s]) ? 1 : 0;
    }
  }
}

// Keeps the best min(n, K) of the n distinct keys buf[0..n) in buf[0..), best
// first: each key's rank is the number of keys above it (broadcast reads of
// the buffer), then the keys of rank < K move to their rank. Wave-private
// buffer: the wave's LDS operations complete in program order.
__device__ __forceinline__ int keep_best(uint64_t* buf, int n, int K, int lane) {
  uint64_t mine[kDiagSlots];
  int rank[kDiagSlots];
  const int ns = (n + kWave - 1) / kWave;
#pragma unroll
  for (int s = 0; s < kDiagSlots; ++s) {
    const int e = lane + s * kWave;
    mine[s] = (s < ns && e < n) ? buf[e] : 0ull;
    rank[s] = 0;
  }
  count_above<kDiagSlots>(buf, n, ns, mine, rank);
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int s = 0; s < kDiagSlots; ++s) {
    const int e = lane + s * kWave;
    if (s < ns && e < n && rank[s] < K) buf[rank[s]] = mine[s];
  }
  __builtin_amdgcn_wave_barrier();
  return n < K ? n : K;
}

// Slot q of a raw tile as fp32 (the order Tile::widen produces).
template <int DT, bool VEC, int Q>
__device__ __forceinline__ float raw_elem(const typename Tile<DT, VEC>::Raw& r) {
  if constexpr (VEC && DT == kBF16) return (Q & 1) ? bf16_hi(r.d[Q / 2]) : bf16_lo(r.d[Q / 2]);
  else return __uint_as_float(r.d[Q]);
}

template <int DT, bool VEC, int G>
__device__ __forceinline__ void diag_terms(const typename Tile<DT, VEC>::Raw& rd,
                                           const typename Tile<DT, VEC>::Raw& rt, float k,
                                           float refT, float refD, float lr, float iD, float& sa,
                                           float& ss, float& sA, float& mx) {
  float pa[8], ps[8], pA[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    float zD, zT;
    // unrolled: u and G are compile-time, so the slot index is too
    switch (u) {
#define SPECV_SLOT(U)                                  \
  case U:                                              \
    zD = raw_elem<DT, VEC, G * 8 + U>(rd);             \
    zT = raw_elem<DT, VEC, G * 8 + U>(rt);             \
    break;
      SPECV_SLOT(0) SPECV_SLOT(1) SPECV_SLOT(2) SPECV_SLOT(3)
      SPECV_SLOT(4) SPECV_SLOT(5) SPECV_SLOT(6) SPECV_SLOT(7)
#undef SPECV_SLOT
    }
    const float eD = term_exp(zD, refD, k);
    const float tD = exp2_hw(eD);
    // min(p, q) = min(tT r, tD) / S^D with r = S^D / S^T, tT r formed as
    // 2^(fl32(z - M) k + log2 r) in one fma (log2 r is of order 1, so the
    // exponent keeps its resolution); the 1 / S^D once per group
    const float tTr = exp2_hw(__builtin_fmaf(zT - refT, k, lr));
    pa[u] = fminf(tTr, tD);
    ps[u] = tD;
    // a masked token (tD = 0, eD = -inf) must add 0: eD is clamped to the
    // lowest finite float, which changes nothing where tD > 0 (eD is finite
    // there) and turns 0 * -inf into -0
    pA[u] = tD * fmaxf(eD, -3.40282347e38f);
    mx = fmaxf(mx, zD);
  }
  sa = tree_sum(pa) * iD;
  ss = tree_sum(ps);
  sA = tree_sum(pA);
}

// What one (position, chunk) wave of pass 2 leaves for the merge of its
// position: its fp64 sums, the keys it kept (best first, in its LDS buffer)
// and the position's row statistics.
struct DiagChunk {
  double sa, ss, sA;
  int count;
  RowStat st_t, st_d;
  float k;
};

// Pass 2 of work item `item` (position j = item / chunks, chunk c = item %
// chunks), by one wave with the LDS buffer `buf`. Returns false, with nothing
// written, for a position that the merge reports as NaN (layout error,
// invalid temperature, unusable row). With STORE the wave writes its sums and
// its list for the merge kernel; else it leaves them in `out` and `buf`.
template <int DT, bool VEC, bool STORE>
__device__ __forceinline__ bool diag_chunk(const DiagArgs& a, int64_t item, int lane,
                                           uint64_t* buf, DiagChunk& out) {
  using TL = Tile<DT, VEC>;
  using Raw = typename TL::Raw;
  constexpr int NE = TL::NE;
  constexpr int NG = NE / 8;
  static_assert(kDiagGroup == 8, "diag_terms and the scan share 8-slot groups");
  constexpr int64_t esz = (DT == kBF16) ? 2 : 4;
  const int64_t j = item / a.chunks;
  const int c = (int)(item - j * a.chunks);
  // The sequence of draft row j: arithmetic in a uniform batch, whose rows
  // are in bounds whatever the gammas hold (the host checked the row
  // totals); otherwise from the plan, which fills it only for a valid layout.
  int64_t b;
  if (a.uniform_g > 0) {
    b = j / a.uniform_g;
  } else {
    const uint32_t st0 = a.status[0];
    const int32_t bs = a.dseq[j];
    if (st0 & kLayoutError) return false;
    b = bs;
  }
  const int64_t tr = j + b;
  const void* trow = static_cast<const char*>(a.target) + tr * a.V * esz;
  const void* drow = static_cast<const char*>(a.draft) + j * a.V * esz;
  const int64_t tiles = (a.V + TL::EPI - 1) / TL::EPI;
  const int n_iter = (int)((tiles - c + a.chunks - 1) / a.chunks);  // >= 1: c < chunks <= tiles
  auto tile_start = [&](int it) { return ((int64_t)c + (int64_t)it * a.chunks) * TL::EPI; };
  auto fetch_row = [&](const void* row, int it, Raw& r) {
    const int64_t e0 = tile_start(it);
    if (e0 + TL::EPI <= a.V) TL::template load_raw<false>(row, e0, a.V, 0, lane, r);
    else TL::template load_raw<true>(row, e0, a.V, 0, lane, r);
  };
  // The draft row's first tile and the row partials go out before anything
  // that waits on memory; the target row's first tile once the temperature
  // says the position samples.
  Raw da, ta;
  fetch_row(drow, 0, da);
  RowPart qt[4], qd[4];
  load_parts4(a.tparts + tr * a.chunks, a.chunks, qt);
  load_parts4(a.dparts + j * a.chunks, a.chunks, qd);
  const int K = a.K;
  float thz = (K > 0) ? a.bar[j * a.chunks + c] : ninf();  // logit of th
  const float k = diag_scale(a, j, b);
  if (a.uniform_g > 0 && (a.status[0] & kLayoutError)) return false;
  if (!(k >= 0.f)) return false;  // invalid temperature: the merge reports NaN
  const bool sampling = k > 0.f;
  if (sampling) fetch_row(trow, 0, ta);
  const RowStat st_t = merge_row_from(qt, a.tparts + tr * a.chunks, a.chunks, k, sampling);
  const RowStat st_d = merge_row_from(qd, a.dparts + j * a.chunks, a.chunks, k, sampling);
  if (!st_t.valid || !st_d.valid) return false;
  const float lTD = sampling ? (float)log2(st_d.s / st_t.s) : 0.f;  // log2 (S^D / S^T)
  const float iD = sampling ? (float)(1.0 / st_d.s) : 0.f;
  const int limit = (2 * K > kWave) ? 2 * K : kWave;
  double sa = 0.0, ss = 0.0, sA = 0.0;
  int count = 0;          // keys in the buffer
  // The first bar (thz, loaded above) comes from pass 1: the K-th largest
  // lane maximum of this chunk, a logit with at least K logits of the chunk
  // at or above it, so keys below its value cannot reach the best K.
  uint64_t th = rank_key(thz, INT32_MAX);  // keys at or below th cannot reach the best K
  auto fetch = [&](int it, Raw& rd, Raw& rt) {
    fetch_row(drow, it, rd);
    if (sampling) fetch_row(trow, it, rt);
  };
  // the top-k step of one slot group: one compare per slot against the bar's
  // logit, the exact key test only where some lane may hold a candidate
  auto scan_group = [&](const Raw& rd, int64_t e0, auto gq) {
    constexpr int G = decltype(gq)::value;
#define SPECV_SCAN(U)                                                       \
  {                                                                         \
    const float z = raw_elem<DT, VEC, G * kDiagGroup + U>(rd);              \
    if (ballot(z >= thz) != 0) {                                            \
      const int64_t id = TL::index(e0, 0, lane, G * kDiagGroup + U);        \
      const uint64_t key = rank_key(z, (int32_t)id);                        \
      const bool cand = id < a.V && key > th;                               \
      const uint64_t m = ballot(cand);                                      \
      if (cand) buf[count + lanes_below(m)] = key;                          \
      count += __popcll(m);                                                 \
      if (count > limit) {                                                  \
        count = keep_best(buf, count, K, lane);                             \
        th = buf[K - 1];                                                    \
        thz = key_value(th);                                                \
      }                                                                     \
    }                                                                       \
  }
    SPECV_SCAN(0) SPECV_SCAN(1) SPECV_SCAN(2) SPECV_SCAN(3)
    SPECV_SCAN(4) SPECV_SCAN(5) SPECV_SCAN(6) SPECV_SCAN(7)
#undef SPECV_SCAN
  };
  auto process = [&](const Raw& rd, const Raw& rt, int it) {
    const int64_t e0 = tile_start(it);
    float gm[NG];  // the lane's maximum draft logit in each 8-slot group
#pragma unroll
    for (int g = 0; g < NG; ++g) gm[g] = ninf();
    if (sampling) {
      float ga[NG], gs[NG], gA[NG];
      diag_terms<DT, VEC, 0>(rd, rt, k, st_t.ref, st_d.ref, lTD, iD, ga[0], gs[0], gA[0], gm[0]);
      diag_terms<DT, VEC, 1>(rd, rt, k, st_t.ref, st_d.ref, lTD, iD, ga[1], gs[1], gA[1], gm[1]);
      if constexpr (NG == 4) {
        diag_terms<DT, VEC, 2>(rd, rt, k, st_t.ref, st_d.ref, lTD, iD, ga[2], gs[2], gA[2], gm[2]);
        diag_terms<DT, VEC, 3>(rd, rt, k, st_t.ref, st_d.ref, lTD, iD, ga[3], gs[3], gA[3], gm[3]);
      }
      sa += (double)tree_sum(ga);
      ss += (double)tree_sum(gs);
      sA += (double)tree_sum(gA);
    } else if (K > 0) {
      float z[NE];
      TL::widen(rd, z);
#pragma unroll
      for (int q = 0; q < NE; ++q) gm[q / 8] = fmaxf(gm[q / 8], z[q]);
    }
    if (K == 0) return;
    float mx = gm[0];
#pragma unroll
    for (int g = 1; g < NG; ++g) mx = fmaxf(mx, gm[g]);
    if (ballot(mx >= thz) == 0) return;
    // a group is scanned only where some lane's group maximum reaches the
    // bar (which may have risen since the tile's check)
    if (ballot(gm[0] >= thz) != 0) scan_group(rd, e0, std::integral_constant<int, 0>{});
    if (ballot(gm[1] >= thz) != 0) scan_group(rd, e0, std::integral_constant<int, 1>{});
    if constexpr (NE / kDiagGroup == 4) {
      if (ballot(gm[2] >= thz) != 0) scan_group(rd, e0, std::integral_constant<int, 2>{});
      if (ballot(gm[3] >= thz) != 0) scan_group(rd, e0, std::integral_constant<int, 3>{});
    }
  };
  // single-buffered: one tile (both rows) in flight at a time per wave; the
  // first one was issued above
  for (int it = 0; it < n_iter; ++it) {
    if (it > 0) fetch(it, da, ta);
    process(da, ta, it);
  }
  const int64_t slot = j * a.chunks + c;
  if (sampling) {
    sa = wave_sum(sa);
    ss = wave_sum(ss);
    sA = wave_sum(sA);
  }
  if (K > 0) count = keep_best(buf, count, K, lane);
  if constexpr (STORE) {
    if (lane == 0) a.parts[slot] = DiagPart{sa, ss, sA};
    if (K > 0 && lane < K) {
      const bool have = lane < count;
      const uint64_t key = have ? buf[lane] : 0ull;
      a.topz[slot * K + lane] = have ? key_value(key) : ninf();
      a.topi[slot * K + lane] = have ? key_index(key) : INT32_MAX;
    }
  } else {
    out = DiagChunk{sa, ss, sA, count, st_t, st_d, k};
  }
  return true;
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void k5_diag_pass(DiagArgs a) {
  __shared__ __attribute__((aligned(16))) uint64_t sbuf[kWavesPerBlock][kDiagCap];
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t item = wave_uniform((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  if (item >= a.total_d * a.chunks) return;
  DiagChunk unused;
  (void)diag_chunk<DT, VEC, true>(a, item, lane, sbuf[threadIdx.x >> 6], unused);
}

// Pass 2 and the merge in one launch, for 1, 2 or 4 chunks per position and
// at most 64 NS keys in a position's lists: the chunk waves of a position are
// then in one workgroup (item = 4 blockIdx + wave), leave their sums and kept
// keys in LDS, and after a workgroup barrier the chunk-0 wave merges them
// exactly as k6_diag_merge does from global memory (the same reductions in
// the same order, so the same bits). Every wave of the workgroup reaches the
// barrier: nothing returns before it.
template <int DT, bool VEC, int NS>
__global__ __launch_bounds__(kBlock) void k5_diag_pass_merge(DiagArgs a) {
  __shared__ __attribute__((aligned(16))) uint64_t sbuf[kWavesPerBlock][kDiagCap];
  __shared__ __attribute__((aligned(16))) uint64_t mbuf[kWavesPerBlock * kMaxTopK];
  __shared__ DiagPart mpart[kWavesPerBlock];
  __shared__ int mcount[kWavesPerBlock];
  const int lane = threadIdx.x & (kWave - 1);
  const int w = (int)(threadIdx.x >> 6);
  const int64_t item = wave_uniform((int64_t)blockIdx.x * kWavesPerBlock + w);
  const bool in_range = item < a.total_d * a.chunks;
  DiagChunk o{};
  const bool valid = in_range && diag_chunk<DT, VEC, false>(a, item, lane, sbuf[w], o);
  if (lane == 0) {
    mpart[w] = valid ? DiagPart{o.sa, o.ss, o.sA} : DiagPart{0.0, 0.0, 0.0};
    mcount[w] = valid ? o.count : 0;
  }
  __syncthreads();
  const int C = a.chunks;
  if (!in_range || w % C != 0) return;
  const int64_t j = item / C;
  const int K = a.K;
  if (!valid) {
    if (lane == 0) {
      a.out_alpha[j] = __builtin_nan("");
      a.out_entropy[j] = __builtin_nan("");
    }
    if (lane < K) {
      a.out_index[j * K + lane] = -1;
      a.out_prob[j * K + lane] = __builtin_nan("");
    }
    return;
  }
  const bool sampling = o.k > 0.f;
  double alpha, entropy;
  if (sampling) {
    const DiagPart part = (lane < C) ? mpart[w + lane] : DiagPart{0.0, 0.0, 0.0};
    alpha = wave_sum(part.alpha);
    const double S = wave_sum(part.s), A = wave_sum(part.a);
    entropy = log(S) - 0.69314718055994530942 * A / S;
  } else {
    alpha = (o.st_t.arg == o.st_d.arg) ? 1.0 : 0.0;
    entropy = 0.0;
  }
  if (lane == 0) {
    a.out_alpha[j] = alpha;
    a.out_entropy[j] = entropy;
  }
  if (K == 0) return;
  // the union of the chunk lists, chunk by chunk, empty places as key 0
  const int n = C * K;
  const int ns = (n + kWave - 1) / kWave;
  const int stride = (n + 7) / 8 * 8;
  uint64_t* mb = mbuf + (w / C) * stride;
  uint64_t mine[NS];  // n <= 64 NS (checked at launch)
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int e = lane + s * kWave;
    uint64_t key = 0ull;
    if (s < ns && e < n) {
      const int cc = e / K, l = e - cc * K;
      if (l < mcount[w + cc]) key = sbuf[w + cc][l];
      mb[e] = key;
    }
    mine[s] = key;
  }
  __builtin_amdgcn_wave_barrier();
  int rank[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) rank[s] = 0;
  count_above<NS>(mb, n, ns, mine, rank);
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (s < ns && mine[s] != 0ull && rank[s] < K) {
      const float z = key_value(mine[s]);
      double q;
      if (sampling) q = exp2(((double)z - (double)o.st_d.ref) * (double)o.k) / o.st_d.s;
      else q = (rank[s] == 0) ? 1.0 : 0.0;
      a.out_index[j * K + rank[s]] = key_index(mine[s]);
      a.out_prob[j * K + rank[s]] = q;
    }
  }
}

// One wave per position: sums the chunk partials and ranks the union of the
// chunk lists (at most 16 * 64 keys, in LDS); a key's rank is its place in
// the merged list. Padding entries (index INT32_MAX) take no part: the
// chunks hold at least K real entries between them, since K <= V. NS: 64-key
// slots per lane, the smallest power of two with 64 NS >= chunks * K (chosen
// at launch), so small lists keep few registers. Every load that depends
// only on the position is issued before the checks that may end the wave.
//
// LDS: kWavesPerBlock buffers of chunks * K keys (rounded up to a multiple of
// 8 keys), sized at launch.
constexpr int kMergeCap = 16 * kMaxTopK;

template <int NS>
__global__ __launch_bounds__(kBlock) void k6_diag_merge(DiagArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint64_t merge_lds[];
  const int lane = threadIdx.x & (kWave - 1);
  const int stride = (a.chunks * a.K + 7) / 8 * 8;
  uint64_t* buf = merge_lds + (threadIdx.x >> 6) * stride;
  const int64_t j = wave_uniform((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  if (j >= a.total_d) return;
  const int K = a.K;
  const int n = a.chunks * K;
  const int ns = (n + kWave - 1) / kWave;
  // independent loads
  const uint32_t status = a.status[0];
  const int64_t b = diag_seq(a, j);
  const float k = diag_scale(a, j, b);
  DiagPart part{0.0, 0.0, 0.0};
  if (lane < a.chunks) part = a.parts[j * a.chunks + lane];
  int32_t ids[NS];
  float zs[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int e = lane + s * kWave;
    ids[s] = INT32_MAX;
    zs[s] = 0.f;
    if (s < ns && e < n) {
      ids[s] = a.topi[j * n + e];
      zs[s] = a.topz[j * n + e];
    }
  }
  auto fail = [&]() {
    if (lane == 0) {
      a.out_alpha[j] = __builtin_nan("");
      a.out_entropy[j] = __builtin_nan("");
    }
    if (lane < K) {
      a.out_index[j * K + lane] = -1;
      a.out_prob[j * K + lane] = __builtin_nan("");
    }
  };
  if (status & kLayoutError) return fail();
  if (!(k >= 0.f)) return fail();
  const bool sampling = k > 0.f;
  const int64_t tr = j + b;
  const RowStat st_t = merge_row(a.tparts + tr * a.chunks, a.chunks, k, sampling);
  const RowStat st_d = merge_row(a.dparts + j * a.chunks, a.chunks, k, sampling);
  if (!st_t.valid || !st_d.valid) return fail();
  double alpha, entropy;
  if (sampling) {
    alpha = wave_sum(part.alpha);
    const double S = wave_sum(part.s), A = wave_sum(part.a);
    entropy = log(S) - 0.69314718055994530942 * A / S;
  } else {
    alpha = (st_t.arg == st_d.arg) ? 1.0 : 0.0;
    entropy = 0.0;
  }
  if (lane == 0) {
    a.out_alpha[j] = alpha;
    a.out_entropy[j] = entropy;
  }
  if (K == 0) return;
  uint64_t mine[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int e = lane + s * kWave;
    const uint64_t key = (ids[s] != INT32_MAX) ? rank_key(zs[s], ids[s]) : 0ull;
    if (s < ns && e < n) buf[e] = key;
    mine[s] = key;
  }
  __builtin_amdgcn_wave_barrier();
  int rank[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) rank[s] = 0;
  count_above<NS>(buf, n, ns, mine, rank);
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (s < ns && mine[s] != 0ull && rank[s] < K) {
      const float z = key_value(mine[s]);
      double q;
      if (sampling) q = exp2(((double)z - (double)st_d.ref) * (double)k) / st_d.s;
      else q = (rank[s] == 0) ? 1.0 : 0.0;
      a.out_index[j * K + rank[s]] = key_index(mine[s]);
      a.out_prob[j * K + rank[s]] = q;
    }
  }
}

}  // namespace specv
