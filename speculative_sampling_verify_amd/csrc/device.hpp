// device.hpp -- wave-level building blocks of libspecverify's kernels (gfx950).
//
// Everything here is device code for CDNA4: 64-lane wavefronts, raw v_exp_f32,
// cross-lane exchange with __shfl_xor / __shfl_up (ds_swizzle / DPP / bpermute,
// no LDS storage), ballots as 64-bit masks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace specv {

constexpr int kWave = 64;
constexpr int kBlock = 256;                     // 4 waves per workgroup
constexpr int kWavesPerBlock = kBlock / kWave;  // each wave is an independent work item

enum : int { kF32 = 0, kBF16 = 1 };

// Device status word bits (mirrored in the public header).
constexpr uint32_t kSeqError = 1u;
constexpr uint32_t kLayoutError = 2u;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float ninf() { return -__builtin_huge_valf(); }
__device__ __forceinline__ float pinf() { return __builtin_huge_valf(); }

// bf16 is the upper half of an IEEE binary32: widening is exact.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 2^x on the transcendental unit (v_exp_f32). Results below the smallest
// normal flush to 0; -inf -> 0; NaN -> NaN.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// log2(e) / T in fp32: exp((z - m) / T) = 2^((z - m) * k). Every kernel that
// evaluates a softmax at temperature T derives k through this one function.
// It overflows to +inf for T below about 4.2e-39, which the callers treat as
// an invalid temperature.
__device__ __forceinline__ float temp_scale(float T) {
  return (float)(1.4426950408889634074 / (double)T);
}

// A sampling temperature: T > 0, finite, and log2(e)/T finite in fp32.
__device__ __forceinline__ bool sampling_temperature(float T) {
  return T > 0.f && T < pinf() && temp_scale(T) < pinf();
}

// Per-sequence scale: k = log2(e)/T for a sampling temperature, 0 for a
// greedy sequence (T = 0), -1 for an invalid temperature.
__device__ __forceinline__ float seq_scale(float T) {
  return sampling_temperature(T) ? temp_scale(T) : (T == 0.f ? 0.f : -1.f);
}

// Reference logit of a row or span with maximum m: m itself, or 0 for an
// all-masked (-inf) span. Terms are 2^(fl32(fl32(z - ref) k)) (term_exp):
// the maximum's term is exactly 1 and none overflows, at any finite logits
// and any finite k (a difference that overflows to -inf gives 0). A
// reference m * k instead would carry that product's rounding error into
// every term, which overflows the exponent range once |m k| passes 2^31
// (logits masked with the most negative finite value, tiny T).
__device__ __forceinline__ float ref_logit(float m) { return (m == ninf()) ? 0.f : m; }
__device__ __forceinline__ float term_exp(float z, float ref, float k) { return (z - ref) * k; }

// Factor that moves a sum taken relative to maximum m onto the reference of
// maximum mn >= m, from v_exp_f32 (within 1 ulp; exactly 1 when m == mn); 0
// for an all-masked sum (keeps NaN payloads: NaN * 0).
__device__ __forceinline__ float rescale32(float m, float mn, float k) {
  if (m == ninf()) return 0.f;
  return exp2_hw(term_exp(m, ref_logit(mn), k));
}

template <int DT>
__device__ __forceinline__ float load_logit(const void* base, int64_t idx) {
  if constexpr (DT == kBF16) {
    const uint16_t h = static_cast<const uint16_t*>(base)[idx];
    return __uint_as_float((uint32_t)h << 16);
  } else {
    return static_cast<const float*>(base)[idx];
  }
}

// ---------------------------------------------------------------------------
// Tiles: what one wave reads per loop iteration from a row chunk starting at
// element e0. Each lane owns NE elements, in increasing index order within
// the lane and across iterations (the argmax tie rule relies on it).
//   bf16, vector path: 4 x 16-byte loads per lane = 32 elements; one wave
//                      instruction covers 1 KiB of contiguous row.
//   fp32, vector path: 4 x 16-byte loads per lane = 16 elements.
//   scalar path (rows not 16-byte aligned): 16 strided 2- or 4-byte loads.
// A tile is loaded raw (RD dwords per lane) and widened to fp32 separately,
// so a kernel can issue the next tile's loads before it works on this one.
// ---------------------------------------------------------------------------
template <int DT, bool VEC>
struct Tile {
  static constexpr int NE = (VEC && DT == kBF16) ? 32 : 16;
  static constexpr int EPI = kWave * NE;  // elements per wave iteration
  static constexpr int VE = (DT == kBF16) ? 8 : 4;  // elements per 16-byte vector
  static constexpr int RD = VEC ? 16 : NE;           // raw dwords per lane

  struct Raw {
    uint32_t d[RD];
  };

  // Element index of slot j of lane `lane` in iteration `it`.
  __device__ static __forceinline__ int64_t index(int64_t e0, int it, int lane, int j) {
    if constexpr (VEC) {
      const int64_t vec = (int64_t)(it * 4 + j / VE) * kWave + lane;
      return e0 + vec * VE + (j % VE);
    } else {
      return e0 + (int64_t)(it * NE + j) * kWave + lane;
    }
  }

  // Where element `off` (0 <= off < EPI) of a tile lands in the raw dwords
  // load_raw reads, packed with the chunk iteration `it` that holds the tile:
  // (it << 11) | (dword << 7) | (high half << 6) | lane. The element's fp32
  // bits are that dword (fp32, or bf16 widened on load), or its high half or
  // its low half shifted up (two bf16 per dword).
  __device__ static __forceinline__ int32_t capture_code(int it, int off) {
    int dw, hi = 0, ln;
    if constexpr (VEC) {
      const int vec = off / VE;
      ln = vec % kWave;
      const int u = vec / kWave, e = off % VE;
      if constexpr (DT == kBF16) {
        dw = u * 4 + e / 2;
        hi = e & 1;
      } else {
        dw = u * 4 + e;
      }
    } else {
      dw = off / kWave;
      ln = off % kWave;
    }
    return (it << 11) | (dw << 7) | (hi << 6) | ln;
  }
  __device__ static __forceinline__ uint32_t bits_of(uint32_t w, int32_t cap) {
    if constexpr (VEC && DT == kBF16) return ((cap >> 6) & 1) ? (w & 0xffff0000u) : (w << 16);
    else return w;
  }

  // Raw load of iteration `it`; slots at or past e1 read as -inf when MASK.
  template <bool MASK>
  __device__ static __forceinline__ void load_raw(const void* row, int64_t e0, int64_t e1, int it,
                                                  int lane, Raw& r) {
    if constexpr (VEC) {
      const u32x4* p = reinterpret_cast<const u32x4*>(
          static_cast<const char*>(row) + e0 * (DT == kBF16 ? 2 : 4));
      constexpr uint32_t kNegInf = (DT == kBF16) ? 0xff80ff80u : 0xff800000u;  // -inf
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t vec = (int64_t)(it * 4 + u) * kWave + lane;
        u32x4 q;
        if (MASK && e0 + vec * VE >= e1)
          q = u32x4{kNegInf, kNegInf, kNegInf, kNegInf};
        else
          q = __builtin_nontemporal_load(p + vec);
        r.d[4 * u + 0] = q.x; r.d[4 * u + 1] = q.y; r.d[4 * u + 2] = q.z; r.d[4 * u + 3] = q.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < NE; ++j) {
        const int64_t idx = e0 + (int64_t)(it * NE + j) * kWave + lane;
        float v;
        if (MASK && idx >= e1)
          v = ninf();
        else if constexpr (DT == kBF16)
          v = __uint_as_float((uint32_t)__builtin_nontemporal_load(static_cast<const uint16_t*>(row) + idx) << 16);
        else
          v = __builtin_nontemporal_load(static_cast<const float*>(row) + idx);
        r.d[j] = __float_as_uint(v);
      }
    }
  }

  // Stores the raw tile of iteration `it` as load_raw read it (the same
  // slots), skipping slots at or past e1; non-temporal 16-byte stores on the
  // vector path.
  __device__ static __forceinline__ void store_raw(void* row, int64_t e0, int64_t e1, int it,
                                                   int lane, const Raw& r) {
    if constexpr (VEC) {
      u32x4* p = reinterpret_cast<u32x4*>(static_cast<char*>(row) + e0 * (DT == kBF16 ? 2 : 4));
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t vec = (int64_t)(it * 4 + u) * kWave + lane;
        if (e0 + vec * VE < e1)
          __builtin_nontemporal_store(u32x4{r.d[4 * u], r.d[4 * u + 1], r.d[4 * u + 2], r.d[4 * u + 3]},
                                      p + vec);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NE; ++j) {
        const int64_t idx = e0 + (int64_t)(it * NE + j) * kWave + lane;
        if (idx < e1) {
          if constexpr (DT == kBF16)
            static_cast<uint16_t*>(row)[idx] = (uint16_t)(r.d[j] >> 16);
          else
            static_cast<uint32_t*>(row)[idx] = r.d[j];
        }
      }
    }
  }

  __device__ static __forceinline__ void load_raw(const void* row, int64_t e0, int64_t e1, int it,
                                                  int n_full, int lane, Raw& r) {
    if (it < n_full) load_raw<false>(row, e0, e1, it, lane, r);
    else load_raw<true>(row, e0, e1, it, lane, r);
  }

  // The raw tile of a row of V <= EPI elements (vector path, so V is a
  // multiple of VE) with no branch around a load: a vector past the row's end
  // loads the row's last vector again and reads as -inf, the values
  // load_raw<true> gives it.
  __device__ static __forceinline__ void load_only_tile(const void* row, int64_t V, int lane, Raw& r) {
    static_assert(VEC, "vector path only");
    const u32x4* p = static_cast<const u32x4*>(row);
    constexpr uint32_t kNegInf = (DT == kBF16) ? 0xff80ff80u : 0xff800000u;  // -inf
    const int last = (int)(V / VE) - 1;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int vec = u * kWave + lane;
      const u32x4 q = __builtin_nontemporal_load(p + (vec < last ? vec : last));
      const bool past = vec > last;
      r.d[4 * u + 0] = past ? kNegInf : q.x;
      r.d[4 * u + 1] = past ? kNegInf : q.y;
      r.d[4 * u + 2] = past ? kNegInf : q.z;
      r.d[4 * u + 3] = past ? kNegInf : q.w;
    }
  }

  __device__ static __forceinline__ void widen(const Raw& r, float (&z)[NE]) {
    if constexpr (VEC && DT == kBF16) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        z[2 * q] = bf16_lo(r.d[q]);
        z[2 * q + 1] = bf16_hi(r.d[q]);
      }
    } else {
#pragma unroll
      for (int q = 0; q < NE; ++q) z[q] = __uint_as_float(r.d[q]);
    }
  }

  template <bool MASK>
  __device__ static __forceinline__ void load(const void* row, int64_t e0, int64_t e1, int it,
                                              int lane, float (&z)[NE]) {
    Raw r;
    load_raw<MASK>(row, e0, e1, it, lane, r);
    widen(r, z);
  }
};

// Pairwise (tree) sum of N floats, N a power of two: fixed order, log2(N)
// rounding levels.
template <int N>
__device__ __forceinline__ float tree_sum(float (&e)[N]) {
#pragma unroll
  for (int w = N / 2; w >= 1; w >>= 1) {
#pragma unroll
    for (int j = 0; j < w; ++j) e[j] += e[j + w];
  }
  return e[0];
}

template <int N>
__device__ __forceinline__ float tile_max(const float (&z)[N]) {
  float g = z[0];
#pragma unroll
  for (int j = 1; j < N; ++j) g = fmaxf(g, z[j]);
  return g;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) v = min(v, __shfl_xor(v, off, kWave));
  return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Inclusive prefix sum across the wave (lane order).
__device__ __forceinline__ double wave_inclusive_scan(double v, int lane) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const double o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ int first_lane(uint64_t mask) { return __ffsll((long long)mask) - 1; }

__device__ __forceinline__ int64_t wave_uniform(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds; each round
// multiplies counter words 0 and 2 by the two Philox multipliers, folds the
// high halves into words 1 and 3 with the round key, and the key advances by
// the two Weyl increments after every round.
// ---------------------------------------------------------------------------
struct PhiloxBlock {
  uint32_t w0, w1, w2, w3;
};

__device__ __forceinline__ PhiloxBlock philox4x32_10(uint64_t seed, uint32_t c0, uint32_t c1,
                                                     uint32_t c2, uint32_t c3) {
  constexpr uint32_t kMulA = 0xD2511F53u, kMulB = 0xCD9E8D57u;
  constexpr uint32_t kWeylA = 0x9E3779B9u, kWeylB = 0xBB67AE85u;
  uint32_t ka = (uint32_t)seed, kb = (uint32_t)(seed >> 32);
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const uint32_t hi_a = __umulhi(kMulA, c0), lo_a = kMulA * c0;
    const uint32_t hi_b = __umulhi(kMulB, c2), lo_b = kMulB * c2;
    c0 = hi_b ^ c1 ^ ka;
    c1 = lo_b;
    c2 = hi_a ^ c3 ^ kb;
    c3 = lo_a;
    ka += kWeylA;
    kb += kWeylB;
  }
  return PhiloxBlock{c0, c1, c2, c3};
}

// 24 random bits -> (0, 1]: ((w >> 8) + 1) * 2^-24, exact in fp32.
__device__ __forceinline__ float uniform24(uint32_t w) {
  return (float)((w >> 8) + 1u) * 5.9604644775390625e-08f;
}

}  // namespace specv
