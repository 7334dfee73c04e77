/*
 * oracle_stress.c -- drives every entry point of the CPU oracle over random
 * shapes, for sanitizer builds (AddressSanitizer + UndefinedBehaviorSanitizer,
 * or ThreadSanitizer): ragged batches with gamma from 0, greedy, sampling and
 * invalid temperatures, masked tokens, NaN and +inf rows, draft tokens outside
 * [0, V), layout errors, injected uniforms, every lenience; diagnostics with
 * random top-k; bigram decode loops; vertical cascades with k2 below, equal to
 * and above k1, bad start tokens and the planted-mistake switch. A sanitizer
 * report ends the run with a nonzero status. Test infrastructure.
 *
 *   oracle_stress [cases] [seed]
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "specv_oracle.h"

static uint64_t g_state;

static uint64_t next_u64(void) { /* splitmix64 */
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static int64_t below(int64_t n) { return n > 0 ? (int64_t)(next_u64() % (uint64_t)n) : 0; }
static double unit(void) { return ((next_u64() >> 11) + 0.5) / 9007199254740992.0; }
static double normal(void) { return sqrt(-2.0 * log(unit())) * cos(6.283185307179586 * unit()); }

static uint16_t to_bf16(float f) { /* round to nearest even; NaN stays NaN */
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x7fffffu)) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static void* xmalloc(size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p) {
    fprintf(stderr, "out of memory\n");
    exit(2);
  }
  return p;
}

/* rows [rows, V] of logits in `dtype`, N(0, scale^2), some masked, maybe bad */
static void* make_rows(int64_t rows, int64_t V, int dtype, double scale, int allow_bad) {
  const size_t esz = dtype == ORACLE_BF16 ? 2 : 4;
  void* p = xmalloc((size_t)(rows * V) * esz);
  for (int64_t r = 0; r < rows; ++r) {
    const int masked = below(4) == 0;
    const int bad = allow_bad && below(12) == 0;
    for (int64_t v = 0; v < V; ++v) {
      float f = (float)(normal() * scale);
      if (masked && V > 1 && below(3) == 0) f = -INFINITY;
      if (bad && v == V / 2) f = below(2) ? NAN : INFINITY;
      if (dtype == ORACLE_BF16) ((uint16_t*)p)[r * V + v] = to_bf16(f);
      else ((float*)p)[r * V + v] = f;
    }
  }
  return p;
}

static float pick_temperature(void) {
  switch (below(10)) {
    case 0: return 0.0f;
    case 1: return 0.0f;
    case 2: return 0.5f;
    case 3: return 2.0f;
    case 4: return below(4) == 0 ? -1.0f : 1.0f;
    case 5: return below(4) == 0 ? NAN : 0.7f;
    default: return 1.0f;
  }
}

static void stress_verify(void) {
  static const int64_t Vs[] = {1, 2, 7, 64, 513, 1000, 3000};
  const int64_t V = Vs[below(7)];
  const int dtype = (int)below(2);
  const int64_t B = 1 + below(12);
  const int64_t mg = below(10);
  int32_t* gamma = xmalloc((size_t)B * 4);
  float* T = xmalloc((size_t)B * 4);
  int64_t tt = 0, td = 0;
  for (int64_t b = 0; b < B; ++b) {
    gamma[b] = (int32_t)below(mg + 1);
    T[b] = pick_temperature();
    tt += gamma[b] + 1;
    td += gamma[b];
  }
  const int layout_error = below(15) == 0;
  if (layout_error && B > 1) gamma[0] = gamma[0] == 0 ? 1 : 0; /* totals no longer match */
  void* target = make_rows(tt, V, dtype, 0.5 + 2.0 * unit(), 1);
  void* draft = make_rows(td, V, dtype, 0.5 + 2.0 * unit(), 1);
  int32_t* tokens = xmalloc((size_t)td * 4);
  for (int64_t i = 0; i < td; ++i) tokens[i] = below(20) == 0 ? (int32_t)(below(2) ? -1 : V)
                                                                : (int32_t)below(V);
  const int inject = below(3) == 0;
  float* r = NULL;
  float* u = NULL;
  if (inject) {
    r = xmalloc((size_t)(B * (mg ? mg : 1)) * 4);
    u = xmalloc((size_t)B * 4);
    for (int64_t i = 0; i < B * (mg ? mg : 1); ++i) r[i] = (float)((below(1 << 24) + 1) / 16777216.0);
    for (int64_t b = 0; b < B; ++b) u[b] = (float)((below(1 << 24) + 1) / 16777216.0);
  }
  static const float eps[] = {1.0f, 0.5f, 0.05f};
  const int kind = (int)below(4);
  int32_t* n = xmalloc((size_t)B * 4);
  int32_t* next = xmalloc((size_t)B * 4);
  double* margin = xmalloc((size_t)B * 8);
  uint8_t* near = xmalloc((size_t)B);
  double* ratio = xmalloc((size_t)(B * (mg ? mg : 1)) * 8);
  double* resmass = xmalloc((size_t)B * 8);
  double* am = xmalloc((size_t)B * 8);
  double* dm = xmalloc((size_t)B * 8);
  int32_t* win = xmalloc((size_t)B * 5 * 4);
  double* np = xmalloc((size_t)B * 8);
  oracle_verify(B, V, mg, dtype, tt, td, target, draft, tokens, gamma, T, next_u64(), below(1000),
                kind, eps[below(3)], r, u, n, next, margin, near, ratio, resmass, am, dm, win, np,
                (int)(1 + below(4)));
  for (int64_t b = 0; b < B; ++b)
    if (n[b] < -1 || n[b] > mg || next[b] < -1 || next[b] >= V) {
      fprintf(stderr, "verify: outcome out of range (%d, %d)\n", n[b], next[b]);
      exit(3);
    }
  if (!layout_error) {
    const int64_t K = below(V < 8 ? V + 1 : 9);
    double* alpha = xmalloc((size_t)td * 8);
    double* ent = xmalloc((size_t)td * 8);
    int32_t* idx = xmalloc((size_t)(td * K) * 4);
    double* prob = xmalloc((size_t)(td * K) * 8);
    oracle_position_diagnostics(B, V, dtype, tt, td, target, draft, gamma, T, K, alpha, ent, idx,
                                prob);
    free(alpha); free(ent); free(idx); free(prob);
    float* Trow = xmalloc((size_t)tt * 4);
    double* m = xmalloc((size_t)tt * 8);
    double* s = xmalloc((size_t)tt * 8);
    int32_t* a = xmalloc((size_t)tt * 4);
    uint8_t* ok = xmalloc((size_t)tt);
    for (int64_t i = 0; i < tt; ++i) Trow[i] = below(3) ? 1.0f : 0.0f;
    oracle_row_stats(target, dtype, tt, V, Trow, m, s, a, ok);
    double* p = xmalloc((size_t)V * 8);
    oracle_softmax_row(target, dtype, V, below(tt), 0.8f, p);
    free(Trow); free(m); free(s); free(a); free(ok); free(p);
  }
  free(gamma); free(T); free(target); free(draft); free(tokens); free(r); free(u); free(n);
  free(next); free(margin); free(near); free(ratio); free(resmass); free(am); free(dm); free(win);
  free(np);
}

static int32_t* start_tokens(int64_t B, int64_t V) {
  int32_t* s = xmalloc((size_t)B * 4);
  for (int64_t b = 0; b < B; ++b) s[b] = below(10) == 0 ? (int32_t)(below(2) ? -3 : V) : (int32_t)below(V);
  return s;
}

static float* temperatures(int64_t B) {
  float* T = xmalloc((size_t)B * 4);
  for (int64_t b = 0; b < B; ++b) T[b] = pick_temperature();
  return T;
}

static void stress_decode(void) {
  static const int64_t Vs[] = {1, 3, 17, 64};
  const int64_t V = Vs[below(4)], B = 1 + below(6), g = below(6), R = below(4);
  const int dtype = (int)below(2);
  void* t = make_rows(V, V, dtype, 1.5, 0);
  void* d = make_rows(V, V, dtype, 1.5, 0);
  int32_t* start = start_tokens(B, V);
  float* T = temperatures(B);
  int32_t* tokens = xmalloc((size_t)(B * R * (g + 1)) * 4);
  int32_t* length = xmalloc((size_t)B * 4);
  int32_t* accepted = xmalloc((size_t)(B * R) * 4);
  int32_t* first_near = xmalloc((size_t)B * 4);
  oracle_decode_bigram(B, V, g, R, dtype, t, d, T, start, next_u64(), below(100), tokens, length,
                       accepted, first_near, (int)(1 + below(3)));
  free(t); free(d); free(start); free(T); free(tokens); free(length); free(accepted);
  free(first_near);
}

static void stress_cascade(void) {
  static const int64_t Vs[] = {1, 3, 17, 64};
  const int64_t V = Vs[below(4)], B = 1 + below(5), k1 = below(6), k2 = below(7), R = below(3);
  const int dtype = (int)below(2);
  void* t = make_rows(V, V, dtype, 1.5, 0);
  void* m1 = make_rows(V, V, dtype, 1.5, 0);
  void* m2 = make_rows(V, V, dtype, 1.5, 0);
  int32_t* start = start_tokens(B, V);
  float* T = temperatures(B);
  int32_t* tokens = xmalloc((size_t)(B * R * (k1 + 1)) * 4);
  int32_t* length = xmalloc((size_t)B * 4);
  int32_t* accepted = xmalloc((size_t)(B * R) * 4);
  int32_t* first_near = xmalloc((size_t)B * 4);
  static const float eps[] = {1.0f, 0.5f, 0.1f};
  oracle_cascade_bigram(B, V, k1, k2, R, dtype, t, m1, m2, T, start, (int)below(4), eps[below(3)],
                        next_u64(), below(100), (int)below(2), tokens, length, accepted,
                        first_near, (int)(1 + below(3)));
  free(t); free(m1); free(m2); free(start); free(T); free(tokens); free(length); free(accepted);
  free(first_near);
}

int main(int argc, char** argv) {
  const int cases = argc > 1 ? atoi(argv[1]) : 40;
  g_state = argc > 2 ? strtoull(argv[2], NULL, 10) : 1;
  uint32_t ctr[8] = {1, 2, 3, 4, 5, 6, 7, 8}, out[8];
  oracle_philox_blocks(next_u64(), ctr, out, 2);
  for (int c = 0; c < cases; ++c) {
    stress_verify();
    stress_decode();
    stress_cascade();
  }
  /* the planted mistakes take other branches of the same code */
  for (int m = 1; m <= 4; ++m) {
    oracle_set_mutant(m);
    stress_verify();
  }
  oracle_set_mutant(0);
  printf("oracle_stress: %d cases ok\n", cases);
  return 0;
}
