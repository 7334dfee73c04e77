/*
 * specv_oracle.c -- plain CPU oracle for the speculative-sampling verify step.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load or call this library. The product path (the HIP
 * library) never links, imports or falls back to it, and this file shares no
 * source, header or constant table with it.
 *
 * What it computes, and where the method is defined:
 *   - DistillSpec (Zhou et al., ICLR 2024), Appendix A.3, Algorithm A.1
 *     "Speculative decoding step": compute the thresholds
 *     f(p_i(x_i), eps)/q_i(x_i), draw one uniform per draft position, take
 *     n = the first position whose uniform exceeds its threshold (gamma if
 *     none), then draw one more token from norm(max(0, p_n - q_n)) when
 *     n < gamma, or from p_gamma when every draft was accepted. Lossless
 *     decoding is f(p, eps) = p (eps = 1); lossy decoding uses one of the
 *     lenience functions of DistillSpec section 4 (the paragraph on
 *     DistillSpec with lossy SD): f_lin = p/eps, f_sq = p/eps^2, f_exp = p^eps, eps in (0, 1].
 *     The residual of the final draw stays max(0, p - q) as the algorithm
 *     prints it, whatever the lenience.
 *   - The same step as summarised from Leviathan, Kalman and Matias on
 *     "How speculative decoding lets a small model draft and a large one
 *     check" (1-indexed form of the same rule), and in prose in the study
 *     notes "Speculative Decoding and Distillation", Part 1, steps 3-5.
 *   - Temperature softmax sigma_T(z)_i = exp(z_i/T) / sum_j exp(z_j/T), the
 *     same T for the target and the draft rows: "Speculative Decoding and
 *     Distillation", Part 2 "Loss (Hinton)".
 *   - Greedy verification (T = 0) is exact match against argmax p:
 *     "Speculative Decoding and Distillation", Practical considerations
 *     ("Greedy vs sampling"); DISCO (arXiv 2405.04304) section 3 describes
 *     the same as rejection sampling at zero temperature.
 *
 * Precision: every probability, ratio and cumulative sum is float64. Inputs
 * (bf16 or fp32 logits, fp32 temperatures) convert to float64 exactly.
 *
 * Readings where the pages leave a step open (all restated in the design
 * notes of the repository):
 *   - uniforms come from Philox4x32-10 (Salmon, Moraes, Dror and Shaw,
 *     "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11), key = seed,
 *     counter = (row lo, row hi, position, 0) with row = row_offset + b;
 *     word 0 gives r_i, word 1 at position n gives the final-draw uniform u;
 *   - a 32-bit word w maps to U(w) = ((w >> 8) + 1) * 2^-24, in (0, 1];
 *   - reject iff r_i > ratio_i (equality accepts); q_i(x_i) = 0 gives an
 *     infinite ratio (accept);
 *   - the final draw is the inverse CDF in index order: the smallest v with
 *     u * C_{V-1} <= C_v, C the inclusive prefix sum of the weights; if the
 *     residual mass is exactly 0 the weights fall back to p_n;
 *   - greedy argmax ties resolve to the lowest index, on the raw logits;
 *   - a sequence whose needed rows hold NaN or +inf, or hold no finite logit,
 *     or whose tokens fall outside [0, V), or whose T is NaN, negative,
 *     +inf or below the fp32 range of log2(e)/T (temperature_invalid),
 *     yields (n, token) = (-1, -1); a gamma outside [0, max_gamma], or
 *     row totals that disagree with the gammas, make every sequence (-1, -1).
 *
 * Parity pins: see the test suite (Philox against rocRAND's implementation,
 * softmax against torch float64, injected-uniform hand cases, quadrature
 * over the uniforms on tiny inputs, and chi-square tests of the output law).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "specv_oracle.h"

#define ORACLE_NEAR_TIE 1e-6

/* Negative controls for the statistical tests: each value plants one known
 * mistake so that the tests can show they would catch it. 0 = correct. */
#define MUTANT_NONE 0
#define MUTANT_RESIDUAL_IS_P 1 /* residual replaced by p_n            */
#define MUTANT_RESIDUAL_IS_Q 2 /* residual replaced by q_n            */
#define MUTANT_N_PLUS_ONE 3    /* accepted count off by one (capped)  */
#define MUTANT_LENIENCE_TIMES 4 /* f_lin applied as p * eps, not p / eps */
static int g_mutant = MUTANT_NONE;

void oracle_set_mutant(int m) { g_mutant = m; }

/* ------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon et al., SC'11): 10 rounds of the 4x32 S-box.  */
/* Each round multiplies words 0 and 2 by the two Philox constants,    */
/* mixes the high halves with words 1 and 3 and the round key, and the */
/* key advances by the two Weyl constants between rounds.              */
/* ------------------------------------------------------------------ */
void oracle_philox4x32_10(uint64_t seed, const uint32_t ctr_in[4], uint32_t out[4]) {
  const uint32_t mul_a = 0xD2511F53u, mul_b = 0xCD9E8D57u;
  const uint32_t weyl_a = 0x9E3779B9u, weyl_b = 0xBB67AE85u;
  uint32_t key_a = (uint32_t)seed, key_b = (uint32_t)(seed >> 32);
  uint32_t x0 = ctr_in[0], x1 = ctr_in[1], x2 = ctr_in[2], x3 = ctr_in[3];
  for (int round = 0; round < 10; ++round) {
    uint64_t prod_a = (uint64_t)mul_a * (uint64_t)x0;
    uint64_t prod_b = (uint64_t)mul_b * (uint64_t)x2;
    uint32_t y0 = (uint32_t)(prod_b >> 32) ^ x1 ^ key_a;
    uint32_t y1 = (uint32_t)prod_b;
    uint32_t y2 = (uint32_t)(prod_a >> 32) ^ x3 ^ key_b;
    uint32_t y3 = (uint32_t)prod_a;
    x0 = y0; x1 = y1; x2 = y2; x3 = y3;
    key_a += weyl_a;
    key_b += weyl_b;
  }
  out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/* U(w) = ((w >> 8) + 1) / 2^24: 24 random bits, in (0, 1], exact in fp32. */
double oracle_uniform24(uint32_t w) { return (double)((w >> 8) + 1u) / 16777216.0; }

void oracle_uniform24_many(const uint32_t* w, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_uniform24(w[i]);
}

/* The two uniforms the step uses for sequence row `row` and position `pos`. */
static void draw_uniforms(uint64_t seed, uint64_t row, uint32_t pos, double* r_word0,
                          double* u_word1) {
  uint32_t ctr[4] = {(uint32_t)row, (uint32_t)(row >> 32), pos, 0u};
  uint32_t w[4];
  oracle_philox4x32_10(seed, ctr, w);
  if (r_word0) *r_word0 = oracle_uniform24(w[0]);
  if (u_word1) *u_word1 = oracle_uniform24(w[1]);
}

/* ------------------------------------------------------------------ */
/* Input decoding: bf16 is the top half of an IEEE binary32.           */
/* ------------------------------------------------------------------ */
static double bf16_to_double(uint16_t h) {
  uint32_t bits = (uint32_t)h << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

void oracle_decode_bf16(const uint16_t* in, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_to_double(in[i]);
}

/* Copy row `row` of a [rows, V] logit matrix into z[0..V) as float64. */
static void load_row(const void* base, int dtype, int64_t V, int64_t row, double* z) {
  if (dtype == ORACLE_BF16) {
    const uint16_t* p = (const uint16_t*)base + row * V;
    for (int64_t v = 0; v < V; ++v) z[v] = bf16_to_double(p[v]);
  } else {
    const float* p = (const float*)base + row * V;
    for (int64_t v = 0; v < V; ++v) z[v] = (double)p[v];
  }
}

/* A temperature outside the step's domain: NaN, negative or +inf, or a
 * positive T so small that the logit scale log2(e)/T is not a finite fp32
 * number (T below about 4.2e-39). The second part is a stated limit of the
 * library's fp32 arithmetic, not of the method; the test is exact: the
 * quotient in float64 rounds to +inf in fp32 from 2^128 - 2^103 on. */
static int temperature_invalid(double T) {
  if (isnan(T) || T < 0.0 || isinf(T)) return 1;
  if (T == 0.0) return 0;
  return 1.4426950408889634074 / T >= 0x1.ffffffp127;
}

/* A row is usable when it has no NaN, no +inf and at least one finite value
 * (-inf marks a masked token of probability 0). */
static int row_is_valid(const double* z, int64_t V) {
  int any_finite = 0;
  for (int64_t v = 0; v < V; ++v) {
    if (isnan(z[v])) return 0;
    if (isinf(z[v]) && z[v] > 0) return 0;
    if (isfinite(z[v])) any_finite = 1;
  }
  return any_finite;
}

/* argmax over raw logits, lowest index on ties. */
static int64_t row_argmax(const double* z, int64_t V) {
  int64_t best = 0;
  for (int64_t v = 1; v < V; ++v)
    if (z[v] > z[best]) best = v;
  return best;
}

/* Temperature softmax: m = max z, S = sum exp((z - m)/T) in index order,
 * p_v = exp((z_v - m)/T) / S. Writes p when p != NULL. */
static void row_softmax(const double* z, int64_t V, double T, double* m_out, double* s_out,
                        double* p) {
  double m = -INFINITY;
  for (int64_t v = 0; v < V; ++v)
    if (z[v] > m) m = z[v];
  double s = 0.0;
  for (int64_t v = 0; v < V; ++v) s += exp((z[v] - m) / T);
  if (p)
    for (int64_t v = 0; v < V; ++v) p[v] = exp((z[v] - m) / T) / s;
  if (m_out) *m_out = m;
  if (s_out) *s_out = s;
}

/* ------------------------------------------------------------------ */
/* The verify step.                                                    */
/* ------------------------------------------------------------------ */

/* Lenience functions (DistillSpec section 4, lossy SD paragraph, and the
 * thresholds of Algorithm A.1): f is
 * increasing in p and decreasing in eps, and f(p, 1) = p for all three. */
static double lenience(double p, int kind, double eps) {
  switch (kind) {
    case ORACLE_LENIENCE_LIN:
      return g_mutant == MUTANT_LENIENCE_TIMES ? p * eps : p / eps;
    case ORACLE_LENIENCE_SQ:
      return p / (eps * eps);
    case ORACLE_LENIENCE_EXP:
      return pow(p, eps);
    default:
      return p;
  }
}

typedef struct {
  int64_t batch, vocab, max_gamma;
  int dtype;
  int64_t total_target_rows, total_draft_rows;
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const int32_t* gamma;
  const float* temperature;
  uint64_t seed, row_offset;
  int lenience;       /* ORACLE_LENIENCE_*                              */
  double eps;         /* lenience parameter, in (0, 1]                  */
  const float* inj_r; /* [batch * max_gamma] or NULL: injected r_i      */
  const float* inj_u; /* [batch] or NULL: injected final-draw uniforms  */
  int32_t* out_n;
  int32_t* out_next;
  double* out_margin;  /* [batch] or NULL: min(accept margin, draw margin) */
  uint8_t* out_near;   /* [batch] or NULL: margin < ORACLE_NEAR_TIE */
  double* out_accept_margin; /* [batch] or NULL: smallest |r_i - ratio_i| / ratio_i, decisive i */
  double* out_draw_margin;   /* [batch] or NULL: distance of u * C to the nearest CDF step / C */
  int32_t* out_window;       /* [batch, 5] or NULL: tok_lo, tok_hi, alt_n, alt_lo, alt_hi */
  double* out_near_prob;     /* [batch] or NULL: chance that the decisive uniforms fall in a window */
  double* out_ratio;   /* [batch * max_gamma] or NULL: f(p_i(x_i))/q_i(x_i) */
  double* out_resmass; /* [batch] or NULL: total weight of the final draw */
  const int64_t* toff;
  const int64_t* doff;
  int layout_ok;
  int nthreads;
} job_t;

typedef struct {
  double* z;  /* V   */
  double* zq; /* V   */
  double* p;  /* V   */
  double* q;  /* V   */
  double* w;  /* V   */
} scratch_t;

/* Outcome of one sequence: n, the token, the two margins and the windows.
 * tok_lo..tok_hi are the tokens whose CDF interval meets [t - d, t + d], d =
 * ORACLE_NEAR_TIE * C (only the drawn token when the draw is not a near-tie);
 * alt_* is the outcome with the first near-tie accept decision reversed
 * (alt_n = -2 when there is none). */
typedef struct {
  int64_t n, tok, tok_lo, tok_hi;
  double accept_margin, draw_margin;
  int64_t near_pos; /* first decisive position with accept margin < ORACLE_NEAR_TIE, or -1 */
  double near_prob; /* probability over the uniforms that a decisive one lands in its window */
} outcome_t;

static void set_result(const job_t* J, int64_t b, const outcome_t* o, const outcome_t* alt) {
  const double margin = o->accept_margin < o->draw_margin ? o->accept_margin : o->draw_margin;
  J->out_n[b] = (int32_t)o->n;
  J->out_next[b] = (int32_t)o->tok;
  if (J->out_margin) J->out_margin[b] = margin;
  if (J->out_near) J->out_near[b] = (uint8_t)(margin < ORACLE_NEAR_TIE);
  if (J->out_accept_margin) J->out_accept_margin[b] = o->accept_margin;
  if (J->out_draw_margin) J->out_draw_margin[b] = o->draw_margin;
  if (J->out_near_prob) J->out_near_prob[b] = o->near_prob;
  if (J->out_window) {
    int32_t* w = J->out_window + 5 * b;
    w[0] = (int32_t)o->tok_lo;
    w[1] = (int32_t)o->tok_hi;
    w[2] = alt ? (int32_t)alt->n : -2;
    w[3] = alt ? (int32_t)alt->tok_lo : -2;
    w[4] = alt ? (int32_t)alt->tok_hi : -2;
  }
}

static void set_failed(const job_t* J, int64_t b) {
  outcome_t o = {-1, -1, -1, -1, INFINITY, INFINITY, -1, 0.0};
  set_result(J, b, &o, NULL);
}

static void set_greedy(const job_t* J, int64_t b, int64_t n, int64_t tok) {
  outcome_t o = {n, tok, tok, tok, INFINITY, INFINITY, -1, 0.0};
  set_result(J, b, &o, NULL);
}

/* Inverse-CDF draw in index order over weights w[0..V): the smallest v with
 * t <= C_v where t = u * C_{V-1}. Returns -1 when the total is 0. Also the
 * draw margin (distance of t to the nearer end of the token's CDF interval,
 * over the total) and the window [*lo, *hi] of tokens whose interval meets
 * [t - d, t + d], d = ORACLE_NEAR_TIE * total. */
static int64_t cdf_search(const double* w, int64_t V, double t) {
  /* smallest v with t <= C_v; rounding past the last prefix gives the last
   * token of positive weight */
  double c = 0.0;
  for (int64_t v = 0; v < V; ++v) {
    c += w[v];
    if (t <= c) return v;
  }
  for (int64_t v = V - 1; v >= 0; --v)
    if (w[v] > 0.0) return v;
  return -1;
}

static int64_t inverse_cdf(const double* w, int64_t V, double u, double* margin, double* total_out,
                           int64_t* lo, int64_t* hi) {
  double total = 0.0;
  for (int64_t v = 0; v < V; ++v) total += w[v];
  if (total_out) *total_out = total;
  if (!(total > 0.0)) return -1;
  const double t = u * total;
  double c = 0.0, prev = 0.0;
  int64_t tok = -1;
  for (int64_t v = 0; v < V; ++v) {
    prev = c;
    c += w[v];
    if (t <= c) {
      const double below = t - prev, above = c - t;
      *margin = (below < above ? below : above) / total;
      tok = v;
      break;
    }
  }
  if (tok < 0) {
    /* Unreachable in exact arithmetic (t <= total); rounding could leave t a
     * hair above the last prefix: take the last token of positive weight. */
    tok = cdf_search(w, V, 2.0 * total);
    *margin = 0.0;
  }
  if (lo && hi) {
    const double d = ORACLE_NEAR_TIE * total;
    /* the lower end stays above 0: a weight-0 prefix is never drawn (u > 0) */
    const double tl = t - d > 0.0 ? t - d : 0x1p-1074;
    *lo = cdf_search(w, V, tl);
    *hi = cdf_search(w, V, t + d);
    if (*lo > tok) *lo = tok;
    if (*hi < tok) *hi = tok;
  }
  return tok;
}

/* The sampling step of one sequence whose rows are valid: the accept walk
 * (Algorithm A.1 steps 5-7) and the final draw (steps 8-11). With flip >= 0
 * the decision at position flip is reversed (used for the outcome on the
 * other side of a near-tie); flip < 0 is the step itself. */
static void sample_outcome(const job_t* J, int64_t b, scratch_t* S, int64_t flip, outcome_t* o) {
  const int64_t V = J->vocab;
  const int64_t g = J->gamma[b];
  const double T = (double)J->temperature[b];
  const int64_t t0 = J->toff[b], d0 = J->doff[b];
  const uint64_t philox_row = J->row_offset + (uint64_t)b;
  o->accept_margin = INFINITY;
  o->draw_margin = INFINITY;
  o->near_pos = -1;
  o->near_prob = 0.0;

  /* Accept walk: ratio_i = f(p_i(x_i), eps) / q_i(x_i); reject at the first
   * i with r_i > ratio_i. */
  int64_t n = g;
  for (int64_t i = 0; i < g; ++i) {
    const int32_t x = J->tokens[d0 + i];
    double mp, sp, mq, sq;
    load_row(J->target, J->dtype, V, t0 + i, S->z);
    row_softmax(S->z, V, T, &mp, &sp, NULL);
    const double p_x = exp((S->z[x] - mp) / T) / sp;
    load_row(J->draft, J->dtype, V, d0 + i, S->zq);
    row_softmax(S->zq, V, T, &mq, &sq, NULL);
    const double q_x = exp((S->zq[x] - mq) / T) / sq;
    const double ratio = (q_x == 0.0) ? INFINITY : lenience(p_x, J->lenience, J->eps) / q_x;
    if (flip < 0 && J->out_ratio) J->out_ratio[b * J->max_gamma + i] = ratio;
    double r;
    if (J->inj_r)
      r = (double)J->inj_r[b * J->max_gamma + i];
    else
      draw_uniforms(J->seed, philox_row, (uint32_t)i, &r, NULL);
    if (isfinite(ratio)) {
      const double mg = fabs(r - ratio) / ratio;
      if (mg < o->accept_margin) o->accept_margin = mg;
      if (mg < ORACLE_NEAR_TIE && o->near_pos < 0) o->near_pos = i;
      /* r is uniform on (0, 1]: the window of relative half-width 1e-6
       * around a ratio below 1 has that much chance */
      if (ratio < 1.0) o->near_prob += 2.0 * ORACLE_NEAR_TIE * ratio;
    }
    int reject = r > ratio;
    if (i == flip) reject = !reject;
    if (reject) {
      n = i;
      break;
    }
  }
  if (g_mutant == MUTANT_N_PLUS_ONE && n < g) n = n + 1;

  /* Final draw. */
  double u;
  if (J->inj_u)
    u = (double)J->inj_u[b];
  else
    draw_uniforms(J->seed, philox_row, (uint32_t)n, NULL, &u);

  load_row(J->target, J->dtype, V, t0 + n, S->z);
  row_softmax(S->z, V, T, NULL, NULL, S->p);
  if (n < g && g_mutant != MUTANT_RESIDUAL_IS_P) {
    load_row(J->draft, J->dtype, V, d0 + n, S->zq);
    row_softmax(S->zq, V, T, NULL, NULL, S->q);
    for (int64_t v = 0; v < V; ++v) {
      double d = S->p[v] - S->q[v];
      S->w[v] = d > 0.0 ? d : 0.0;
    }
    if (g_mutant == MUTANT_RESIDUAL_IS_Q)
      for (int64_t v = 0; v < V; ++v) S->w[v] = S->q[v];
  } else {
    for (int64_t v = 0; v < V; ++v) S->w[v] = S->p[v];
  }
  double total = 0.0;
  int64_t lo = -1, hi = -1;
  int64_t tok = inverse_cdf(S->w, V, u, &o->draw_margin, &total, &lo, &hi);
  if (tok < 0) {
    /* The residual has no mass (p_n == q_n up to rounding): draw from p_n. */
    tok = inverse_cdf(S->p, V, u, &o->draw_margin, &total, &lo, &hi);
  } else if (n < g && total < ORACLE_NEAR_TIE) {
    /* A residual this small is not resolved by fp32 weights: a computation
     * in fp32 may find no mass at all and draw from p_n instead. */
    o->draw_margin = 0.0;
    lo = 0;
    hi = V - 1;
  }
  if (flip < 0 && J->out_resmass) J->out_resmass[b] = total;
  if (o->draw_margin == 0.0 && lo == 0 && hi == V - 1) {
    o->near_prob += 1.0; /* a residual below the window: flagged whatever u is */
  } else if (total > 0.0) {
    /* u * C is uniform on (0, C]: the part of it within d = 1e-6 C of a step
     * of the CDF, summed over the tokens' intervals */
    const double* wd = (total > 0.0 && tok >= 0 && S->w[tok] > 0.0) ? S->w : S->p;
    double tw = 0.0;
    for (int64_t v = 0; v < V; ++v) tw += wd[v];
    for (int64_t v = 0; v < V; ++v) {
      const double f = wd[v] / tw;
      o->near_prob += f < 2.0 * ORACLE_NEAR_TIE ? f : 2.0 * ORACLE_NEAR_TIE;
    }
  }
  o->n = n;
  o->tok = tok;
  o->tok_lo = lo;
  o->tok_hi = hi;
}

static void verify_sequence(const job_t* J, int64_t b, scratch_t* S) {
  const int64_t V = J->vocab;
  if (!J->layout_ok) {
    set_failed(J, b);
    return;
  }
  const int64_t g = J->gamma[b];
  const double T = (double)J->temperature[b];
  const int64_t t0 = J->toff[b], d0 = J->doff[b];
  if (temperature_invalid(T)) {
    set_failed(J, b);
    return;
  }
  for (int64_t i = 0; i < g; ++i) {
    int32_t x = J->tokens[d0 + i];
    if (x < 0 || x >= V) {
      set_failed(J, b);
      return;
    }
  }

  if (T == 0.0) {
    /* Greedy: accept while the draft token equals the target argmax; emit
     * argmax of the first disagreeing (or the bonus) target row. Every
     * target row is checked for validity; draft rows are not read. */
    int64_t n = g, next = -1;
    int64_t first_bad = -1;
    for (int64_t i = 0; i <= g; ++i) {
      load_row(J->target, J->dtype, V, t0 + i, S->z);
      if (!row_is_valid(S->z, V)) {
        first_bad = i;
        break;
      }
      int64_t a = row_argmax(S->z, V);
      if (i < g && n == g && J->tokens[d0 + i] != a) n = i;
      if (i == n && next < 0) next = a;
    }
    if (first_bad >= 0) {
      set_failed(J, b);
      return;
    }
    if (g_mutant == MUTANT_N_PLUS_ONE && n < g) {
      n = n + 1;
      load_row(J->target, J->dtype, V, t0 + n, S->z);
      next = row_argmax(S->z, V);
    }
    set_greedy(J, b, n, next);
    return;
  }

  /* Sampling. Validate every needed row first (target 0..g, draft 0..g-1). */
  for (int64_t i = 0; i <= g; ++i) {
    load_row(J->target, J->dtype, V, t0 + i, S->z);
    if (!row_is_valid(S->z, V)) {
      set_failed(J, b);
      return;
    }
  }
  for (int64_t i = 0; i < g; ++i) {
    load_row(J->draft, J->dtype, V, d0 + i, S->zq);
    if (!row_is_valid(S->zq, V)) {
      set_failed(J, b);
      return;
    }
  }
  outcome_t o, alt;
  sample_outcome(J, b, S, -1, &o);
  if (o.near_pos >= 0 && J->out_window) {
    /* the other side of the first near-tie accept decision */
    sample_outcome(J, b, S, o.near_pos, &alt);
    set_result(J, b, &o, &alt);
  } else {
    set_result(J, b, &o, NULL);
  }
}

typedef struct {
  const job_t* J;
  int tid;
} worker_arg_t;

static void* worker(void* arg) {
  worker_arg_t* A = (worker_arg_t*)arg;
  const job_t* J = A->J;
  scratch_t S;
  size_t bytes = (size_t)J->vocab * sizeof(double);
  S.z = (double*)malloc(bytes);
  S.zq = (double*)malloc(bytes);
  S.p = (double*)malloc(bytes);
  S.q = (double*)malloc(bytes);
  S.w = (double*)malloc(bytes);
  for (int64_t b = A->tid; b < J->batch; b += J->nthreads) verify_sequence(J, b, &S);
  free(S.z); free(S.zq); free(S.p); free(S.q); free(S.w);
  return NULL;
}

/* Packed ragged layout: target rows of sequence b start at
 * toff[b] = sum_{b' < b} (gamma_b' + 1), draft rows at doff[b] = sum gamma_b'. */
static int plan_offsets(job_t* J, int64_t* toff, int64_t* doff) {
  int64_t st = 0, sd = 0;
  int ok = 1;
  for (int64_t b = 0; b < J->batch; ++b) {
    int64_t g = J->gamma[b];
    if (g < 0 || g > J->max_gamma) ok = 0;
    toff[b] = st;
    doff[b] = sd;
    if (g < 0) g = 0;
    st += g + 1;
    sd += g;
  }
  if (st != J->total_target_rows || sd != J->total_draft_rows) ok = 0;
  return ok;
}

static int run_job(job_t* J) {
  int64_t* toff = (int64_t*)malloc((size_t)(J->batch + 1) * sizeof(int64_t));
  int64_t* doff = (int64_t*)malloc((size_t)(J->batch + 1) * sizeof(int64_t));
  J->layout_ok = plan_offsets(J, toff, doff);
  J->toff = toff;
  J->doff = doff;
  int nt = J->nthreads < 1 ? 1 : J->nthreads;
  if (nt > J->batch) nt = (int)(J->batch > 0 ? J->batch : 1);
  J->nthreads = nt;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nt);
  worker_arg_t* args = (worker_arg_t*)malloc(sizeof(worker_arg_t) * (size_t)nt);
  for (int t = 0; t < nt; ++t) {
    args[t].J = J;
    args[t].tid = t;
    pthread_create(&th[t], NULL, worker, &args[t]);
  }
  for (int t = 0; t < nt; ++t) pthread_join(th[t], NULL);
  free(th); free(args); free(toff); free(doff);
  return J->layout_ok ? 0 : 1;
}

/* Returns 0 when the layout is consistent, 1 when every sequence was given
 * (-1, -1) because a gamma or a row total was out of range. */
int oracle_verify(int64_t batch, int64_t vocab, int64_t max_gamma, int dtype,
                  int64_t total_target_rows, int64_t total_draft_rows, const void* target,
                  const void* draft, const int32_t* tokens, const int32_t* gamma,
                  const float* temperature, uint64_t seed, uint64_t row_offset,
                  int lenience_kind, float eps,
                  const float* inj_r, const float* inj_u, int32_t* out_n, int32_t* out_next,
                  double* out_margin, uint8_t* out_near, double* out_ratio, double* out_resmass,
                  double* out_accept_margin, double* out_draw_margin, int32_t* out_window,
                  double* out_near_prob, int nthreads) {
  job_t J;
  memset(&J, 0, sizeof J);
  J.batch = batch; J.vocab = vocab; J.max_gamma = max_gamma; J.dtype = dtype;
  J.total_target_rows = total_target_rows; J.total_draft_rows = total_draft_rows;
  J.target = target; J.draft = draft; J.tokens = tokens; J.gamma = gamma;
  J.temperature = temperature; J.seed = seed; J.row_offset = row_offset;
  J.lenience = lenience_kind; J.eps = (double)eps;
  J.inj_r = inj_r; J.inj_u = inj_u;
  J.out_n = out_n; J.out_next = out_next; J.out_margin = out_margin; J.out_near = out_near;
  J.out_ratio = out_ratio; J.out_resmass = out_resmass;
  J.out_accept_margin = out_accept_margin; J.out_draw_margin = out_draw_margin;
  J.out_window = out_window;
  J.out_near_prob = out_near_prob;
  J.nthreads = nthreads;
  return run_job(&J);
}

/* Per-row statistics of rows [0, rows) of one logit matrix at temperature
 * T_row[r]: m (max), S (sum exp((z - m)/T), NaN when T_row[r] == 0), the
 * argmax (lowest index) and a validity flag. */
void oracle_row_stats(const void* logits, int dtype, int64_t rows, int64_t vocab,
                      const float* T_row, double* out_m, double* out_s, int32_t* out_arg,
                      uint8_t* out_valid) {
  double* z = (double*)malloc((size_t)vocab * sizeof(double));
  for (int64_t r = 0; r < rows; ++r) {
    load_row(logits, dtype, vocab, r, z);
    out_valid[r] = (uint8_t)row_is_valid(z, vocab);
    out_arg[r] = (int32_t)row_argmax(z, vocab);
    const double T = (double)T_row[r];
    if (T > 0.0) {
      row_softmax(z, vocab, T, &out_m[r], &out_s[r], NULL);
    } else {
      double m = -INFINITY;
      for (int64_t v = 0; v < vocab; ++v)
        if (z[v] > m) m = z[v];
      out_m[r] = m;
      out_s[r] = NAN;
    }
  }
  free(z);
}

/* Probabilities p_v = exp((z_v - m)/T)/S of one row. */
void oracle_softmax_row(const void* logits, int dtype, int64_t vocab, int64_t row, float T,
                        double* out_p) {
  double* z = (double*)malloc((size_t)vocab * sizeof(double));
  load_row(logits, dtype, vocab, row, z);
  row_softmax(z, vocab, (double)T, NULL, NULL, out_p);
  free(z);
}

/* Batched Philox blocks: out[4k..4k+4) = Philox4x32-10(seed, ctr[4k..4k+4)). */
void oracle_philox_blocks(uint64_t seed, const uint32_t* ctr, uint32_t* out, int64_t count) {
  for (int64_t k = 0; k < count; ++k) oracle_philox4x32_10(seed, ctr + 4 * k, out + 4 * k);
}

/* ------------------------------------------------------------------ */
/* Per-position diagnostics of a packed batch.                         */
/* ------------------------------------------------------------------ */

/* For every draft position i < gamma_b of every sequence b (output index:
 * the packed draft row doff[b] + i), with p = p_i and q = q_i the
 * temperature softmaxes of target row i and draft row i:
 *   alpha   = sum_v min(p_v, q_v): the acceptance probability of a token
 *             drafted from q (DistillSpec section 3, and its section 4
 *             reading 1 - alpha as the total variation distance);
 *   entropy = -sum_v q_v ln q_v (0 ln 0 = 0), the Ent(y^D_i) feature of
 *             DISCO's stopping classifier (DISCO section 3, Eq. 2);
 *   top-k   = the k most probable draft tokens and their q, the Top_k(y^D_i)
 *             feature of the same equation, most probable first; equal
 *             logits rank the lower index first.
 * Greedy sequences (T = 0) use the zero-temperature limits that greedy
 * verification uses: p and q one-hot at their argmax (lowest index), so
 * alpha is 1 when the two argmaxes agree and 0 otherwise, the entropy is 0
 * and the top-1 probability is 1. A position whose target or draft row is
 * unusable (NaN, +inf, no finite logit) or whose T is NaN, negative or +inf
 * gets alpha = entropy = NaN, indices -1 and probabilities NaN.
 * Returns 1 (and writes nothing) when the gammas and row totals disagree. */
int oracle_position_diagnostics(int64_t batch, int64_t vocab, int dtype, int64_t total_target_rows,
                                int64_t total_draft_rows, const void* target, const void* draft,
                                const int32_t* gamma, const float* temperature, int64_t top_k,
                                double* out_alpha, double* out_entropy, int32_t* out_topk_index,
                                double* out_topk_prob) {
  int64_t st = 0, sd = 0;
  for (int64_t b = 0; b < batch; ++b) {
    if (gamma[b] < 0) return 1;
    st += gamma[b] + 1;
    sd += gamma[b];
  }
  if (st != total_target_rows || sd != total_draft_rows) return 1;
  const int64_t V = vocab;
  double* zp = (double*)malloc((size_t)V * sizeof(double));
  double* zq = (double*)malloc((size_t)V * sizeof(double));
  double* p = (double*)malloc((size_t)V * sizeof(double));
  double* q = (double*)malloc((size_t)V * sizeof(double));
  uint8_t* taken = (uint8_t*)malloc((size_t)V);
  int64_t t0 = 0, d0 = 0;
  for (int64_t b = 0; b < batch; ++b) {
    const int64_t g = gamma[b];
    const double T = (double)temperature[b];
    for (int64_t i = 0; i < g; ++i) {
      const int64_t j = d0 + i;
      load_row(target, dtype, V, t0 + i, zp);
      load_row(draft, dtype, V, d0 + i, zq);
      const int ok = row_is_valid(zp, V) && row_is_valid(zq, V) && !temperature_invalid(T);
      if (!ok) {
        out_alpha[j] = NAN;
        out_entropy[j] = NAN;
        for (int64_t k = 0; k < top_k; ++k) {
          out_topk_index[j * top_k + k] = -1;
          out_topk_prob[j * top_k + k] = NAN;
        }
        continue;
      }
      if (T == 0.0) {
        const int64_t ap = row_argmax(zp, V), aq = row_argmax(zq, V);
        for (int64_t v = 0; v < V; ++v) {
          p[v] = (v == ap) ? 1.0 : 0.0;
          q[v] = (v == aq) ? 1.0 : 0.0;
        }
      } else {
        row_softmax(zp, V, T, NULL, NULL, p);
        row_softmax(zq, V, T, NULL, NULL, q);
      }
      double a = 0.0, h = 0.0;
      for (int64_t v = 0; v < V; ++v) {
        a += p[v] < q[v] ? p[v] : q[v];
        if (q[v] > 0.0) h -= q[v] * log(q[v]);
      }
      out_alpha[j] = a;
      out_entropy[j] = h;
      /* top-k by repeated selection of the best token not yet taken */
      memset(taken, 0, (size_t)V);
      for (int64_t k = 0; k < top_k; ++k) {
        int64_t best = -1;
        for (int64_t v = 0; v < V; ++v)
          if (!taken[v] && (best < 0 || zq[v] > zq[best])) best = v;
        taken[best] = 1;
        out_topk_index[j * top_k + k] = (int32_t)best;
        out_topk_prob[j * top_k + k] = q[best];
      }
    }
    t0 += g + 1;
    d0 += g;
  }
  free(zp); free(zq); free(p); free(q); free(taken);
  return 0;
}

/* ------------------------------------------------------------------ */
/* Multi-round decoding with bigram "models".                          */
/* ------------------------------------------------------------------ */

/* Speculative decoding over several rounds (DistillSpec Algorithm A.1,
 * repeated: the context grows by the n accepted draft tokens and the one
 * token of the final draw each round). The models are bigram tables: the
 * target's logits for the next token are row `prev` of ttab [V, V], the
 * draft's are row `prev` of dtab, prev being the last token of the context.
 * Each round and sequence b (Philox row = row_offset + r * batch + b):
 *   drafting: x_i ~ softmax(dtab[prev] / T_b) for i = 0..gamma-1, prev = the
 *     context's last token, then x_{i-1}; by inverse CDF in index order with
 *     u = U(word 0 of Philox(seed; row, i, 1)); T_b = 0 drafts the argmax;
 *   verification: the step above on target rows ttab[prev_i], i = 0..gamma,
 *     and draft rows dtab[prev_i], i < gamma, with the same row.
 * out_tokens [batch, rounds * (gamma + 1)] holds the generated tokens,
 * out_length [batch] their count (-1 once a round fails: a start token
 * outside [0, V) or a data error in verification), out_accepted
 * [batch, rounds] the n of each round (-1 after a failure), and
 * out_first_near [batch] the first round with a near-tie in drafting or
 * verification (rounds if none). */
int oracle_decode_bigram(int64_t batch, int64_t vocab, int64_t gamma, int64_t rounds, int dtype,
                         const void* ttab, const void* dtab, const float* temperature,
                         const int32_t* start, uint64_t seed, uint64_t row_offset,
                         int32_t* out_tokens, int32_t* out_length, int32_t* out_accepted,
                         int32_t* out_first_near, int nthreads) {
  const int64_t V = vocab, B = batch, g = gamma;
  const size_t esz = dtype == ORACLE_BF16 ? 2 : 4;
  const size_t row_bytes = (size_t)V * esz;
  const int64_t cap = rounds * (g + 1);
  char* tpack = (char*)malloc((size_t)(B * (g + 1)) * row_bytes + 1);
  char* dpack = (char*)malloc((size_t)(B * g) * row_bytes + 1);
  int32_t* tokens = (int32_t*)malloc((size_t)(B * g + 1) * sizeof(int32_t));
  int32_t* gam = (int32_t*)malloc((size_t)(B + 1) * sizeof(int32_t));
  int32_t* cur = (int32_t*)malloc((size_t)(B + 1) * sizeof(int32_t));
  int32_t* len = (int32_t*)malloc((size_t)(B + 1) * sizeof(int32_t));
  uint8_t* failed = (uint8_t*)malloc((size_t)B + 1);
  uint8_t* dnear = (uint8_t*)malloc((size_t)B + 1);
  int32_t* n_out = (int32_t*)malloc((size_t)(B + 1) * sizeof(int32_t));
  int32_t* next_out = (int32_t*)malloc((size_t)(B + 1) * sizeof(int32_t));
  uint8_t* vnear = (uint8_t*)malloc((size_t)B + 1);
  double* z = (double*)malloc((size_t)V * sizeof(double));
  double* q = (double*)malloc((size_t)V * sizeof(double));
  for (int64_t b = 0; b < B; ++b) {
    gam[b] = (int32_t)g;
    failed[b] = (uint8_t)(start[b] < 0 || start[b] >= V);
    cur[b] = failed[b] ? 0 : start[b];
    len[b] = 0;
    out_first_near[b] = (int32_t)rounds;
  }
  for (int64_t r = 0; r < rounds; ++r) {
    for (int64_t b = 0; b < B; ++b) {
      const double T = (double)temperature[b];
      const uint64_t prow = row_offset + (uint64_t)(r * B + b);
      int32_t prev = cur[b];
      dnear[b] = 0;
      for (int64_t i = 0; i <= g; ++i) {
        memcpy(tpack + (size_t)(b * (g + 1) + i) * row_bytes,
               (const char*)ttab + (size_t)prev * row_bytes, row_bytes);
        if (i == g) break;
        memcpy(dpack + (size_t)(b * g + i) * row_bytes, (const char*)dtab + (size_t)prev * row_bytes,
               row_bytes);
        load_row(dtab, dtype, V, prev, z);
        int64_t x = 0;
        if (!row_is_valid(z, V) || temperature_invalid(T)) {
          x = 0; /* verification reports the sequence */
        } else if (T == 0.0) {
          x = row_argmax(z, V);
        } else {
          row_softmax(z, V, T, NULL, NULL, q);
          uint32_t ctr[4] = {(uint32_t)prow, (uint32_t)(prow >> 32), (uint32_t)i, 1u};
          uint32_t w[4];
          oracle_philox4x32_10(seed, ctr, w);
          double margin = INFINITY;
          x = inverse_cdf(q, V, oracle_uniform24(w[0]), &margin, NULL, NULL, NULL);
          if (x < 0) x = 0;
          if (margin < ORACLE_NEAR_TIE) dnear[b] = 1;
        }
        tokens[b * g + i] = (int32_t)x;
        prev = (int32_t)x;
      }
    }
    oracle_verify(B, V, g, dtype, B * (g + 1), B * g, tpack, dpack, tokens, gam, temperature, seed,
                  row_offset + (uint64_t)(r * B), ORACLE_LENIENCE_NONE, 1.0f, NULL, NULL, n_out,
                  next_out, NULL, vnear, NULL, NULL, NULL, NULL, NULL, NULL, nthreads);
    for (int64_t b = 0; b < B; ++b) {
      if (!failed[b] && n_out[b] < 0) failed[b] = 1;
      if (failed[b]) {
        out_accepted[b * rounds + r] = -1;
        continue;
      }
      const int32_t n = n_out[b];
      for (int32_t i = 0; i < n; ++i) out_tokens[b * cap + len[b] + i] = tokens[b * g + i];
      out_tokens[b * cap + len[b] + n] = next_out[b];
      len[b] += n + 1;
      cur[b] = next_out[b];
      out_accepted[b * rounds + r] = n;
      if ((dnear[b] || vnear[b]) && out_first_near[b] == rounds) out_first_near[b] = (int32_t)r;
    }
  }
  for (int64_t b = 0; b < B; ++b) out_length[b] = failed[b] ? -1 : len[b];
  free(tpack); free(dpack); free(tokens); free(gam); free(cur); free(len); free(failed);
  free(dnear); free(n_out); free(next_out); free(vnear); free(z); free(q);
  return 0;
}

/* ------------------------------------------------------------------ */
/* Vertical cascade with bigram "models".                              */
/* ------------------------------------------------------------------ */

/* The target's review of one sequence's cascade draft (outer round of the
 * vertical cascade), in float64 throughout: Algorithm A.1 without lenience,
 * with the target's rows p_i = softmax(ttab[prev_i] / T), prev_0 = the last
 * token, prev_i = draft token i - 1, and at each drafted position the law the
 * token was drawn from (see oracle_cascade_bigram): Q = min(q2, f(p1)) +
 * (1 - beta) norm(max(0, p1 - q2)) for a token from an inner position below
 * k2, Q = p1 for a token from the inner bonus position (p1, q2: the mid and
 * small softmaxes after the token's predecessor). Accept x_i while
 * r_i <= p_i(x_i) / Q_i(x_i); the final draw is from norm(max(0, p_n - Q_n)),
 * or from p_k1 when all k1 are accepted. Greedy (T = 0): exact match with the
 * target's argmax. Sets *n = -1 on an unusable target row; *near when a
 * decisive uniform lies within the near-tie window. */
typedef struct {
  double* zt; /* V: target logits of one row */
  double* zm; /* V */
  double* p1; /* V */
  double* q2; /* V */
  double* pt; /* V: target probabilities */
  double* Q;  /* V: law of the draft token */
  double* w;  /* V */
} review_scratch_t;

static void cascade_law(int64_t V, int dtype, const void* m1tab, const void* m2tab, double T,
                        int32_t prev, int bonus, int kind, double eps, int mutant_q_is_p1,
                        review_scratch_t* S) {
  load_row(m1tab, dtype, V, prev, S->zm);
  row_softmax(S->zm, V, T, NULL, NULL, S->p1);
  if (bonus || mutant_q_is_p1) {
    for (int64_t v = 0; v < V; ++v) S->Q[v] = S->p1[v];
    return;
  }
  load_row(m2tab, dtype, V, prev, S->zm);
  row_softmax(S->zm, V, T, NULL, NULL, S->q2);
  double beta = 0.0, rmass = 0.0;
  for (int64_t v = 0; v < V; ++v) {
    const double f = lenience(S->p1[v], kind, eps);
    beta += S->q2[v] < f ? S->q2[v] : f;
    const double d = S->p1[v] - S->q2[v];
    rmass += d > 0.0 ? d : 0.0;
  }
  for (int64_t v = 0; v < V; ++v) {
    const double f = lenience(S->p1[v], kind, eps);
    double q = S->q2[v] < f ? S->q2[v] : f;
    const double d = S->p1[v] - S->q2[v];
    if (rmass > 0.0 && d > 0.0) q += (1.0 - beta) * d / rmass;
    S->Q[v] = q;
  }
}

static void cascade_review(int64_t V, int64_t k1, int dtype, const void* ttab, const void* m1tab,
                           const void* m2tab, double T, int32_t start, const int32_t* dtok,
                           const int32_t* dprev, const int8_t* dbonus, int kind, double eps,
                           int mutant_q_is_p1, uint64_t seed, uint64_t philox_row, int32_t* n_out,
                           int32_t* next_out, uint8_t* near, review_scratch_t* S) {
  *near = 0;
  /* every target row the review reads must be usable */
  for (int64_t i = 0; i <= k1; ++i) {
    const int32_t prev = i == 0 ? start : dtok[i - 1];
    load_row(ttab, dtype, V, prev, S->zt);
    if (!row_is_valid(S->zt, V)) {
      *n_out = -1;
      *next_out = -1;
      return;
    }
  }
  if (T == 0.0) {
    int64_t n = k1;
    for (int64_t i = 0; i < k1; ++i) {
      load_row(ttab, dtype, V, i == 0 ? start : dtok[i - 1], S->zt);
      if (dtok[i] != row_argmax(S->zt, V)) {
        n = i;
        break;
      }
    }
    load_row(ttab, dtype, V, n == 0 ? start : dtok[n - 1], S->zt);
    *n_out = (int32_t)n;
    *next_out = (int32_t)row_argmax(S->zt, V);
    return;
  }
  int64_t n = k1;
  for (int64_t i = 0; i < k1; ++i) {
    const int32_t x = dtok[i];
    load_row(ttab, dtype, V, i == 0 ? start : dtok[i - 1], S->zt);
    row_softmax(S->zt, V, T, NULL, NULL, S->pt);
    cascade_law(V, dtype, m1tab, m2tab, T, dprev[i], dbonus[i], kind, eps, mutant_q_is_p1, S);
    const double ratio = S->Q[x] == 0.0 ? INFINITY : S->pt[x] / S->Q[x];
    double r;
    draw_uniforms(seed, philox_row, (uint32_t)i, &r, NULL);
    if (isfinite(ratio) && fabs(r - ratio) / ratio < ORACLE_NEAR_TIE) *near = 1;
    if (r > ratio) {
      n = i;
      break;
    }
  }
  double u;
  draw_uniforms(seed, philox_row, (uint32_t)n, NULL, &u);
  load_row(ttab, dtype, V, n == 0 ? start : dtok[n - 1], S->zt);
  row_softmax(S->zt, V, T, NULL, NULL, S->pt);
  if (n < k1) {
    cascade_law(V, dtype, m1tab, m2tab, T, dprev[n], dbonus[n], kind, eps, mutant_q_is_p1, S);
    for (int64_t v = 0; v < V; ++v) {
      const double d = S->pt[v] - S->Q[v];
      S->w[v] = d > 0.0 ? d : 0.0;
    }
  } else {
    for (int64_t v = 0; v < V; ++v) S->w[v] = S->pt[v];
  }
  double margin = INFINITY, total = 0.0;
  int64_t tok = inverse_cdf(S->w, V, u, &margin, &total, NULL, NULL);
  if (tok < 0) {
    tok = inverse_cdf(S->pt, V, u, &margin, &total, NULL, NULL);
  } else if (n < k1 && total < ORACLE_NEAR_TIE) {
    margin = 0.0; /* a residual below the window (see sample_outcome) */
  }
  if (margin < ORACLE_NEAR_TIE) *near = 1;
  *n_out = (int32_t)n;
  *next_out = (int32_t)tok;
}

/* CS Drafting's vertical cascade (Chen et al., "Cascade Speculative
 * Drafting for Even Faster LLM Inference", sections 3.1 and 3.4) over three
 * bigram tables: target t, intermediate drafter m1, smallest drafter m2.
 * Outer round r of sequence b builds a draft of k1 tokens for the target by
 * inner rounds j = 0, 1, ...: m2 drafts k2 tokens (as in the decode loop),
 * m1 reviews them with the lenience (kind, eps) -- the step of Algorithm A.1
 * with threshold f(p1, eps)/q2 -- and its n accepted tokens plus its drawn
 * token join the draft, until the draft holds k1 tokens (the excess of the
 * last inner round is dropped). The target then reviews the draft without
 * lenience. Its draft distribution at each position is the one that token
 * was drawn from, given everything before it:
 *   a token from an inner position i < k2 (an accepted draft or the draw
 *   after a rejection): Q = min(q2, f(p1)) + (1 - beta) * norm(max(0, p1 -
 *   q2)), beta = sum_v min(q2(v), f(p1(v))) -- the law of that step's output;
 *   a token from the bonus position k2 (all k2 drafts accepted): Q = p1.
 * With that Q the target review keeps the target's output law whatever the
 * inner lenience: the reading under which the paper's claim, that a target
 * review without lenience leaves the output law unchanged, holds exactly.
 * The target review computes p and Q in float64 from the tables
 * (cascade_review): the ratio p(x)/Q(x) and the residual max(0, p - Q).
 * Greedy sequences (T = 0) use exact-match reviews throughout.
 * Philox rows: outer round r uses the block row_offset + r * (k1 + 1) *
 * batch (+ b), inner round j the block row_offset + (r * (k1 + 1) + 1 + j)
 * * batch; drafting draws word 0 of counter (row, i, 1), reviews use the
 * verify step's counters.
 * Every inner round drafts and reviews k2 tokens for every sequence; the
 * result of a sequence whose draft is already complete is not used.
 * Outputs as oracle_decode_bigram, with out_tokens [batch, rounds * (k1 + 1)],
 * out_accepted the target review's n per round, and out_first_near the first
 * round with a near-tie anywhere in it. mutant_q_is_p1 = 1 makes the target
 * review use p1 as the draft distribution at every position (a negative
 * control: wrong unless eps = 1). */
int oracle_cascade_bigram(int64_t batch, int64_t vocab, int64_t k1, int64_t k2, int64_t rounds,
                          int dtype, const void* ttab, const void* m1tab, const void* m2tab,
                          const float* temperature, const int32_t* start, int lenience_kind,
                          float eps, uint64_t seed, uint64_t row_offset, int mutant_q_is_p1,
                          int32_t* out_tokens, int32_t* out_length, int32_t* out_accepted,
                          int32_t* out_first_near, int nthreads) {
  const int64_t V = vocab, B = batch;
  const size_t esz = dtype == ORACLE_BF16 ? 2 : 4;
  const size_t row_bytes = (size_t)V * esz;
  const int64_t cap = rounds * (k1 + 1);
  const int64_t dcap = k1 + k2 + 1; /* draft buffer per sequence */
  /* inner review buffers (table dtype) */
  char* itpack = (char*)malloc((size_t)(B * (k2 + 1)) * row_bytes + 1);
  char* idpack = (char*)malloc((size_t)(B * k2) * row_bytes + 1);
  int32_t* itok = (int32_t*)malloc((size_t)(B * k2 + 1) * 4);
  int32_t* ipack = (int32_t*)malloc((size_t)(B * k2 + 1) * 4); /* packed inner draft tokens */
  int32_t* igam = (int32_t*)malloc((size_t)(B + 1) * 4);
  /* the target review's rows, float64 */
  review_scratch_t rvs;
  review_scratch_t* rv = &rvs;
  rv->zt = (double*)malloc((size_t)V * 8);
  rv->zm = (double*)malloc((size_t)V * 8);
  rv->p1 = (double*)malloc((size_t)V * 8);
  rv->q2 = (double*)malloc((size_t)V * 8);
  rv->pt = (double*)malloc((size_t)V * 8);
  rv->Q = (double*)malloc((size_t)V * 8);
  rv->w = (double*)malloc((size_t)V * 8);
  /* per-sequence state */
  int32_t* dtok = (int32_t*)malloc((size_t)(B * dcap + 1) * 4);   /* draft tokens      */
  int32_t* dprev = (int32_t*)malloc((size_t)(B * dcap + 1) * 4);  /* their prev token  */
  int8_t* dbonus = (int8_t*)malloc((size_t)(B * dcap + 1));       /* from a bonus slot */
  int64_t* dlen = (int64_t*)malloc((size_t)(B + 1) * 8);
  int32_t* cur = (int32_t*)malloc((size_t)(B + 1) * 4);
  int32_t* len = (int32_t*)malloc((size_t)(B + 1) * 4);
  uint8_t* failed = (uint8_t*)malloc((size_t)B + 1);
  uint8_t* near = (uint8_t*)malloc((size_t)B + 1);
  uint8_t* vnear = (uint8_t*)malloc((size_t)B + 1);
  uint8_t* dnear = (uint8_t*)malloc((size_t)B + 1);
  int32_t* n_out = (int32_t*)malloc((size_t)(B + 1) * 4);
  int32_t* next_out = (int32_t*)malloc((size_t)(B + 1) * 4);
  int32_t* ipr = (int32_t*)malloc((size_t)(B * (k2 + 1) + 1) * 4); /* inner prev per slot */
  double* z = (double*)malloc((size_t)V * 8);
  double* p1 = (double*)malloc((size_t)V * 8);
  double* q2 = (double*)malloc((size_t)V * 8);
  for (int64_t b = 0; b < B; ++b) {
    failed[b] = (uint8_t)(start[b] < 0 || start[b] >= V);
    cur[b] = failed[b] ? 0 : start[b];
    len[b] = 0;
    out_first_near[b] = (int32_t)rounds;
  }
  for (int64_t r = 0; r < rounds; ++r) {
    for (int64_t b = 0; b < B; ++b) {
      dlen[b] = 0;
      near[b] = 0;
    }
    /* inner rounds: at most k1 (each adds at least one token) */
    for (int64_t j = 0; j < k1; ++j) {
      const uint64_t rbase = row_offset + (uint64_t)((r * (k1 + 1) + 1 + j) * B);
      for (int64_t b = 0; b < B; ++b) {
        igam[b] = (int32_t)k2;
        const double T = (double)temperature[b];
        int32_t prev = dlen[b] > 0 ? dtok[b * dcap + dlen[b] - 1] : cur[b];
        const int64_t g = igam[b];
        dnear[b] = 0;
        /* packed offsets of this inner batch: sequence b's rows start at
         * sum_{b' < b} (g_b' + 1) and sum g_b' (computed below) */
        for (int64_t i = 0; i <= g; ++i) {
          ipr[b * (k2 + 1) + i] = prev;
          if (i == g) break;
          load_row(m2tab, dtype, V, prev, z);
          int64_t x = 0;
          if (!row_is_valid(z, V) || temperature_invalid(T)) {
            x = 0;
          } else if (T == 0.0) {
            x = row_argmax(z, V);
          } else {
            row_softmax(z, V, T, NULL, NULL, q2);
            const uint64_t prow = rbase + (uint64_t)b;
            uint32_t ctr[4] = {(uint32_t)prow, (uint32_t)(prow >> 32), (uint32_t)i, 1u};
            uint32_t w[4];
            oracle_philox4x32_10(seed, ctr, w);
            double margin = INFINITY;
            x = inverse_cdf(q2, V, oracle_uniform24(w[0]), &margin, NULL, NULL, NULL);
            if (x < 0) x = 0;
            if (margin < ORACLE_NEAR_TIE) dnear[b] = 1;
          }
          itok[b * k2 + i] = (int32_t)x;
          prev = (int32_t)x;
        }
      }
      /* pack the inner review (ragged: inactive sequences have gamma 0) */
      int64_t tt = 0, td = 0;
      for (int64_t b = 0; b < B; ++b) {
        const int64_t g = igam[b];
        for (int64_t i = 0; i <= g; ++i)
          memcpy(itpack + (size_t)(tt + i) * row_bytes,
                 (const char*)m1tab + (size_t)ipr[b * (k2 + 1) + i] * row_bytes, row_bytes);
        for (int64_t i = 0; i < g; ++i) {
          memcpy(idpack + (size_t)(td + i) * row_bytes,
                 (const char*)m2tab + (size_t)ipr[b * (k2 + 1) + i] * row_bytes, row_bytes);
          ipack[td + i] = itok[b * k2 + i];
        }
        tt += g + 1;
        td += g;
      }
      oracle_verify(B, V, k2, dtype, tt, td, itpack, idpack, ipack, igam, temperature, seed, rbase,
                    lenience_kind, eps, NULL, NULL, n_out, next_out, NULL, vnear, NULL, NULL, NULL,
                    NULL, NULL, NULL, nthreads);
      for (int64_t b = 0; b < B; ++b) {
        if (dlen[b] >= k1) continue; /* draft already complete: result unused */
        if (n_out[b] < 0) {
          failed[b] = 1;
          /* nothing more to draft: pad with token 0 so that every row the
           * target review addresses exists; the result is not used */
          for (int64_t d = dlen[b]; d < k1; ++d) {
            dtok[b * dcap + d] = 0;
            dprev[b * dcap + d] = 0;
            dbonus[b * dcap + d] = 0;
          }
          dlen[b] = k1;
          continue;
        }
        if (vnear[b] || dnear[b]) near[b] = 1;
        const int32_t n = n_out[b];
        for (int32_t i = 0; i <= n; ++i) {
          const int64_t d = dlen[b] + i;
          dtok[b * dcap + d] = i < n ? itok[b * k2 + i] : next_out[b];
          dprev[b * dcap + d] = ipr[b * (k2 + 1) + i];
          dbonus[b * dcap + d] = (int8_t)(i == k2);
        }
        dlen[b] += n + 1;
      }
    }
    /* the target review of the first k1 draft tokens, without lenience */
    const uint64_t obase = row_offset + (uint64_t)(r * (k1 + 1) * B);
    for (int64_t b = 0; b < B; ++b) {
      vnear[b] = 0;
      if (failed[b]) {
        n_out[b] = -1;
        continue;
      }
      const double T = (double)temperature[b];
      if (temperature_invalid(T)) {
        n_out[b] = -1;
        next_out[b] = -1;
        continue;
      }
      cascade_review(V, k1, dtype, ttab, m1tab, m2tab, T, cur[b], dtok + b * dcap,
                     dprev + b * dcap, dbonus + b * dcap, lenience_kind, (double)eps,
                     mutant_q_is_p1, seed, obase + (uint64_t)b, &n_out[b], &next_out[b],
                     &vnear[b], rv);
    }
    for (int64_t b = 0; b < B; ++b) {
      if (!failed[b] && n_out[b] < 0) failed[b] = 1;
      if (failed[b]) {
        out_accepted[b * rounds + r] = -1;
        continue;
      }
      const int32_t n = n_out[b];
      for (int32_t i = 0; i < n; ++i) out_tokens[b * cap + len[b] + i] = dtok[b * dcap + i];
      out_tokens[b * cap + len[b] + n] = next_out[b];
      len[b] += n + 1;
      cur[b] = next_out[b];
      out_accepted[b * rounds + r] = n;
      if ((near[b] || vnear[b]) && out_first_near[b] == rounds) out_first_near[b] = (int32_t)r;
    }
  }
  for (int64_t b = 0; b < B; ++b) out_length[b] = failed[b] ? -1 : len[b];
  free(itpack); free(idpack); free(itok); free(ipack); free(igam);
  free(rv->zt); free(rv->zm); free(rv->p1); free(rv->q2); free(rv->pt); free(rv->Q); free(rv->w);
  free(dtok); free(dprev); free(dbonus); free(dlen); free(cur); free(len);
  free(failed); free(near); free(vnear); free(dnear); free(n_out); free(next_out); free(ipr); free(z);
  free(p1); free(q2);
  return 0;
}
