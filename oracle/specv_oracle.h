/*
 * specv_oracle.h -- prototypes of the CPU oracle's entry points
 * (oracle/specv_oracle.c).
 *
 * TEST INFRASTRUCTURE: only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use the oracle; the HIP library never
 * includes this header. Logit arrays are [rows, vocab] row-major, bf16 as
 * uint16 bit patterns (dtype ORACLE_BF16) or float32 (ORACLE_F32), in the
 * packed layout of the verify step.
 */
#ifndef SPECV_ORACLE_H
#define SPECV_ORACLE_H

#include <stdint.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1

#define ORACLE_LENIENCE_NONE 0
#define ORACLE_LENIENCE_LIN 1
#define ORACLE_LENIENCE_SQ 2
#define ORACLE_LENIENCE_EXP 3

void oracle_set_mutant(int m);
void oracle_philox4x32_10(uint64_t seed, const uint32_t ctr_in[4], uint32_t out[4]);
double oracle_uniform24(uint32_t w);
void oracle_uniform24_many(const uint32_t* w, double* out, int64_t n);
void oracle_decode_bf16(const uint16_t* in, double* out, int64_t n);
void oracle_philox_blocks(uint64_t seed, const uint32_t* ctr, uint32_t* out, int64_t count);

/* The verify step over a packed batch; every output pointer from out_margin
 * on may be NULL. out_window is [batch, 5]: tok_lo, tok_hi, alt_n, alt_lo,
 * alt_hi. Returns 1 after a layout error (every sequence (-1, -1)). */
int oracle_verify(int64_t batch, int64_t vocab, int64_t max_gamma, int dtype,
                  int64_t total_target_rows, int64_t total_draft_rows, const void* target,
                  const void* draft, const int32_t* tokens, const int32_t* gamma,
                  const float* temperature, uint64_t seed, uint64_t row_offset,
                  int lenience_kind, float eps,
                  const float* inj_r, const float* inj_u, int32_t* out_n, int32_t* out_next,
                  double* out_margin, uint8_t* out_near, double* out_ratio, double* out_resmass,
                  double* out_accept_margin, double* out_draw_margin, int32_t* out_window,
                  double* out_near_prob, int nthreads);

void oracle_row_stats(const void* logits, int dtype, int64_t rows, int64_t vocab,
                      const float* T_row, double* out_m, double* out_s, int32_t* out_arg,
                      uint8_t* out_valid);
void oracle_softmax_row(const void* logits, int dtype, int64_t vocab, int64_t row, float T,
                        double* out_p);

int oracle_position_diagnostics(int64_t batch, int64_t vocab, int dtype, int64_t total_target_rows,
                                int64_t total_draft_rows, const void* target, const void* draft,
                                const int32_t* gamma, const float* temperature, int64_t top_k,
                                double* out_alpha, double* out_entropy, int32_t* out_topk_index,
                                double* out_topk_prob);

int oracle_decode_bigram(int64_t batch, int64_t vocab, int64_t gamma, int64_t rounds, int dtype,
                         const void* ttab, const void* dtab, const float* temperature,
                         const int32_t* start, uint64_t seed, uint64_t row_offset,
                         int32_t* out_tokens, int32_t* out_length, int32_t* out_accepted,
                         int32_t* out_first_near, int nthreads);

int oracle_cascade_bigram(int64_t batch, int64_t vocab, int64_t k1, int64_t k2, int64_t rounds,
                          int dtype, const void* ttab, const void* m1tab, const void* m2tab,
                          const float* temperature, const int32_t* start, int lenience_kind,
                          float eps, uint64_t seed, uint64_t row_offset, int mutant_q_is_p1,
                          int32_t* out_tokens, int32_t* out_length, int32_t* out_accepted,
                          int32_t* out_first_near, int nthreads);

#endif /* SPECV_ORACLE_H */
