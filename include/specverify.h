/*
 * specverify.h -- C ABI of libspecverify, the speculative-sampling verify
 * step on AMD Instinct MI355X (gfx950).
 *
 * The operation (DistillSpec, Zhou et al., ICLR 2024, Appendix A.3,
 * Algorithm A.1 "Speculative decoding step", lossless: lenience eps = 1; the
 * same rule as summarised from Leviathan et al. on "How speculative decoding
 * lets a small model draft and a large one check"):
 *
 *   For each sequence b with gamma_b draft tokens x_0..x_{gamma_b - 1}:
 *     p_i = softmax(target logits row i / T_b),  i = 0..gamma_b
 *     q_i = softmax(draft  logits row i / T_b),  i = 0..gamma_b - 1
 *     r_i ~ U(0, 1];  n = first i with r_i > p_i(x_i) / q_i(x_i), else gamma_b
 *     next token ~ norm(max(0, p_n - q_n))  if n < gamma_b
 *                ~ p_{gamma_b}              if n == gamma_b
 *   Greedy sequences (T_b == 0) accept x_i while it equals argmax p_i and
 *   emit argmax p_n ("Speculative Decoding and Distillation" notes,
 *   Practical considerations: greedy acceptance is exact match). The
 *   temperature softmax is the one in the same notes, Part 2 "Loss (Hinton)",
 *   with one T shared by target and draft.
 *   The caller appends x_0..x_{n-1} and the next token: at least one and at
 *   most gamma_b + 1 tokens per call and sequence.
 *
 * Uniforms: Philox4x32-10 (Salmon et al., SC'11) with key = seed and counter
 * (row lo, row hi, i, 0), row = philox_row_offset + b. Word 0 of block i is
 * r_i; word 1 of block n is the uniform of the final draw. A word w becomes
 * ((w >> 8) + 1) * 2^-24, in (0, 1]. The final draw is the inverse CDF in
 * index order: the smallest v with u * C_{V-1} <= C_v. Argmax ties resolve to
 * the lowest index.
 *
 * Layout (every tensor pointer below is a DEVICE pointer, caller-owned):
 *   target_logits  [sum_b (gamma_b + 1), V] row-major, row stride V, packed by
 *                  sequence: sequence b's rows start at sum_{b'<b}(gamma_b'+1)
 *   draft_logits   [sum_b gamma_b, V], sequence b's rows at sum_{b'<b} gamma_b'
 *   draft_tokens   [sum_b gamma_b] int32, same packing as the draft rows
 *   gamma_per_row  [B] int32 in [0, max_gamma]
 *   temperature    [B] float32: > 0 sampling, == 0 greedy
 *   out_n_accepted [B] int32, out_next_token [B] int32
 * Both logit tensors share one dtype (bf16 or fp32). -inf logits are legal
 * (masked tokens), and so is any finite logit: masks with the most negative
 * finite value work as -inf would. A sampling T_b must keep log2(e)/T_b, the
 * fp32 scale of the logits, finite: T_b above about 4.2e-39 (exactly: the
 * float64 quotient log2(e)/T_b below 2^128 - 2^103).
 *
 * Asynchrony: every entry point that takes a stream only enqueues work on it
 * and returns; results are valid after the stream is synchronised. Nothing
 * allocates device memory: scratch space is the caller's workspace, sized by
 * specv_workspace_bytes() (specv_verify_noalloc: a static array). Calls that
 * share a workspace must not overlap.
 *
 * Errors:
 *   - argument errors (null pointers, sizes out of range, row totals that
 *     cannot match, misaligned logits, workspace too small) return a status
 *     before anything is enqueued;
 *   - a failed launch returns SPECV_ERR_HIP;
 *   - data errors found on the device give that sequence (-1, -1) and set a
 *     bit in the status word at byte offset 0 of the workspace: a gamma_b
 *     outside [0, max_gamma] or gammas that disagree with the row totals
 *     (every sequence gets (-1, -1)); T_b NaN, negative, +inf or too small for
 *     the fp32 scale log2(e)/T_b; a draft token
 *     outside [0, V); a needed row with NaN or +inf or no finite logit
 *     (needed rows: all target rows; draft rows only of sampling sequences).
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPECV_MAX_GAMMA 63

typedef enum { SPECV_F32 = 0, SPECV_BF16 = 1 } specv_dtype_t;

typedef enum {
  SPECV_OK = 0,
  SPECV_ERR_INVALID_ARGUMENT = 1,
  SPECV_ERR_WORKSPACE = 2,
  SPECV_ERR_HIP = 3,
  SPECV_ERR_UNSUPPORTED = 4,
  SPECV_ERR_SCRATCH_LIMIT = 5 /* specv_verify_noalloc: shape too large for its scratch */
} specv_status_t;

/* Device status word: uint32 at byte offset 0 of the workspace after a call. */
#define SPECV_WORKSPACE_STATUS_OFFSET 0
#define SPECV_DEV_SEQ_ERROR 1u    /* at least one sequence got (-1, -1)        */
#define SPECV_DEV_LAYOUT_ERROR 2u /* gammas out of range or row totals differ  */

/* Host struct describing one call. */
typedef struct {
  int32_t batch;               /* B >= 0 (B == 0: nothing to do)             */
  int32_t vocab;               /* V >= 1                                     */
  int32_t max_gamma;           /* 0 <= max_gamma <= SPECV_MAX_GAMMA          */
  specv_dtype_t dtype;         /* dtype of both logit tensors                */
  int64_t total_target_rows;   /* sum_b (gamma_b + 1) == total_draft_rows + B;
                                  at most 2^29, and total_target_rows * V at most 2^40 */
  int64_t total_draft_rows;    /* sum_b gamma_b <= B * max_gamma             */
} specv_shape_t;

/* Bytes of device workspace specv_verify needs for `shape`; 0 if the shape
 * is invalid (a valid shape always needs at least 256 bytes). */
size_t specv_workspace_bytes(const specv_shape_t* shape);

/* The verify step (DistillSpec Algorithm A.1, eps = 1), all sequences at
 * once. `workspace` is a device buffer of at least specv_workspace_bytes()
 * bytes, 256-byte aligned; its contents need no initialisation. */
specv_status_t specv_verify(const specv_shape_t* shape, const void* target_logits,
                            const void* draft_logits, const int32_t* draft_tokens,
                            const int32_t* gamma_per_row, const float* temperature,
                            uint64_t seed, uint64_t philox_row_offset,
                            int32_t* out_n_accepted, int32_t* out_next_token,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): specv_verify
 * with no workspace argument. Its scratch is a static device array of
 * SPECV_NOALLOC_SCRATCH_BYTES per GPU, created with the library's code object
 * on that GPU and held until the process ends; its address is looked up once
 * per device (the current device, which must be the stream's). The call
 * allocates nothing and frees nothing. A shape whose workspace
 * (specv_workspace_bytes) exceeds SPECV_NOALLOC_SCRATCH_BYTES returns
 * SPECV_ERR_SCRATCH_LIMIT before anything is enqueued. Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (other streams, other
 * threads) race and must be serialised by the caller. The array keeps the
 * last call's contents; nothing in it needs clearing (every call writes what
 * it reads). out_status: NULL, or a device uint32 that receives the status
 * word of specv_verify's workspace (byte offset 0) once the call's kernels
 * have run, by one more small launch on `stream` (0 for an empty batch).
 * Everything else as specv_verify. */
#define SPECV_NOALLOC_SCRATCH_BYTES (16u << 20)
specv_status_t specv_verify_noalloc(const specv_shape_t* shape, const void* target_logits,
                                    const void* draft_logits, const int32_t* draft_tokens,
                                    const int32_t* gamma_per_row, const float* temperature,
                                    uint64_t seed, uint64_t philox_row_offset,
                                    int32_t* out_n_accepted, int32_t* out_next_token,
                                    uint32_t* out_status, hipStream_t stream);

/* Same as specv_verify with the uniforms given instead of drawn: r is
 * [B, max_gamma] float32 (r_i of sequence b at r[b * max_gamma + i]) and u is
 * [B] float32, device pointers. Values are used as given (expected in
 * (0, 1]). Decouples the random stream from the accept/draw logic. */
specv_status_t specv_verify_with_uniforms(const specv_shape_t* shape, const void* target_logits,
                                          const void* draft_logits, const int32_t* draft_tokens,
                                          const int32_t* gamma_per_row, const float* temperature,
                                          const float* r, const float* u,
                                          int32_t* out_n_accepted, int32_t* out_next_token,
                                          void* workspace, size_t workspace_bytes,
                                          hipStream_t stream);

/* Lenience functions of lossy verification (DistillSpec section 4, the
 * paragraph on DistillSpec with lossy SD, and the rejection thresholds of
 * Algorithm A.1): a drafted token x is accepted with probability
 * min(1, f(p(x), eps) / q(x)) instead of min(1, p(x) / q(x)). Each f grows
 * with p, shrinks with eps, and f(p, 1) = p. */
typedef enum {
  SPECV_LENIENCE_NONE = 0, /* f = p: lossless                */
  SPECV_LENIENCE_LIN = 1,  /* f = p / eps                    */
  SPECV_LENIENCE_SQ = 2,   /* f = p / eps^2                  */
  SPECV_LENIENCE_EXP = 3   /* f = p^eps                      */
} specv_lenience_t;

/* The verify step with lenience f and parameter epsilon in (0, 1] (ignored
 * for SPECV_LENIENCE_NONE; epsilon == 1 is the lossless step). The final
 * draw after a rejection still samples norm(max(0, p_n - q_n)), as
 * Algorithm A.1 prints it, so for epsilon < 1 the output no longer follows
 * the target distribution. Greedy sequences (T_b == 0) are unaffected: their
 * p is one-hot, f(0, eps) = 0 and f(1, eps) >= 1. The f value, threshold and
 * comparison are float64. r and u: both NULL draws the uniforms from Philox
 * as specv_verify does; both given injects them as in
 * specv_verify_with_uniforms (r may be NULL when max_gamma == 0). An
 * unknown lenience, an epsilon outside (0, 1] (NaN included) or r without u
 * is SPECV_ERR_INVALID_ARGUMENT. `events` is NULL or stage events as in
 * specv_verify_profiled. Everything else as specv_verify. */
specv_status_t specv_verify_lenient(const specv_shape_t* shape, const void* target_logits,
                                    const void* draft_logits, const int32_t* draft_tokens,
                                    const int32_t* gamma_per_row, const float* temperature,
                                    specv_lenience_t lenience, float epsilon, uint64_t seed,
                                    uint64_t philox_row_offset, const float* r, const float* u,
                                    int32_t* out_n_accepted, int32_t* out_next_token,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream,
                                    hipEvent_t* events);

/* Per-position diagnostics. For every draft position i < gamma_b of every
 * sequence b, written at the packed draft-row index doff_b + i, with
 * p = p_i and q = q_i the temperature softmaxes of target row i and draft
 * row i:
 *   out_alpha[j]   = sum_v min(p_v, q_v), the probability that a token drafted
 *                    from q is accepted (DistillSpec section 3; 1 - alpha is
 *                    the total variation distance of its section 4);
 *   out_entropy[j] = -sum_v q_v ln q_v (nats);
 *   out_topk_index[j * top_k + l], out_topk_prob[j * top_k + l]: the l-th most
 *                    probable draft token and its q (larger logit first, equal
 *                    logits lower index first).
 * Entropy and top-k are the Ent and Top_k features of DISCO's stopping
 * classifier (DISCO section 3, Eq. 2). Greedy sequences (T_b == 0) use the
 * zero-temperature limits of greedy verification: p and q one-hot at their
 * argmax, so alpha is 1 or 0, the entropy 0 and the top-1 probability 1.
 * A position whose target or draft row holds NaN or +inf or no finite logit,
 * or whose T_b is invalid (as for specv_verify), gets NaN alpha and entropy, index
 * -1 and probability NaN; after a layout error (as in specv_verify) every
 * position reads so, and the status bit is set. 0 <= top_k <= min(V,
 * SPECV_MAX_TOP_K); with top_k == 0 the top-k pointers may be NULL.
 * Precision: alpha and entropy are float64 sums of fp32 terms; the top-k
 * selection compares raw logits (exact); its probabilities are float64.
 * Device output arrays are caller-owned; `workspace` is at least
 * specv_diagnostics_workspace_bytes(shape, top_k) bytes, 256-byte aligned.
 * `events` is NULL or 2 * SPECV_NUM_STAGES events recorded around the
 * stages as in specv_verify_profiled; the stages here are the plan, pass 1
 * (row statistics of every target and draft row), pass 2 (SPECV_STAGE_
 * ACCEPT_MASS slot: the per-position sums and top-k lists) and the merge
 * (SPECV_STAGE_DRAW slot; it shares pass 2's launch, and its events are
 * recorded back to back, when a position has 1, 2 or 4 pass-1 chunks and
 * chunks * top_k <= 64). */
#define SPECV_MAX_TOP_K 64
size_t specv_diagnostics_workspace_bytes(const specv_shape_t* shape, int32_t top_k);
specv_status_t specv_position_diagnostics(const specv_shape_t* shape, const void* target_logits,
                                          const void* draft_logits, const int32_t* gamma_per_row,
                                          const float* temperature, int32_t top_k,
                                          double* out_alpha, double* out_entropy,
                                          int32_t* out_topk_index, double* out_topk_prob,
                                          void* workspace, size_t workspace_bytes,
                                          hipStream_t stream, hipEvent_t* events);

/* Multi-round speculative decoding with bigram "models" (DistillSpec
 * Algorithm A.1 repeated: each round extends every sequence by its n
 * accepted draft tokens and the drawn token). The models are bigram logit
 * tables [V, V] (row s: the logits of the next token after token s), one for
 * the target and one for the draft, in `dtype`, row-major, device memory.
 * Round r, sequence b, with row = philox_row_offset + r * batch + b and prev
 * the sequence's last token (start_token[b] before round 0):
 *   drafting: x_i ~ softmax(draft_table[prev_i] / T_b), prev_0 = prev,
 *     prev_{i+1} = x_i, i < gamma: the inverse CDF in index order (smallest
 *     v with u * C_{V-1} <= C_v) with u = U(word 0 of Philox(seed; counter
 *     (row lo, row hi, i, 1))); T_b == 0 drafts the argmax (lowest index);
 *   verification: specv_verify on target rows target_table[prev_i],
 *     i = 0..gamma, and draft rows draft_table[prev_i], i < gamma, with
 *     philox_row_offset + r * batch as its row offset.
 * Outputs (device, caller-owned): out_tokens [batch, rounds * (gamma + 1)]
 * (generated tokens, -1 past the end), out_length [batch] (tokens generated;
 * -1 for a sequence whose start token is outside [0, V) or whose round hit a
 * data error), out_accepted [batch, rounds] (n of each round, -1 from a
 * failed round on). Rows of the draft table used by greedy sequences are not
 * checked for NaN. `events`: NULL, or 2 * SPECV_NUM_STAGES events recorded
 * around the stages of the last round: drafting (SPECV_STAGE_PLAN slot), the
 * row gather, which also forms the verify step's pass-1 statistics (ROWSTATS
 * slot), the rest of the verify step (ACCEPT_MASS slot) and the append (DRAW
 * slot). Argument errors as for specv_verify; the workspace
 * is specv_decode_workspace_bytes(shape) bytes, 256-byte aligned. */
typedef struct {
  int32_t batch;   /* >= 0                               */
  int32_t vocab;   /* V >= 1; the tables are [V, V]      */
  int32_t gamma;   /* draft tokens per round, 0..63      */
  int32_t rounds;  /* >= 0                               */
  specv_dtype_t dtype;
} specv_decode_shape_t;

/* Workspace bytes for a decode call; 0 for an invalid shape. Size limits:
 * V * V and batch * rounds * (gamma + 1) at most 2^40, and the verify step
 * of a round (batch * (gamma + 1) target rows of V) within specv_shape_t's. */
size_t specv_decode_workspace_bytes(const specv_decode_shape_t* shape);
specv_status_t specv_decode_bigram(const specv_decode_shape_t* shape, const void* target_table,
                                   const void* draft_table, const float* temperature,
                                   const int32_t* start_token, uint64_t seed,
                                   uint64_t philox_row_offset, int32_t* out_tokens,
                                   int32_t* out_length, int32_t* out_accepted, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream,
                                   hipEvent_t* events);

/* CS Drafting's vertical cascade ("Cascade Speculative Drafting for Even
 * Faster LLM Inference", sections 3.1 and 3.4) with three bigram tables
 * [V, V] of one dtype: target, intermediate drafter (mid) and smallest
 * drafter (small). Outer round r of sequence b: inner rounds j = 0, 1, ...
 * let the small table draft k2 tokens (drafting as in specv_decode_bigram)
 * and the mid table review them with the given lenience (specv_verify_lenient
 * rule), and the n accepted tokens plus the drawn one join a draft, until it
 * holds k1 tokens (the excess is dropped). The target table then reviews the
 * first k1 draft tokens without lenience, against the law each was drawn
 * from: min(q2, f(p1)) + (1 - beta) norm(max(0, p1 - q2)) with beta =
 * sum_v min(q2(v), f(p1(v))) for a token from an inner position < k2, p1
 * for a token from the inner bonus position (p1, q2: the mid and small
 * softmaxes after the token's predecessor). With that law the output follows
 * the target's distribution whatever the inner lenience; this is the reading
 * under which the paper's claim holds exactly. The target review runs in
 * fp32 (target rows converted exactly, draft rows fl32(T ln law)).
 * Every inner round drafts and reviews all sequences (at most k1 inner
 * rounds per outer round); results of a sequence whose draft is complete are
 * unused. Philox rows: the target review of round r uses row offset
 * philox_row_offset + r (k1 + 1) batch, inner round j uses philox_row_offset
 * + (r (k1 + 1) + 1 + j) batch (drafting on counter word 3 = 1). Outputs and
 * failure rules as specv_decode_bigram, with out_tokens [batch, rounds
 * (k1 + 1)] and out_accepted the target review's n. Lenience and epsilon as
 * in specv_verify_lenient. `events`: NULL, or 2 * SPECV_NUM_STAGES events
 * recorded in the last outer round: around the first inner round's drafting
 * (SPECV_STAGE_PLAN slot), its row gather with the review's pass 1
 * (ROWSTATS slot) and the rest of its review (ACCEPT_MASS slot), and around
 * the whole target review with its append
 * (DRAW slot). */
typedef struct {
  int32_t batch;   /* >= 0                                    */
  int32_t vocab;   /* V >= 1; the tables are [V, V]           */
  int32_t k1;      /* draft tokens per target review, 0..63   */
  int32_t k2;      /* small-table drafts per inner round, 0..63 */
  int32_t rounds;  /* >= 0                                    */
  specv_dtype_t dtype;
} specv_cascade_shape_t;

/* Workspace bytes for a cascade call; 0 for an invalid shape. Size limits:
 * V * V and batch * rounds * (k1 + 1) at most 2^40, and both reviews
 * (batch * (k1 + 1) and batch * (k2 + 1) target rows of V) within
 * specv_shape_t's. */
size_t specv_cascade_workspace_bytes(const specv_cascade_shape_t* shape);
specv_status_t specv_cascade_bigram(const specv_cascade_shape_t* shape, const void* target_table,
                                    const void* mid_table, const void* small_table,
                                    const float* temperature, const int32_t* start_token,
                                    specv_lenience_t lenience, float epsilon, uint64_t seed,
                                    uint64_t philox_row_offset, int32_t* out_tokens,
                                    int32_t* out_length, int32_t* out_accepted, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream,
                                    hipEvent_t* events);

/* Stages of one call, in launch order. A stage is one kernel, with two
 * exceptions whose event pairs are then recorded back to back and time
 * nothing: there is no plan launch for a uniform batch (every gamma_b ==
 * max_gamma; pass 1 checks the gammas) nor for a ragged batch of at most
 * 1024 sequences (pass 1's first workgroup writes the offsets and checks the
 * gammas, and each pass-1 wave finds its row's sequence itself), and the
 * draw shares the launch of the accept step and pass 2 when one workgroup
 * holds a sequence's pass-2 waves (16 waves at most: 512 or more sequences,
 * or V <= 32768). */
#define SPECV_STAGE_PLAN 0        /* offsets of the packed rows, per-row T scale */
#define SPECV_STAGE_ROWSTATS 1    /* pass 1: max, sum of exp (argmax) per row    */
#define SPECV_STAGE_ACCEPT_MASS 2 /* ratios, uniforms, n; pass 2 weight masses   */
#define SPECV_STAGE_DRAW 3        /* inverse-CDF draw of the next token          */
#define SPECV_NUM_STAGES 4

/* specv_verify that also records events[2 s] before and events[2 s + 1]
 * after stage s on `stream` (events: 2 * SPECV_NUM_STAGES hipEvent_t created
 * by the caller, or NULL; a NULL entry is skipped). For timing the stages of
 * a call. */
specv_status_t specv_verify_profiled(const specv_shape_t* shape, const void* target_logits,
                                     const void* draft_logits, const int32_t* draft_tokens,
                                     const int32_t* gamma_per_row, const float* temperature,
                                     uint64_t seed, uint64_t philox_row_offset,
                                     int32_t* out_n_accepted, int32_t* out_next_token,
                                     void* workspace, size_t workspace_bytes,
                                     hipStream_t stream, hipEvent_t* events);

/* Row statistics of pass 1, merged per row (the values specv_verify uses):
 * m = max z, s = sum_v exp((z_v - m) / T_b) (float64; NaN for rows of greedy
 * sequences and for rows with NaN/+inf), arg = argmax z (lowest index).
 * Outputs are device arrays of total_target_rows / total_draft_rows entries;
 * draft rows of greedy sequences are not read: m = NaN, s = NaN, arg = -1. */
specv_status_t specv_row_stats(const specv_shape_t* shape, const void* target_logits,
                               const void* draft_logits, const int32_t* gamma_per_row,
                               const float* temperature, float* out_target_max,
                               double* out_target_sum, int32_t* out_target_argmax,
                               float* out_draft_max, double* out_draft_sum,
                               int32_t* out_draft_argmax, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/* Temperature-softmax probabilities of selected rows, as the final draw
 * evaluates them: rows[k] >= 0 selects target row rows[k], rows[k] < 0
 * selects draft row -rows[k] - 1 (device int64 array of n_rows entries);
 * out_probs is [n_rows, V] float32. The row's sequence must be sampling. */
specv_status_t specv_softmax_rows(const specv_shape_t* shape, const void* target_logits,
                                  const void* draft_logits, const int32_t* gamma_per_row,
                                  const float* temperature, const int64_t* rows, int64_t n_rows,
                                  float* out_probs, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/* Raw Philox4x32-10 blocks of the device generator: out[4k..4k+4) for key =
 * seed and counter ctr[4k..4k+4) (device arrays, n blocks). */
specv_status_t specv_philox4x32_10(uint64_t seed, const uint32_t* ctr, uint32_t* out, int64_t n,
                                   hipStream_t stream);

/* Device copy of `bytes` bytes (16-byte aligned pointers, bytes a multiple
 * of 16): whole 64 KiB segments with the read probe's tiled pattern (two
 * sibling waves per segment on alternate 4 KiB tiles, non-temporal loads and
 * stores), a shorter tail by a grid-stride copy. A calibration kernel for
 * memory counters and copy bandwidth. */
specv_status_t specv_copy_bytes(void* dst, const void* src, size_t bytes, hipStream_t stream);

/* Read-only stream of `bytes` bytes at src (device, 16-byte aligned; bytes a
 * multiple of 65,536) with the access pattern of pass 1: each 64 KiB segment
 * is read by two sibling waves taking alternate 4 KiB tiles with 16-byte
 * non-temporal loads. sink (device, bytes / 32,768 words) receives one XOR
 * checksum of the dwords each wave read: wave 2s + h of segment s reads its
 * tiles h, h + 2, ..., h + 14. A calibration kernel: the read bandwidth this
 * part reaches with that pattern. Invalid sizes or pointers return
 * SPECV_ERR_INVALID_ARGUMENT before anything is enqueued. */
specv_status_t specv_read_bytes(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

const char* specv_status_string(specv_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
