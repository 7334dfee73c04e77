// specverify.hip -- host side of libspecverify: argument checks, workspace
// carve-up and kernel launches on the caller's stream. The C ABI is declared
// in include/specverify.h.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <mutex>

#include "cascade.hpp"
#include "decode.hpp"
#include "diagnostics.hpp"
#include "kernels.hpp"
#include "specverify.h"

using namespace specv;

namespace {

constexpr size_t kAlign = 256;

// Enum fields and arguments of the C ABI arrive from C and ctypes callers as
// plain 32-bit integers, so any value may be there; reading a C++ enum object
// that holds a value outside its enumerators' range is undefined, so checks
// read the integer bits instead.
template <typename E>
int32_t enum_bits(const E& e) {
  static_assert(sizeof(E) == sizeof(int32_t), "the C ABI's enums are 32-bit");
  int32_t v;
  memcpy(&v, &e, sizeof v);
  return v;
}

bool dtype_ok(const specv_dtype_t& dt) {
  const int32_t v = enum_bits(dt);
  return v == SPECV_F32 || v == SPECV_BF16;
}

bool lenience_ok(const specv_lenience_t& l, float epsilon) {
  const int32_t v = enum_bits(l);
  if (v < SPECV_LENIENCE_NONE || v > SPECV_LENIENCE_EXP) return false;
  return v == SPECV_LENIENCE_NONE || (epsilon > 0.f && epsilon <= 1.f);
}
// Tuning constants (measured on MI355X; see the design notes).
#ifndef SPECV_K1_CHUNK_BF16
#define SPECV_K1_CHUNK_BF16 32768
#endif
#ifndef SPECV_K1_CHUNK_F32
#define SPECV_K1_CHUNK_F32 24576
#endif
#ifndef SPECV_K1_TWO_CHUNKS_ABOVE
#define SPECV_K1_TWO_CHUNKS_ABOVE 2048
#endif
#ifndef SPECV_MASS_WAVES
#define SPECV_MASS_WAVES 8192
#endif
// pass-1 work item: about this many elements of one row (swept per dtype)
constexpr int64_t kK1ChunkBF16 = SPECV_K1_CHUNK_BF16;
constexpr int64_t kK1ChunkF32 = SPECV_K1_CHUNK_F32;
constexpr int64_t kMaxChunks1 = 16;                  // pass-1 chunks per row (at most)
#ifndef SPECV_MIN_PASS1_WAVES
#define SPECV_MIN_PASS1_WAVES 512
#endif
constexpr int64_t kMinPass1Waves = SPECV_MIN_PASS1_WAVES;  // two per compute unit
#ifndef SPECV_MIN_WAVES_CHUNK_CAP
#define SPECV_MIN_WAVES_CHUNK_CAP 4
#endif
constexpr int kDrawStep = kBlock * 8; // elements per workgroup scan step of the draw
constexpr int64_t kTargetMassItems = SPECV_MASS_WAVES;  // pass-2 waves to aim for
constexpr int64_t kMassStepsPerWave = 5;      // draw steps per wave of a one-workgroup split
constexpr int64_t kFusedMinWaves = 2048;      // ... if it still gives this many waves in all
constexpr int64_t kTargetUnfusedItems = 3072;  // else unfused waves to aim for
// Accept step, pass 2 and draw in one launch when a sequence's pass-2 waves fit
// one workgroup and its sub-block masses fit this much LDS.
#ifndef SPECV_INLINE_PLAN
#define SPECV_INLINE_PLAN 1  // ragged batches of at most 1024 sequences: no plan launch
#endif
#ifndef SPECV_CAPTURE
#define SPECV_CAPTURE 1  // 0: the accept step reads the draft tokens' logits from the rows
#endif
#ifndef SPECV_FUSED_DRAW
#define SPECV_FUSED_DRAW 1
#endif
#ifndef SPECV_DRAW_FROM_LDS
#define SPECV_DRAW_FROM_LDS 1  // one wave, one sub-block: the draw walks the weights left in LDS
#endif
#ifndef SPECV_SHORT_ROWS
#define SPECV_SHORT_ROWS 2  // rows per pass-1 wave for rows of one tile (0: one row per wave)
#endif
constexpr size_t kFusedDrawLds = 64 * 1024;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Plan {
  int dt;
  int64_t B, V, max_gamma, tt, td;
  int64_t esz;
  int chunks1;
  int chunks3, chunk3_elems;
  int64_t nsub;
  bool fused_draw;  // k3_accept_mass_draw instead of k3_accept_mass + k4_draw
  size_t off_toff, off_doff, off_tk, off_dk, off_tparts, off_dparts, off_sel, off_sub;
  size_t off_ttok;  // draft-token index per target row (the plan launch's table)
  size_t bytes;
  // per-position diagnostics (after the verify layout)
  size_t off_dseq, off_bar, off_dgparts, off_topz, off_topi;
  size_t diag_bytes;
};

bool shape_ok(const specv_shape_t* s) {
  if (!s) return false;
  if (s->batch < 0 || s->vocab < 1 || s->max_gamma < 0 || s->max_gamma > SPECV_MAX_GAMMA) return false;
  if (!dtype_ok(s->dtype)) return false;
  if (s->total_draft_rows < 0 || s->total_target_rows < 0) return false;
  // draft rows bounded first (B * max_gamma < 2^37), so the sum cannot overflow
  if (s->total_draft_rows > (int64_t)s->batch * s->max_gamma) return false;
  if (s->total_target_rows != s->total_draft_rows + s->batch) return false;
  // packed element offsets must fit int64 comfortably
  if (s->total_target_rows > ((int64_t)1 << 40) / s->vocab) return false;
  // every launch grid stays below 2^31 workgroups (at most 2^30 rows of both
  // kinds, a few chunks each; many chunks only where V, and so 2^40 / V, bound
  // the rows)
  if (s->total_target_rows > ((int64_t)1 << 29)) return false;
  return true;
}

void make_plan(const specv_shape_t* s, Plan* p) {
  p->dt = (s->dtype == SPECV_BF16) ? kBF16 : kF32;
  p->B = s->batch;
  p->V = s->vocab;
  p->max_gamma = s->max_gamma;
  p->tt = s->total_target_rows;
  p->td = s->total_draft_rows;
  p->esz = (p->dt == kBF16) ? 2 : 4;
  // pass 1: about kK1Chunk* elements per (row, chunk) work item, but two
  // chunks at least once a row is longer than 2048 elements (two waves on
  // a row read it faster than one), and at most 16 (the accept step merges
  // them). A chunk is every C-th tile of its row and a tile holds at most
  // 2048 elements, so C never exceeds the row's tile count.
  const int64_t per = (p->dt == kBF16) ? kK1ChunkBF16 : kK1ChunkF32;
  int64_t c1 = (p->V + per - 1) / per;
  if (c1 < 2 && p->V > SPECV_K1_TWO_CHUNKS_ABOVE) c1 = 2;
  // a batch too small to fill the part (a few sequences) gets more, shorter
  // chunks: at least kMinPass1Waves waves while a row has tiles to give
  const int64_t rows = p->tt + p->td;
  if (rows > 0 && rows * c1 < kMinPass1Waves) {
    const int64_t want = (kMinPass1Waves + rows - 1) / rows;
    const int64_t tiles = (p->V + 2047) / 2048;  // the fewest tiles of any path's tiling
    int64_t cap = tiles < SPECV_MIN_WAVES_CHUNK_CAP ? tiles : SPECV_MIN_WAVES_CHUNK_CAP;
    cap = cap > c1 ? cap : c1;
    c1 = want < cap ? want : cap;
  }
  c1 = c1 < 1 ? 1 : (c1 > kMaxChunks1 ? kMaxChunks1 : c1);
  p->chunks1 = (int)c1;
  // pass 2: enough chunks per sequence to give about kTargetMassItems waves.
  // Where that needs more than the 16 waves one workgroup holds (so the draw
  // takes a launch of its own), a split with about kMassStepsPerWave draw
  // steps per wave that fits one workgroup is taken instead if it still gives
  // kFusedMinWaves waves in all; else fewer, longer unfused chunks (about
  // kTargetUnfusedItems waves). Swept on this part per workload.
  const int64_t Bp = p->B > 0 ? p->B : 1;
  const int64_t max_c3 = (p->V + kDrawStep - 1) / kDrawStep;
  auto chunks_for = [&](int64_t c3, int64_t* elems) {
    c3 = c3 < 1 ? 1 : (c3 > max_c3 ? max_c3 : c3);
    int64_t ch3 = (p->V + c3 - 1) / c3;
    ch3 = (ch3 + kDrawStep - 1) / kDrawStep * kDrawStep;
    *elems = ch3;
    return (p->V + ch3 - 1) / ch3;
  };
  int64_t ch3;
  int64_t c3 = chunks_for((kTargetMassItems + Bp - 1) / Bp, &ch3);
  if (c3 * kWave > 1024) {
    int64_t chf;
    const int64_t cf = chunks_for((max_c3 + kMassStepsPerWave - 1) / kMassStepsPerWave, &chf);
    if (cf * kWave <= 1024 && Bp * cf >= kFusedMinWaves) {
      c3 = cf;
      ch3 = chf;
    } else {
      c3 = chunks_for((kTargetUnfusedItems + Bp - 1) / Bp, &ch3);
    }
  }
  p->chunk3_elems = (int)ch3;
  p->chunks3 = (int)c3;
  size_t off = kAlign;  // [0, 256): status word
  p->off_toff = off; off = align_up(off + (size_t)(p->B + 1) * 8);
  p->off_doff = off; off = align_up(off + (size_t)(p->B + 1) * 8);
  p->off_tk = off; off = align_up(off + (size_t)p->tt * 4);
  p->off_dk = off; off = align_up(off + (size_t)p->td * 4);
  p->off_tparts = off; off = align_up(off + (size_t)p->tt * p->chunks1 * sizeof(RowPart));
  p->off_dparts = off; off = align_up(off + (size_t)p->td * p->chunks1 * sizeof(RowPart));
  p->off_sel = off; off = align_up(off + (size_t)p->B * sizeof(Select));
  p->nsub = (p->V + kSub - 1) / kSub;
  p->fused_draw = SPECV_FUSED_DRAW && p->chunks3 * kWave <= 1024 &&
                  (size_t)p->nsub * sizeof(double) <= kFusedDrawLds;
  p->off_sub = off; off = align_up(off + (size_t)p->B * p->nsub * sizeof(double));
  p->off_ttok = off; off = align_up(off + (size_t)p->tt * 4);
  p->bytes = off;
}

// Workspace of specv_position_diagnostics with top-k lists of K entries.
void make_diag_plan(Plan* p, int K) {
  size_t off = p->bytes;
  const size_t items = (size_t)p->td * p->chunks1;
  p->off_dseq = off; off = align_up(off + (size_t)p->td * 4);
  p->off_bar = off; off = align_up(off + items * 4);
  p->off_dgparts = off; off = align_up(off + items * sizeof(DiagPart));
  p->off_topz = off; off = align_up(off + items * K * 4);
  p->off_topi = off; off = align_up(off + items * K * 4);
  p->diag_bytes = off;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

struct Call {
  const specv_shape_t* shape;
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const int32_t* gamma;
  const float* temperature;
  uint64_t seed, row_offset;
  const float* inj_r;
  const float* inj_u;
  int32_t* out_n;
  int32_t* out_next;
  void* ws;
  size_t ws_bytes;
  hipStream_t stream;
  hipEvent_t* events;
  int32_t lenience = kLenNone;
  float eps = 1.f;
  // Pass 1 already done (uniform batch only): the pass-1 partials and the
  // status word are in the workspace, written by a producer of the rows
  // (k_dec_gather_stats), so the call starts at the accept step.
  bool skip_pass1 = false;
};

specv_status_t check_common(const specv_shape_t* shape, const void* target, const void* draft,
                            const int32_t* gamma, const float* temperature, void* ws,
                            size_t ws_bytes, Plan* p) {
  if (!shape_ok(shape)) return SPECV_ERR_INVALID_ARGUMENT;
  make_plan(shape, p);
  if (p->B == 0) return SPECV_OK;
  if (!gamma || !temperature) return SPECV_ERR_INVALID_ARGUMENT;
  if (!target) return SPECV_ERR_INVALID_ARGUMENT;
  if (p->td > 0 && !draft) return SPECV_ERR_INVALID_ARGUMENT;
  if (!aligned(target, (size_t)p->esz) || (draft && !aligned(draft, (size_t)p->esz)))
    return SPECV_ERR_INVALID_ARGUMENT;
  if (!ws || ws_bytes < p->bytes || !aligned(ws, kAlign)) return SPECV_ERR_WORKSPACE;
  return SPECV_OK;
}

bool vector_path(const Plan& p, const void* target, const void* draft) {
  return (p.V * p.esz) % 16 == 0 && aligned(target, 16) && (!draft || aligned(draft, 16));
}

inline specv_status_t launched() {
  return hipGetLastError() == hipSuccess ? SPECV_OK : SPECV_ERR_HIP;
}

inline void mark(hipEvent_t* ev, int idx, hipStream_t s) {
  if (ev && ev[idx]) (void)hipEventRecord(ev[idx], s);
}

// Workgroups for `waves` waves. The shape checks keep every grid far below
// 2^31 workgroups; a count past that gives 0, which the launch rejects,
// rather than a truncated grid.
inline unsigned blocks_for(int64_t waves) {
  const int64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
  return blocks > 0x7fffffff ? 0u : (unsigned)blocks;
}

// A batch is uniform when its row totals equal B * (max_gamma + 1): with
// every gamma_b <= max_gamma (checked on the device) all equal max_gamma.
bool uniform_batch(const Plan& p) { return p.B > 0 && p.tt == p.B * (p.max_gamma + 1); }

specv_status_t launch_plan(const Plan& p, const int32_t* gamma, const float* temperature, void* ws,
                           hipStream_t st, int32_t* dseq = nullptr, int32_t* ttok = nullptr) {
  PlanArgs a;
  a.gamma = gamma;
  a.temperature = temperature;
  a.toff = at<int64_t>(ws, p.off_toff);
  a.doff = at<int64_t>(ws, p.off_doff);
  a.tk = at<float>(ws, p.off_tk);
  a.dk = at<float>(ws, p.off_dk);
  a.dseq = dseq;
  a.ttok = ttok;
  a.status = at<uint32_t>(ws, 0);
  a.total_t = p.tt;
  a.total_d = p.td;
  a.B = (int32_t)p.B;
  a.max_gamma = (int32_t)p.max_gamma;
  hipLaunchKernelGGL(k0_plan, dim3(1), dim3(1024), 0, st, a);
  return launched();
}

specv_status_t launch_row_stats(const Plan& p, bool vec, const void* target, const void* draft,
                                void* ws, hipStream_t st, bool with_argmax = false,
                                bool all_drafts = false, int bar_k = 0, float* bar = nullptr,
                                const float* temperature = nullptr, bool uniform = false,
                                const int32_t* plan_gamma = nullptr, bool inline_plan = false,
                                const int32_t* tokens = nullptr) {
  RowStatsArgs a;
  a.target = target;
  a.draft = draft;
  a.tk = at<float>(ws, p.off_tk);
  a.dk = at<float>(ws, p.off_dk);
  a.tparts = at<RowPart>(ws, p.off_tparts);
  a.dparts = at<RowPart>(ws, p.off_dparts);
  a.status = at<uint32_t>(ws, 0);
  a.total_t = p.tt;
  a.total_d = p.td;
  a.V = p.V;
  a.B = (int32_t)p.B;
  a.chunks = p.chunks1;
  a.all_drafts = all_drafts ? 1 : 0;
  a.bar_k = bar_k;
  a.bar = bar;
  a.uniform_g = uniform ? (int32_t)p.max_gamma : -1;
  a.temperature = temperature;
  a.gamma = (uniform || inline_plan) ? plan_gamma : nullptr;
  a.status_out = at<uint32_t>(ws, 0);
  a.inline_plan = inline_plan ? 1 : 0;
  a.max_gamma = (int32_t)p.max_gamma;
  a.toff = at<int64_t>(ws, p.off_toff);
  a.doff = at<int64_t>(ws, p.off_doff);
  // tokens given: capture the draft tokens' logits for the accept step
  a.tokens = tokens;
  a.ttok = (tokens && !uniform && !inline_plan) ? at<int32_t>(ws, p.off_ttok) : nullptr;
  const int64_t waves = (p.tt + p.td) * p.chunks1;
  if (waves == 0) return SPECV_OK;
  // rows of one tile: several rows per wave, the next one's tile in flight
  const int64_t epi = (p.dt == kBF16) ? Tile<kBF16, true>::EPI : Tile<kF32, true>::EPI;
  if (SPECV_SHORT_ROWS > 0 && vec && p.chunks1 == 1 && p.V <= epi && !with_argmax && !all_drafts &&
      bar_k == 0 && !inline_plan) {
    constexpr int R = SPECV_SHORT_ROWS > 0 ? SPECV_SHORT_ROWS : 2;
    const dim3 grid(blocks_for((p.tt + p.td + R - 1) / R)), block(kBlock);
    if (p.dt == kBF16) hipLaunchKernelGGL((k1_short_rows<kBF16, R>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((k1_short_rows<kF32, R>), grid, block, 0, st, a);
    return launched();
  }
  const dim3 grid(blocks_for(waves)), block(kBlock);
  // specv_verify needs no argmax of sampling rows; the diagnostics export does
  if (with_argmax) {
    if (p.dt == kBF16) {
      if (vec) hipLaunchKernelGGL((k1_row_stats<kBF16, true, true>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((k1_row_stats<kBF16, false, true>), grid, block, 0, st, a);
    } else {
      if (vec) hipLaunchKernelGGL((k1_row_stats<kF32, true, true>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((k1_row_stats<kF32, false, true>), grid, block, 0, st, a);
    }
  } else {
    if (p.dt == kBF16) {
      if (vec) hipLaunchKernelGGL((k1_row_stats<kBF16, true, false>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((k1_row_stats<kBF16, false, false>), grid, block, 0, st, a);
    } else {
      if (vec) hipLaunchKernelGGL((k1_row_stats<kF32, true, false>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((k1_row_stats<kF32, false, false>), grid, block, 0, st, a);
    }
  }
  return launched();
}

// Pass 1 of specv_verify records the draft tokens' logits for the accept
// step (one dependent memory round trip less at its head): the wave whose
// chunk holds a token takes its logit from the tile in its registers, so
// nothing is loaded for it.
bool capture_logits(const Plan& p) { return p.td > 0 && SPECV_CAPTURE; }

// log2 of pass 1's tile length (elements) on the path `vec` picks
int tile_shift(const Plan& p, bool vec) {
  const int epi = (p.dt == kBF16) ? (vec ? Tile<kBF16, true>::EPI : Tile<kBF16, false>::EPI)
                                   : (vec ? Tile<kF32, true>::EPI : Tile<kF32, false>::EPI);
  int sh = 0;
  while ((1 << sh) < epi) ++sh;
  return sh;
}

AcceptArgs accept_args(const Plan& p, const Call& c, bool vec) {
  AcceptArgs a;
  a.target = c.target;
  a.draft = c.draft;
  a.tokens = c.tokens;
  a.gamma = c.gamma;
  a.temperature = c.temperature;
  a.toff = at<int64_t>(c.ws, p.off_toff);
  a.doff = at<int64_t>(c.ws, p.off_doff);
  a.tparts = at<RowPart>(c.ws, p.off_tparts);
  a.dparts = at<RowPart>(c.ws, p.off_dparts);
  a.status = at<uint32_t>(c.ws, 0);
  a.sel = at<Select>(c.ws, p.off_sel);
  a.out_n = c.out_n;
  a.out_next = c.out_next;
  a.inj_r = c.inj_r;
  a.inj_u = c.inj_u;
  a.seed = c.seed;
  a.row_offset = c.row_offset;
  a.V = p.V;
  a.B = (int32_t)p.B;
  a.max_gamma = (int32_t)p.max_gamma;
  a.chunks = p.chunks1;
  a.lenience = c.lenience;
  a.eps = c.eps;
  a.uniform_g = uniform_batch(p) ? (int32_t)p.max_gamma : -1;
  const bool captured = !c.skip_pass1 && capture_logits(p);  // pass 1 of run() recorded them
  a.cap_shift = captured ? tile_shift(p, vec) : 0;
  return a;
}

DrawArgs draw_args(const Plan& p, const Call& c) {
  DrawArgs a;
  a.target = c.target;
  a.draft = c.draft;
  a.sel = at<Select>(c.ws, p.off_sel);
  a.sub = at<double>(c.ws, p.off_sub);
  a.out_next = c.out_next;
  a.V = p.V;
  a.B = (int32_t)p.B;
  a.chunks3 = p.chunks3;
  a.nsub = (int32_t)p.nsub;
  a.weights_in_lds = (p.fused_draw && p.chunks3 == 1 && p.nsub == 1 && SPECV_DRAW_FROM_LDS) ? 1 : 0;
  return a;
}

specv_status_t launch_accept_mass(const Plan& p, bool vec, const Call& c) {
  const AcceptArgs acc = accept_args(p, c, vec);
  const DrawArgs a = draw_args(p, c);
  if (p.fused_draw) {
    // one workgroup per sequence, one wave per pass-2 chunk; masses in LDS
    const dim3 grid((unsigned)p.B), block((unsigned)(p.chunks3 * kWave));
    // one wave and one sub-block: the draw's weights stay in LDS too
    const size_t lds = a.weights_in_lds ? 2 * sizeof(double) + kSub * sizeof(float)
                                        : (size_t)p.nsub * sizeof(double);
    if (p.dt == kBF16) {
      if (vec) hipLaunchKernelGGL((k3_accept_mass_draw<kBF16, true>), grid, block, lds, c.stream, acc, a);
      else hipLaunchKernelGGL((k3_accept_mass_draw<kBF16, false>), grid, block, lds, c.stream, acc, a);
    } else {
      if (vec) hipLaunchKernelGGL((k3_accept_mass_draw<kF32, true>), grid, block, lds, c.stream, acc, a);
      else hipLaunchKernelGGL((k3_accept_mass_draw<kF32, false>), grid, block, lds, c.stream, acc, a);
    }
    return launched();
  }
  const dim3 grid(blocks_for(p.B * p.chunks3)), block(kBlock);
  if (p.dt == kBF16) {
    if (vec) hipLaunchKernelGGL((k3_accept_mass<kBF16, true>), grid, block, 0, c.stream, acc, a);
    else hipLaunchKernelGGL((k3_accept_mass<kBF16, false>), grid, block, 0, c.stream, acc, a);
  } else {
    if (vec) hipLaunchKernelGGL((k3_accept_mass<kF32, true>), grid, block, 0, c.stream, acc, a);
    else hipLaunchKernelGGL((k3_accept_mass<kF32, false>), grid, block, 0, c.stream, acc, a);
  }
  return launched();
}

specv_status_t launch_draw(const Plan& p, bool vec, const Call& c) {
  if (p.fused_draw) return SPECV_OK;  // drawn by k3_accept_mass_draw
  const DrawArgs a = draw_args(p, c);
  const dim3 grid(blocks_for(p.B)), block(kBlock);
  if (p.dt == kBF16) {
    if (vec) hipLaunchKernelGGL((k4_draw<kBF16, true>), grid, block, 0, c.stream, a);
    else hipLaunchKernelGGL((k4_draw<kBF16, false>), grid, block, 0, c.stream, a);
  } else {
    if (vec) hipLaunchKernelGGL((k4_draw<kF32, true>), grid, block, 0, c.stream, a);
    else hipLaunchKernelGGL((k4_draw<kF32, false>), grid, block, 0, c.stream, a);
  }
  return launched();
}

specv_status_t run(const Call& c) {
  Plan p;
  specv_status_t st = check_common(c.shape, c.target, c.draft, c.gamma, c.temperature, c.ws,
                                   c.ws_bytes, &p);
  if (st != SPECV_OK || p.B == 0) return st;
  if (!c.out_n || !c.out_next) return SPECV_ERR_INVALID_ARGUMENT;
  if (p.td > 0 && !c.tokens) return SPECV_ERR_INVALID_ARGUMENT;
  if ((c.inj_r == nullptr) != (c.inj_u == nullptr)) return SPECV_ERR_INVALID_ARGUMENT;
  const bool vec = vector_path(p, c.target, c.draft);
  const bool uniform = uniform_batch(p);
  if (c.skip_pass1 && !uniform) return SPECV_ERR_INVALID_ARGUMENT;
  // A uniform batch has no plan launch: pass 1's first workgroup checks the
  // gammas and sets the status word. Nor has a ragged batch of at most
  // kInlinePlanMax sequences: pass 1's first workgroup writes its offsets and
  // status word, and each pass-1 wave finds its row's sequence itself.
  const bool inline_plan = !uniform && !c.skip_pass1 && SPECV_INLINE_PLAN &&
                           p.B <= kInlinePlanMax;
  mark(c.events, 2 * SPECV_STAGE_PLAN, c.stream);
  if (!uniform && !inline_plan &&
      (st = launch_plan(p, c.gamma, c.temperature, c.ws, c.stream, nullptr,
                        at<int32_t>(c.ws, p.off_ttok))) != SPECV_OK)
    return st;
  mark(c.events, 2 * SPECV_STAGE_PLAN + 1, c.stream);
  mark(c.events, 2 * SPECV_STAGE_ROWSTATS, c.stream);
  if (!c.skip_pass1 &&
      (st = launch_row_stats(p, vec, c.target, c.draft, c.ws, c.stream, false, false, 0, nullptr,
                             c.temperature, uniform, c.gamma, inline_plan,
                             capture_logits(p) ? c.tokens : nullptr)) != SPECV_OK)
    return st;
  mark(c.events, 2 * SPECV_STAGE_ROWSTATS + 1, c.stream);
  mark(c.events, 2 * SPECV_STAGE_ACCEPT_MASS, c.stream);
  if ((st = launch_accept_mass(p, vec, c)) != SPECV_OK) return st;
  mark(c.events, 2 * SPECV_STAGE_ACCEPT_MASS + 1, c.stream);
  mark(c.events, 2 * SPECV_STAGE_DRAW, c.stream);
  if ((st = launch_draw(p, vec, c)) != SPECV_OK) return st;
  mark(c.events, 2 * SPECV_STAGE_DRAW + 1, c.stream);
  return SPECV_OK;
}

struct DecodePlan {
  specv_shape_t vshape;  // the verify step's shape for one round
  Plan vp;
  int64_t esz, row_bytes, cap;
  size_t off_tpack, off_dpack, off_drafts, off_tsrc, off_dsrc, off_gam, off_cur, off_len, off_fail,
      off_vn, off_vnext;
  size_t bytes;
};

bool decode_shape_ok(const specv_decode_shape_t* s) {
  if (!s) return false;
  if (s->batch < 0 || s->vocab < 1 || s->gamma < 0 || s->gamma > SPECV_MAX_GAMMA || s->rounds < 0)
    return false;
  if (!dtype_ok(s->dtype)) return false;
  // the [V, V] tables and the token buffer must be addressable
  if ((int64_t)s->vocab * s->vocab > ((int64_t)1 << 40)) return false;
  if ((int64_t)s->batch * s->rounds > ((int64_t)1 << 40) / (s->gamma + 1)) return false;  // no overflow
  return true;
}

bool make_decode_plan(const specv_decode_shape_t* s, DecodePlan* d) {
  d->vshape.batch = s->batch;
  d->vshape.vocab = s->vocab;
  d->vshape.max_gamma = s->gamma;
  d->vshape.dtype = s->dtype;
  d->vshape.total_target_rows = (int64_t)s->batch * (s->gamma + 1);
  d->vshape.total_draft_rows = (int64_t)s->batch * s->gamma;
  if (!shape_ok(&d->vshape)) return false;
  make_plan(&d->vshape, &d->vp);
  d->esz = (s->dtype == SPECV_BF16) ? 2 : 4;
  d->row_bytes = (int64_t)s->vocab * d->esz;
  d->cap = (int64_t)s->rounds * (s->gamma + 1);
  const int64_t B = s->batch, g = s->gamma;
  size_t off = d->vp.bytes;
  d->off_tpack = off; off = align_up(off + (size_t)(B * (g + 1)) * d->row_bytes);
  d->off_dpack = off; off = align_up(off + (size_t)(B * g) * d->row_bytes);
  d->off_drafts = off; off = align_up(off + (size_t)(B * g) * 4);
  d->off_tsrc = off; off = align_up(off + (size_t)(B * (g + 1)) * 4);
  d->off_dsrc = off; off = align_up(off + (size_t)(B * g) * 4);
  d->off_gam = off; off = align_up(off + (size_t)B * 4);
  d->off_cur = off; off = align_up(off + (size_t)B * 4);
  d->off_len = off; off = align_up(off + (size_t)B * 4);
  d->off_fail = off; off = align_up(off + (size_t)B * 4);
  d->off_vn = off; off = align_up(off + (size_t)B * 4);
  d->off_vnext = off; off = align_up(off + (size_t)B * 4);
  d->bytes = off;
  return true;
}

__global__ __launch_bounds__(kBlock) void k_fill_i32(int32_t* p, int64_t n, int32_t value) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < n) p[t] = value;
}

struct CascadePlan {
  specv_shape_t vin, vout;  // inner (m1 vs m2) and target review shapes
  Plan pin, pout;
  int64_t esz, row_bytes, cap, dcap;
  size_t vbytes;  // verify workspace shared by both reviews (stream-ordered)
  size_t off_itp, off_idp, off_otp, off_odp, off_itok, off_ipr, off_iprd, off_igam, off_ogam,
      off_otok, off_cur, off_icur, off_fail, off_len, off_dlen, off_dtok, off_dprev, off_dbonus,
      off_vn, off_vnext;
  size_t bytes;
};

bool cascade_shape_ok(const specv_cascade_shape_t* s) {
  if (!s) return false;
  if (s->batch < 0 || s->vocab < 1 || s->rounds < 0) return false;
  if (s->k1 < 0 || s->k1 > SPECV_MAX_GAMMA || s->k2 < 0 || s->k2 > SPECV_MAX_GAMMA) return false;
  if (!dtype_ok(s->dtype)) return false;
  if ((int64_t)s->vocab * s->vocab > ((int64_t)1 << 40)) return false;
  if ((int64_t)s->batch * s->rounds > ((int64_t)1 << 40) / (s->k1 + 1)) return false;  // no overflow
  return true;
}

bool make_cascade_plan(const specv_cascade_shape_t* s, CascadePlan* c) {
  const int64_t B = s->batch, k1 = s->k1, k2 = s->k2;
  c->vin = specv_shape_t{s->batch, s->vocab, s->k2, s->dtype, B * (k2 + 1), B * k2};
  c->vout = specv_shape_t{s->batch, s->vocab, s->k1, SPECV_F32, B * (k1 + 1), B * k1};
  if (!shape_ok(&c->vin) || !shape_ok(&c->vout)) return false;
  make_plan(&c->vin, &c->pin);
  make_plan(&c->vout, &c->pout);
  c->esz = (s->dtype == SPECV_BF16) ? 2 : 4;
  c->row_bytes = (int64_t)s->vocab * c->esz;
  c->cap = (int64_t)s->rounds * (k1 + 1);
  c->dcap = k1 + k2 + 1;
  const int64_t V = s->vocab;
  size_t off = align_up(c->pin.bytes > c->pout.bytes ? c->pin.bytes : c->pout.bytes);
  c->vbytes = off;
  c->off_itp = off; off = align_up(off + (size_t)(B * (k2 + 1)) * c->row_bytes);
  c->off_idp = off; off = align_up(off + (size_t)(B * k2) * c->row_bytes);
  c->off_otp = off; off = align_up(off + (size_t)(B * (k1 + 1) * V) * 4);
  c->off_odp = off; off = align_up(off + (size_t)(B * k1 * V) * 4);
  c->off_itok = off; off = align_up(off + (size_t)(B * k2) * 4);
  c->off_ipr = off; off = align_up(off + (size_t)(B * (k2 + 1)) * 4);
  c->off_iprd = off; off = align_up(off + (size_t)(B * k2) * 4);
  c->off_igam = off; off = align_up(off + (size_t)B * 4);
  c->off_ogam = off; off = align_up(off + (size_t)B * 4);
  c->off_otok = off; off = align_up(off + (size_t)(B * k1) * 4);
  c->off_cur = off; off = align_up(off + (size_t)B * 4);
  c->off_icur = off; off = align_up(off + (size_t)B * 4);
  c->off_fail = off; off = align_up(off + (size_t)B * 4);
  c->off_len = off; off = align_up(off + (size_t)B * 4);
  c->off_dlen = off; off = align_up(off + (size_t)B * 4);
  c->off_dtok = off; off = align_up(off + (size_t)(B * c->dcap) * 4);
  c->off_dprev = off; off = align_up(off + (size_t)(B * c->dcap) * 4);
  c->off_dbonus = off; off = align_up(off + (size_t)(B * c->dcap) * 4);
  c->off_vn = off; off = align_up(off + (size_t)B * 4);
  c->off_vnext = off; off = align_up(off + (size_t)B * 4);
  c->bytes = off;
  return true;
}

// The workgroup row builder is instantiated per lenience kind.
template <int DT, bool VEC>
void launch_cas_rows_wg(dim3 g, dim3 wg, hipStream_t stream, const CascadeArgs& ca) {
  switch (ca.lenience) {
    case kLenLin: hipLaunchKernelGGL((k_cas_outer_rows_wg<DT, VEC, kLenLin>), g, wg, 0, stream, ca); break;
    case kLenSq: hipLaunchKernelGGL((k_cas_outer_rows_wg<DT, VEC, kLenSq>), g, wg, 0, stream, ca); break;
    case kLenExp: hipLaunchKernelGGL((k_cas_outer_rows_wg<DT, VEC, kLenExp>), g, wg, 0, stream, ca); break;
    default: hipLaunchKernelGGL((k_cas_outer_rows_wg<DT, VEC, kLenNone>), g, wg, 0, stream, ca); break;
  }
}

// The static scratch of specv_verify_noalloc: one array per GPU, held until
// the process ends. Host code never uses the array's name as an address; the
// device address comes from hipGetSymbolAddress, looked up once per device
// with that device current.
__device__ __align__(256) unsigned char scratch[SPECV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_address[kMaxDevices] = {};

specv_status_t scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SPECV_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_address[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SPECV_ERR_HIP;
    g_scratch_address[dev] = p;
  }
  *out = g_scratch_address[dev];
  return SPECV_OK;
}

// The status word of a no-allocation call, copied to the caller's output
// (0 when the batch was empty and nothing ran).
__global__ void k_copy_status(const uint32_t* status, uint32_t* out) {
  if (threadIdx.x == 0) out[0] = status ? status[0] : 0u;
}

}  // namespace

extern "C" {

size_t specv_workspace_bytes(const specv_shape_t* shape) {
  if (!shape_ok(shape)) return 0;
  Plan p;
  make_plan(shape, &p);
  return p.bytes;
}

specv_status_t specv_verify(const specv_shape_t* shape, const void* target_logits,
                            const void* draft_logits, const int32_t* draft_tokens,
                            const int32_t* gamma_per_row, const float* temperature,
                            uint64_t seed, uint64_t philox_row_offset,
                            int32_t* out_n_accepted, int32_t* out_next_token,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Call c{shape, target_logits, draft_logits, draft_tokens, gamma_per_row, temperature,
         seed, philox_row_offset, nullptr, nullptr, out_n_accepted, out_next_token,
         workspace, workspace_bytes, stream, nullptr};
  return run(c);
}

specv_status_t specv_verify_noalloc(const specv_shape_t* shape, const void* target_logits,
                                    const void* draft_logits, const int32_t* draft_tokens,
                                    const int32_t* gamma_per_row, const float* temperature,
                                    uint64_t seed, uint64_t philox_row_offset,
                                    int32_t* out_n_accepted, int32_t* out_next_token,
                                    uint32_t* out_status, hipStream_t stream) {
  if (!shape_ok(shape)) return SPECV_ERR_INVALID_ARGUMENT;
  Plan p;
  make_plan(shape, &p);
  if (p.bytes > (size_t)SPECV_NOALLOC_SCRATCH_BYTES) return SPECV_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  specv_status_t st = SPECV_OK;
  if (p.B > 0 && (st = scratch_address(&ws)) != SPECV_OK) return st;
  Call c{shape, target_logits, draft_logits, draft_tokens, gamma_per_row, temperature,
         seed, philox_row_offset, nullptr, nullptr, out_n_accepted, out_next_token,
         ws, (size_t)SPECV_NOALLOC_SCRATCH_BYTES, stream, nullptr};
  if ((st = run(c)) != SPECV_OK) return st;
  if (out_status) {
    hipLaunchKernelGGL(k_copy_status, dim3(1), dim3(64), 0, stream,
                       p.B > 0 ? static_cast<const uint32_t*>(ws) : nullptr, out_status);
    return launched();
  }
  return SPECV_OK;
}

specv_status_t specv_verify_profiled(const specv_shape_t* shape, const void* target_logits,
                                     const void* draft_logits, const int32_t* draft_tokens,
                                     const int32_t* gamma_per_row, const float* temperature,
                                     uint64_t seed, uint64_t philox_row_offset,
                                     int32_t* out_n_accepted, int32_t* out_next_token,
                                     void* workspace, size_t workspace_bytes,
                                     hipStream_t stream, hipEvent_t* events) {
  Call c{shape, target_logits, draft_logits, draft_tokens, gamma_per_row, temperature,
         seed, philox_row_offset, nullptr, nullptr, out_n_accepted, out_next_token,
         workspace, workspace_bytes, stream, events};
  return run(c);
}

specv_status_t specv_verify_with_uniforms(const specv_shape_t* shape, const void* target_logits,
                                          const void* draft_logits, const int32_t* draft_tokens,
                                          const int32_t* gamma_per_row, const float* temperature,
                                          const float* r, const float* u,
                                          int32_t* out_n_accepted, int32_t* out_next_token,
                                          void* workspace, size_t workspace_bytes,
                                          hipStream_t stream) {
  if (!u || (!r && shape && shape->max_gamma > 0 && shape->batch > 0))
    return SPECV_ERR_INVALID_ARGUMENT;
  // with max_gamma == 0 there are no r entries; any non-null pointer will do
  Call c{shape, target_logits, draft_logits, draft_tokens, gamma_per_row, temperature,
         0, 0, r ? r : u, u, out_n_accepted, out_next_token,
         workspace, workspace_bytes, stream, nullptr};
  return run(c);
}

specv_status_t specv_verify_lenient(const specv_shape_t* shape, const void* target_logits,
                                    const void* draft_logits, const int32_t* draft_tokens,
                                    const int32_t* gamma_per_row, const float* temperature,
                                    specv_lenience_t lenience, float epsilon, uint64_t seed,
                                    uint64_t philox_row_offset, const float* r, const float* u,
                                    int32_t* out_n_accepted, int32_t* out_next_token,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream,
                                    hipEvent_t* events) {
  if (!lenience_ok(lenience, epsilon)) return SPECV_ERR_INVALID_ARGUMENT;
  const bool need_r = shape && shape->max_gamma > 0 && shape->batch > 0;
  if (u ? (need_r && !r) : (r != nullptr)) return SPECV_ERR_INVALID_ARGUMENT;
  Call c{shape, target_logits, draft_logits, draft_tokens, gamma_per_row, temperature,
         seed, philox_row_offset, u ? (r ? r : u) : nullptr, u, out_n_accepted, out_next_token,
         workspace, workspace_bytes, stream, events};
  // f(p, 1) = p for every lenience function: eps = 1 is the lossless step
  c.lenience = (epsilon == 1.f) ? kLenNone : (int32_t)lenience;
  c.eps = epsilon;
  return run(c);
}

size_t specv_diagnostics_workspace_bytes(const specv_shape_t* shape, int32_t top_k) {
  if (!shape_ok(shape) || top_k < 0 || top_k > kMaxTopK || top_k > shape->vocab) return 0;
  Plan p;
  make_plan(shape, &p);
  make_diag_plan(&p, top_k);
  return p.diag_bytes;
}

specv_status_t specv_position_diagnostics(const specv_shape_t* shape, const void* target_logits,
                                          const void* draft_logits, const int32_t* gamma_per_row,
                                          const float* temperature, int32_t top_k,
                                          double* out_alpha, double* out_entropy,
                                          int32_t* out_topk_index, double* out_topk_prob,
                                          void* workspace, size_t workspace_bytes,
                                          hipStream_t stream, hipEvent_t* events) {
  if (top_k < 0 || top_k > kMaxTopK || (shape && top_k > shape->vocab))
    return SPECV_ERR_INVALID_ARGUMENT;
  Plan p;
  specv_status_t st = check_common(shape, target_logits, draft_logits, gamma_per_row, temperature,
                                   workspace, workspace_bytes, &p);
  if (st != SPECV_OK || p.B == 0) return st;
  make_diag_plan(&p, top_k);
  if (workspace_bytes < p.diag_bytes) return SPECV_ERR_WORKSPACE;
  if (p.td > 0 && (!out_alpha || !out_entropy)) return SPECV_ERR_INVALID_ARGUMENT;
  if (p.td > 0 && top_k > 0 && (!out_topk_index || !out_topk_prob))
    return SPECV_ERR_INVALID_ARGUMENT;
  const bool vec = vector_path(p, target_logits, draft_logits);
  int32_t* dseq = at<int32_t>(workspace, p.off_dseq);
  // A uniform batch with draft rows has no plan launch: pass 1 checks the
  // gammas and sets the status word, and the row -> sequence map is j / gamma.
  const bool uniform = uniform_batch(p) && p.td > 0;
  mark(events, 2 * SPECV_STAGE_PLAN, stream);
  if (!uniform &&
      (st = launch_plan(p, gamma_per_row, temperature, workspace, stream, dseq)) != SPECV_OK)
    return st;
  mark(events, 2 * SPECV_STAGE_PLAN + 1, stream);
  mark(events, 2 * SPECV_STAGE_ROWSTATS, stream);
  float* bar = at<float>(workspace, p.off_bar);
  if (p.td > 0 && (st = launch_row_stats(p, vec, target_logits, draft_logits, workspace, stream,
                                         false, true, top_k, bar, temperature, uniform,
                                         gamma_per_row)) != SPECV_OK)
    return st;
  mark(events, 2 * SPECV_STAGE_ROWSTATS + 1, stream);
  DiagArgs a;
  a.target = target_logits;
  a.draft = draft_logits;
  a.dk = at<float>(workspace, p.off_dk);
  a.dseq = dseq;
  a.bar = bar;
  a.tparts = at<RowPart>(workspace, p.off_tparts);
  a.dparts = at<RowPart>(workspace, p.off_dparts);
  a.status = at<uint32_t>(workspace, 0);
  a.parts = at<DiagPart>(workspace, p.off_dgparts);
  a.topz = at<float>(workspace, p.off_topz);
  a.topi = at<int32_t>(workspace, p.off_topi);
  a.out_alpha = out_alpha;
  a.out_entropy = out_entropy;
  a.out_index = out_topk_index;
  a.out_prob = out_topk_prob;
  a.total_d = p.td;
  a.V = p.V;
  a.chunks = p.chunks1;
  a.K = top_k;
  a.uniform_g = uniform ? (int32_t)p.max_gamma : -1;
  a.temperature = temperature;
  const dim3 grid(blocks_for(p.td * p.chunks1)), block(kBlock);
  mark(events, 2 * SPECV_STAGE_ACCEPT_MASS, stream);
  // with 1, 2 or 4 chunks per position a workgroup holds whole positions, and
  // for lists of at most 64 keys in all the merge runs in the pass-2 launch
  // (its event pair then times nothing); longer lists rank faster in a launch
  // of their own
  const bool fused_merge = kWavesPerBlock % p.chunks1 == 0 && p.chunks1 * top_k <= kWave;
  if (p.td == 0) {
    // nothing to compute
  } else if (fused_merge) {
    if (p.dt == kBF16) {
      if (vec) hipLaunchKernelGGL((k5_diag_pass_merge<kBF16, true, 1>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((k5_diag_pass_merge<kBF16, false, 1>), grid, block, 0, stream, a);
    } else {
      if (vec) hipLaunchKernelGGL((k5_diag_pass_merge<kF32, true, 1>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((k5_diag_pass_merge<kF32, false, 1>), grid, block, 0, stream, a);
    }
  } else if (p.dt == kBF16) {
    if (vec) hipLaunchKernelGGL((k5_diag_pass<kBF16, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((k5_diag_pass<kBF16, false>), grid, block, 0, stream, a);
  } else {
    if (vec) hipLaunchKernelGGL((k5_diag_pass<kF32, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((k5_diag_pass<kF32, false>), grid, block, 0, stream, a);
  }
  if ((st = launched()) != SPECV_OK) return st;
  mark(events, 2 * SPECV_STAGE_ACCEPT_MASS + 1, stream);
  mark(events, 2 * SPECV_STAGE_DRAW, stream);
  const size_t merge_lds = (size_t)kWavesPerBlock * ((p.chunks1 * top_k + 7) / 8 * 8) * 8;
  if (p.td > 0 && !fused_merge) {
    // 64-key slots per lane for the union of the chunk lists
    const int n = p.chunks1 * top_k, ns = (n + kWave - 1) / kWave;
    const dim3 mg(blocks_for(p.td));
    if (ns <= 1) hipLaunchKernelGGL(k6_diag_merge<1>, mg, block, merge_lds, stream, a);
    else if (ns <= 2) hipLaunchKernelGGL(k6_diag_merge<2>, mg, block, merge_lds, stream, a);
    else if (ns <= 4) hipLaunchKernelGGL(k6_diag_merge<4>, mg, block, merge_lds, stream, a);
    else if (ns <= 8) hipLaunchKernelGGL(k6_diag_merge<8>, mg, block, merge_lds, stream, a);
    else hipLaunchKernelGGL(k6_diag_merge<16>, mg, block, merge_lds, stream, a);
  }
  if ((st = launched()) != SPECV_OK) return st;
  mark(events, 2 * SPECV_STAGE_DRAW + 1, stream);
  return SPECV_OK;
}

// The gather of one round with the verify step's pass 1 folded in: the
// partials go to the verify workspace `vws` laid out by plan `vp`.
specv_status_t launch_gather_stats(bool bf16, bool vec, const GatherArgs& ga, const Plan& vp,
                                   void* vws, const float* temperature, const int32_t* gam,
                                   hipStream_t stream) {
  RowStatsArgs a{};
  a.tparts = at<RowPart>(vws, vp.off_tparts);
  a.dparts = at<RowPart>(vws, vp.off_dparts);
  a.status = at<uint32_t>(vws, 0);
  a.total_t = vp.tt;
  a.total_d = vp.td;
  a.V = vp.V;
  a.B = (int32_t)vp.B;
  a.chunks = vp.chunks1;
  a.uniform_g = (int32_t)vp.max_gamma;
  a.temperature = temperature;
  a.gamma = gam;
  a.status_out = at<uint32_t>(vws, 0);
  const int64_t waves = (vp.tt + vp.td) * vp.chunks1;
  if (waves == 0) return SPECV_OK;
  const dim3 grid(blocks_for(waves)), block(kBlock);
  if (bf16) {
    if (vec) hipLaunchKernelGGL((k_dec_gather_stats<kBF16, true>), grid, block, 0, stream, ga, a);
    else hipLaunchKernelGGL((k_dec_gather_stats<kBF16, false>), grid, block, 0, stream, ga, a);
  } else {
    if (vec) hipLaunchKernelGGL((k_dec_gather_stats<kF32, true>), grid, block, 0, stream, ga, a);
    else hipLaunchKernelGGL((k_dec_gather_stats<kF32, false>), grid, block, 0, stream, ga, a);
  }
  return launched();
}

// Drafting of one round: a workgroup per sequence when its rows fit the
// workgroup's registers (V <= 8192), else one wave per sequence streaming the row.
specv_status_t launch_draft(bool bf16, bool vec, const DecodeArgs& a, int64_t B, hipStream_t stream) {
  const dim3 block(kBlock);
  if (a.V <= kDecResident) {
    const dim3 g((unsigned)B), wg(kDecWaves * kWave);
    if (bf16) {
      if (vec) hipLaunchKernelGGL((k_dec_draft_wg<kBF16, true>), g, wg, 0, stream, a);
      else hipLaunchKernelGGL((k_dec_draft_wg<kBF16, false>), g, wg, 0, stream, a);
    } else {
      if (vec) hipLaunchKernelGGL((k_dec_draft_wg<kF32, true>), g, wg, 0, stream, a);
      else hipLaunchKernelGGL((k_dec_draft_wg<kF32, false>), g, wg, 0, stream, a);
    }
  } else if (bf16) {
    if (vec) hipLaunchKernelGGL((k_dec_draft<kBF16, true>), dim3(blocks_for(B)), block, 0, stream, a);
    else hipLaunchKernelGGL((k_dec_draft<kBF16, false>), dim3(blocks_for(B)), block, 0, stream, a);
  } else {
    if (vec) hipLaunchKernelGGL((k_dec_draft<kF32, true>), dim3(blocks_for(B)), block, 0, stream, a);
    else hipLaunchKernelGGL((k_dec_draft<kF32, false>), dim3(blocks_for(B)), block, 0, stream, a);
  }
  return launched();
}

size_t specv_decode_workspace_bytes(const specv_decode_shape_t* shape) {
  if (!decode_shape_ok(shape)) return 0;
  DecodePlan d;
  if (!make_decode_plan(shape, &d)) return 0;
  return d.bytes;
}

specv_status_t specv_decode_bigram(const specv_decode_shape_t* shape, const void* target_table,
                                   const void* draft_table, const float* temperature,
                                   const int32_t* start_token, uint64_t seed,
                                   uint64_t philox_row_offset, int32_t* out_tokens,
                                   int32_t* out_length, int32_t* out_accepted, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream,
                                   hipEvent_t* events) {
  if (!decode_shape_ok(shape)) return SPECV_ERR_INVALID_ARGUMENT;
  DecodePlan d;
  if (!make_decode_plan(shape, &d)) return SPECV_ERR_INVALID_ARGUMENT;
  const int64_t B = shape->batch, g = shape->gamma, R = shape->rounds;
  if (B == 0) return SPECV_OK;
  if (!target_table || !draft_table || !temperature || !start_token || !out_length)
    return SPECV_ERR_INVALID_ARGUMENT;
  if (R > 0 && (!out_tokens || !out_accepted)) return SPECV_ERR_INVALID_ARGUMENT;
  if (!aligned(target_table, (size_t)d.esz) || !aligned(draft_table, (size_t)d.esz))
    return SPECV_ERR_INVALID_ARGUMENT;
  if (!workspace || workspace_bytes < d.bytes || !aligned(workspace, kAlign))
    return SPECV_ERR_WORKSPACE;
  DecodeArgs a;
  a.ttab = target_table;
  a.dtab = draft_table;
  a.temperature = temperature;
  a.start = start_token;
  a.cur = at<int32_t>(workspace, d.off_cur);
  a.drafts = at<int32_t>(workspace, d.off_drafts);
  a.trow_src = at<int32_t>(workspace, d.off_tsrc);
  a.drow_src = at<int32_t>(workspace, d.off_dsrc);
  a.gam = at<int32_t>(workspace, d.off_gam);
  a.len = at<int32_t>(workspace, d.off_len);
  a.fail = at<int32_t>(workspace, d.off_fail);
  a.vn = at<int32_t>(workspace, d.off_vn);
  a.vnext = at<int32_t>(workspace, d.off_vnext);
  a.out_tokens = out_tokens;
  a.out_length = out_length;
  a.out_accepted = out_accepted;
  a.seed = seed;
  a.V = shape->vocab;
  a.cap = d.cap;
  a.B = (int32_t)B;
  a.gamma = (int32_t)g;
  a.rounds = (int32_t)R;
  a.round = 0;
  a.row_base = philox_row_offset;
  const dim3 block(kBlock);
  const unsigned seq_blocks = (unsigned)((B + kBlock - 1) / kBlock);
  hipLaunchKernelGGL(k_dec_init, dim3(seq_blocks < 1024 ? seq_blocks : 1024), block, 0, stream, a);
  specv_status_t st = launched();
  if (st != SPECV_OK) return st;
  GatherArgs ga;
  ga.ttab = target_table;
  ga.dtab = draft_table;
  ga.trow_src = a.trow_src;
  ga.drow_src = a.drow_src;
  ga.tdst = at<char>(workspace, d.off_tpack);
  ga.ddst = at<char>(workspace, d.off_dpack);
  ga.row_bytes = d.row_bytes;
  ga.n_t = B * (g + 1);
  ga.n_d = B * g;
  const bool vec = d.row_bytes % 16 == 0 && aligned(target_table, 16) && aligned(draft_table, 16);
  for (int64_t r = 0; r < R; ++r) {
    a.round = (int32_t)r;
    a.row_base = philox_row_offset + (uint64_t)(r * B);
    const bool last = r + 1 == R;
    hipEvent_t* ev = last ? events : nullptr;
    mark(ev, 2 * SPECV_STAGE_PLAN, stream);
    if ((st = launch_draft(shape->dtype == SPECV_BF16, vec, a, B, stream)) != SPECV_OK) return st;
    mark(ev, 2 * SPECV_STAGE_PLAN + 1, stream);
    mark(ev, 2 * SPECV_STAGE_ROWSTATS, stream);
    if ((st = launch_gather_stats(shape->dtype == SPECV_BF16, vec, ga, d.vp, workspace, temperature,
                                  a.gam, stream)) != SPECV_OK)
      return st;
    mark(ev, 2 * SPECV_STAGE_ROWSTATS + 1, stream);
    mark(ev, 2 * SPECV_STAGE_ACCEPT_MASS, stream);
    Call c{&d.vshape, ga.tdst, ga.ddst, a.drafts, a.gam, temperature, seed, a.row_base, nullptr,
           nullptr, at<int32_t>(workspace, d.off_vn), at<int32_t>(workspace, d.off_vnext),
           workspace, d.vp.bytes, stream, nullptr};
    c.skip_pass1 = true;
    if ((st = run(c)) != SPECV_OK) return st;
    mark(ev, 2 * SPECV_STAGE_ACCEPT_MASS + 1, stream);
    mark(ev, 2 * SPECV_STAGE_DRAW, stream);
    hipLaunchKernelGGL(k_dec_append, dim3(seq_blocks), block, 0, stream, a);
    if ((st = launched()) != SPECV_OK) return st;
    mark(ev, 2 * SPECV_STAGE_DRAW + 1, stream);
  }
  hipLaunchKernelGGL(k_dec_finish, dim3(seq_blocks), block, 0, stream, a);
  return launched();
}

size_t specv_cascade_workspace_bytes(const specv_cascade_shape_t* shape) {
  if (!cascade_shape_ok(shape)) return 0;
  CascadePlan c;
  if (!make_cascade_plan(shape, &c)) return 0;
  return c.bytes;
}

specv_status_t specv_cascade_bigram(const specv_cascade_shape_t* shape, const void* target_table,
                                    const void* mid_table, const void* small_table,
                                    const float* temperature, const int32_t* start_token,
                                    specv_lenience_t lenience, float epsilon, uint64_t seed,
                                    uint64_t philox_row_offset, int32_t* out_tokens,
                                    int32_t* out_length, int32_t* out_accepted, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream,
                                    hipEvent_t* events) {
  if (!cascade_shape_ok(shape)) return SPECV_ERR_INVALID_ARGUMENT;
  if (!lenience_ok(lenience, epsilon)) return SPECV_ERR_INVALID_ARGUMENT;
  CascadePlan c;
  if (!make_cascade_plan(shape, &c)) return SPECV_ERR_INVALID_ARGUMENT;
  const int64_t B = shape->batch, k1 = shape->k1, k2 = shape->k2, R = shape->rounds;
  if (B == 0) return SPECV_OK;
  if (!target_table || !mid_table || !small_table || !temperature || !start_token || !out_length)
    return SPECV_ERR_INVALID_ARGUMENT;
  if (R > 0 && (!out_tokens || !out_accepted)) return SPECV_ERR_INVALID_ARGUMENT;
  if (!aligned(target_table, (size_t)c.esz) || !aligned(mid_table, (size_t)c.esz) ||
      !aligned(small_table, (size_t)c.esz))
    return SPECV_ERR_INVALID_ARGUMENT;
  if (!workspace || workspace_bytes < c.bytes || !aligned(workspace, kAlign))
    return SPECV_ERR_WORKSPACE;
  const bool bf16 = shape->dtype == SPECV_BF16;
  const int32_t len_kind = (lenience == SPECV_LENIENCE_NONE || epsilon == 1.f) ? kLenNone
                                                                                : (int32_t)lenience;
  // target-review side: the decode loop's state and append
  DecodeArgs dd{};
  dd.temperature = temperature;
  dd.start = start_token;
  dd.cur = at<int32_t>(workspace, c.off_cur);
  dd.drafts = at<int32_t>(workspace, c.off_otok);
  dd.gam = at<int32_t>(workspace, c.off_ogam);
  dd.len = at<int32_t>(workspace, c.off_len);
  dd.fail = at<int32_t>(workspace, c.off_fail);
  dd.vn = at<int32_t>(workspace, c.off_vn);
  dd.vnext = at<int32_t>(workspace, c.off_vnext);
  dd.out_tokens = out_tokens;
  dd.out_length = out_length;
  dd.out_accepted = out_accepted;
  dd.seed = seed;
  dd.V = shape->vocab;
  dd.cap = c.cap;
  dd.B = (int32_t)B;
  dd.gamma = (int32_t)k1;
  dd.rounds = (int32_t)R;
  // inner drafting: the decode loop's drafting kernel on the smallest table
  DecodeArgs di = dd;
  di.dtab = small_table;
  di.cur = at<int32_t>(workspace, c.off_icur);
  di.drafts = at<int32_t>(workspace, c.off_itok);
  di.trow_src = at<int32_t>(workspace, c.off_ipr);
  di.drow_src = at<int32_t>(workspace, c.off_iprd);
  di.gamma = (int32_t)k2;
  CascadeArgs ca{};
  ca.ttab = target_table;
  ca.m1tab = mid_table;
  ca.m2tab = small_table;
  ca.temperature = temperature;
  ca.cur = dd.cur;
  ca.icur = di.cur;
  ca.fail = dd.fail;
  ca.dlen = at<int32_t>(workspace, c.off_dlen);
  ca.dtok = at<int32_t>(workspace, c.off_dtok);
  ca.dprev = at<int32_t>(workspace, c.off_dprev);
  ca.dbonus = at<int32_t>(workspace, c.off_dbonus);
  ca.itok = di.drafts;
  ca.ipr = di.trow_src;
  ca.vn = dd.vn;
  ca.vnext = dd.vnext;
  ca.otpack = at<float>(workspace, c.off_otp);
  ca.odpack = at<float>(workspace, c.off_odp);
  ca.otok = dd.drafts;
  ca.lenience = len_kind;
  ca.eps = epsilon;
  ca.V = shape->vocab;
  ca.dcap = c.dcap;
  ca.B = (int32_t)B;
  ca.k1 = (int32_t)k1;
  ca.k2 = (int32_t)k2;
  GatherArgs ga;
  ga.ttab = mid_table;
  ga.dtab = small_table;
  ga.trow_src = di.trow_src;
  ga.drow_src = di.drow_src;
  ga.tdst = at<char>(workspace, c.off_itp);
  ga.ddst = at<char>(workspace, c.off_idp);
  ga.row_bytes = c.row_bytes;
  ga.n_t = B * (k2 + 1);
  ga.n_d = B * k2;
  const bool vec = c.row_bytes % 16 == 0 && aligned(mid_table, 16) && aligned(small_table, 16);
  const dim3 block(kBlock);
  const unsigned seq_blocks = (unsigned)((B + kBlock - 1) / kBlock);
  specv_status_t st;
  hipLaunchKernelGGL(k_dec_init, dim3(seq_blocks < 1024 ? seq_blocks : 1024), block, 0, stream, dd);
  if ((st = launched()) != SPECV_OK) return st;
  hipLaunchKernelGGL(k_fill_i32, dim3(seq_blocks), block, 0, stream,
                     at<int32_t>(workspace, c.off_igam), B, (int32_t)k2);
  if ((st = launched()) != SPECV_OK) return st;
  for (int64_t r = 0; r < R; ++r) {
    hipLaunchKernelGGL(k_cas_round_init, dim3(seq_blocks), block, 0, stream, ca);
    if ((st = launched()) != SPECV_OK) return st;
    const bool last = r + 1 == R;
    for (int64_t j = 0; j < k1; ++j) {
      hipEvent_t* ev = (last && j == 0) ? events : nullptr;  // the last round's first inner round
      di.row_base = philox_row_offset + (uint64_t)((r * (k1 + 1) + 1 + j) * B);
      mark(ev, 2 * SPECV_STAGE_PLAN, stream);
      if ((st = launch_draft(bf16, vec, di, B, stream)) != SPECV_OK) return st;
      mark(ev, 2 * SPECV_STAGE_PLAN + 1, stream);
      mark(ev, 2 * SPECV_STAGE_ROWSTATS, stream);
      if ((st = launch_gather_stats(bf16, vec, ga, c.pin, workspace, temperature,
                                    at<int32_t>(workspace, c.off_igam), stream)) != SPECV_OK)
        return st;
      mark(ev, 2 * SPECV_STAGE_ROWSTATS + 1, stream);
      mark(ev, 2 * SPECV_STAGE_ACCEPT_MASS, stream);
      Call ci{&c.vin, ga.tdst, ga.ddst, di.drafts, at<int32_t>(workspace, c.off_igam), temperature,
              seed, di.row_base, nullptr, nullptr, at<int32_t>(workspace, c.off_vn),
              at<int32_t>(workspace, c.off_vnext), workspace, c.vbytes, stream, nullptr};
      ci.lenience = len_kind;
      ci.eps = epsilon;
      ci.skip_pass1 = true;
      if ((st = run(ci)) != SPECV_OK) return st;
      mark(ev, 2 * SPECV_STAGE_ACCEPT_MASS + 1, stream);
      hipLaunchKernelGGL(k_cas_inner_append, dim3(seq_blocks), block, 0, stream, ca);
      if ((st = launched()) != SPECV_OK) return st;
    }
    hipEvent_t* evo = last ? events : nullptr;
    mark(evo, 2 * SPECV_STAGE_DRAW, stream);
    const int64_t ow = B * (k1 + 1);
    // fp32 review rows are 16-byte aligned when V is a multiple of 4 (table
    // rows: a 16-byte multiple, the same condition as the gather's)
    const bool ovec = vec && shape->vocab % 4 == 0 && aligned(target_table, 16);
    if (shape->vocab <= kCasResident) {
      // a workgroup per (sequence, position): both drafter rows stay in registers
      const dim3 g((unsigned)ow), wg(kCasWaves * kWave);
      if (bf16) {
        if (ovec) launch_cas_rows_wg<kBF16, true>(g, wg, stream, ca);
        else launch_cas_rows_wg<kBF16, false>(g, wg, stream, ca);
      } else {
        if (ovec) launch_cas_rows_wg<kF32, true>(g, wg, stream, ca);
        else launch_cas_rows_wg<kF32, false>(g, wg, stream, ca);
      }
    } else if (bf16) {
      if (ovec) hipLaunchKernelGGL((k_cas_outer_rows<kBF16, true>), dim3(blocks_for(ow)), block, 0, stream, ca);
      else hipLaunchKernelGGL((k_cas_outer_rows<kBF16, false>), dim3(blocks_for(ow)), block, 0, stream, ca);
    } else {
      if (ovec) hipLaunchKernelGGL((k_cas_outer_rows<kF32, true>), dim3(blocks_for(ow)), block, 0, stream, ca);
      else hipLaunchKernelGGL((k_cas_outer_rows<kF32, false>), dim3(blocks_for(ow)), block, 0, stream, ca);
    }
    if ((st = launched()) != SPECV_OK) return st;
    Call co{&c.vout, ca.otpack, ca.odpack, ca.otok, dd.gam, temperature, seed,
            philox_row_offset + (uint64_t)(r * (k1 + 1) * B), nullptr, nullptr,
            at<int32_t>(workspace, c.off_vn), at<int32_t>(workspace, c.off_vnext), workspace,
            c.vbytes, stream, nullptr};
    if ((st = run(co)) != SPECV_OK) return st;
    dd.round = (int32_t)r;
    hipLaunchKernelGGL(k_dec_append, dim3(seq_blocks), block, 0, stream, dd);
    if ((st = launched()) != SPECV_OK) return st;
    mark(evo, 2 * SPECV_STAGE_DRAW + 1, stream);
  }
  hipLaunchKernelGGL(k_dec_finish, dim3(seq_blocks), block, 0, stream, dd);
  return launched();
}

specv_status_t specv_row_stats(const specv_shape_t* shape, const void* target_logits,
                               const void* draft_logits, const int32_t* gamma_per_row,
                               const float* temperature, float* out_target_max,
                               double* out_target_sum, int32_t* out_target_argmax,
                               float* out_draft_max, double* out_draft_sum,
                               int32_t* out_draft_argmax, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  Plan p;
  specv_status_t st = check_common(shape, target_logits, draft_logits, gamma_per_row, temperature,
                                   workspace, workspace_bytes, &p);
  if (st != SPECV_OK || p.B == 0) return st;
  if (!out_target_max || !out_target_sum || !out_target_argmax) return SPECV_ERR_INVALID_ARGUMENT;
  if (p.td > 0 && (!out_draft_max || !out_draft_sum || !out_draft_argmax))
    return SPECV_ERR_INVALID_ARGUMENT;
  const bool vec = vector_path(p, target_logits, draft_logits);
  if ((st = launch_plan(p, gamma_per_row, temperature, workspace, stream)) != SPECV_OK) return st;
  if ((st = launch_row_stats(p, vec, target_logits, draft_logits, workspace, stream, true)) !=
      SPECV_OK)
    return st;
  MergeArgs a;
  a.tparts = at<RowPart>(workspace, p.off_tparts);
  a.dparts = at<RowPart>(workspace, p.off_dparts);
  a.tk = at<float>(workspace, p.off_tk);
  a.dk = at<float>(workspace, p.off_dk);
  a.status = at<uint32_t>(workspace, 0);
  a.out_tm = out_target_max;
  a.out_ts = out_target_sum;
  a.out_ta = out_target_argmax;
  a.out_dm = out_draft_max;
  a.out_ds = out_draft_sum;
  a.out_da = out_draft_argmax;
  a.total_t = p.tt;
  a.total_d = p.td;
  a.B = (int32_t)p.B;
  a.chunks = p.chunks1;
  const int64_t rows = p.tt + p.td;
  hipLaunchKernelGGL(k_merge_rows, dim3((unsigned)((rows + kBlock - 1) / kBlock)), dim3(kBlock), 0,
                     stream, a);
  return launched();
}

specv_status_t specv_softmax_rows(const specv_shape_t* shape, const void* target_logits,
                                  const void* draft_logits, const int32_t* gamma_per_row,
                                  const float* temperature, const int64_t* rows, int64_t n_rows,
                                  float* out_probs, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  Plan p;
  specv_status_t st = check_common(shape, target_logits, draft_logits, gamma_per_row, temperature,
                                   workspace, workspace_bytes, &p);
  if (st != SPECV_OK || p.B == 0 || n_rows == 0) return st;
  if (n_rows < 0 || n_rows > 65535 || !rows || !out_probs) return SPECV_ERR_INVALID_ARGUMENT;
  const bool vec = vector_path(p, target_logits, draft_logits);
  if ((st = launch_plan(p, gamma_per_row, temperature, workspace, stream)) != SPECV_OK) return st;
  if ((st = launch_row_stats(p, vec, target_logits, draft_logits, workspace, stream)) != SPECV_OK)
    return st;
  ProbArgs a;
  a.target = target_logits;
  a.draft = draft_logits;
  a.tparts = at<RowPart>(workspace, p.off_tparts);
  a.dparts = at<RowPart>(workspace, p.off_dparts);
  a.tk = at<float>(workspace, p.off_tk);
  a.dk = at<float>(workspace, p.off_dk);
  a.rows = rows;
  a.out = out_probs;
  a.V = p.V;
  a.n_rows = n_rows;
  a.total_t = p.tt;
  a.total_d = p.td;
  a.B = (int32_t)p.B;
  a.chunks = p.chunks1;
  const dim3 grid((unsigned)((p.V + 2047) / 2048), (unsigned)n_rows);
  if (p.dt == kBF16) hipLaunchKernelGGL((k_softmax_rows<kBF16>), grid, dim3(kBlock), 0, stream, a);
  else hipLaunchKernelGGL((k_softmax_rows<kF32>), grid, dim3(kBlock), 0, stream, a);
  return launched();
}

specv_status_t specv_philox4x32_10(uint64_t seed, const uint32_t* ctr, uint32_t* out, int64_t n,
                                   hipStream_t stream) {
  if (n < 0 || (n > 0 && (!ctr || !out))) return SPECV_ERR_INVALID_ARGUMENT;
  if (n == 0) return SPECV_OK;
  hipLaunchKernelGGL(k_philox, dim3((unsigned)((n + kBlock - 1) / kBlock)), dim3(kBlock), 0, stream,
                     seed, ctr, out, n);
  return launched();
}

specv_status_t specv_copy_bytes(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return SPECV_OK;
  if (!dst || !src || bytes % 16 != 0 || !aligned(dst, 16) || !aligned(src, 16))
    return SPECV_ERR_INVALID_ARGUMENT;
  // whole 64 KiB segments with the tiled copy, a shorter tail grid-stride
  const int64_t segments = (int64_t)(bytes / kProbeSegBytes);
  const int64_t tail16 = (int64_t)(bytes % kProbeSegBytes) / 16;
  u32x4* d = static_cast<u32x4*>(dst);
  const u32x4* s = static_cast<const u32x4*>(src);
  if (segments > 0) {
    hipLaunchKernelGGL(k_copy_tiled, dim3(blocks_for(2 * segments)), dim3(kBlock), 0, stream, d, s,
                       segments);
    const specv_status_t st = launched();
    if (st != SPECV_OK) return st;
  }
  if (tail16 > 0) {
    const int64_t off = segments * (kProbeSegBytes / 16);
    hipLaunchKernelGGL(k_copy, dim3((unsigned)((tail16 + kBlock - 1) / kBlock)), dim3(kBlock), 0,
                       stream, d + off, s + off, tail16);
    return launched();
  }
  return SPECV_OK;
}

specv_status_t specv_read_bytes(const void* src, size_t bytes, uint32_t* sink,
                                hipStream_t stream) {
  if (bytes == 0) return SPECV_OK;
  if (!src || !sink || bytes % kProbeSegBytes != 0 || !aligned(src, 16) || !aligned(sink, 4))
    return SPECV_ERR_INVALID_ARGUMENT;
  const int64_t segments = (int64_t)(bytes / kProbeSegBytes);
  hipLaunchKernelGGL(k_read_probe, dim3(blocks_for(2 * segments)), dim3(kBlock), 0, stream,
                     static_cast<const u32x4*>(src), segments, sink);
  return launched();
}

const char* specv_status_string(specv_status_t status) {
  switch (enum_bits(status)) {
    case SPECV_OK: return "ok";
    case SPECV_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SPECV_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case SPECV_ERR_HIP: return "HIP launch failed";
    case SPECV_ERR_UNSUPPORTED: return "unsupported";
    case SPECV_ERR_SCRATCH_LIMIT:
      return "the call needs more scratch than specv_verify_noalloc's static buffer holds";
  }
  return "unknown status";
}

}  // extern "C"
