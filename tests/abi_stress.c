/*
 * abi_stress.c -- drives the argument checks of libspecverify's C ABI for a
 * sanitizer build of the library's host code (AddressSanitizer +
 * UndefinedBehaviorSanitizer): shape descriptors with extreme fields (the
 * checks' integer arithmetic must not overflow), the workspace queries of
 * every entry point, and calls with null, misaligned or fake pointers that
 * must be refused before anything is enqueued, so no GPU is needed. Exits
 * nonzero on a wrong status or a sanitizer report. Test infrastructure.
 *
 *   abi_stress [cases] [seed]
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "specverify.h"

static uint64_t g_state;

static uint64_t next_u64(void) { /* splitmix64 */
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static int32_t any_i32(void) {
  switch (next_u64() % 4) {
    case 0: return (int32_t)(next_u64() % 80) - 3;
    case 1: return (int32_t)(next_u64() & 0xffffffffu);
    case 2: return (next_u64() & 1) ? INT32_MAX : INT32_MIN;
    default: return (int32_t)(next_u64() % 300000);
  }
}

static int64_t any_i64(void) {
  switch (next_u64() % 4) {
    case 0: return (int64_t)(next_u64() % 400) - 3;
    case 1: return (int64_t)next_u64();
    case 2: return (next_u64() & 1) ? INT64_MAX : INT64_MIN;
    default: return (int64_t)(next_u64() % (1ull << 42));
  }
}

static int g_failures;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    fprintf(stderr, "%s: status %d, expected %d\n", what, got, want);
    ++g_failures;
  }
}

#define FAKE ((void*)0x100000)

int main(int argc, char** argv) {
  const int cases = argc > 1 ? atoi(argv[1]) : 20000;
  g_state = argc > 2 ? strtoull(argv[2], NULL, 10) : 1;
  for (int c = 0; c < cases; ++c) {
    specv_shape_t s;
    s.batch = any_i32();
    s.vocab = any_i32();
    s.max_gamma = any_i32();
    s.dtype = (specv_dtype_t)((int)(next_u64() % 5) - 1);
    s.total_draft_rows = any_i64();
    /* often the consistent total (wrapping like the hardware, not overflowing in C) */
    s.total_target_rows = (next_u64() & 1)
                              ? (int64_t)((uint64_t)s.total_draft_rows + (uint64_t)(int64_t)s.batch)
                              : any_i64();
    const size_t ws = specv_workspace_bytes(&s);
    (void)specv_diagnostics_workspace_bytes(&s, any_i32());
    if (ws == 0) {
      expect(specv_verify(&s, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0, FAKE, FAKE, FAKE, (size_t)1 << 30,
                          NULL),
             SPECV_ERR_INVALID_ARGUMENT, "verify, invalid shape");
      expect(specv_verify_noalloc(&s, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0, FAKE, FAKE, NULL, NULL),
             SPECV_ERR_INVALID_ARGUMENT, "noalloc, invalid shape");
    } else if (s.batch > 0) {
      /* a valid shape with a workspace one byte short */
      expect(specv_verify(&s, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0, FAKE, FAKE, FAKE, ws - 1, NULL),
             SPECV_ERR_WORKSPACE, "verify, short workspace");
      if (ws > SPECV_NOALLOC_SCRATCH_BYTES)
        expect(specv_verify_noalloc(&s, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0, FAKE, FAKE, NULL, NULL),
               SPECV_ERR_SCRATCH_LIMIT, "noalloc, beyond the scratch");
    }
    specv_decode_shape_t d = {any_i32(), any_i32(), any_i32(), any_i32(),
                              (specv_dtype_t)((int)(next_u64() % 4) - 1)};
    (void)specv_decode_workspace_bytes(&d);
    specv_cascade_shape_t k = {any_i32(), any_i32(), any_i32(), any_i32(), any_i32(),
                               (specv_dtype_t)((int)(next_u64() % 4) - 1)};
    (void)specv_cascade_workspace_bytes(&k);
  }
  /* argument errors on a valid shape */
  specv_shape_t s = {4, 1000, 3, SPECV_BF16, 16, 12};
  expect(specv_verify(NULL, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0, FAKE, FAKE, FAKE, 1 << 30, NULL),
         SPECV_ERR_INVALID_ARGUMENT, "null shape");
  expect(specv_verify(&s, NULL, FAKE, FAKE, FAKE, FAKE, 0, 0, FAKE, FAKE, FAKE, 1 << 30, NULL),
         SPECV_ERR_INVALID_ARGUMENT, "null target");
  expect(specv_verify(&s, (void*)0x100001, FAKE, FAKE, FAKE, FAKE, 0, 0, FAKE, FAKE, FAKE, 1 << 30,
                      NULL),
         SPECV_ERR_INVALID_ARGUMENT, "misaligned target");
  expect(specv_verify(&s, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0, FAKE, FAKE, (void*)0x100010, 1 << 30,
                      NULL),
         SPECV_ERR_WORKSPACE, "misaligned workspace");
  expect(specv_verify_lenient(&s, FAKE, FAKE, FAKE, FAKE, FAKE, SPECV_LENIENCE_LIN, 0.0f, 0, 0, NULL,
                              NULL, FAKE, FAKE, FAKE, 1 << 30, NULL, NULL),
         SPECV_ERR_INVALID_ARGUMENT, "epsilon 0");
  expect(specv_position_diagnostics(&s, FAKE, FAKE, FAKE, FAKE, 65, FAKE, FAKE, FAKE, FAKE, FAKE,
                                    1 << 30, NULL, NULL),
         SPECV_ERR_INVALID_ARGUMENT, "top_k 65");
  expect(specv_softmax_rows(&s, FAKE, FAKE, FAKE, FAKE, FAKE, -1, FAKE, FAKE, 1 << 30, NULL),
         SPECV_ERR_INVALID_ARGUMENT, "negative row count");
  expect(specv_copy_bytes(FAKE, FAKE, 15, NULL), SPECV_ERR_INVALID_ARGUMENT, "copy of 15 bytes");
  expect(specv_read_bytes(FAKE, 65536 + 16, FAKE, NULL), SPECV_ERR_INVALID_ARGUMENT, "partial segment");
  expect(specv_philox4x32_10(0, FAKE, FAKE, -1, NULL), SPECV_ERR_INVALID_ARGUMENT, "negative count");
  for (int st = 0; st <= 6; ++st)
    if (!specv_status_string((specv_status_t)st)) ++g_failures;
  if (g_failures) {
    fprintf(stderr, "abi_stress: %d failures\n", g_failures);
    return 1;
  }
  printf("abi_stress: %d cases ok\n", cases);
  return 0;
}
