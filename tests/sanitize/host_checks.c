/* Host-side argument checks of every entry point, built with AddressSanitizer
 * and UndefinedBehaviorSanitizer on the host code (tests/test_host_sanitizers.py).
 * Every call here is rejected (or, with M_cap == 0, finished) before any HIP
 * runtime call, so no GPU is needed. The pointers are fake, aligned addresses
 * that are never dereferenced. Exit status: the number of failed checks. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "grouped_gemm.h"

static int failures = 0;

static void expect(const char *what, gg_status_t got, gg_status_t want) {
  if (got != want) {
    printf("FAIL %s: status %d, expected %d\n", what, (int)got, (int)want);
    ++failures;
  }
}

#define P(x) ((void *)(uintptr_t)(x))

/* the four entry points with the plain argument list */
typedef gg_status_t (*plain_fn)(const void *, const void *, const int32_t *, void *, int32_t,
                                int32_t, int32_t, int32_t, int32_t, void *);

static gg_status_t bf16_fp32(const void *A, const void *B, const int32_t *off, void *C, int32_t E,
                             int32_t K, int32_t N, int32_t M, int32_t bm, void *s) {
  return gg_grouped_gemm_bf16(A, B, off, (float *)C, E, K, N, M, bm, s);
}

static gg_status_t fp8w(const void *A, const void *B, const int32_t *off, void *C, int32_t E,
                        int32_t K, int32_t N, int32_t M, int32_t bm, void *s) {
  return gg_grouped_gemm_fp8w(A, B, (const float *)P(0x200), off, (float *)C, E, K, N, M, bm, s);
}

struct plain_case {
  const char *name;
  uintptr_t A, B, off, C;
  int32_t E, K, N, M, bm;
  gg_status_t want;
};

int main(void) {
  const struct plain_case cases[] = {
      {"null A", 0, 32, 64, 128, 4, 256, 256, 29, 0, GG_ERR_INVALID_VALUE},
      {"null B", 16, 0, 64, 128, 4, 256, 256, 29, 0, GG_ERR_INVALID_VALUE},
      {"null offsets", 16, 32, 0, 128, 4, 256, 256, 29, 0, GG_ERR_INVALID_VALUE},
      {"null C", 16, 32, 64, 0, 4, 256, 256, 29, 0, GG_ERR_INVALID_VALUE},
      {"E = 0", 16, 32, 64, 128, 0, 256, 256, 29, 0, GG_ERR_INVALID_VALUE},
      {"E < 0", 16, 32, 64, 128, -7, 256, 256, 29, 0, GG_ERR_INVALID_VALUE},
      {"K = 0", 16, 32, 64, 128, 4, 0, 256, 29, 0, GG_ERR_INVALID_VALUE},
      {"N < 0", 16, 32, 64, 128, 4, 256, -8, 29, 0, GG_ERR_INVALID_VALUE},
      {"M_cap < 0", 16, 32, 64, 128, 4, 256, 256, -1, 0, GG_ERR_INVALID_VALUE},
      {"bm = 48", 16, 32, 64, 128, 4, 256, 256, 29, 48, GG_ERR_INVALID_VALUE},
      {"bm = -16", 16, 32, 64, 128, 4, 256, 256, 29, -16, GG_ERR_INVALID_VALUE},
      {"A misaligned", 24, 32, 64, 128, 4, 256, 256, 29, 0, GG_ERR_MISALIGNED},
      {"offsets misaligned", 16, 32, 66, 128, 4, 256, 256, 29, 0, GG_ERR_MISALIGNED},
      {"K % 8", 16, 32, 64, 128, 4, 252, 256, 29, 0, GG_ERR_MISALIGNED},
      {"N % 8", 16, 32, 64, 128, 4, 256, 100, 29, 0, GG_ERR_MISALIGNED},
      {"E too large", 16, 32, 64, 128, GG_MAX_EXPERTS + 1, 256, 256, 29, 0, GG_ERR_UNSUPPORTED},
      {"K too large", 16, 32, 64, 128, 4, GG_MAX_K + 8, 256, 29, 0, GG_ERR_UNSUPPORTED},
      {"N too large", 16, 32, 64, 128, 4, 256, GG_MAX_N + 8, 29, 0, GG_ERR_UNSUPPORTED},
      {"M_cap near INT32_MAX", 16, 32, 64, 128, 4, 256, 256, INT32_MAX, 16, GG_ERR_UNSUPPORTED},
      {"extreme sizes", 16, 32, 64, 128, GG_MAX_EXPERTS, GG_MAX_K, GG_MAX_N, INT32_MAX - 1, 0,
       GG_ERR_UNSUPPORTED},
      {"M_cap = 0 (nothing to do)", 16, 32, 64, 128, 4, 256, 256, 0, 0, GG_OK},
  };
  const struct {
    const char *name;
    plain_fn fn;
  } fns[] = {{"bf16", bf16_fp32},
             {"bf16out", gg_grouped_gemm_bf16_bf16out},
             {"swiglu", gg_grouped_gemm_bf16_swiglu},
             {"fp8w", fp8w}};
  char what[160];
  for (size_t f = 0; f < sizeof(fns) / sizeof(fns[0]); ++f)
    for (size_t i = 0; i < sizeof(cases) / sizeof(cases[0]); ++i) {
      const struct plain_case *c = &cases[i];
      snprintf(what, sizeof what, "%s: %s", fns[f].name, c->name);
      expect(what, fns[f].fn(P(c->A), P(c->B), (const int32_t *)P(c->off), P(c->C), c->E, c->K,
                             c->N, c->M, c->bm, NULL),
             c->want);
    }

  /* fp8 weights need their scales */
  expect("fp8w: null scales",
         gg_grouped_gemm_fp8w(P(16), P(32), NULL, (const int32_t *)P(64), (float *)P(128), 4, 256,
                              256, 29, 0, NULL),
         GG_ERR_INVALID_VALUE);
  expect("fp8w: misaligned scales",
         gg_grouped_gemm_fp8w(P(16), P(32), (const float *)P(0x204), (const int32_t *)P(64),
                              (float *)P(128), 4, 256, 256, 29, 0, NULL),
         GG_ERR_MISALIGNED);

  /* fp8 activations and weights */
  expect("fp8: null row scales",
         gg_grouped_gemm_fp8(P(16), NULL, P(32), (const float *)P(64), (const int32_t *)P(96),
                             (float *)P(128), 4, 256, 256, 29, 0, NULL),
         GG_ERR_INVALID_VALUE);
  expect("fp8: K not a multiple of 16",
         gg_grouped_gemm_fp8(P(16), (const float *)P(48), P(32), (const float *)P(64),
                             (const int32_t *)P(96), (float *)P(128), 4, 264, 256, 29, 0, NULL),
         GG_ERR_MISALIGNED);
  expect("fp8: misaligned row scales",
         gg_grouped_gemm_fp8(P(16), (const float *)P(50), P(32), (const float *)P(64),
                             (const int32_t *)P(96), (float *)P(128), 4, 256, 256, 29, 0, NULL),
         GG_ERR_MISALIGNED);
  expect("fp8: nothing to do",
         gg_grouped_gemm_fp8(P(16), (const float *)P(48), P(32), (const float *)P(64),
                             (const int32_t *)P(96), (float *)P(128), 4, 256, 256, 0, 0, NULL),
         GG_OK);

  /* gather / scatter */
  expect("gather: null src_rows",
         gg_grouped_gemm_bf16_gather(P(16), 10, NULL, P(32), (const int32_t *)P(64),
                                     (float *)P(128), NULL, 4, 256, 256, 29, 0, NULL),
         GG_ERR_INVALID_VALUE);
  expect("gather: n_src < 0",
         gg_grouped_gemm_bf16_gather(P(16), -1, (const int32_t *)P(96), P(32),
                                     (const int32_t *)P(64), (float *)P(128), NULL, 4, 256, 256,
                                     29, 0, NULL),
         GG_ERR_INVALID_VALUE);
  expect("gather: misaligned dst_rows",
         gg_grouped_gemm_bf16_gather(P(16), 10, (const int32_t *)P(96), P(32),
                                     (const int32_t *)P(64), (float *)P(128),
                                     (const int32_t *)P(98), 4, 256, 256, 29, 0, NULL),
         GG_ERR_MISALIGNED);
  expect("gather: X beyond 2^31 bytes",
         gg_grouped_gemm_bf16_gather(P(16), (1 << 22) + 1, (const int32_t *)P(96), P(32),
                                     (const int32_t *)P(64), (float *)P(128), NULL, 4, 256, 256,
                                     29, 0, NULL),
         GG_ERR_UNSUPPORTED);

  /* gather + weighted combine */
  expect("combine: null dst_rows",
         gg_grouped_gemm_bf16_gather_combine(P(16), 10, (const int32_t *)P(96), P(32),
                                             (const int32_t *)P(64), NULL, (const float *)P(48),
                                             (float *)P(128), 10, 4, 256, 256, 29, 0, NULL),
         GG_ERR_INVALID_VALUE);
  expect("combine: null weights",
         gg_grouped_gemm_bf16_gather_combine(P(16), 10, (const int32_t *)P(96), P(32),
                                             (const int32_t *)P(64), (const int32_t *)P(80), NULL,
                                             (float *)P(128), 10, 4, 256, 256, 29, 0, NULL),
         GG_ERR_INVALID_VALUE);
  expect("combine: n_dst < 0",
         gg_grouped_gemm_bf16_gather_combine(P(16), 10, (const int32_t *)P(96), P(32),
                                             (const int32_t *)P(64), (const int32_t *)P(80),
                                             (const float *)P(48), (float *)P(128), -1, 4, 256,
                                             256, 29, 0, NULL),
         GG_ERR_INVALID_VALUE);
  expect("combine: misaligned weights",
         gg_grouped_gemm_bf16_gather_combine(P(16), 10, (const int32_t *)P(96), P(32),
                                             (const int32_t *)P(64), (const int32_t *)P(80),
                                             (const float *)P(50), (float *)P(128), 10, 4, 256,
                                             256, 29, 0, NULL),
         GG_ERR_MISALIGNED);

  /* tile schedule */
  expect("schedule: null count",
         gg_tile_schedule((const int32_t *)P(64), 4, 256, 29, 0, (int32_t *)P(128), NULL, 10,
                          NULL),
         GG_ERR_INVALID_VALUE);
  expect("schedule: null tiles with room",
         gg_tile_schedule((const int32_t *)P(64), 4, 256, 29, 0, NULL, (int32_t *)P(132), 10,
                          NULL),
         GG_ERR_INVALID_VALUE);
  expect("schedule: bad bm",
         gg_tile_schedule((const int32_t *)P(64), 4, 256, 29, 24, (int32_t *)P(128),
                          (int32_t *)P(132), 10, NULL),
         GG_ERR_INVALID_VALUE);

  /* status strings: every code, and an unknown one */
  for (int s = 0; s <= 5; ++s) {
    const char *m = gg_status_string((gg_status_t)s);
    if (m == NULL || strlen(m) == 0) {
      printf("FAIL status string %d\n", s);
      ++failures;
    }
  }
  printf("host checks: %d failure(s)\n", failures);
  return failures;
}
