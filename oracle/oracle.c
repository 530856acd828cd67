/*
 * CPU oracle for the ragged-M grouped GEMM -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the CPU-baseline leg of the benchmark
 * load this file's library. The product path (the HIP library) never links,
 * calls or includes anything here, and this file includes nothing of it.
 *
 * What it computes, and where that is defined:
 *   "Grouped GEMM for Imbalanced Experts on Blackwell: A WIP Worklog",
 *   section "What I am measuring" and section 2 ("The Grouped Problem and the
 *   flat tile list"): after routing, rows are grouped by expert and expert e
 *   computes an independent product [m_e, K] x [K, N]; K and N are fixed,
 *   m_e is decided at runtime and may be zero. The InferenceX glossary entry
 *   "Grouped GEMM" ("Technical definition") states the same: independent
 *   matrix multiplications with different row counts in one launch.
 *
 *   So, for every expert e and every row i in [off[e], off[e+1]) and every
 *   column j < N:
 *       C[i][j] = sum_{k<K} a(A[i][k]) * a(B[e][k][j])
 *   where a(x) is the exact value of the bfloat16 bit pattern x. The sum is
 *   taken in IEEE binary64 in the order k = 0, 1, ..., K-1. Rows of A and C
 *   outside every group are neither read nor written.
 *
 *   Alongside C the oracle returns S[i][j] = sum_k |a(A[i][k]) * a(B[e][k][j])|
 *   (the scale of the per-element error bound a floating-point result of the
 *   same sum may carry) and the number of multiply-adds it performed.
 *
 * Layouts (row-major, last index fastest):
 *   A [M_cap][K] bf16 bits, B [E][K][N] bf16 bits, off [E+1] int32,
 *   C and S [M_cap][N] double.
 *
 * Every function here is pinned by CPU tests against brute force, a library
 * matrix product, closed forms and the pages' printed figures.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* exact value of a bfloat16 bit pattern: it is the high half of a binary32 word */
static double bf16_value(uint16_t bits) {
  uint32_t w = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads later calls run on (n >= 1); used to time the loop on one core. */
void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/*
 * Full grouped product. Returns 0 on success, -1 on malformed offsets
 * (off[0] != 0, decreasing, or off[E] > M_cap). S may be NULL.
 * *madds receives the number of multiply-adds performed (sum_e m_e*K*N).
 */
int oracle_grouped_gemm(const uint16_t *A, const uint16_t *B, const int32_t *off,
                        int E, int K, int N, int M_cap,
                        double *C, double *S, int64_t *madds) {
  if (E < 1 || K < 1 || N < 1 || M_cap < 0) return -1;
  if (off[0] != 0) return -1;
  for (int e = 0; e < E; ++e)
    if (off[e + 1] < off[e]) return -1;
  if (off[E] > M_cap) return -1;

  int64_t count = 0;
  for (int e = 0; e < E; ++e) {
    const int r0 = off[e], r1 = off[e + 1];
    const uint16_t *Be = B + (size_t)e * K * N;
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = r0; i < r1; ++i) {
      double *acc = (double *)calloc((size_t)N, sizeof(double));
      double *sab = (double *)calloc((size_t)N, sizeof(double));
      const uint16_t *Ai = A + (size_t)i * K;
      for (int k = 0; k < K; ++k) {
        const double a = bf16_value(Ai[k]);
        const uint16_t *Bk = Be + (size_t)k * N;
        for (int j = 0; j < N; ++j) {
          const double p = a * bf16_value(Bk[j]);
          acc[j] += p;
          sab[j] += fabs(p);
        }
      }
      memcpy(C + (size_t)i * N, acc, (size_t)N * sizeof(double));
      if (S) memcpy(S + (size_t)i * N, sab, (size_t)N * sizeof(double));
      free(acc);
      free(sab);
    }
    count += (int64_t)(r1 - r0) * K * N;
  }
  if (madds) *madds = count;
  return 0;
}

/*
 * Selected entries of the same product, one dot product each, for problems
 * too large to compute whole. For n entries (rows[t], cols[t]) it writes
 * c[t] = C[rows[t]][cols[t]] and s[t] = S[rows[t]][cols[t]]. A row outside
 * every group gets c = s = NaN. Returns 0, or -1 on malformed offsets.
 */
int oracle_grouped_gemm_entries(const uint16_t *A, const uint16_t *B, const int32_t *off,
                                int E, int K, int N, int M_cap,
                                const int64_t *rows, const int64_t *cols, int64_t n,
                                double *c, double *s) {
  if (E < 1 || K < 1 || N < 1 || M_cap < 0 || off[0] != 0) return -1;
  for (int e = 0; e < E; ++e)
    if (off[e + 1] < off[e]) return -1;
  if (off[E] > M_cap) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < n; ++t) {
    const int64_t i = rows[t], j = cols[t];
    int ex = -1;
    for (int e = 0; e < E; ++e)
      if (i >= off[e] && i < off[e + 1]) { ex = e; break; }
    if (ex < 0 || j < 0 || j >= N) { c[t] = NAN; s[t] = NAN; continue; }
    const uint16_t *Ai = A + (size_t)i * K;
    const uint16_t *Be = B + (size_t)ex * K * N;
    double acc = 0.0, sab = 0.0;
    for (int k = 0; k < K; ++k) {
      const double p = bf16_value(Ai[k]) * bf16_value(Be[(size_t)k * N + j]);
      acc += p;
      sab += fabs(p);
    }
    c[t] = acc;
    s[t] = sab;
  }
  return 0;
}
