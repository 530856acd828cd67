/*
 * Ragged-M grouped GEMM for AMD Instinct MI355X (gfx950) -- C ABI.
 *
 * One call computes E independent bf16 products with fp32 accumulation,
 *     C[off[e]:off[e+1], :] = A[off[e]:off[e+1], :] x B[e]      for e < E,
 * where the row count m_e = off[e+1] - off[e] of every group is read on the
 * device at run time and may be zero or heavily skewed. This is the
 * expert-FFN projection of a Mixture-of-Experts layer after routing, as
 * defined by "Grouped GEMM for Imbalanced Experts on Blackwell: A WIP
 * Worklog" (section "What I am measuring" and section 2, "The Grouped
 * Problem and the flat tile list") and by the InferenceX glossary entry
 * "Grouped GEMM" ("Technical definition"): rows arrive grouped by expert,
 * K and N are fixed, the group sizes are only known at run time, and every
 * expert's product runs in a single launch.
 *
 * Conventions shared by every entry point below:
 *  - All array pointers are DEVICE pointers owned by the caller; the library
 *    keeps no reference to them after the call returns and allocates no
 *    device memory.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). The
 *    call only enqueues work on it: no host synchronisation, no device to
 *    host copy. Results are ready when the stream reaches that point.
 *  - Errors the host can see (bad sizes, null or misaligned pointers,
 *    unsupported shapes) return a status and enqueue nothing.
 *  - Malformed offsets (off[0] != 0, decreasing entries, entries outside
 *    [0, M_cap]) are the caller's bug; they never make the kernel read or
 *    write outside A[0:M_cap], B[0:E] and C[0:M_cap]: every offset is clamped
 *    into [0, M_cap] and a group whose clamped end precedes its clamped start
 *    is treated as empty. Decreasing offsets can make clamped groups
 *    overlap; if the tiles of all groups then outnumber what M_cap rows can
 *    produce with nondecreasing offsets, ((M_cap / h) + E) * ceil(N / 256)
 *    for the smallest height h in use, the call computes nothing at all.
 *  - Calls on different streams may run concurrently; the library holds no
 *    mutable state besides a per-device cache of launch limits.
 */
#ifndef MOE_RAGGED_GROUPED_AMD_GROUPED_GEMM_H
#define MOE_RAGGED_GROUPED_AMD_GROUPED_GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GG_OK = 0,
  GG_ERR_INVALID_VALUE = 1, /* null pointer, non-positive size, bad bm        */
  GG_ERR_MISALIGNED = 2,    /* pointer not 16-byte aligned, K or N not 8k     */
  GG_ERR_UNSUPPORTED = 3,   /* E, K or N above its limit, or index range beyond int32 */
  GG_ERR_LAUNCH = 4         /* the HIP runtime refused the launch             */
} gg_status_t;

/* Largest number of groups one call accepts (the per-group tables live in LDS). */
#define GG_MAX_EXPERTS 1024
/* Largest K and N gg_grouped_gemm_bf16 accepts. */
#define GG_MAX_K (1 << 22)
#define GG_MAX_N (1 << 24)

/*
 * gg_grouped_gemm_bf16 -- the grouped product (worklog section 2; glossary
 * "Technical definition").
 *
 *   A   bf16 [M_cap][K], row-major (K fastest). Rows are grouped by expert:
 *       rows off[e] .. off[e+1]-1 belong to expert e. Rows at or beyond
 *       off[E] are never read.
 *   B   bf16 [E][K][N], row-major (N fastest): B[e] is expert e's weight.
 *       The slice of an expert with no rows is never read.
 *   group_offsets  int32 [E+1] on the device: 0 = off[0] <= off[1] <= ...
 *       <= off[E] = M_tot <= M_cap.
 *   C   fp32 [M_cap][N], row-major. Rows [0, M_tot) are overwritten with the
 *       product (not accumulated into); rows [M_tot, M_cap) are not touched.
 *   E in [1, GG_MAX_EXPERTS]; K >= 8 and N >= 8, both multiples of 8;
 *   K <= GG_MAX_K and N <= GG_MAX_N (the kernels address a tile's A rows and
 *   a K slice of B with 32-bit byte offsets);
 *   M_cap >= 0 (0: nothing is enqueued).
 *   bm  tile height: 16, 32, 64, 128 or 256 for every expert, or 0 to let
 *       the device choose per expert from its row count (the trade between
 *       padding in the last tile and per-tile work that the worklog
 *       describes in sections 2.1, 6 and 7).
 *   A, B and C must be 16-byte aligned; group_offsets 4-byte aligned.
 *
 * Accumulation is fp32 inside the matrix cores; a result differs from the
 * exact sum by at most a few units of K * 2^-24 relative to sum_k |a*b|.
 */
gg_status_t gg_grouped_gemm_bf16(const void *A, const void *B, const int32_t *group_offsets,
                                 float *C, int32_t E, int32_t K, int32_t N, int32_t M_cap,
                                 int32_t bm, void *stream);

/*
 * gg_grouped_gemm_bf16_bf16out -- the same product with bf16 output C.
 *
 * The worklog's compulsory-traffic model (section 2.1, about 474 MB at 16k)
 * counts C as 2-byte values. Every argument and rule is that of
 * gg_grouped_gemm_bf16 except C:
 *   C   bf16 [M_cap][N], row-major, 16-byte aligned. Each element is the fp32
 *       matrix-core result rounded once to the nearest bf16 (ties to even),
 *       so it is within half a bf16 unit (2^-9 relative) of the fp32 result
 *       gg_grouped_gemm_bf16 returns for the same inputs, and equal to that
 *       result rounded to bf16.
 */
gg_status_t gg_grouped_gemm_bf16_bf16out(const void *A, const void *B,
                                         const int32_t *group_offsets, void *C, int32_t E,
                                         int32_t K, int32_t N, int32_t M_cap, int32_t bm,
                                         void *stream);

/*
 * gg_grouped_gemm_bf16_swiglu -- the gate and up projections with the SwiGLU
 * activation applied in the epilogue.
 *
 * The Pearl Pulse page "Pearl's grouped GEMM kernel for MoE models,
 * explained" (section "What the 15% measures") benchmarks the kernel on
 * the gate and up projections of MoE models; the activation between them
 * and the next projection is silu(gate) * up. Here B holds both projections
 * with their columns interleaved, so the product's two columns of one output
 * are computed by the same lane and need no exchange:
 *   B   bf16 [E][K][N], N = 2 * I: column 2j is gate column j and column
 *       2j+1 is up column j (a caller holding [W_gate | W_up] interleaves
 *       the columns once, when the weights are loaded).
 *   H   bf16 [M_cap][N/2], row-major, 16-byte aligned:
 *       H[r][j] = silu(C[r][2j]) * C[r][2j+1], silu(x) = x / (1 + e^-x),
 *       where C is the fp32 product gg_grouped_gemm_bf16 computes for the
 *       same inputs. The activation is evaluated in fp32 as
 *       x * rcp(1 + 2^(-x log2 e)) with the hardware exp2 and reciprocal,
 *       within (|gate| + 3.5) * 2^-23 of the exact value relative to first
 *       order (-0 where e^-gate overflows, for gate below about -88.7), and
 *       rounded once to the nearest bf16 (ties to even). Rows at or past
 *       off[E] are not written.
 * A, group_offsets, E, K, N, M_cap, bm, the stream, the status codes and
 * the conditions for them are those of gg_grouped_gemm_bf16 (N a multiple
 * of 8, so I is a multiple of 4).
 */
gg_status_t gg_grouped_gemm_bf16_swiglu(const void *A, const void *B,
                                        const int32_t *group_offsets, void *H, int32_t E,
                                        int32_t K, int32_t N, int32_t M_cap, int32_t bm,
                                        void *stream);

/*
 * gg_grouped_gemm_bf16_gather -- the product with the expert grouping done by
 * index instead of by copying rows (the worklog's "What I am measuring" puts
 * the token permutation on either side of the grouped GEMM; here it is folded
 * into the A loads and the C stores).
 *
 *   X         bf16 [n_src][K], row-major, 16-byte aligned: the unpermuted
 *             rows (e.g. token activations).
 *   src_rows  int32 [M_cap] on the device, 4-byte aligned: grouped row r
 *             (expert e owns grouped rows off[e] .. off[e+1]-1, exactly as
 *             in gg_grouped_gemm_bf16) reads its A row from X[src_rows[r]].
 *             An index outside [0, n_src) reads a row of zeros. Entries at
 *             or past off[E] are never read.
 *   dst_rows  int32 [M_cap] on the device, 4-byte aligned, or NULL: grouped
 *             row r is written to C row dst_rows[r]; an index outside
 *             [0, M_cap) is not written. With NULL, grouped row r is written
 *             to C row r, as in gg_grouped_gemm_bf16. Two grouped rows that
 *             name the same C row race (either result may land).
 *   C         fp32 [M_cap][N], row-major; rows no grouped row names are not
 *             touched.
 *   n_src >= 0 and n_src * K * 2 <= 2^31 (GG_ERR_UNSUPPORTED otherwise).
 * The other arguments, rules and the accuracy are those of
 * gg_grouped_gemm_bf16. The result equals gg_grouped_gemm_bf16 applied to
 * A = X[src_rows] followed by C[dst_rows[r]] = C_grouped[r].
 */
gg_status_t gg_grouped_gemm_bf16_gather(const void *X, int32_t n_src, const int32_t *src_rows,
                                        const void *B, const int32_t *group_offsets, float *C,
                                        const int32_t *dst_rows, int32_t E, int32_t K, int32_t N,
                                        int32_t M_cap, int32_t bm, void *stream);

/*
 * gg_grouped_gemm_bf16_gather_combine -- the gathered product with the
 * weighted combine folded into the epilogue.
 *
 * After the expert products, each token's routed rows are weighted and
 * summed back into the token's row (the worklog's "What I am measuring"
 * places the permutation on either side of the grouped GEMM; the InferenceX
 * glossary's "Engineering details" name the weighted combine). Here:
 *   Y[dst_rows[r]][n] += row_weights[r] * C[r][n]
 * for every grouped row r < off[E] whose destination lies in [0, n_dst),
 * where C[r] is the product gg_grouped_gemm_bf16_gather computes for that
 * row (A row X[src_rows[r]], weights B[e] of its expert).
 *   X, n_src, src_rows, B, group_offsets, E, K, N, M_cap, bm, stream: as in
 *             gg_grouped_gemm_bf16_gather.
 *   dst_rows     int32 [M_cap] on the device, 4-byte aligned, required.
 *                Several grouped rows may name the same Y row (top-k).
 *   row_weights  fp32 [M_cap] on the device, 4-byte aligned, required.
 *   Y            fp32 [n_dst][N], row-major, 16-byte aligned, in device
 *                memory (hipMalloc; the adds are the GPU's fp32 atomics):
 *                accumulated into, not overwritten -- clear it first for a
 *                plain combine. Rows no grouped row names keep their values.
 *   n_dst >= 0.
 * Each term is the fp32 product row times its weight, rounded once; the
 * terms meeting in one element are added with fp32 atomic adds in an
 * unspecified order, so the result may differ between runs by the rounding
 * of that order (the product itself is as accurate as gg_grouped_gemm_bf16).
 * Status codes as for gg_grouped_gemm_bf16_gather; a null dst_rows or
 * row_weights, or n_dst < 0, is GG_ERR_INVALID_VALUE.
 */
gg_status_t gg_grouped_gemm_bf16_gather_combine(const void *X, int32_t n_src,
                                                const int32_t *src_rows, const void *B,
                                                const int32_t *group_offsets,
                                                const int32_t *dst_rows,
                                                const float *row_weights, float *Y, int32_t n_dst,
                                                int32_t E, int32_t K, int32_t N, int32_t M_cap,
                                                int32_t bm, void *stream);

/*
 * gg_grouped_gemm_fp8w -- the product with fp8 weights and per-column scales
 * (the Pearl Pulse page, "What the 15% measures", notes that its kernel
 * ships with an FP8 scheme; the scheme below is this library's reading).
 *
 *   C[r][n] = scale[e][n] * sum_k A[r][k] * dec(Bq[e][k][n])   for r in group e
 *
 *   A        bf16 [M_cap][K], as in gg_grouped_gemm_bf16.
 *   Bq       uint8 [E][K][N], row-major, 16-byte aligned: OCP fp8 E4M3 codes
 *            (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; 0x7F and
 *            0xFF are NaN; largest finite magnitude 448).
 *   b_scale  fp32 [E][N] on the device, 16-byte aligned: one scale per expert
 *            and output column.
 *   C        fp32 [M_cap][N].
 * The weights stay fp8 in LDS and each is widened exactly to bf16 as the
 * matrix cores' operand is read from there; the products accumulate in fp32
 * in the bf16 matrix cores, and the epilogue multiplies by the column scale
 * (one more fp32 rounding). Weight bytes in HBM are halved;
 * this is a separate precision from gg_grouped_gemm_bf16, not a replacement.
 * Other arguments and rules are those of gg_grouped_gemm_bf16; b_scale NULL
 * is GG_ERR_INVALID_VALUE, misaligned b_scale GG_ERR_MISALIGNED.
 */
gg_status_t gg_grouped_gemm_fp8w(const void *A, const void *Bq, const float *b_scale,
                                 const int32_t *group_offsets, float *C, int32_t E, int32_t K,
                                 int32_t N, int32_t M_cap, int32_t bm, void *stream);

/*
 * gg_grouped_gemm_fp8 -- fp8 activations and fp8 weights on the fp8 matrix
 * cores (the article's FP8 scheme, read as one scale per activation row and
 * one per weight column).
 *
 *   C[r][n] = a_scale[r] * b_scale[e][n] * sum_k dec(Aq[r][k]) * dec(Bq[e][k][n])
 *
 *   Aq       uint8 [M_cap][K], row-major, 16-byte aligned: E4M3 codes, rows
 *            grouped by expert as A in gg_grouped_gemm_bf16.
 *   a_scale  fp32 [M_cap] on the device, 4-byte aligned: one scale per row.
 *   Bq       uint8 [E][K][N], 16-byte aligned: E4M3 codes, as for
 *            gg_grouped_gemm_fp8w.
 *   b_scale  fp32 [E][N], 16-byte aligned: one scale per expert and column.
 *   C        fp32 [M_cap][N].
 *   K and N must be multiples of 16 (GG_ERR_MISALIGNED otherwise).
 * The products of two E4M3 values are exact; they accumulate in fp32 in the
 * matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4 with unit block scales),
 * and the epilogue multiplies by the row and the column scale (two fp32
 * roundings). Other arguments and rules are those of gg_grouped_gemm_bf16;
 * a NULL scale pointer is GG_ERR_INVALID_VALUE.
 */
gg_status_t gg_grouped_gemm_fp8(const void *Aq, const float *a_scale, const void *Bq,
                                const float *b_scale, const int32_t *group_offsets, float *C,
                                int32_t E, int32_t K, int32_t N, int32_t M_cap, int32_t bm,
                                void *stream);

/*
 * gg_grouped_gemm_fp8_bf16out -- gg_grouped_gemm_fp8 with bf16 output: C is
 * bf16 [M_cap][N], 16-byte aligned, each element the fp32 result of
 * gg_grouped_gemm_fp8 (scales applied) rounded once to the nearest bf16
 * (ties to even). Every other argument and rule is that of
 * gg_grouped_gemm_fp8.
 */
gg_status_t gg_grouped_gemm_fp8_bf16out(const void *Aq, const float *a_scale, const void *Bq,
                                        const float *b_scale, const int32_t *group_offsets,
                                        void *C, int32_t E, int32_t K, int32_t N, int32_t M_cap,
                                        int32_t bm, void *stream);

/*
 * gg_grouped_gemm_fp8_swiglu -- gg_grouped_gemm_fp8 for the gate and up
 * projections with the SwiGLU of gg_grouped_gemm_bf16_swiglu in the
 * epilogue: Bq's columns interleave gate (even) and up (odd), and
 *   H[r][j] = silu(C[r][2j]) * C[r][2j+1]   (bf16 [M_cap][N/2], 16-byte aligned)
 * where C is the scaled fp32 result gg_grouped_gemm_fp8 computes. The
 * activation and its rounding are those of gg_grouped_gemm_bf16_swiglu;
 * every other argument and rule is that of gg_grouped_gemm_fp8.
 */
gg_status_t gg_grouped_gemm_fp8_swiglu(const void *Aq, const float *a_scale, const void *Bq,
                                       const float *b_scale, const int32_t *group_offsets,
                                       void *H, int32_t E, int32_t K, int32_t N, int32_t M_cap,
                                       int32_t bm, void *stream);

/*
 * gg_tile_schedule -- the flat tile list the product kernel consumes,
 * written out (worklog section 2: one descriptor per output tile of one
 * expert, expert-major order, tiles stopping at expert boundaries, empty
 * experts contributing none).
 *
 * The device builds it from group_offsets with exactly the code the product
 * kernel runs; tile t of the list is written as 5 int32
 *     tiles[5t .. 5t+4] = { expert, row0, rows, col0, bm }
 * in the order the product kernel walks tile ids. The set of descriptors is
 * the worklog's; the order is expert by expert, and inside an expert the M
 * tiles are taken in groups of up to 8 with the N tile outer and the M tile
 * inner in each group (so consecutive tiles share a column slice of the
 * expert's weights). Tiles are 256 columns wide, except when every expert
 * with rows has 16-row tiles: then they are 512 wide. At most
 * max_tiles descriptors are written; *n_tiles (a device int32) receives the
 * full count even when it exceeds max_tiles (0 for malformed offsets whose
 * overlapping groups exceed the bound stated at the top of this file).
 * Arguments E, N, M_cap, bm and the offsets rules are those of
 * gg_grouped_gemm_bf16; tiles may be NULL when max_tiles == 0.
 */
gg_status_t gg_tile_schedule(const int32_t *group_offsets, int32_t E, int32_t N, int32_t M_cap,
                             int32_t bm, int32_t *tiles, int32_t *n_tiles, int32_t max_tiles,
                             void *stream);

/* Static English text for a status code. */
const char *gg_status_string(gg_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_RAGGED_GROUPED_AMD_GROUPED_GEMM_H */
