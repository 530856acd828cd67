/*
 * Per-tile timeline of the grouped product -- the tracing build's C ABI.
 *
 * A diagnostic for callers who measure the kernel, not part of the product
 * path: these entry points exist only in libmoe_ragged_grouped_amd_trace.so,
 * which is built from the same sources with GG_TILE_TRACE defined
 * (moe_ragged_grouped_amd/build.py). The product library carries no tracing
 * code. The timeline shows how long each tile takes and how evenly the
 * workgroups of the persistent launch finish once tiles of different heights
 * share the machine.
 *
 * The traced kernel is the product kernel with one workgroup barrier and
 * three reads of the constant-rate real-time counter added per tile, so its
 * tiles run a little slower than the product's. The tracing library also
 * exports the entry points of grouped_gemm.h; they compute what the product
 * library's do and record nothing.
 */
#ifndef MOE_RAGGED_GROUPED_AMD_GROUPED_GEMM_TRACE_H
#define MOE_RAGGED_GROUPED_AMD_GROUPED_GEMM_TRACE_H

#include <stdint.h>

#include "grouped_gemm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Workgroup records at the start of every trace buffer. */
#define GG_TRACE_WORKGROUPS 1024
/* uint64_t values per record. */
#define GG_TRACE_RECORD 8

/*
 * gg_trace_grouped_gemm_bf16 -- gg_grouped_gemm_bf16 (same arguments, same
 * result, same status codes) that also records a timeline.
 *
 *   trace  DEVICE buffer of uint64_t, 8-byte aligned, owned by the caller,
 *          holding GG_TRACE_RECORD * (GG_TRACE_WORKGROUPS + max_tiles) values:
 *          one record of GG_TRACE_RECORD values per workgroup, then one per
 *          tile. Times are counter ticks (gg_trace_clock_khz). The call writes
 *          - for workgroup b < GG_TRACE_WORKGROUPS of the launch, record b:
 *            the time it started, the time its tile list was built, its
 *            hardware location (the HIP __smid() value: XCC id in bits 6 and
 *            up, shader engine in bits 4-5, CU in bits 0-3), the number of
 *            tiles it ran, then zeros;
 *          - for tile t < max_tiles of the launch's tile list, record
 *            GG_TRACE_WORKGROUPS + t: its start (after the workgroup barrier
 *            that opens it), the time its descriptor was decoded, its end
 *            (after the barrier that closes its K loop), its height bm, the
 *            workgroup that ran it, its expert, valid rows and first column.
 *          Records of workgroups the launch does not have and of tiles past
 *          its tile count are left as they were: clear the buffer first.
 *   max_tiles  tiles to record (>= 0).
 * Errors: GG_ERR_INVALID_VALUE for a null trace or max_tiles < 0,
 * GG_ERR_MISALIGNED for a misaligned trace, else those of
 * gg_grouped_gemm_bf16.
 */
gg_status_t gg_trace_grouped_gemm_bf16(const void *A, const void *B,
                                       const int32_t *group_offsets, float *C, int32_t E,
                                       int32_t K, int32_t N, int32_t M_cap, int32_t bm,
                                       uint64_t *trace, int32_t max_tiles, void *stream);

/*
 * gg_trace_clock_khz -- the rate of the trace's counter on the current
 * device, in kHz (the HIP wall-clock rate attribute), written to the host
 * int *khz. GG_ERR_INVALID_VALUE for a null khz, GG_ERR_LAUNCH if the HIP
 * runtime cannot report it.
 */
gg_status_t gg_trace_clock_khz(int32_t *khz);

#ifdef __cplusplus
}
#endif

#endif /* MOE_RAGGED_GROUPED_AMD_GROUPED_GEMM_TRACE_H */
