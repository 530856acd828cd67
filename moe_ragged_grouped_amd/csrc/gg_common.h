// Shared device types and small helpers for the gfx950 grouped-GEMM kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gg {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) short s16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// LDS-typed pointers: keep every shared-memory access a ds_* instruction
// (a generic pointer would turn them into flat accesses that also wait on
// outstanding global loads).
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

constexpr int kThreads = 256;  // four 64-lane waves per workgroup
constexpr int kWave = 64;

__device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

// Global-memory typed pointers: keep loads and stores global_* instructions
// even where the compiler cannot see where a pointer came from (a generic
// pointer would become flat_* accesses, which also count against the LDS
// wait counter).
typedef __attribute__((address_space(1))) const u32x4 gbl_cu32x4;
typedef __attribute__((address_space(1))) f32x4 gbl_f32x4;

// One 16-byte global load (global_load_dwordx4).
__device__ __forceinline__ u32x4 ld_g16(const void *p) { return *(gbl_cu32x4 *)p; }

// One 16-byte global store (global_store_dwordx4).
__device__ __forceinline__ void st_g16(float *p, f32x4 v) { *(gbl_f32x4 *)p = v; }

// Transposing LDS read of a 4 (rows) x 16 (16-bit columns) block per 16-lane
// group (ds_read_b64_tr_b16). Lane 16g + s supplies the address of 4
// consecutive 16-bit values; the instruction returns to lane 16g + i the
// values (i % 4) of lanes 16g + i/4, 16g + 4 + i/4, 16g + 8 + i/4 and
// 16g + 12 + i/4. With lane 16g + s pointing at row s/4, columns 4(s%4)..+3
// of a row-major block, lane 16g + i receives column i of rows 0..3.
__device__ __forceinline__ s16x4 lds_read_tr16(const lds_u16 *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
}

}  // namespace gg
