// Shared device types and small helpers for the gfx950 grouped-GEMM kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int kThreads = 512;  // eight 64-lane waves per workgroup
constexpr int kWave = 64;

__device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

__host__ __device__ constexpr int gcd(int a, int b) { return b == 0 ? a : gcd(b, a % b); }
__host__ __device__ constexpr int lcm(int a, int b) { return a / gcd(a, b) * b; }

// f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time.
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// Global-memory typed pointer: keeps the epilogue stores global_*
// instructions even where the compiler cannot see where a pointer came from
// (a generic pointer would become flat_* accesses, which also count against
// the LDS wait counter).
typedef __attribute__((address_space(1))) f32x4 gbl_f32x4;

// Raw buffer access (buffer_load_dwordx4 with a per-lane byte offset). The
// resource holds a base address and a size in bytes; a lane whose offset
// lies at or past the size reads zeros without touching memory. That range
// check is the zero fill of padding rows, of K past its end and of columns
// past N, with no branch and a 32-bit offset per lane instead of a 64-bit
// address.
typedef __amdgpu_buffer_rsrc_t buf_rsrc;
constexpr int kBufWord3 = 0x00020000;  // gfx9-family raw buffer, no swizzle
// A byte offset past every buffer this library describes (their sizes stay
// at or below 2^31).
constexpr uint32_t kOob = 0x80000000u;

__device__ __forceinline__ buf_rsrc make_buf(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           kBufWord3);
}

// Cache-policy operand of a buffer access (gfx950): nt marks the data as
// streaming, so it does not displace lines that other tiles will reuse.
constexpr int kCacheDefault = 0;
constexpr int kCacheStream = 2;  // nt

// One 16-byte load at base + voff + soff; zeros when the offset is out of range.
template <int POLICY = kCacheDefault>
__device__ __forceinline__ u32x4 ld_buf16(buf_rsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, POLICY);
}

// One 4-byte global load of an index (global_load_dword).
typedef __attribute__((address_space(1))) const int32_t gbl_ci32;
__device__ __forceinline__ int ld_g4(const int32_t *p) { return *(gbl_ci32 *)p; }

// One 4-byte global load of a float (global_load_dword).
typedef __attribute__((address_space(1))) const float gbl_cf32;
__device__ __forceinline__ float ld_g4f(const float *p) { return *(gbl_cf32 *)p; }

// One 16-byte global load of four floats (global_load_dwordx4).
typedef __attribute__((address_space(1))) const f32x4 gbl_cf32x4;
__device__ __forceinline__ f32x4 ld_g16f(const float *p) { return *(gbl_cf32x4 *)p; }

// Two fp8 e4m3 values (OCP, as v_cvt_scalef32_pk_bf16_fp8 reads them), the
// 16-bit half HIGH of a dword, -> two bf16 values in order. The scale
// operand is 1, so the conversion is exact.
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
template <bool HIGH>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HIGH));
}

// One 16-byte global store (global_store_dwordx4).
__device__ __forceinline__ void st_g16(float *p, f32x4 v) { *(gbl_f32x4 *)p = v; }

// What the epilogue writes: C in fp32, C rounded to bf16, the SwiGLU of
// interleaved (gate, up) column pairs rounded to bf16 (half as many columns),
// or (AddF32) each row times its weight added into fp32 destination rows.
enum class Out { F32, BF16, SwiGluBF16, AddF32 };

typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((address_space(1))) bf16x4 gbl_bf16x4;

// Four fp32 values rounded to bf16 (v_cvt_pk_bf16_f32, round to nearest even)
// and stored as one 8-byte global store.
__device__ __forceinline__ void st_g8_bf16(uint16_t *p, f32x4 v) {
  *(gbl_bf16x4 *)p = __builtin_convertvector(v, bf16x4);
}

// SwiGLU of one lane's four columns, taken as two (gate, up) pairs:
// v = (g0, u0, g1, u1) -> silu(g0) * u0, silu(g1) * u1 with
// silu(x) = x / (1 + e^-x) = x * rcp(1 + 2^(-x log2 e)), evaluated in fp32
// with the hardware exp2 and reciprocal (v_exp_f32, v_rcp_f32, each within
// one ulp). Rounding -x log2 e moves the exponent by up to |x| log2(e) 2^-23,
// so the result is within about (|x| + 3.5) 2^-23 of silu(x) * u relative; e^-x
// overflows to infinity for x below about -88.7, giving -0 where the exact
// value is below 3e-37. Each result is rounded once to bf16 (ties to even)
// and the pair stored as one 4-byte global store.
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((address_space(1))) bf16x2 gbl_bf16x2;
__device__ __forceinline__ float silu(float x) {
  constexpr float kLog2e = 1.4426950408889634f;
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * kLog2e));
}
__device__ __forceinline__ void st_g4_swiglu_bf16(uint16_t *p, f32x4 v) {
  const f32x2 h = {silu(v.x) * v.y, silu(v.z) * v.w};
  *(gbl_bf16x2 *)p = __builtin_convertvector(h, bf16x2);
}

// *p += v: one fp32 atomic add (global_atomic_add_f32, no return value;
// device memory). Adds to one element from several lanes or workgroups land
// in an unspecified order, each rounded once.
typedef __attribute__((address_space(1))) float gbl_f32;
__device__ __forceinline__ void atomic_add(float *p, float v) {
  __builtin_amdgcn_global_atomic_fadd_f32((gbl_f32 *)p, v);
}

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
