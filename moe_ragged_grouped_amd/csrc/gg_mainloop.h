// One output tile of one expert on gfx950 bf16 matrix cores.
//
// The workgroup owns the tile's whole K reduction, so no cross-workgroup
// reduction exists ("Grouped GEMM for Imbalanced Experts on Blackwell: A WIP
// Worklog", Fig. 2 caption). Rows past the tile's valid count are padding:
// they are loaded as zeros, multiplied, and never stored (section 2.1 and the
// register-direct epilogue of section 4.1).
//
// MI355X mapping:
//  * v_mfma_f32_16x16x32_bf16 computes C^T blocks: the first operand is a
//    16 (n) x 32 (k) slice of B^T, the second a 32 (k) x 16 (m) slice of A^T.
//    Both operands then want 8 consecutive k per lane. A rows are already
//    K-contiguous (one 16-byte LDS read per lane); B is [K][N] N-contiguous,
//    so its fragments come from ds_read_b64_tr_b16, which transposes a
//    4 x 16 row-major block per 16-lane group on the way out of LDS.
//  * The accumulator layout of C^T gives every lane 4 consecutive columns of
//    one row of C, so the epilogue is one 16-byte store per lane per block,
//    straight from registers with a per-lane row guard.
//  * Global -> LDS staging: every thread moves 16-byte chunks
//    (global_load_dwordx4 / ds_write_b128); the next K slice is fetched into
//    registers while the matrix cores work on the current LDS stage (two LDS
//    stages, one barrier per K slice).
#pragma once

#include "gg_common.h"

namespace gg {

template <int BM_, int BN_, int BK_, int WM_, int WN_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
  static_assert(WM * WN == kThreads / kWave, "four waves per workgroup");
  static constexpr int WTM = BM / WM;  // rows of C per wave
  static constexpr int WTN = BN / WN;  // columns of C per wave
  static_assert(WTM % 16 == 0 && WTN % 16 == 0 && BK % 32 == 0, "16x16x32 blocks");
  static constexpr int MI = WTM / 16;
  static constexpr int NI = WTN / 16;
  static constexpr int A_LD = BK + 8;   // LDS row pitch (elements) of the A stage
  static constexpr int B_LD = BN + 8;   // LDS row pitch (elements) of the B stage
  static constexpr int A_STAGE = BM * A_LD;
  static constexpr int B_STAGE = BK * B_LD;
  static constexpr int A_CHUNKS = BM * BK / 8;  // 16-byte chunks per K slice
  static constexpr int B_CHUNKS = BK * BN / 8;
  static constexpr int A_PER_T = (A_CHUNKS + kThreads - 1) / kThreads;
  static constexpr int B_PER_T = (B_CHUNKS + kThreads - 1) / kThreads;
  static constexpr int LDS_BYTES = 2 * (A_STAGE + B_STAGE) * 2;
};

// Tile configurations per tile height (the tile width is 128 for all).
using Cfg16 = TileCfg<16, 128, 64, 1, 4>;
using Cfg32 = TileCfg<32, 128, 64, 1, 4>;
using Cfg64 = TileCfg<64, 128, 64, 1, 4>;
using Cfg128 = TileCfg<128, 128, 64, 2, 2>;

template <class C>
struct Staging {
  u32x4 a[C::A_PER_T];
  u32x4 b[C::B_PER_T];
};

// Global -> registers for K slice starting at k0. Out-of-range chunks are zero.
template <class C>
__device__ __forceinline__ void load_slice(Staging<C> &st, const uint16_t *__restrict__ A,
                                           const uint16_t *__restrict__ Be, int row0, int rows,
                                           int col0, int k0, int K, int N) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < C::A_PER_T; ++i) {
    const int c = tid + i * kThreads;
    const int r = c / (C::BK / 8), kc = c % (C::BK / 8);
    const int k = k0 + 8 * kc;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (c < C::A_CHUNKS && r < rows && k < K) v = ld_g16(A + (size_t)(row0 + r) * K + k);
    st.a[i] = v;
  }
#pragma unroll
  for (int i = 0; i < C::B_PER_T; ++i) {
    const int c = tid + i * kThreads;
    const int kr = c / (C::BN / 8), nc = c % (C::BN / 8);
    const int k = k0 + kr, n = col0 + 8 * nc;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (c < C::B_CHUNKS && k < K && n < N) v = ld_g16(Be + (size_t)k * N + n);
    st.b[i] = v;
  }
}

// Registers -> LDS stage.
template <class C>
__device__ __forceinline__ void store_slice(const Staging<C> &st, lds_u16 *As, lds_u16 *Bs) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < C::A_PER_T; ++i) {
    const int c = tid + i * kThreads;
    const int r = c / (C::BK / 8), kc = c % (C::BK / 8);
    if (c < C::A_CHUNKS) *(lds_u32x4 *)(As + r * C::A_LD + 8 * kc) = st.a[i];
  }
#pragma unroll
  for (int i = 0; i < C::B_PER_T; ++i) {
    const int c = tid + i * kThreads;
    const int kr = c / (C::BN / 8), nc = c % (C::BN / 8);
    if (c < C::B_CHUNKS) *(lds_u32x4 *)(Bs + kr * C::B_LD + 8 * nc) = st.b[i];
  }
}

// Matrix-core work on one LDS stage.
template <class C>
__device__ __forceinline__ void mma_stage(f32x4 (&acc)[C::NI][C::MI], const lds_u16 *As,
                                          const lds_u16 *Bs, int wm0, int wn0) {
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, s = lane % 16;
#pragma unroll
  for (int ks = 0; ks < C::BK / 32; ++ks) {
    bf16x8 y[C::MI];
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi) {
      const lds_u16 *p = As + (wm0 + mi * 16 + s) * C::A_LD + ks * 32 + 8 * g;
      y[mi] = __builtin_bit_cast(bf16x8, *(const lds_u32x4 *)p);
    }
    bf16x8 x[C::NI];
#pragma unroll
    for (int ni = 0; ni < C::NI; ++ni) {
      const lds_u16 *p = Bs + (ks * 32 + 8 * g + s / 4) * C::B_LD + wn0 + ni * 16 + 4 * (s % 4);
      const s16x4 lo = lds_read_tr16(p);
      const s16x4 hi = lds_read_tr16(p + 4 * C::B_LD);
      const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      x[ni] = __builtin_bit_cast(bf16x8, v);
    }
#pragma unroll
    for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
      for (int mi = 0; mi < C::MI; ++mi)
        acc[ni][mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x[ni], y[mi], acc[ni][mi], 0, 0, 0);
  }
}

// Full K loop and epilogue for one tile. lds must hold C::LDS_BYTES.
// Ends with a workgroup barrier, so the caller may reuse the LDS at once.
template <class C>
__device__ __forceinline__ void run_tile(const uint16_t *__restrict__ A,
                                         const uint16_t *__restrict__ Be, float *__restrict__ Cout,
                                         int row0, int rows, int col0, int K, int N, lds_u16 *lds) {
  // stage s: A at lds + s * A_STAGE, B at lds + 2 * A_STAGE + s * B_STAGE
  lds_u16 *const As0 = lds;
  lds_u16 *const Bs0 = lds + 2 * C::A_STAGE;
  const int wave = threadIdx.x / kWave;
  const int wm0 = (wave / C::WN) * C::WTM;
  const int wn0 = (wave % C::WN) * C::WTN;

  f32x4 acc[C::NI][C::MI];
#pragma unroll
  for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi) acc[ni][mi] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int KT = cdiv(K, C::BK);
  Staging<C> st;
  load_slice<C>(st, A, Be, row0, rows, col0, 0, K, N);
  store_slice<C>(st, As0, Bs0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const bool more = kt + 1 < KT;
    const int cur = kt & 1, nxt = cur ^ 1;
    if (more) load_slice<C>(st, A, Be, row0, rows, col0, (kt + 1) * C::BK, K, N);
    mma_stage<C>(acc, As0 + cur * C::A_STAGE, Bs0 + cur * C::B_STAGE, wm0, wn0);
    if (more) store_slice<C>(st, As0 + nxt * C::A_STAGE, Bs0 + nxt * C::B_STAGE);
    __syncthreads();
  }

  // epilogue: lane holds C[m][n..n+3] for m = s, n = 4g within each 16x16 block
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, s = lane % 16;
#pragma unroll
  for (int mi = 0; mi < C::MI; ++mi) {
    const int m = wm0 + mi * 16 + s;
    if (m < rows) {
      float *crow = Cout + (size_t)(row0 + m) * N;
#pragma unroll
      for (int ni = 0; ni < C::NI; ++ni) {
        const int n = col0 + wn0 + ni * 16 + 4 * g;
        if (n < N) *reinterpret_cast<f32x4 *>(crow + n) = acc[ni][mi];
      }
    }
  }
}

}  // namespace gg
