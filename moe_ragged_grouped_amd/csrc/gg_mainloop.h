// One output tile of one expert on gfx950 bf16 matrix cores.
//
// The workgroup owns the tile's whole K reduction, so no cross-workgroup
// reduction exists ("Grouped GEMM for Imbalanced Experts on Blackwell: A WIP
// Worklog", Fig. 2 caption). Rows past the tile's valid count are padding:
// they are loaded as zeros, multiplied, and never stored (section 2.1 and the
// register-direct epilogue of section 4.1).
//
// MI355X mapping:
//  * Two workgroups of four waves per CU (at most 256 registers per wave, at
//    most 80 KiB of LDS per workgroup): for the weight-streaming shapes the
//    bytes in flight per CU, not the tile shape, set the achieved HBM
//    bandwidth, and a second resident workgroup doubles them.
//  * K runs in slices of BK: every thread moves 16-byte chunks global ->
//    registers (global_load_dwordx4) for slice k+1 while the matrix cores work
//    on slice k out of LDS, then writes them to the other of two LDS stages
//    (ds_write_b128); one barrier per slice.
//  * v_mfma_f32_16x16x32_bf16 computes C^T blocks: the first operand is a
//    16 (n) x 32 (k) slice of B^T, the second a 32 (k) x 16 (m) slice of A^T.
//    Both operands want 8 consecutive k per lane. A rows are K-contiguous in
//    LDS (one ds_read_b128 per lane); B is [K][N] N-contiguous, and its
//    fragments come from ds_read_b64_tr_b16, which transposes a 4 x 16
//    row-major block per 16-lane group on the way out of LDS. Rows of both
//    stages are padded by 16 bytes. The transposing read moves about 97 bytes
//    per clock per CU against 172 for ds_read_b128, so tall wave tiles (fewer
//    B fragments per flop) are preferred.
//  * The accumulator layout of C^T gives every lane 4 consecutive columns of
//    one row of C, so the epilogue is one 16-byte store per lane per block,
//    straight from registers with a per-lane row guard.
#pragma once

#include "gg_common.h"
#include "gg_schedule.h"

namespace gg {

template <int BM_, int BK_, int WM_, int WN_>
struct TileCfg {
  static constexpr int BM = BM_, BN = width_of(BM_), BK = BK_, WM = WM_, WN = WN_;
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

// Tile configurations per tile height (all 128 columns wide).
using Cfg16 = TileCfg<16, 64, 1, 4>;    // wave tile 16 x 32
using Cfg32 = TileCfg<32, 64, 1, 4>;    // wave tile 32 x 32
using Cfg64 = TileCfg<64, 64, 1, 4>;    // wave tile 64 x 32
using Cfg128 = TileCfg<128, 64, 2, 2>;  // wave tile 64 x 64
using Cfg256 = TileCfg<256, 32, 2, 2>;  // wave tile 128 x 64 (32-deep slices fit 2 stages)

struct TileArgs {
  const uint16_t *A;   // A rows of this tile: row r at A + r * K
  const uint16_t *B;   // B[e] + col0: element (k, n) at B + k * N + n
  float *C;            // C + row0 * N + col0
  int rows, K, N, ncols;  // ncols = valid columns in this tile (<= BN)
};

template <class C>
struct Staging {
  u32x4 a[C::A_PER_T];
  u32x4 b[C::B_PER_T];
};

// Global -> registers for the K slice starting at k0. Out-of-range chunks
// (rows past the tile's valid rows, K past the end, columns past N) are zero.
template <class C>
__device__ __forceinline__ void load_slice(Staging<C> &st, const TileArgs &t, int k0) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < C::A_PER_T; ++i) {
    const int c = tid + i * kThreads;
    const int r = c / (C::BK / 8), kc = c % (C::BK / 8);
    const int k = k0 + 8 * kc;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (c < C::A_CHUNKS && r < t.rows && k < t.K) v = ld_g16(t.A + (size_t)r * t.K + k);
    st.a[i] = v;
  }
#pragma unroll
  for (int i = 0; i < C::B_PER_T; ++i) {
    const int c = tid + i * kThreads;
    const int kr = c / (C::BN / 8), nc = c % (C::BN / 8);
    const int k = k0 + kr, n = 8 * nc;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (c < C::B_CHUNKS && k < t.K && n < t.ncols) v = ld_g16(t.B + (size_t)k * t.N + n);
    st.b[i] = v;
  }
}

// Registers -> one LDS stage.
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

// Matrix-core work on one LDS stage (BK/32 K steps of 32). The B fragments
// of a step are read first and kept; the A fragments are streamed one 16-row
// block at a time, which keeps a tall wave tile's register footprint small.
template <class C>
__device__ __forceinline__ void mma_stage(f32x4 (&acc)[C::NI][C::MI], const lds_u16 *As,
                                          const lds_u16 *Bs, int wm0, int wn0) {
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, s = lane % 16;
#pragma unroll
  for (int ks = 0; ks < C::BK / 32; ++ks) {
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
    for (int mi = 0; mi < C::MI; ++mi) {
      const lds_u16 *p = As + (wm0 + mi * 16 + s) * C::A_LD + ks * 32 + 8 * g;
      const bf16x8 y = __builtin_bit_cast(bf16x8, *(const lds_u32x4 *)p);
#pragma unroll
      for (int ni = 0; ni < C::NI; ++ni)
        acc[ni][mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x[ni], y, acc[ni][mi], 0, 0, 0);
    }
  }
}

// Full K loop and epilogue for one tile. lds must hold C::LDS_BYTES. Ends with
// a workgroup barrier, so the next tile may refill the stages at once.
template <class C>
__device__ __forceinline__ void run_tile(const TileArgs &t, lds_u16 *lds) {
  lds_u16 *const As0 = lds;                       // stage s: As0 + s * A_STAGE
  lds_u16 *const Bs0 = lds + 2 * C::A_STAGE;      // stage s: Bs0 + s * B_STAGE
  const int wave = threadIdx.x / kWave;
  const int wm0 = (wave / C::WN) * C::WTM;
  const int wn0 = (wave % C::WN) * C::WTN;

  f32x4 acc[C::NI][C::MI];
#pragma unroll
  for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi) acc[ni][mi] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int KT = cdiv(t.K, C::BK);
  Staging<C> st;
  load_slice<C>(st, t, 0);
  store_slice<C>(st, As0, Bs0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const bool more = kt + 1 < KT;
    const int cur = kt & 1, nxt = cur ^ 1;
    if (more) load_slice<C>(st, t, (kt + 1) * C::BK);
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
    if (m < t.rows) {
      float *crow = t.C + (size_t)m * t.N;
#pragma unroll
      for (int ni = 0; ni < C::NI; ++ni) {
        const int n = wn0 + ni * 16 + 4 * g;
        if (n < t.ncols) st_g16(crow + n, acc[ni][mi]);
      }
    }
  }
}

}  // namespace gg
