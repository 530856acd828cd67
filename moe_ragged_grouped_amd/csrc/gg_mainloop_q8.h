// One output tile with fp8 activations and fp8 weights on the gfx950 fp8
// matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4, both operands OCP E4M3,
// unit block scales).
//
//   C[r][n] = a_scale[r] * b_scale[e][n] * sum_k dec(Aq[r][k]) * dec(Bq[e][k][n])
//
// The Pearl Pulse page "Pearl's grouped GEMM kernel for MoE models,
// explained" (section "What the 15% measures") says the kernel ships with an
// FP8 scheme and gives no details; one fp32 scale per activation row
// and one per weight column is the reading taken. The tile walk, the tile
// heights and widths, the buffer-resource zero fill and the epilogue layout
// are those of the bf16 kernel (gg_mainloop.h); what changes:
//  * a K slice is 128 deep and one matrix instruction covers it (16 x 16
//    outputs, 128 products per output), twice the products per byte of a
//    bf16 slice;
//  * both LDS stages hold bytes; rows are padded by 16 bytes;
//  * a lane's operand is 32 consecutive k of one row (A) or one column (B).
//    The hardware pairs byte j of the A lane with byte j of the B lane of the
//    same 16-lane group, so any k order shared by both operands is the same
//    product; here lane group g holds k = 32g .. 32g + 31 in order. A comes
//    from two ds_read_b128 per lane; B, stored [k][n] in LDS, from four
//    ds_read_b64_tr_b8, each of which hands lane i of a 16-lane group column
//    i of an 8 (k) x 16 (n) byte block (lane s of the group supplies the
//    address of row s/2, bytes 8 (s%2) .. 8 (s%2) + 7; both layouts were
//    checked by an in-bounds probe).
#pragma once

#include "gg_common.h"
#include "gg_mainloop.h"
#include "gg_schedule.h"

namespace gg {

typedef __attribute__((ext_vector_type(8))) int i32x8;

template <int BM_, int WM_, int WN_, int AD_, int BD_, int BN_ = kTileN>
struct TileCfgQ8 {
  static constexpr bool Q8 = true;
  static constexpr bool FP8B = true;  // per-column weight scales
  static constexpr int A_ELEM = 1, B_ELEM = 1;
  static constexpr int BM = BM_, BN = BN_, BK = 128, WM = WM_, WN = WN_;
  static constexpr int AD = AD_, BD = BD_;
  static_assert(WM * WN == kThreads / kWave, "one wave per wave tile");
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "16x16 blocks");
  static constexpr int MI = WTM / 16, NI = WTN / 16;
  static constexpr int A_LD = BK + 16;  // LDS row pitch of A (bytes)
  static constexpr int B_LD = BN + 16;  // LDS row pitch of B (bytes), one row per k
  static constexpr int A_STAGE = BM * A_LD, B_STAGE = BK * B_LD;  // bytes
  static constexpr int A_CHUNKS = BM * BK / 16, B_CHUNKS = BK * BN / 16;  // 16-byte chunks
  static constexpr int A_PER_T = (A_CHUNKS + kThreads - 1) / kThreads;
  static constexpr int B_PER_T = (B_CHUNKS + kThreads - 1) / kThreads;
  static constexpr int LDS_BYTES = 2 * (A_STAGE + B_STAGE);
  static_assert(kThreads % (BK / 16) == 0 && kThreads % (BN / 16) == 0, "chunk layout");
};

// Heights as in gg_mainloop.h. Every slice of these carries 32 KB of weights
// per 256 columns, as a 64-deep bf16 slice does, so the weight prefetch
// depths are the bf16 ones.
using CfgQ16 = TileCfgQ8<16, 1, 8, 1, 2>;
using CfgQ16W = TileCfgQ8<16, 1, 8, 1, 1, kWideN>;
using CfgQ32 = TileCfgQ8<32, 1, 8, 1, 2>;
using CfgQ64 = TileCfgQ8<64, 1, 8, 1, 2>;
using CfgQ128 = TileCfgQ8<128, 2, 4, 1, 2>;
using CfgQ256 = TileCfgQ8<256, 2, 4, 1, 1>;

template <class C>
struct LoadsQ8 {
  buf_rsrc a;                  // the tile's valid A rows: rows * K bytes
  uint32_t a_off[C::A_PER_T];  // chunk i of this thread at k0 = 0, or kOob
  uint32_t b_off[C::B_PER_T];  // chunk i of this thread inside a slice, or kOob
  int a_k;                     // K position of this thread's A chunks in a slice
};

template <class C>
struct StagingQ8 {
  u32x4 a[C::AD][C::A_PER_T];
  u32x4 b[C::BD][C::B_PER_T];
};

// Host limits keep every offset below 2^31 (rows * K <= 256 * K, 128 * N).
// K and N are multiples of 16, so no chunk straddles the end of a row.
template <class C>
__device__ __forceinline__ void init_loads_q8(LoadsQ8<C> &L, const TileArgs &t) {
  const int tid = t.tid;
  const int kc = tid % (C::BK / 16);
  L.a_k = 16 * kc;
  L.a = make_buf(t.A, (uint32_t)t.rows * (uint32_t)t.K);
#pragma unroll
  for (int i = 0; i < C::A_PER_T; ++i) {
    const int c = tid + i * kThreads;
    const uint32_t r = c / (C::BK / 16);
    L.a_off[i] = c < C::A_CHUNKS ? r * (uint32_t)t.K + 16u * kc : kOob;
  }
  const int n = 16 * (tid % (C::BN / 16));
#pragma unroll
  for (int i = 0; i < C::B_PER_T; ++i) {
    const int c = tid + i * kThreads;
    const uint32_t kr = c / (C::BN / 16);
    L.b_off[i] = (c < C::B_CHUNKS && n < t.ncols) ? kr * (uint32_t)t.N + n : kOob;
  }
}

template <class C>
__device__ __forceinline__ void load_a_q8(u32x4 (&a)[C::A_PER_T], const LoadsQ8<C> &L,
                                          const TileArgs &t, int k0) {
  const bool kin = k0 + L.a_k < t.K;
#pragma unroll
  for (int i = 0; i < C::A_PER_T; ++i) a[i] = ld_buf16(L.a, kin ? L.a_off[i] : kOob, (uint32_t)k0);
}

template <class C>
__device__ __forceinline__ void load_b_q8(u32x4 (&b)[C::B_PER_T], const LoadsQ8<C> &L,
                                          const TileArgs &t, int k0) {
  const long long rem = t.b_bytes - (long long)k0 * t.N;
  const uint32_t size = rem <= 0 ? 0u : (rem < kOob ? (uint32_t)rem : kOob);
  const buf_rsrc r = make_buf((const char *)t.B + (size_t)k0 * t.N, size);
#pragma unroll
  for (int i = 0; i < C::B_PER_T; ++i) b[i] = ld_buf16<kCacheStream>(r, L.b_off[i], 0u);
}

template <class C>
__device__ __forceinline__ void store_a_q8(const u32x4 (&a)[C::A_PER_T], lds_u8 *As, int tid) {
#pragma unroll
  for (int i = 0; i < C::A_PER_T; ++i) {
    const int c = tid + i * kThreads;
    const int r = c / (C::BK / 16), kc = c % (C::BK / 16);
    if (C::A_CHUNKS % kThreads == 0 || c < C::A_CHUNKS)
      *(lds_u32x4 *)(As + r * C::A_LD + 16 * kc) = a[i];
  }
}

template <class C>
__device__ __forceinline__ void store_b_q8(const u32x4 (&b)[C::B_PER_T], lds_u8 *Bs, int tid) {
#pragma unroll
  for (int i = 0; i < C::B_PER_T; ++i) {
    const int c = tid + i * kThreads;
    const int kr = c / (C::BN / 16), nc = c % (C::BN / 16);
    if (C::B_CHUNKS % kThreads == 0 || c < C::B_CHUNKS)
      *(lds_u32x4 *)(Bs + kr * C::B_LD + 16 * nc) = b[i];
  }
}

// The 128-deep slice in one stage: B^T operands (32 k of one column per
// lane) are read first and kept, A^T operands streamed per 16-row block.
// blk(mi) runs right after block mi's products (a no-op but in a tile's last
// slice, where block mi's accumulators are then final).
template <class C, class Blk>
__device__ __forceinline__ void mma_stage_q8(f32x4 (&acc)[C::NI][C::MI], const lds_u8 *As,
                                             const lds_u8 *Bs, int wm0, int wn0, int lane,
                                             Blk &&blk) {
  const int g = lane / 16, s = lane % 16;
  i32x8 x[C::NI];
#pragma unroll
  for (int ni = 0; ni < C::NI; ++ni) {
    const lds_u8 *p = Bs + (32 * g + s / 2) * C::B_LD + wn0 + ni * 16 + 8 * (s % 2);
    i32x2 q[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      q[j] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)(p + 8 * j * C::B_LD));
    x[ni] = i32x8{q[0].x, q[0].y, q[1].x, q[1].y, q[2].x, q[2].y, q[3].x, q[3].y};
  }
#pragma unroll
  for (int mi = 0; mi < C::MI; ++mi) {
    const lds_u8 *p = As + (wm0 + mi * 16 + s) * C::A_LD + 32 * g;
    const u32x4 lo = *(const lds_u32x4 *)p;
    const u32x4 hi = *(const lds_u32x4 *)(p + 16);
    const i32x8 y = __builtin_bit_cast(
        i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
    for (int ni = 0; ni < C::NI; ++ni)
      // formats 0, 0 = E4M3 for both operands; block scales 127 = 2^0
      acc[ni][mi] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x[ni], y, acc[ni][mi], 0, 0,
                                                                     0, 127, 0, 127);
    blk(mi);
  }
}

// The K-loop operations of the fp8 x fp8 tiles (see k_loop in gg_mainloop.h).
template <class C>
struct KOpsQ8 {
  LoadsQ8<C> &L;
  StagingQ8<C> &st;
  const TileArgs &t;
  lds_u8 *As0, *Bs0;
  f32x4 (*acc)[C::NI][C::MI];
  int wm0, wn0, lane;
  template <int J>
  __device__ __forceinline__ void load_a(Slot<J>, int kt) { load_a_q8<C>(st.a[J], L, t, kt * C::BK); }
  template <int J>
  __device__ __forceinline__ void load_b(Slot<J>, int kt) { load_b_q8<C>(st.b[J], L, t, kt * C::BK); }
  template <int J>
  __device__ __forceinline__ void store_a(Slot<J>, int stage) {
    store_a_q8<C>(st.a[J], As0 + stage * C::A_STAGE, t.tid);
  }
  template <int J>
  __device__ __forceinline__ void store_b(Slot<J>, int stage) {
    store_b_q8<C>(st.b[J], Bs0 + stage * C::B_STAGE, t.tid);
  }
  // one 128-deep K step per stage: mid() (the B loads) runs before it, then
  // blk(-1) (the last slice's epilogue set-up), then the products with
  // blk(mi) after block mi
  template <class Mid, class Blk>
  __device__ __forceinline__ void mma(int stage, Mid &&mid, Blk &&blk) {
    mid();
    __builtin_amdgcn_sched_barrier(0);
    blk(-1);
    mma_stage_q8<C>(*acc, As0 + stage * C::A_STAGE, Bs0 + stage * C::B_STAGE, wm0, wn0, lane,
                    blk);
  }
};

// Full K loop and epilogue of one fp8 tile (grouped rows; C in fp32, rounded
// once to bf16 when O is Out::BF16, or the bf16 SwiGLU of interleaved (gate,
// up) column pairs when O is Out::SwiGluBF16). The loop is the shared k_loop:
// A one slice and B BD slices ahead in registers, two LDS stages, one barrier
// per slice, a branch-free unrolled steady state.
template <class C, Out O>
__device__ __forceinline__ void run_tile_q8(const TileArgs &t, lds_u16 *lds_base) {
  lds_u8 *const lds = (lds_u8 *)lds_base;
  lds_u8 *const As0 = lds;                       // stage s: As0 + s * A_STAGE
  lds_u8 *const Bs0 = lds + 2 * C::A_STAGE;      // stage s: Bs0 + s * B_STAGE
  const int wave = __builtin_amdgcn_readfirstlane(t.tid / kWave);
  const int lane = t.tid % kWave;
  const int wm0 = (wave / C::WN) * C::WTM;
  const int wn0 = (wave % C::WN) * C::WTN;

  f32x4 acc[C::NI][C::MI];
#pragma unroll
  for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi) acc[ni][mi] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int KT = cdiv(t.K, C::BK);
  LoadsQ8<C> L;
  init_loads_q8<C>(L, t);
  StagingQ8<C> st;
  KOpsQ8<C> ops{L, st, t, As0, Bs0, &acc, wm0, wn0, lane};
  // epilogue: lane holds C[m][n..n+3] for m = s, n = 4g within each 16x16
  // block, times the row's activation scale and the columns' weight scales.
  // It runs inside the last slice: blk(-1) loads the scales (the staging
  // registers are free by then, as no slice follows), and each block is
  // stored right after its final products, so the stores drain while the
  // later blocks are multiplied.
  const int g = lane / 16, s = lane % 16;
  // C (or H) at row m, columns n..n+3, from the scaled accumulators v
  auto put = [&](int m, int n, f32x4 v) {
    if constexpr (O == Out::F32)
      st_g16((float *)t.C + (size_t)m * t.N + n, v);
    else if constexpr (O == Out::BF16)
      st_g8_bf16((uint16_t *)t.C + (size_t)m * t.N + n, v);
    else  // SwiGLU of the (gate, up) pairs (n, n+1), (n+2, n+3), scales applied
      st_g4_swiglu_bf16((uint16_t *)t.C + (size_t)m * (t.N / 2) + n / 2, v);
  };
  f32x4 bsc[C::NI];
  float asc[C::MI];
  auto epilogue = [&](int mi) {
    if (mi < 0) {
#pragma unroll
      for (int ni = 0; ni < C::NI; ++ni) {
        const int n = wn0 + ni * 16 + 4 * g;
        bsc[ni] = n < t.ncols ? ld_g16f(t.scale + n) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int i = 0; i < C::MI; ++i) {
        const int m = wm0 + i * 16 + s;
        asc[i] = m < t.rows ? ld_g4f(t.a_scale + m) : 0.f;
      }
      return;
    }
    const int m = wm0 + mi * 16 + s;
    if (m < t.rows) {
#pragma unroll
      for (int ni = 0; ni < C::NI; ++ni) {
        const int n = wn0 + ni * 16 + 4 * g;
        if (n < t.ncols) put(m, n, acc[ni][mi] * asc[mi] * bsc[ni]);
      }
    }
  };
  if constexpr (C::MI <= 4) {
    k_loop<C::AD, C::BD, 2>(KT, ops, epilogue);
  } else {
    // The tallest tile's registers do not hold the scales through its last
    // slice (it spilled), so it stores after the loop. Loading a scale per
    // block there would wait on the stores already issued (one counter
    // covers both), so the scales go through LDS, free once the loop's final
    // barrier has passed: each thread loads one row or column scale.
    // Measured against per-block loads (one box, outputs bitwise equal):
    // uniform16k 86.0 -> 80.3 us, skew16k 124.8 -> 116.7 us.
    static_assert(C::BM + C::BN <= kThreads, "one scale per thread");
    k_loop<C::AD, C::BD, 2>(KT, ops);
    lds_f32 *const sc = (lds_f32 *)lds_base;  // [BM] row scales, then [BN] column scales
    if (t.tid < C::BM) {
      sc[t.tid] = t.tid < t.rows ? ld_g4f(t.a_scale + t.tid) : 0.f;
    } else if (t.tid < C::BM + C::BN) {
      const int n = t.tid - C::BM;
      sc[C::BM + n] = n < t.ncols ? ld_g4f(t.scale + n) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi) {
      const int m = wm0 + mi * 16 + s;
      if (m < t.rows) {
        const float sa = sc[m];
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni) {
          const int n = wn0 + ni * 16 + 4 * g;
          if (n < t.ncols) put(m, n, acc[ni][mi] * sa * *(const lds_f32x4 *)(sc + C::BM + n));
        }
      }
    }
    __syncthreads();  // the next tile's first stage stores overwrite the scales
  }
}

}  // namespace gg
