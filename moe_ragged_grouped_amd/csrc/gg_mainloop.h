// One output tile of one expert on gfx950 bf16 matrix cores.
//
// The workgroup owns the tile's whole K reduction, so no cross-workgroup
// reduction exists ("Grouped GEMM for Imbalanced Experts on Blackwell: A WIP
// Worklog", Fig. 2 caption). Rows past the tile's valid count are padding:
// they are loaded as zeros, multiplied, and never stored (section 2.1 and the
// register-direct epilogue of section 4.1).
//
// MI355X mapping:
//  * One workgroup of eight waves per CU (two waves per SIMD, at most 256
//    registers per wave; up to 141 KiB of LDS). Tiles are 256 columns wide
//    (512 for the 16-row tiles of a launch whose tiles are all 16 rows high),
//    so a tile's A rows are fetched once per 256 output columns. What
//    limits these kernels is how many bytes each CU's vector memory path
//    (address unit and L1) keeps in flight against the L2/HBM latency, so the
//    design minimises the bytes each CU must fetch (wide tiles, 128-byte row
//    segments from 64-deep K slices) and keeps two slices of B in flight.
//  * K runs in slices of BK: every thread moves 16-byte chunks global ->
//    registers (buffer_load_dwordx4) ahead of their use while the matrix
//    cores work on slice k out of LDS, then writes them to the other of two
//    LDS stages (ds_write_b128); one barrier per slice.
//  * v_mfma_f32_16x16x32_bf16 computes C^T blocks: the first operand is a
//    16 (n) x 32 (k) slice of B^T, the second a 32 (k) x 16 (m) slice of A^T.
//    Both operands want 8 consecutive k per lane. A rows are K-contiguous in
//    LDS (one ds_read_b128 per lane); B is [K][N] N-contiguous, and its
//    fragments come from ds_read_b64_tr_b16, which transposes a 4 x 16
//    row-major block per 16-lane group on the way out of LDS. Rows of both
//    operands are XOR-swizzled by 16-byte chunks (a_chunk, b_chunk below), so
//    no fragment read has a bank conflict. The transposing read moves at most
//    about 128 bytes per clock per CU (half the 16-byte read's rate), so
//    tall wave tiles (fewer B fragments per flop) are preferred.
//  * The accumulator layout of C^T gives every lane 4 consecutive columns of
//    one row of C, so the epilogue is one 16-byte store (fp32 C) or one 8-byte
//    store (bf16 C) per lane per block, straight from registers with a
//    per-lane row guard.
#pragma once

#include "gg_common.h"
#include "gg_schedule.h"

namespace gg {

template <int BM_, int BK_, int WM_, int WN_, int AD_, int BD_, bool FP8B_ = false, int NS_ = 2,
          int BN_ = kTileN>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
  // K slices of A and of B held in registers ahead of the LDS stage
  static constexpr int AD = AD_, BD = BD_;
  // LDS stages: 2 = the next slice is written while the current one is read
  // (one barrier per slice); 1 = write after a second barrier (half the LDS)
  static constexpr int NS = NS_;
  static_assert(NS == 1 || NS == 2, "LDS stages");
  static constexpr bool Q8 = false;  // bf16 activations (see gg_mainloop_q8.h)
  // B in HBM: bf16 (2 bytes) or fp8 e4m3 (1 byte, kept as fp8 in LDS and
  // widened to bf16 as its operand is read); one 16-byte global chunk holds
  // B_CE elements of a B row
  static constexpr bool FP8B = FP8B_;
  static constexpr int A_ELEM = 2;  // bytes per A element (bf16)
  static constexpr int B_ELEM = FP8B ? 1 : 2;
  static constexpr int B_CE = 16 / B_ELEM;
  static_assert(WM * WN == kThreads / kWave, "one wave per wave tile");
  static_assert(AD >= 1 && AD <= 3 && BD >= 1 && BD <= 4, "prefetch depths");
  static constexpr int WTM = BM / WM;  // rows of C per wave
  static constexpr int WTN = BN / WN;  // columns of C per wave
  static_assert(WTM % 16 == 0 && WTN % 16 == 0 && BK % 32 == 0, "16x16x32 blocks");
  static constexpr int MI = WTM / 16;
  static constexpr int NI = WTN / 16;
  // LDS row pitches (elements). Both operands' rows are XOR-swizzled by
  // 16-byte chunks so that a fragment read touches every bank once:
  //  * A rows are unpadded (BK elements, A_CH chunks); chunk c of row r sits
  //    at chunk c ^ (r % A_CH) (a_chunk). Measured with the kernel's own lane
  //    addresses (eight waves per CU): 4 LDS cycles per ds_read_b128, none
  //    of them bank conflicts, 234 bytes per clock per CU; rows padded to 144
  //    bytes (or 272 for 128-deep slices) take 8 cycles, half of them
  //    conflicts, 128 bytes per clock.
  //  * bf16 B rows are unpadded (BN elements); chunk c of row k sits at
  //    chunk c ^ b_swz(k) (b_chunk): 2 LDS cycles per ds_read_b64_tr_b16, no
  //    conflicts, against 4 cycles, half of them conflicts, with rows padded
  //    by 16 bytes (the 8-byte reads move at most 111-128 bytes per clock per
  //    CU either way).
  // Stores (ds_write_b128) take 8 cycles per instruction, counted as
  // conflict-free, with every layout here.
  static constexpr int A_LD = BK;
  static constexpr int A_CH = BK / 8;
  static_assert(A_CH == 8 || A_CH == 16, "A swizzle: 8 or 16 chunks per row");
  static constexpr int B_LD = BN;  // bf16 B rows, in elements
  // B row pitch in bytes. fp8 weights stay fp8 in LDS and are widened to
  // bf16 after the read, so that LDS holds and moves half the weight bytes.
  // Rows are padded by 16 bytes: the 8-bit transposing read then takes 2 LDS
  // cycles with no conflicts (32 bytes of padding: 4 cycles, half of them
  // conflicts; none: 32 cycles).
  static constexpr int B_LDB = FP8B ? BN + 16 : 2 * B_LD;
  static constexpr int A_STAGE = BM * A_LD;
  static constexpr int B_STAGE = BK * B_LDB / 2;  // in 16-bit units
  static constexpr int A_CHUNKS = BM * BK / 8;  // 16-byte chunks per K slice
  static constexpr int B_CHUNKS = BK * BN / B_CE;
  static constexpr int A_PER_T = (A_CHUNKS + kThreads - 1) / kThreads;
  static constexpr int B_PER_T = (B_CHUNKS + kThreads - 1) / kThreads;
  static constexpr int LDS_BYTES = NS * (A_STAGE + B_STAGE) * 2;
};

// Tile configurations per tile height (256 columns wide, and 512 for the
// 16-row tiles of launches whose tiles are all 16 rows high; eight waves).
using Cfg16 = TileCfg<16, 64, 1, 8, 1, 2>;    // wave tile 16 x 32
// 512 wide, B one slice ahead: a 64 KB slice per CU is already enough in
// flight (measured on the decode shape: one slice ahead 234 us, two 237,
// three 239; fp8 weights, half the bytes per slice, want two).
using Cfg16W = TileCfg<16, 64, 1, 8, 1, 1, false, 2, kWideN>;  // wave tile 16 x 64
using Cfg32 = TileCfg<32, 64, 1, 8, 1, 2>;    // wave tile 32 x 32
using Cfg64 = TileCfg<64, 64, 1, 8, 1, 2>;    // wave tile 64 x 32
using Cfg128 = TileCfg<128, 64, 2, 4, 1, 2>;  // wave tile 64 x 64
using Cfg256 = TileCfg<256, 64, 2, 4, 1, 2>;  // wave tile 128 x 64

// The same shapes with fp8 weights. A 64-deep fp8 slice of B is half the
// bytes of a bf16 one; the weight-streaming heights take 128-deep slices so
// that each CU keeps as many weight bytes in flight as with bf16.
using Cfg16F = TileCfg<16, 128, 1, 8, 1, 2, true>;
using Cfg16FW = TileCfg<16, 64, 1, 8, 1, 2, true, 2, kWideN>;  // 512 wide: a 64-deep slice
using Cfg32F = TileCfg<32, 128, 1, 8, 1, 2, true>;
using Cfg64F = TileCfg<64, 64, 1, 8, 1, 2, true>;
using Cfg128F = TileCfg<128, 64, 2, 4, 1, 2, true>;
using Cfg256F = TileCfg<256, 64, 2, 4, 1, 2, true>;

// Where a tile's A rows come from and where its C rows go.
//  Grouped: row r of the tile is row row0 + r of A and of C.
//  Indexed: row r reads X[src[r]] (src = src_rows + row0) and, when dst is
//  given, writes C[dst[r]] (dst = dst_rows + row0); otherwise C row row0 + r.
enum class Rows { Grouped, Indexed };

struct TileArgs {
  const void *A;       // Grouped: A rows of this tile (row r at A + r * K); Indexed: X
  const char *B;       // B[e] + col0: element (k, n) at byte (k * N + n) * B_ELEM
  void *C;             // C + row0 * N + col0 (C + col0 when dst is given); for SwiGLU
                       // output H + row0 * N/2 + col0/2
  int rows, K, N, ncols;  // ncols = valid columns in this tile (<= BN)
  long long b_bytes;   // bytes from B to the end of B[e]: (K * N - col0) * B_ELEM
  const float *scale;  // fp8 B: scale[e][col0 ..], one per output column; else null
  const float *a_scale;  // fp8 A: a_scale[row0 ..], one per row; else null
  int tid;             // threadIdx.x, re-derived per tile (see tile_body)
  // Indexed rows only
  const int32_t *src;  // src_rows + row0
  const int32_t *dst;  // dst_rows + row0, or null
  int n_src;           // rows of X; a source index outside [0, n_src) reads zeros
  int n_dst;           // rows of C; a destination outside [0, n_dst) is not written
  const float *wts;    // combine only: row_weights + row0 (grouped row r adds wts[r] * C)
};

// Register staging: the A chunks of the next AD K slices (slice s in
// a[s % AD]) and the B chunks of the next BD slices (slice s in b[s % BD]).
template <class C>
struct Staging {
  u32x4 a[C::AD][C::A_PER_T];
  u32x4 b[C::BD][C::B_PER_T];
};

// Per-thread load offsets of one tile. A thread's chunks of a K slice share
// one K position (A) or one column position (B), because the chunk index
// steps by the thread count, a multiple of the chunks per row.
template <class C>
struct Loads {
  static_assert(kThreads % (C::BK / 8) == 0 && kThreads % (C::BN / C::B_CE) == 0, "chunk layout");
  buf_rsrc a;                   // the tile's valid A rows: rows * K * 2 bytes
  uint32_t a_off[C::A_PER_T];   // chunk i of this thread at k0 = 0, or kOob
  uint32_t b_off[C::B_PER_T];   // chunk i of this thread inside a slice, or kOob
  int a_k;                      // K position of this thread's A chunks in a slice
};

// Host limits keep every offset below 2^31: rows * K * 2 <= 256 * K * 2 and
// BK * N * 2 <= 64 * N * 2.
template <class C, Rows R>
__device__ __forceinline__ void init_loads(Loads<C> &L, const TileArgs &t) {
  const int tid = t.tid;
  const int kc = tid % (C::BK / 8);
  L.a_k = 8 * kc;
  if constexpr (R == Rows::Grouped) {
    L.a = make_buf(t.A, (uint32_t)t.rows * (uint32_t)t.K * 2u);
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
      const int c = tid + i * kThreads;
      const uint32_t r = c / (C::BK / 8);
      L.a_off[i] = c < C::A_CHUNKS ? (r * (uint32_t)t.K + 8u * kc) * 2u : kOob;
    }
  } else {
    // the resource spans all of X (n_src * K * 2 <= 2^31 bytes, checked on
    // the host); a chunk's offset is its source row's, or kOob for padding
    // rows and for source indices outside [0, n_src)
    L.a = make_buf(t.A, (uint32_t)t.n_src * (uint32_t)t.K * 2u);
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
      const int c = tid + i * kThreads;
      const int r = c / (C::BK / 8);
      uint32_t off = kOob;
      if (c < C::A_CHUNKS && r < t.rows) {
        const int x = ld_g4(t.src + r);
        if (x >= 0 && x < t.n_src) off = ((uint32_t)x * (uint32_t)t.K + 8u * kc) * 2u;
      }
      L.a_off[i] = off;
    }
  }
  const int n = C::B_CE * (tid % (C::BN / C::B_CE));
#pragma unroll
  for (int i = 0; i < C::B_PER_T; ++i) {
    const int c = tid + i * kThreads;
    const uint32_t kr = c / (C::BN / C::B_CE);
    L.b_off[i] = (c < C::B_CHUNKS && n < t.ncols) ? (kr * (uint32_t)t.N + n) * C::B_ELEM : kOob;
  }
}

// Global -> registers for the K slice starting at k0. Rows past the tile's
// valid rows, K past its end and columns past N read as zero: the A resource
// ends at the last valid row, K-tail chunks of A get kOob, and the B resource
// of a slice ends where B[e] ends (a slice at or past K has size 0).
template <class C>
__device__ __forceinline__ void load_a(u32x4 (&a)[C::A_PER_T], const Loads<C> &L,
                                       const TileArgs &t, int k0) {
  const bool kin = k0 + L.a_k < t.K;
#pragma unroll
  for (int i = 0; i < C::A_PER_T; ++i) a[i] = ld_buf16(L.a, kin ? L.a_off[i] : kOob, 2u * k0);
}

// B is loaded as streaming data (nt): each weight byte feeds only the tiles
// of one column slice, which run side by side, and is not needed again.
// Measured on the whole launch: decode shape 258 -> 242 us, 16k uniform
// 142 -> 132 us; the same hint on A (reused by every column tile of an
// expert) or on the C stores made the 16k shapes slower.
template <class C>
__device__ __forceinline__ void load_b(u32x4 (&b)[C::B_PER_T], const Loads<C> &L,
                                       const TileArgs &t, int k0) {
  // bytes from the slice start to the end of B[e]; none for a slice past K
  const long long rem = t.b_bytes - (long long)k0 * t.N * C::B_ELEM;
  const uint32_t size = rem <= 0 ? 0u : (rem < kOob ? (uint32_t)rem : kOob);
  const buf_rsrc r = make_buf(t.B + (size_t)k0 * t.N * C::B_ELEM, size);
#pragma unroll
  for (int i = 0; i < C::B_PER_T; ++i) b[i] = ld_buf16<kCacheStream>(r, L.b_off[i], 0u);
}

// LDS chunk that holds 16-byte chunk c of A row r (the swizzle of TileCfg).
template <class C>
__device__ __forceinline__ int a_chunk(int r, int c) {
  return c ^ (r & (C::A_CH - 1));
}

// Registers -> one LDS stage.
template <class C>
__device__ __forceinline__ void store_a(const u32x4 (&a)[C::A_PER_T], lds_u16 *As, int tid) {
#pragma unroll
  for (int i = 0; i < C::A_PER_T; ++i) {
    const int c = tid + i * kThreads;
    const int r = c / C::A_CH, kc = c % C::A_CH;
    if (C::A_CHUNKS % kThreads == 0 || c < C::A_CHUNKS)
      *(lds_u32x4 *)(As + r * C::A_LD + 8 * a_chunk<C>(r, kc)) = a[i];
  }
}

// LDS chunk that holds 16-byte chunk c (columns 8c .. 8c + 7) of bf16 B row
// k. A transposing read instruction touches 16 rows, 8g + k' for lane group
// g (and 8g + 4 + k' for its second half), k' < 4, 32 bytes of each; the
// XOR moves those 32-byte pieces of rows k' and 8 + k' to eight different
// places within 256 bytes.
__device__ __forceinline__ int b_swz(int k) { return ((k & 3) << 1) | (((k >> 3) & 1) << 3); }
__device__ __forceinline__ int b_chunk(int k, int c) { return c ^ b_swz(k); }

template <class C>
__device__ __forceinline__ void store_b(const u32x4 (&b)[C::B_PER_T], lds_u16 *Bs, int tid) {
#pragma unroll
  for (int i = 0; i < C::B_PER_T; ++i) {
    const int c = tid + i * kThreads;
    const int kr = c / (C::BN / C::B_CE), nc = c % (C::BN / C::B_CE);
    if (C::B_CHUNKS % kThreads == 0 || c < C::B_CHUNKS) {
      if constexpr (C::FP8B) {
        // 16 fp8 values as they are
        *(lds_u32x4 *)((lds_u8 *)Bs + kr * C::B_LDB + 16 * nc) = b[i];
      } else {
        *(lds_u32x4 *)(Bs + kr * C::B_LD + 8 * b_chunk(kr, nc)) = b[i];
      }
    }
  }
}

// Matrix-core work on one LDS stage (BK/32 K steps of 32). The B fragments
// of a step are read first and kept; the A fragments are streamed one 16-row
// block at a time, which keeps a tall wave tile's register footprint small.
// mid() runs after the first half of the K steps (at the end when there is
// only one). blk(mi) runs in the last K step right after the products of
// 16-row block mi, whose accumulators are then final.
template <class C, class Mid, class Blk>
__device__ __forceinline__ void mma_stage(f32x4 (&acc)[C::NI][C::MI], const lds_u16 *As,
                                          const lds_u16 *Bs, int wm0, int wn0, int lane,
                                          Mid &&mid, Blk &&blk) {
  constexpr int KS = C::BK / 32;
  const int g = lane / 16, s = lane % 16;
  // bf16 B: byte address of this lane's first transposing read of column
  // block 0 (row 8g + s/4, columns wn0 + 4 (s % 4) ..). The swizzle puts
  // block ni's 32 bytes at block (ni ^ (s/4)) of the row's 32-byte pieces,
  // and nothing else sets address bits 5-6 (stage bases and rows are
  // 512-byte aligned), so block ni's address is this one XOR 32 ni.
  uint32_t b_base = 0;
  if constexpr (!C::FP8B) {
    static_assert(C::B_LD * 2 % 512 == 0 && C::B_STAGE * 2 % 512 == 0, "B rows, stages");
    const int k = 8 * g + s / 4, n = wn0 + 4 * (s % 4);
    b_base = (uint32_t)(uintptr_t)(Bs + k * C::B_LD + 8 * b_chunk(k, n / 8) + n % 8);
  }
#pragma unroll
  for (int ks = 0; ks < C::BK / 32; ++ks) {
    bf16x8 x[C::NI];
#pragma unroll
    for (int ni = 0; ni < C::NI; ++ni) {
      if constexpr (C::FP8B) {
        // ds_read_b64_tr_b8: lane 16g + s addresses row 8g + s/2, columns
        // 8(s%2)..+7 of an 8 x 16 byte block and receives column s of its
        // 8 rows: the 8 k of its operand, widened exactly to bf16
        const lds_u8 *p = (const lds_u8 *)Bs + (ks * 32 + 8 * g + s / 2) * C::B_LDB + wn0 +
                          ni * 16 + 8 * (s % 2);
        const i32x2 q = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)p);
        const u32x4 w = {fp8x2_to_bf16x2<false>((uint32_t)q.x), fp8x2_to_bf16x2<true>((uint32_t)q.x),
                         fp8x2_to_bf16x2<false>((uint32_t)q.y), fp8x2_to_bf16x2<true>((uint32_t)q.y)};
        x[ni] = __builtin_bit_cast(bf16x8, w);
      } else {
        // rows 32 ks + 8g + s/4 and + 4 (the swizzle of a row depends only
        // on its bits 0, 1 and 3), column block ni
        const lds_u16 *p = (const lds_u16 *)(uintptr_t)(b_base ^ (32u * ni)) + ks * 32 * C::B_LD;
        const s16x4 lo = lds_read_tr16(p);
        const s16x4 hi = lds_read_tr16(p + 4 * C::B_LD);
        const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        x[ni] = __builtin_bit_cast(bf16x8, v);
      }
    }
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi) {
      // row wm0 + mi * 16 + s (wm0 is a multiple of 16), chunk 4 ks + g
      const lds_u16 *p = As + (wm0 + mi * 16 + s) * C::A_LD + 8 * a_chunk<C>(s, 4 * ks + g);
      const bf16x8 y = __builtin_bit_cast(bf16x8, *(const lds_u32x4 *)p);
#pragma unroll
      for (int ni = 0; ni < C::NI; ++ni)
        acc[ni][mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x[ni], y, acc[ni][mi], 0, 0, 0);
      if (ks == KS - 1) blk(mi);
    }
    // one K step at a time: hoisting the next step's fragments above this
    // step's products would add their registers on top of the accumulators
    __builtin_amdgcn_sched_barrier(0);
    if (KS > 1 && ks == KS / 2 - 1) {
      mid();
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if constexpr (KS == 1) mid();
}

// The wave's LDS accesses issued so far have completed (so its other lanes
// see its writes), and the compiler moves no memory access across this
// point. A wave's LDS region shared by no other wave needs nothing more.
__device__ __forceinline__ void wave_lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Epilogue of the weighted combine: Y[dst[r]][n] += w[r] * C[r][n].
//
// The accumulator layout gives each lane four adjacent columns of one row,
// so one atomic instruction straight from it would touch 16 rows, 4 values
// of each. The atomic units of the L2 serve requests far faster when a
// wave's 64 lanes hit consecutive addresses (about 4x, measured with plain
// atomic kernels). So each wave stages one 16-row slab of its block at a
// time in LDS (already weighted) and reads it back row-major: every atomic
// instruction then covers 64 consecutive floats, one row of a 64-wide wave
// block or two rows of a 32-wide one. A wave uses only its own LDS region;
// a workgroup barrier at the end keeps the next tile's first LDS stores
// from overwriting a region another wave is still reading.
template <class C>
__device__ __forceinline__ void combine_epilogue(const TileArgs &t, f32x4 (&acc)[C::NI][C::MI],
                                                 lds_f32 *lds, int wave, int lane, int wm0,
                                                 int wn0) {
  constexpr int P = C::WTN + 4;         // row pitch of a staged slab (floats)
  constexpr int RPI = kWave / C::WTN;   // slab rows per atomic instruction
  static_assert(C::WTN * RPI == kWave && 16 % RPI == 0, "a row (or two) per instruction");
  static_assert(kThreads / kWave * 16 * P * 4 <= C::LDS_BYTES, "staging fits the stages");
  lds_f32 *const stage = lds + wave * 16 * P;
  const int g = lane / 16, s = lane % 16;
  const int rr = lane / C::WTN, cc = lane % C::WTN;  // read-back position in a row group
  const bool col_ok = wn0 + cc < t.ncols;
#pragma unroll
  for (int mi = 0; mi < C::MI; ++mi) {
    // lane s (and s + 16, s + 32, s + 48) owns slab row s: its destination
    // (-1 when there is none) and weight
    const int m = wm0 + mi * 16 + s;
    int d = -1;
    float w = 0.0f;
    if (m < t.rows) {
      const int x = ld_g4(t.dst + m);
      if (x >= 0 && x < t.n_dst) {
        d = x;
        w = ld_g4f(t.wts + m);
      }
    }
#pragma unroll
    for (int ni = 0; ni < C::NI; ++ni)
      *(lds_f32x4 *)(stage + s * P + ni * 16 + 4 * g) = acc[ni][mi] * w;
    // the wave's own LDS writes are complete before it reads them back
    wave_lds_fence();
    float v[16 / RPI];
#pragma unroll
    for (int k = 0; k < 16; k += RPI) v[k / RPI] = stage[(k + rr) * P + cc];
    // the reads are complete before the next slab overwrites the region
    wave_lds_fence();
#pragma unroll
    for (int k = 0; k < 16; k += RPI) {
      // destination of slab row k + rr, held by lane k + rr
      const int d0 = __builtin_amdgcn_readlane(d, k);
      const int dr = RPI == 1 ? d0 : (rr == 0 ? d0 : __builtin_amdgcn_readlane(d, k + 1));
      if (dr >= 0 && col_ok) atomic_add((float *)t.C + (size_t)dr * t.N + wn0 + cc, v[k / RPI]);
    }
  }
  __syncthreads();
}

// The K loop every operand type shares. Slices of A and B are loaded AD and
// BD slices ahead of their use. Tiles that share A rows or B columns run side
// by side and request the same lines at about the same time, so most loads
// wait for HBM, not L2. The steady-state loop (every slice but the last) is
// unrolled so that each staging buffer and each LDS stage has a fixed name,
// and its body is free of branches: slices past K are still "loaded" (all
// lanes out of range, so zeros and no memory traffic). The compiler's
// in-order vmcnt accounting then stores slice s+1 while the loads of later
// slices stay in flight.
//
// Where the loads issue matters. A CU's memory pipeline stays full, so a
// wave that issues a load can block until a slot frees. A's loads (one slice
// ahead) go out first, as they need the whole step to land. B's loads (two
// slices ahead) go out halfway through the matrix work, so that the eight
// waves do not all block at the step's start. Measured on one box against
// issuing both at the start: skew16k 178.5 -> 170.6 us, skew2k_wide 320.3 ->
// 305.5 us, uniform16k 130.8 -> 128.2 us, decode unchanged. Issuing A halfway
// instead was slower (skew2k_wide 396 us), and splitting both into quarters
// gained nothing over halves.
//
// Ops supplies, for a compile-time staging slot J: load_a(J, kt) and
// load_b(J, kt) (slice kt, global -> registers), store_a(J, stage) and
// store_b(J, stage) (registers -> LDS stage), and mma(stage, mid, blk), which
// runs mid() at its halfway point and, where the operand type supports it,
// blk(mi) once block mi's accumulators are final. blk is the epilogue of the
// tile's last slice (a no-op elsewhere). Ends with a workgroup barrier, so the
// next tile may refill the stages at once.
template <int J>
using Slot = std::integral_constant<int, J>;

struct NoBlk {
  __device__ __forceinline__ void operator()(int) const {}
};

template <int AD, int BD, int NS, class Ops, class Blk = NoBlk>
__device__ __forceinline__ void k_loop(int KT, Ops &ops, Blk &&last_blk = Blk{}) {
  static_for<(AD > BD ? AD : BD)>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    if constexpr (j < AD) ops.load_a(jc, j);
    if constexpr (j < BD) ops.load_b(jc, j);
  });
  ops.store_a(Slot<0>{}, 0);
  ops.store_b(Slot<0>{}, 0);
  __syncthreads();

  // one steady-state step: slice kt (kt % U == j) from its stage, slice kt + 1
  // into the other
  auto step = [&](auto jc, int kt) {
    constexpr int j = decltype(jc)::value;
    constexpr int cur = j % NS, nxt = (j + 1) % NS;
    ops.load_a(Slot<j % AD>{}, kt + AD);
    // keep the loads ahead of the matrix work (the scheduler would otherwise
    // sink them next to their LDS stores and expose their latency)
    __builtin_amdgcn_sched_barrier(0);
    // a wave in its matrix phase wins issue arbitration over the SIMD's other
    // wave, which meanwhile waits on its loads and LDS stores
    __builtin_amdgcn_s_setprio(1);
    // B's loads go out halfway through the matrix work rather than with A's
    ops.mma(cur, [&] { ops.load_b(Slot<j % BD>{}, kt + BD); }, NoBlk{});
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NS == 1) __syncthreads();  // every wave is done reading the stage
    ops.store_a(Slot<(j + 1) % AD>{}, nxt);
    ops.store_b(Slot<(j + 1) % BD>{}, nxt);
    __syncthreads();
  };
  // unroll factor: a multiple of AD, BD and 2
  constexpr int U = lcm(lcm(AD, BD), 2);
  int kt0 = 0;
  for (; kt0 + U <= KT - 1; kt0 += U)
    static_for<U>([&](auto jc) { step(jc, kt0 + decltype(jc)::value); });
  static_for<U - 1>([&](auto jc) {
    if (kt0 + decltype(jc)::value < KT - 1) step(jc, kt0 + decltype(jc)::value);
  });
  // the last slice sits in stage (KT - 1) % NS
  ops.mma((KT - 1) % NS, [] {}, last_blk);
  __syncthreads();
}

// The K-loop operations of the bf16-activation tiles (bf16 or fp8 weights).
template <class C>
struct KOpsBf16 {
  Loads<C> &L;
  Staging<C> &st;
  const TileArgs &t;
  lds_u16 *As0, *Bs0;
  f32x4 (*acc)[C::NI][C::MI];
  int wm0, wn0, lane;
  template <int J>
  __device__ __forceinline__ void load_a(Slot<J>, int kt) { gg::load_a<C>(st.a[J], L, t, kt * C::BK); }
  template <int J>
  __device__ __forceinline__ void load_b(Slot<J>, int kt) { gg::load_b<C>(st.b[J], L, t, kt * C::BK); }
  template <int J>
  __device__ __forceinline__ void store_a(Slot<J>, int stage) {
    gg::store_a<C>(st.a[J], As0 + stage * C::A_STAGE, t.tid);
  }
  template <int J>
  __device__ __forceinline__ void store_b(Slot<J>, int stage) {
    gg::store_b<C>(st.b[J], Bs0 + stage * C::B_STAGE, t.tid);
  }
  template <class Mid, class Blk>
  __device__ __forceinline__ void mma(int stage, Mid &&mid, Blk &&blk) {
    blk(-1);  // the last slice's epilogue set-up (nothing in other slices)
    mma_stage<C>(*acc, As0 + stage * C::A_STAGE, Bs0 + stage * C::B_STAGE, wm0, wn0, lane, mid,
                 blk);
  }
};

// Full K loop and epilogue for one tile. lds must hold C::LDS_BYTES. Ends with
// a workgroup barrier, so the next tile may refill the stages at once. O is
// what the epilogue writes: fp32 C (the accumulators as they are), bf16 C
// (rounded to nearest even), bf16 SwiGLU of (gate, up) column pairs into an
// output N/2 columns wide, or (indexed rows only) weight * C added into the
// destination rows with fp32 atomics. R says where rows come from and go.
template <class C, Out O, Rows R>
__device__ __forceinline__ void run_tile(const TileArgs &t, lds_u16 *lds) {
  lds_u16 *const As0 = lds;                       // stage s: As0 + s * A_STAGE
  lds_u16 *const Bs0 = lds + C::NS * C::A_STAGE;  // stage s: Bs0 + s * B_STAGE
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
  Loads<C> L;
  init_loads<C, R>(L, t);
  Staging<C> st;
  KOpsBf16<C> ops{L, st, t, As0, Bs0, &acc, wm0, wn0, lane};
  // epilogue: lane holds C[m][n..n+3] for m = s, n = 4g within each 16x16 block
  const int g = lane / 16, s = lane % 16;
  // What the stores need from global memory, loaded at the start of the last
  // slice (blk(-1)), when no slice follows and the staging registers are
  // free: the destination row of each of this lane's rows (gathered rows)
  // and the weight scales of its columns (fp8 weights).
  int dst_of[R == Rows::Indexed ? C::MI : 1];
  f32x4 scale_of[C::FP8B ? C::NI : 1];
  auto store_block = [&](int mi) {
    if (mi < 0) {
      if constexpr (R == Rows::Indexed) {
#pragma unroll
        for (int i = 0; i < C::MI; ++i) {
          const int m = wm0 + i * 16 + s;
          int d = m;
          if (t.dst != nullptr && m < t.rows) {
            d = ld_g4(t.dst + m);
            d = (d >= 0 && d < t.n_dst) ? d : -1;
          }
          dst_of[i] = d;
        }
      }
      if constexpr (C::FP8B) {
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni) {
          const int n = wn0 + ni * 16 + 4 * g;
          scale_of[ni] = n < t.ncols ? ld_g16f(t.scale + n) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
      return;
    }
    const int m = wm0 + mi * 16 + s;
    int dst_row = m;  // row of t.C this lane writes
    if constexpr (R == Rows::Indexed) dst_row = dst_of[mi];
    if (m < t.rows && dst_row >= 0) {
#pragma unroll
      for (int ni = 0; ni < C::NI; ++ni) {
        const int n = wn0 + ni * 16 + 4 * g;
        if (n < t.ncols) {
          f32x4 v = acc[ni][mi];
          if constexpr (C::FP8B) v *= scale_of[ni];  // per-column weight scale
          if constexpr (O == Out::F32)
            st_g16((float *)t.C + (size_t)dst_row * t.N + n, v);
          else if constexpr (O == Out::BF16)
            st_g8_bf16((uint16_t *)t.C + (size_t)dst_row * t.N + n, v);
          else  // H[row][n/2, n/2+1] from pairs (n, n+1), (n+2, n+3)
            st_g4_swiglu_bf16((uint16_t *)t.C + (size_t)dst_row * (t.N / 2) + n / 2, v);
        }
      }
    }
  };
  // Each block is stored during the last slice's matrix work, as soon as its
  // accumulators are final; the stores then drain while the later blocks are
  // multiplied. Measured against storing after the loop (one box, outputs
  // bitwise equal): fp8 weights skew16k 168.6 -> 157.8 us, uniform16k 120.0
  // -> 116.3 us; gathered rows uniform16k 133.8 -> 131.4 us. (The combine
  // stages through the LDS the last slice still reads, so it stores after.)
  constexpr bool kEarly = O != Out::AddF32;
  if constexpr (kEarly) {
    k_loop<C::AD, C::BD, C::NS>(KT, ops, store_block);
    return;
  }
  k_loop<C::AD, C::BD, C::NS>(KT, ops);
  if constexpr (O == Out::AddF32) {
    combine_epilogue<C>(t, acc, (lds_f32 *)lds, wave, lane, wm0, wn0);
    return;
  }
}

}  // namespace gg
