// Ragged-M grouped GEMM for gfx950: kernels and the C-ABI entry points
// declared in include/grouped_gemm.h. Built with GG_TILE_TRACE, the same
// source also gives the tracing library of include/grouped_gemm_trace.h: the
// blocks under that macro record a per-tile timeline, and the product
// library is compiled without them.
//
// One persistent launch serves every expert. Each workgroup rebuilds the
// tile-count prefix from the device-resident group offsets (gg_schedule.h),
// then walks tile ids with a stride of the grid size, decoding each id into
// {expert, row0, rows, col0, bm} and running that tile's K loop and epilogue
// (gg_mainloop.h). The grid is sized from the occupancy of the kernel (one
// eight-wave workgroup per CU once the tallest tiles are compiled in) and the
// CU count, capped by an upper bound of the tile count that the host can
// derive from M_cap alone, so the launch never waits on the group sizes.
//
// XCD-aware order: MI355X hands consecutive workgroup ids round-robin to its
// 8 XCDs, each with a private L2. Workgroup b processes, in its i-th round,
// tile i*G + (b % 8) * (G / 8) + b / 8, so every XCD works on a contiguous
// run of the expert-major list; tiles that share an expert's A rows (same M
// tile) or its weight columns (same N tile) then meet in the same L2.

#include "grouped_gemm.h"  // include/ (on the -I path)
#ifdef GG_TILE_TRACE
#include "grouped_gemm_trace.h"
#endif
#include "gg_common.h"
#include "gg_mainloop.h"
#include "gg_mainloop_q8.h"
#include "gg_schedule.h"

#include <mutex>
#include <type_traits>

namespace gg {

constexpr int kXcds = 8;

// Operand precisions: bf16 A and B; bf16 A with fp8 weights (kept as fp8
// in LDS, widened to bf16 as the operand is read); fp8 A and B on the fp8
// matrix cores.
enum Prec : int { kBf16 = 0, kW8 = 1, kW8A8 = 2 };

template <int P, class Bf16Cfg, class W8Cfg, class Q8Cfg>
using Pick = typename std::conditional<
    P == kW8A8, Q8Cfg, typename std::conditional<P == kW8, W8Cfg, Bf16Cfg>::type>::type;
constexpr int kMaxK = 1 << 22;
constexpr int kMaxN = 1 << 24;

struct Params {
  const uint16_t *A;
  const uint16_t *B;
  const int32_t *off;
  void *C;  // fp32 or bf16 [M_cap][N], or bf16 [M_cap][N/2] for SwiGLU
  int E, K, N, M_cap;
  int bm_fixed;  // 0 = per-expert choice
  // indexed rows (gather / scatter entry point) only
  const int32_t *src_rows;  // [M_cap]: grouped row r reads A row src_rows[r]
  const int32_t *dst_rows;  // [M_cap] or null: grouped row r writes C row dst_rows[r]
  int n_src;                // rows of A in the indexed form
  const float *b_scale;     // fp8 weights only: [E][N] per-column scales
  const float *a_scale;     // fp8 activations only: [M_cap] per-row scales
  int n_dst;                // indexed form: rows of C (M_cap, or the combine's n_dst)
  const float *row_w;       // combine only: [M_cap] weight of each grouped row
  int tile_cap;             // upper bound of the tile count (check_sizes)
#ifdef GG_TILE_TRACE
  unsigned long long *trace;  // the tracing build's records (grouped_gemm_trace.h)
  int trace_tiles;            // tiles with a record
#endif
};

#ifdef GG_TILE_TRACE
// The tracing build's clock: the constant-rate real-time counter, read with
// every earlier scalar read complete so that the reading is not deferred.
__device__ __forceinline__ unsigned long long trace_clock() {
  const unsigned long long c = __builtin_amdgcn_s_memrealtime();
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  return c;
}
#endif

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ const void *uniform_ptr(const void *p) {
  const uint64_t b = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  return (const void *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// One tile of one height: the tile's base pointers and sizes, then its K loop
// and epilogue. Every input is wave-uniform; readfirstlane makes that visible
// to the compiler, so these values live in scalar registers. In the kernel
// that compiles in all five heights this is what keeps the largest height's
// path within 256 VGPRs (two waves per SIMD) without spilling.
template <class Cfg, Out O, Rows R>
__device__ __forceinline__ void tile_body(const Params &p, int row0, int rows, int col0,
                                          int expert, uint32_t lds_addr) {
  const uint16_t *A = p.A, *B = p.B;
  void *C = p.C;
  int K = p.K, N = p.N;
  lds_u16 *const lds = (lds_u16 *)(uintptr_t)uniform((int)lds_addr);
  K = uniform(K);
  N = uniform(N);
  row0 = uniform(row0);
  col0 = uniform(col0);
  expert = uniform(expert);
  TileArgs a;
  a.B = (const char *)uniform_ptr(B) + ((size_t)expert * K * N + col0) * Cfg::B_ELEM;
  a.scale = Cfg::FP8B ? (const float *)uniform_ptr(p.b_scale) + (size_t)expert * N + col0
                      : nullptr;
  a.a_scale = Cfg::Q8 ? (const float *)uniform_ptr(p.a_scale) + row0 : nullptr;
  // bytes per C element, and C elements per product column (SwiGLU writes one
  // bf16 per (gate, up) pair)
  constexpr size_t kOutBytes = (O == Out::F32 || O == Out::AddF32) ? 4 : 2;
  constexpr int kColsPerOut = O == Out::SwiGluBF16 ? 2 : 1;
  if constexpr (R == Rows::Grouped) {
    a.A = (const char *)uniform_ptr(A) + (size_t)row0 * K * Cfg::A_ELEM;
    a.C = (char *)uniform_ptr(C) + ((size_t)row0 * N + col0) / kColsPerOut * kOutBytes;
    a.src = a.dst = nullptr;
    a.n_src = a.n_dst = 0;
  } else {
    a.A = uniform_ptr(A);
    a.src = (const int32_t *)uniform_ptr(p.src_rows) + row0;
    const int32_t *dst = (const int32_t *)uniform_ptr(p.dst_rows);
    a.dst = dst ? dst + row0 : nullptr;
    a.C = (char *)uniform_ptr(C) + ((size_t)(dst ? 0 : row0) * N + col0) * kOutBytes;
    a.n_src = uniform(p.n_src);
    a.n_dst = uniform(p.n_dst);
  }
  a.wts = O == Out::AddF32 ? (const float *)uniform_ptr(p.row_w) + row0 : nullptr;
  a.rows = uniform(rows);
  a.K = K;
  a.N = N;
  a.ncols = min(Cfg::BN, N - col0);
  a.b_bytes = ((long long)K * N - col0) * Cfg::B_ELEM;
  // The per-thread index arithmetic of a tile depends only on threadIdx.x; an
  // opaque copy per tile keeps the compiler from hoisting all of it out of
  // the persistent loop, where it would stay live (and spill) across tiles.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  a.tid = tid;
  if constexpr (Cfg::Q8) {
    static_assert(O != Out::AddF32 && R == Rows::Grouped,
                  "fp8 activations: grouped rows; fp32, bf16 or SwiGLU output");
    run_tile_q8<Cfg, O>(a, lds);
  } else {
    run_tile<Cfg, O, R>(a, lds);
  }
}

template <class Cfg, Out O, Rows R>
__device__ __forceinline__ void tile_call(const Params &p, const Tile &t, uint32_t lds_addr) {
  tile_body<Cfg, O, R>(p, t.row0, t.rows, t.col0, t.expert, lds_addr);
}

// LDS stage bytes a launch needs: the largest of the heights it compiles in.
template <int MASK, int P>
constexpr int lds_bytes() {
  int m = 0;
  if (MASK & 1) m = m > Pick<P, Cfg16, Cfg16F, CfgQ16>::LDS_BYTES ? m : Pick<P, Cfg16, Cfg16F, CfgQ16>::LDS_BYTES;
  if (MASK & 1) m = m > Pick<P, Cfg16W, Cfg16FW, CfgQ16W>::LDS_BYTES ? m : Pick<P, Cfg16W, Cfg16FW, CfgQ16W>::LDS_BYTES;
  if (MASK & 2) m = m > Pick<P, Cfg32, Cfg32F, CfgQ32>::LDS_BYTES ? m : Pick<P, Cfg32, Cfg32F, CfgQ32>::LDS_BYTES;
  if (MASK & 4) m = m > Pick<P, Cfg64, Cfg64F, CfgQ64>::LDS_BYTES ? m : Pick<P, Cfg64, Cfg64F, CfgQ64>::LDS_BYTES;
  if (MASK & 8)
    m = m > Pick<P, Cfg128, Cfg128F, CfgQ128>::LDS_BYTES ? m : Pick<P, Cfg128, Cfg128F, CfgQ128>::LDS_BYTES;
  if (MASK & 16)
    m = m > Pick<P, Cfg256, Cfg256F, CfgQ256>::LDS_BYTES ? m : Pick<P, Cfg256, Cfg256F, CfgQ256>::LDS_BYTES;
  return m;
}

// MASK bit c compiles in tile height 16 << c (16, 32, 64, 128, 256). A launch
// must compile in every height its schedule can produce. O is the element
// type of C; R says whether rows are grouped or gathered/scattered by index;
// P selects the operand precisions (bf16; fp8 weights; fp8 weights and
// activations).
// The launch's LDS: the operand stages from address 0 (the swizzled layouts
// assume 512-byte aligned stages), then the schedule table.
template <int MASK, int P>
constexpr int sched_offset() { return (lds_bytes<MASK, P>() + 15) / 16 * 16; }
template <int MASK, int P>
constexpr int launch_lds_bytes() { return sched_offset<MASK, P>() + (int)sizeof(SchedLds); }

template <int MASK, Out O, Rows R, int P>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(Params p) {
  // the kernel declares no static LDS, so this region starts at address 0
  extern __shared__ __attribute__((aligned(16))) uint16_t lds_dyn[];
  SchedLds &sched = *(SchedLds *)((char *)lds_dyn + sched_offset<MASK, P>());
  // the LDS base as a plain byte address pinned in a scalar register (the
  // empty asm keeps the compiler from rematerialising it in vector registers)
  uint32_t lds = (uint32_t)(uintptr_t)(lds_u16 *)lds_dyn;
  asm volatile("" : "+s"(lds));
#ifdef GG_TILE_TRACE
  const unsigned long long t_entry = trace_clock();
#endif
  const int total = build_schedule(sched, p.off, p.E, p.M_cap, p.N, p.bm_fixed, p.tile_cap);
  const int G = gridDim.x;  // a multiple of kXcds
  const int b = blockIdx.x;
  const int slot = (b % kXcds) * (G / kXcds) + b / kXcds;
#ifdef GG_TILE_TRACE
  const unsigned long long t_built = trace_clock();
  int n_run = 0;
#endif
  for (int base = 0; base < total; base += G) {
    const int t = base + slot;
    if (t >= total) break;
#ifdef GG_TILE_TRACE
    __syncthreads();  // every wave has left the previous tile
    const unsigned long long t_start = trace_clock();
#endif
    const Tile tl = decode_tile(sched, p.off, t, p.E, p.M_cap, p.N, p.bm_fixed);
#ifdef GG_TILE_TRACE
    const unsigned long long t_decoded = trace_clock();
#endif
    switch (tl.bm) {
      case 16:
        if constexpr (MASK & 1) {
          if (tl.bn == kWideN) tile_call<Pick<P, Cfg16W, Cfg16FW, CfgQ16W>, O, R>(p, tl, lds);
          else tile_call<Pick<P, Cfg16, Cfg16F, CfgQ16>, O, R>(p, tl, lds);
        }
        break;
      case 32: if constexpr (MASK & 2) tile_call<Pick<P, Cfg32, Cfg32F, CfgQ32>, O, R>(p, tl, lds); break;
      case 64: if constexpr (MASK & 4) tile_call<Pick<P, Cfg64, Cfg64F, CfgQ64>, O, R>(p, tl, lds); break;
      case 128:
        if constexpr (MASK & 8) tile_call<Pick<P, Cfg128, Cfg128F, CfgQ128>, O, R>(p, tl, lds);
        break;
      default:
        if constexpr (MASK & 16) tile_call<Pick<P, Cfg256, Cfg256F, CfgQ256>, O, R>(p, tl, lds);
        break;
    }
#ifdef GG_TILE_TRACE
    // the tile's K loop ends with a workgroup barrier, so every wave is done
    const unsigned long long t_end = trace_clock();
    ++n_run;
    if (threadIdx.x == 0 && p.trace != nullptr && t < p.trace_tiles) {
      unsigned long long *r = p.trace + GG_TRACE_RECORD * (GG_TRACE_WORKGROUPS + (size_t)t);
      r[0] = t_start;
      r[1] = t_decoded;
      r[2] = t_end;
      r[3] = (unsigned long long)tl.bm;
      r[4] = (unsigned long long)b;
      r[5] = (unsigned long long)tl.expert;
      r[6] = (unsigned long long)tl.rows;
      r[7] = (unsigned long long)tl.col0;
    }
#endif
  }
#ifdef GG_TILE_TRACE
  // the library's other entry points, also in the tracing build, pass no buffer
  if (threadIdx.x == 0 && p.trace != nullptr && b < GG_TRACE_WORKGROUPS) {
    unsigned long long *r = p.trace + GG_TRACE_RECORD * (size_t)b;
    r[0] = t_entry;
    r[1] = t_built;
    r[2] = __smid();  // XCC id << 6 | shader engine << 4 | CU
    r[3] = (unsigned long long)n_run;
  }
#endif
}

__global__ __launch_bounds__(kThreads) void tile_schedule_kernel(const int32_t *off, int E, int N,
                                                                 int M_cap, int bm_fixed,
                                                                 int tile_cap, int32_t *tiles,
                                                                 int32_t *n_tiles, int max_tiles) {
  __shared__ SchedLds sched;
  const int total = build_schedule(sched, off, E, M_cap, N, bm_fixed, tile_cap);
  if (threadIdx.x == 0) *n_tiles = total;
  const int lim = total < max_tiles ? total : max_tiles;
  for (int t = threadIdx.x; t < lim; t += kThreads) {
    const Tile tl = decode_tile(sched, off, t, E, M_cap, N, bm_fixed);
    int32_t *o = tiles + 5 * (size_t)t;
    o[0] = tl.expert;
    o[1] = tl.row0;
    o[2] = tl.rows;
    o[3] = tl.col0;
    o[4] = tl.bm;
  }
}

// Every launch's LDS (stages + the schedule table) must fit one CU's 160 KiB.
constexpr int kLdsPerCu = 160 * 1024;
static_assert(launch_lds_bytes<31, kBf16>() <= kLdsPerCu, "LDS budget");
static_assert(launch_lds_bytes<31, kW8>() <= kLdsPerCu, "LDS budget");
static_assert(launch_lds_bytes<31, kW8A8>() <= kLdsPerCu, "LDS budget");

// Per-device, per-variant launch limits (CU count x resident workgroups).
struct LaunchInfo {
  int grid = 0;
  hipError_t err = hipSuccess;
};

constexpr int kMaxDevices = 64;

template <int MASK, Out O, Rows R, int P>
static LaunchInfo launch_info(int dev) {
  static LaunchInfo cache[kMaxDevices];
  static std::once_flag once[kMaxDevices];
  std::call_once(once[dev], [dev]() {
    LaunchInfo li;
    int cus = 0, per_cu = 0;
    const int lds = launch_lds_bytes<MASK, P>();
    li.err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (li.err == hipSuccess)
      li.err = hipFuncSetAttribute((const void *)grouped_gemm_kernel<MASK, O, R, P>,
                                   hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (li.err == hipSuccess)
      li.err = hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, (const void *)grouped_gemm_kernel<MASK, O, R, P>, kThreads, lds);
    if (li.err == hipSuccess) {
      if (per_cu < 1) per_cu = 1;
      li.grid = cus * per_cu;
      li.grid -= li.grid % kXcds;
      if (li.grid < kXcds) li.grid = kXcds;
    }
    cache[dev] = li;
  });
  return cache[dev];
}

template <int MASK, Out O, Rows R, int P>
static gg_status_t launch(const Params &p, long long tile_bound, hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GG_ERR_LAUNCH;
  const LaunchInfo li = launch_info<MASK, O, R, P>(dev);
  if (li.err != hipSuccess) return GG_ERR_LAUNCH;
  long long g = tile_bound < li.grid ? tile_bound : li.grid;
  g = (g + kXcds - 1) / kXcds * kXcds;  // keep a multiple of the XCD count
  constexpr int lds = launch_lds_bytes<MASK, P>();
  hipLaunchKernelGGL((grouped_gemm_kernel<MASK, O, R, P>), dim3((unsigned)g), dim3(kThreads),
                     lds, stream, p);
  return hipGetLastError() == hipSuccess ? GG_OK : GG_ERR_LAUNCH;
}

static bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Shared argument checks; fills the tile-count upper bound.
static gg_status_t check_sizes(const int32_t *off, int E, int N, int M_cap, int bm,
                               long long *tile_bound) {
  if (off == nullptr) return GG_ERR_INVALID_VALUE;
  if (E < 1 || N < 1 || M_cap < 0) return GG_ERR_INVALID_VALUE;
  if (!(bm == 0 || bm == 16 || bm == 32 || bm == 64 || bm == 128 || bm == 256))
    return GG_ERR_INVALID_VALUE;
  if (E > kMaxExperts) return GG_ERR_UNSUPPORTED;
  if (!aligned(off, 4)) return GG_ERR_MISALIGNED;
  if (N % 8 != 0) return GG_ERR_MISALIGNED;
  const long long hmin = bm ? bm : 16;
  const long long nt = (N + kTileN - 1) / kTileN;
  const long long bound = ((long long)M_cap / hmin + E) * nt;
  // tile ids, rows + tile height and 5*tile indices must stay inside int32
  if (bound > (1LL << 28) || (long long)M_cap + 256 > INT32_MAX) return GG_ERR_UNSUPPORTED;
  *tile_bound = bound;
  return GG_OK;
}

// The product with C of element type O, rows of form R and operand
// precisions P: argument checks, then one launch.
template <Out O, Rows R, int P = kBf16>
static gg_status_t grouped_gemm(Params p, void *stream) {
  long long bound = 0;
  gg_status_t st = check_sizes(p.off, p.E, p.N, p.M_cap, p.bm_fixed, &bound);
  if (st != GG_OK) return st;
  if (p.A == nullptr || p.B == nullptr || p.C == nullptr || p.K < 1) return GG_ERR_INVALID_VALUE;
  if (p.K % 8 != 0) return GG_ERR_MISALIGNED;
  // 32-bit buffer offsets: a tile's A rows (256 * K * 2 bytes) and a K slice
  // of B (64 * N * 2 bytes) must stay below 2^31 bytes
  if (p.K > kMaxK || p.N > kMaxN) return GG_ERR_UNSUPPORTED;
  if (!aligned(p.A, 16) || !aligned(p.B, 16) || !aligned(p.C, 16)) return GG_ERR_MISALIGNED;
  if constexpr (R == Rows::Indexed) {
    if (p.src_rows == nullptr || p.n_src < 0) return GG_ERR_INVALID_VALUE;
    if (!aligned(p.src_rows, 4) || (p.dst_rows && !aligned(p.dst_rows, 4)))
      return GG_ERR_MISALIGNED;
    // the A resource covers all of X with 32-bit offsets
    if ((long long)p.n_src * p.K * 2 > (1LL << 31)) return GG_ERR_UNSUPPORTED;
  }
  if constexpr (O == Out::AddF32) {
    static_assert(R == Rows::Indexed, "the combine scatters by index");
    if (p.dst_rows == nullptr || p.row_w == nullptr || p.n_dst < 0) return GG_ERR_INVALID_VALUE;
    if (!aligned(p.row_w, 4)) return GG_ERR_MISALIGNED;
  }
  if constexpr (P != kBf16) {
    if (p.b_scale == nullptr) return GG_ERR_INVALID_VALUE;
    if (!aligned(p.b_scale, 16)) return GG_ERR_MISALIGNED;
  }
  if constexpr (P == kW8A8) {
    // 16-byte chunks of one row hold 16 fp8 values
    if (p.a_scale == nullptr) return GG_ERR_INVALID_VALUE;
    if (!aligned(p.a_scale, 4) || p.K % 16 != 0 || p.N % 16 != 0) return GG_ERR_MISALIGNED;
  }
  if (p.M_cap == 0 || bound == 0) return GG_OK;
  p.tile_cap = (int)bound;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (p.bm_fixed) {
    case 16: return launch<1, O, R, P>(p, bound, s);
    case 32: return launch<2, O, R, P>(p, bound, s);
    case 64: return launch<4, O, R, P>(p, bound, s);
    case 128: return launch<8, O, R, P>(p, bound, s);
    case 256: return launch<16, O, R, P>(p, bound, s);
    default: return launch<31, O, R, P>(p, bound, s);
  }
}

static Params make_params(const void *A, const void *B, const int32_t *off, void *C, int32_t E,
                          int32_t K, int32_t N, int32_t M_cap, int32_t bm) {
  return Params{static_cast<const uint16_t *>(A), static_cast<const uint16_t *>(B), off, C, E, K,
                N, M_cap, bm, nullptr, nullptr, 0, nullptr, nullptr, M_cap, nullptr, 0};
}

}  // namespace gg

using namespace gg;

extern "C" gg_status_t gg_grouped_gemm_bf16(const void *A, const void *B,
                                            const int32_t *group_offsets, float *C, int32_t E,
                                            int32_t K, int32_t N, int32_t M_cap, int32_t bm,
                                            void *stream) {
  return grouped_gemm<Out::F32, Rows::Grouped>(
      make_params(A, B, group_offsets, C, E, K, N, M_cap, bm), stream);
}

extern "C" gg_status_t gg_grouped_gemm_bf16_bf16out(const void *A, const void *B,
                                                    const int32_t *group_offsets, void *C,
                                                    int32_t E, int32_t K, int32_t N,
                                                    int32_t M_cap, int32_t bm, void *stream) {
  return grouped_gemm<Out::BF16, Rows::Grouped>(
      make_params(A, B, group_offsets, C, E, K, N, M_cap, bm), stream);
}

extern "C" gg_status_t gg_grouped_gemm_bf16_swiglu(const void *A, const void *B,
                                                   const int32_t *group_offsets, void *H,
                                                   int32_t E, int32_t K, int32_t N, int32_t M_cap,
                                                   int32_t bm, void *stream) {
  return grouped_gemm<Out::SwiGluBF16, Rows::Grouped>(
      make_params(A, B, group_offsets, H, E, K, N, M_cap, bm), stream);
}

extern "C" gg_status_t gg_grouped_gemm_bf16_gather(const void *X, int32_t n_src,
                                                   const int32_t *src_rows, const void *B,
                                                   const int32_t *group_offsets, float *C,
                                                   const int32_t *dst_rows, int32_t E, int32_t K,
                                                   int32_t N, int32_t M_cap, int32_t bm,
                                                   void *stream) {
  Params p = make_params(X, B, group_offsets, C, E, K, N, M_cap, bm);
  p.src_rows = src_rows;
  p.dst_rows = dst_rows;
  p.n_src = n_src;
  return grouped_gemm<Out::F32, Rows::Indexed>(p, stream);
}

extern "C" gg_status_t gg_grouped_gemm_bf16_gather_combine(
    const void *X, int32_t n_src, const int32_t *src_rows, const void *B,
    const int32_t *group_offsets, const int32_t *dst_rows, const float *row_weights, float *Y,
    int32_t n_dst, int32_t E, int32_t K, int32_t N, int32_t M_cap, int32_t bm, void *stream) {
  Params p = make_params(X, B, group_offsets, Y, E, K, N, M_cap, bm);
  p.src_rows = src_rows;
  p.dst_rows = dst_rows;
  p.n_src = n_src;
  p.n_dst = n_dst;
  p.row_w = row_weights;
  return grouped_gemm<Out::AddF32, Rows::Indexed>(p, stream);
}

extern "C" gg_status_t gg_grouped_gemm_fp8w(const void *A, const void *Bq, const float *b_scale,
                                            const int32_t *group_offsets, float *C, int32_t E,
                                            int32_t K, int32_t N, int32_t M_cap, int32_t bm,
                                            void *stream) {
  Params p = make_params(A, Bq, group_offsets, C, E, K, N, M_cap, bm);
  p.b_scale = b_scale;
  return grouped_gemm<Out::F32, Rows::Grouped, kW8>(p, stream);
}

extern "C" gg_status_t gg_grouped_gemm_fp8(const void *Aq, const float *a_scale, const void *Bq,
                                           const float *b_scale, const int32_t *group_offsets,
                                           float *C, int32_t E, int32_t K, int32_t N,
                                           int32_t M_cap, int32_t bm, void *stream) {
  Params p = make_params(Aq, Bq, group_offsets, C, E, K, N, M_cap, bm);
  p.a_scale = a_scale;
  p.b_scale = b_scale;
  return grouped_gemm<Out::F32, Rows::Grouped, kW8A8>(p, stream);
}

extern "C" gg_status_t gg_grouped_gemm_fp8_bf16out(const void *Aq, const float *a_scale,
                                                   const void *Bq, const float *b_scale,
                                                   const int32_t *group_offsets, void *C,
                                                   int32_t E, int32_t K, int32_t N,
                                                   int32_t M_cap, int32_t bm, void *stream) {
  Params p = make_params(Aq, Bq, group_offsets, C, E, K, N, M_cap, bm);
  p.a_scale = a_scale;
  p.b_scale = b_scale;
  return grouped_gemm<Out::BF16, Rows::Grouped, kW8A8>(p, stream);
}

extern "C" gg_status_t gg_grouped_gemm_fp8_swiglu(const void *Aq, const float *a_scale,
                                                  const void *Bq, const float *b_scale,
                                                  const int32_t *group_offsets, void *H,
                                                  int32_t E, int32_t K, int32_t N, int32_t M_cap,
                                                  int32_t bm, void *stream) {
  Params p = make_params(Aq, Bq, group_offsets, H, E, K, N, M_cap, bm);
  p.a_scale = a_scale;
  p.b_scale = b_scale;
  return grouped_gemm<Out::SwiGluBF16, Rows::Grouped, kW8A8>(p, stream);
}

extern "C" gg_status_t gg_tile_schedule(const int32_t *group_offsets, int32_t E, int32_t N,
                                        int32_t M_cap, int32_t bm, int32_t *tiles,
                                        int32_t *n_tiles, int32_t max_tiles, void *stream) {
  long long bound = 0;
  gg_status_t st = check_sizes(group_offsets, E, N, M_cap, bm, &bound);
  if (st != GG_OK) return st;
  if (n_tiles == nullptr || max_tiles < 0 || (max_tiles > 0 && tiles == nullptr))
    return GG_ERR_INVALID_VALUE;
  if (!aligned(n_tiles, 4) || (tiles && !aligned(tiles, 4))) return GG_ERR_MISALIGNED;
  hipLaunchKernelGGL(tile_schedule_kernel, dim3(1), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), group_offsets, E, N, M_cap, bm,
                     (int)bound, tiles, n_tiles, max_tiles);
  return hipGetLastError() == hipSuccess ? GG_OK : GG_ERR_LAUNCH;
}

#ifdef GG_TILE_TRACE
extern "C" gg_status_t gg_trace_grouped_gemm_bf16(const void *A, const void *B,
                                                  const int32_t *group_offsets, float *C,
                                                  int32_t E, int32_t K, int32_t N, int32_t M_cap,
                                                  int32_t bm, uint64_t *trace, int32_t max_tiles,
                                                  void *stream) {
  if (trace == nullptr || max_tiles < 0) return GG_ERR_INVALID_VALUE;
  if (!aligned(trace, 8)) return GG_ERR_MISALIGNED;
  Params p = make_params(A, B, group_offsets, C, E, K, N, M_cap, bm);
  p.trace = reinterpret_cast<unsigned long long *>(trace);
  p.trace_tiles = max_tiles;
  return grouped_gemm<Out::F32, Rows::Grouped>(p, stream);
}

extern "C" gg_status_t gg_trace_clock_khz(int32_t *khz) {
  if (khz == nullptr) return GG_ERR_INVALID_VALUE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GG_ERR_LAUNCH;
  return hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, dev) == hipSuccess
             ? GG_OK
             : GG_ERR_LAUNCH;
}
#endif

extern "C" const char *gg_status_string(gg_status_t status) {
  switch (status) {
    case GG_OK: return "success";
    case GG_ERR_INVALID_VALUE: return "invalid argument (null pointer, size or tile height)";
    case GG_ERR_MISALIGNED: return "misaligned pointer, or K or N not a multiple of 8";
    case GG_ERR_UNSUPPORTED: return "unsupported problem (too many experts or rows, K or N too large)";
    case GG_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}
