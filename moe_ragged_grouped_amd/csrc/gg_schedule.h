// Device-built flat tile list.
//
// "Grouped GEMM for Imbalanced Experts on Blackwell: A WIP Worklog", section 2
// (The Grouped Problem and the flat tile list): every output tile of every
// expert becomes one descriptor {expert, first row, valid rows, first column};
// tiles stop at expert boundaries, an expert with no rows has no tiles, and
// the experts follow each other in order. The worklog enumerates the list on
// the host; here every workgroup rebuilds the per-expert prefix of tile counts
// in LDS from the device-resident offsets (the InferenceX glossary entry
// "Grouped GEMM", "Engineering details", describes the same move of group
// metadata generation into the kernel), so the host never needs the group
// sizes and no device-to-host copy sits in front of the launch. A tile id is
// decoded by binary search over that prefix.
//
// Order inside one expert. The worklog runs N tiles innermost. Here the M
// tiles of an expert are taken in groups of up to kGroupM; inside a group the
// N tile is the outer index and the M tile the inner one. Consecutive tile ids
// then share a column slice of the expert's weights (the bulk of the bytes
// when N*K dwarfs m_e*K), and a group's A rows stay hot across its N tiles.
// Experts with at most kGroupM M tiles are simply N-major. The set of tiles is
// the worklog's; only the order differs.
#pragma once

#include "gg_common.h"

namespace gg {

constexpr int kMaxExperts = 1024;  // the tile prefix lives in LDS
constexpr int kGroupM = 8;         // M tiles per group in the within-expert order

// Tile heights this library runs, smallest first. Tiles are kTileN columns
// wide, except in a launch where every expert's tiles are 16 rows high (the
// weight-streaming decode case): there the tiles are kWideN wide, so each
// workgroup streams twice the contiguous weight row per slice and a launch
// has half as many tiles (measured on 32 experts x 16 rows, K=6144,
// N=4096: 242 -> 237 us). In launches that mix heights, 16-row tiles stay
// narrow: wide ones there become the long poles of the launch.
constexpr int kNumHeights = 5;
constexpr int kTileN = 256;
constexpr int kWideN = 512;
__host__ __device__ constexpr int height_of(int cls) { return 16 << cls; }
__host__ __device__ constexpr int width_of(int bm, bool wide16) {
  return (bm == 16 && wide16) ? kWideN : kTileN;
}

// Per-expert tile height when the caller leaves the choice to the device.
// Minimises ceil(m/BM) * (BM + 64) over BM in {16, 32, 64, 128, 256}: the
// first factor counts tiles, the second prices one tile as its rows plus a
// fixed 64-row-equivalent share for the work every tile repeats regardless of
// its height (streaming the expert's weight slice, barriers, epilogue
// set-up). Ties go to the larger height; an expert with no rows gets 16 (no
// tiles).
__device__ __forceinline__ int adaptive_bm(int m) {
  if (m <= 0) return 16;
  int best = 16;
  long long best_cost = (long long)cdiv(m, 16) * (16 + 64);
#pragma unroll
  for (int c = 1; c < kNumHeights; ++c) {
    const int b = height_of(c);
    const long long cost = (long long)cdiv(m, b) * (b + 64);
    if (cost <= best_cost) { best = b; best_cost = cost; }
  }
  return best;
}

struct Tile {
  int expert;
  int row0;   // first row in A and C
  int rows;   // valid rows, 1..bm
  int col0;   // first column in C
  int bm;     // tile height
  int bn;     // tile width: width_of(bm, the launch's wide16 flag)
};

// LDS table: exclusive prefix of tile counts per expert (start[E] = total).
struct SchedLds {
  int start[kMaxExperts + 1];
  long long wave_sum[kThreads / kWave];
  int wave_tall[kThreads / kWave];  // a wave saw an expert with rows and taller tiles
  int wide16;  // every expert with rows has 16-row tiles: they are kWideN wide
};

// Clamped group boundaries: every offset is pulled into [0, M_cap].
__device__ __forceinline__ int clamp_off(const int32_t *off_g, int e, int M_cap) {
  const int v = off_g[e];
  return v < 0 ? 0 : (v > M_cap ? M_cap : v);
}

// All threads of the workgroup must call this (it contains barriers).
// bm_fixed = 0 selects adaptive_bm per expert. Returns the total tile count.
//
// tile_cap is the host's upper bound of the tile count, derived from M_cap
// alone: with nondecreasing offsets the segments are disjoint and the count
// never exceeds it. Offsets that decrease can make clamped segments overlap,
// each up to M_cap rows, so their counts can sum far past it. The counts are
// therefore summed in 64 bits, and a launch whose total exceeds tile_cap
// schedules no tile at all (every later tile index then fits in 32 bits).
__device__ inline int build_schedule(SchedLds &s, const int32_t *__restrict__ off_g, int E,
                                     int M_cap, int N, int bm_fixed, int tile_cap) {
  const int tid = threadIdx.x;
  // each thread owns a run of consecutive experts (E <= 1024 -> at most 2)
  constexpr int kRun = kMaxExperts / kThreads;
  const int e0 = tid * kRun;
  int rows[kRun], height[kRun];
  int tall = 0;  // an expert of this run has rows and taller tiles than 16
  int lo = e0 < E ? clamp_off(off_g, e0, M_cap) : 0;
#pragma unroll
  for (int j = 0; j < kRun; ++j) {
    const int e = e0 + j;
    rows[j] = 0;
    height[j] = 16;
    if (e < E) {
      const int hi = clamp_off(off_g, e + 1, M_cap);
      rows[j] = hi > lo ? hi - lo : 0;
      height[j] = bm_fixed ? bm_fixed : adaptive_bm(rows[j]);
      tall |= rows[j] > 0 && height[j] > 16;
      lo = hi;
    }
  }
  // workgroup-wide OR of 'tall' through one LDS word per wave (a library
  // reduction would reserve LDS of its own ahead of the operand stages)
  const int lane = tid % kWave, wave = tid / kWave;
  const bool wave_tall = __any(tall);
  if (lane == 0) s.wave_tall[wave] = wave_tall;
  __syncthreads();
  bool any_tall = false;
#pragma unroll
  for (int w = 0; w < kThreads / kWave; ++w) any_tall |= s.wave_tall[w] != 0;
  const bool wide16 = !any_tall;
  long long cnt[kRun];
  long long local = 0;
#pragma unroll
  for (int j = 0; j < kRun; ++j) {
    cnt[j] = rows[j] > 0
                 ? (long long)cdiv(rows[j], height[j]) * cdiv(N, width_of(height[j], wide16))
                 : 0;
    local += cnt[j];
  }
  // inclusive scan of 'local' across the 64 lanes of the wave
  long long incl = local;
#pragma unroll
  for (int d = 1; d < kWave; d *= 2) {
    const long long y = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += y;
  }
  if (lane == kWave - 1) s.wave_sum[wave] = incl;
  __syncthreads();
  long long before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kThreads / kWave; ++w) {
    if (w < wave) before += s.wave_sum[w];
    total += s.wave_sum[w];
  }
  if (total > tile_cap) total = 0;  // overlapping malformed segments: no tiles
  long long run = before + incl - local;  // exclusive prefix of this thread's run
#pragma unroll
  for (int j = 0; j < kRun; ++j) {
    const int e = e0 + j;
    if (e < E) s.start[e] = total ? (int)run : 0;
    run += cnt[j];
  }
  if (tid == 0) {
    s.start[E] = (int)total;
    s.wide16 = wide16;
  }
  __syncthreads();
  return (int)total;
}

// Decode tile id t (0 <= t < total) into its descriptor.
__device__ __forceinline__ Tile decode_tile(const SchedLds &s, const int32_t *__restrict__ off_g,
                                            int t, int E, int M_cap, int N, int bm_fixed) {
  int lo = 0, hi = E;  // start[lo] <= t < start[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s.start[mid] <= t) lo = mid; else hi = mid;
  }
  const int r0 = clamp_off(off_g, lo, M_cap);
  const int m = clamp_off(off_g, lo + 1, M_cap) - r0;
  const int b = bm_fixed ? bm_fixed : adaptive_bm(m);
  const int bn = width_of(b, s.wide16 != 0);
  const int NT = cdiv(N, bn);
  const int n_mt = cdiv(m, b);
  const int local = t - s.start[lo];
  // groups of kGroupM M tiles; N outer, M inner inside a group
  const int per_group = kGroupM * NT;
  const int grp = local / per_group;
  const int r = local - grp * per_group;
  const int gm = min(kGroupM, n_mt - grp * kGroupM);  // M tiles in this group
  const int nt = r / gm;
  const int mt = grp * kGroupM + (r - nt * gm);
  Tile tl;
  tl.expert = lo;
  tl.bm = b;
  tl.bn = bn;
  tl.row0 = r0 + mt * b;
  tl.rows = min(b, m - mt * b);
  tl.col0 = nt * bn;
  return tl;
}

}  // namespace gg
