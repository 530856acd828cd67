// Device-built flat tile list.
//
// "Grouped GEMM for Imbalanced Experts on Blackwell: A WIP Worklog", section 2
// (The Grouped Problem and the flat tile list): every output tile of every
// expert becomes one descriptor {expert, first row, valid rows, first column};
// tiles stop at expert boundaries, an expert with no rows has no tiles, and
// the descriptors are ordered expert-major with the N tile innermost. The
// worklog enumerates the list on the host; here every workgroup rebuilds the
// per-expert prefix of tile counts in LDS from the device-resident offsets
// (the InferenceX glossary entry "Grouped GEMM", "Engineering details", notes
// the same move of group-metadata generation into the kernel), so the host
// never needs the group sizes and no device-to-host copy sits in front of the
// launch. A tile id is decoded by binary search over that prefix.
#pragma once

#include "gg_common.h"

namespace gg {

constexpr int kMaxExperts = 1024;  // per-expert tables live in LDS

// Tile heights this library runs, smallest first. Tile width is 128 for all.
constexpr int kBN = 128;

// Per-expert tile height when the caller leaves the choice to the device.
// Minimises ceil(m/BM) * (BM + 64) over BM in {16, 32, 64, 128}: the first
// factor counts tiles, the second prices one tile as its rows plus a fixed
// 64-row-equivalent share for the work every tile repeats regardless of its
// height (streaming the expert's weight slice, barriers, epilogue set-up).
// Ties go to the larger height; an expert with no rows gets 16 (no tiles).
__device__ __forceinline__ int adaptive_bm(int m) {
  if (m <= 0) return 16;
  int best = 16;
  long long best_cost = (long long)cdiv(m, 16) * (16 + 64);
#pragma unroll
  for (int b = 32; b <= 128; b *= 2) {
    const long long c = (long long)cdiv(m, b) * (b + 64);
    if (c <= best_cost) { best = b; best_cost = c; }
  }
  return best;
}

struct Tile {
  int expert;
  int row0;   // first row in A and C
  int rows;   // valid rows, 1..bm
  int col0;   // first column in C
  int bm;     // tile height
};

// LDS tables: clamped offsets and the exclusive prefix of tile counts.
struct SchedLds {
  int off[kMaxExperts + 1];
  int start[kMaxExperts + 1];
  int wave_sum[kThreads / kWave];
};

// All threads of the workgroup must call this (it contains barriers).
// bm_fixed = 0 selects adaptive_bm per expert. Returns the total tile count.
__device__ inline int build_schedule(SchedLds &s, const int32_t *__restrict__ off_g, int E,
                                     int M_cap, int NT, int bm_fixed) {
  const int tid = threadIdx.x;
  for (int e = tid; e <= E; e += kThreads) {
    int v = off_g[e];
    v = v < 0 ? 0 : (v > M_cap ? M_cap : v);
    s.off[e] = v;
  }
  __syncthreads();
  // each thread owns a run of consecutive experts (E <= 1024 -> at most 4)
  constexpr int kRun = kMaxExperts / kThreads;
  const int e0 = tid * kRun;
  int cnt[kRun];
  int local = 0;
#pragma unroll
  for (int j = 0; j < kRun; ++j) {
    const int e = e0 + j;
    int c = 0;
    if (e < E) {
      const int m = s.off[e + 1] - s.off[e];
      if (m > 0) {
        const int b = bm_fixed ? bm_fixed : adaptive_bm(m);
        c = cdiv(m, b) * NT;
      }
    }
    cnt[j] = c;
    local += c;
  }
  // inclusive scan of 'local' across the 64 lanes of the wave
  const int lane = tid % kWave, wave = tid / kWave;
  int incl = local;
#pragma unroll
  for (int d = 1; d < kWave; d *= 2) {
    const int y = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += y;
  }
  if (lane == kWave - 1) s.wave_sum[wave] = incl;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int w = 0; w < kThreads / kWave; ++w)
    if (w < wave) before += s.wave_sum[w];
  int run = before + incl - local;  // exclusive prefix of this thread's run
#pragma unroll
  for (int j = 0; j < kRun; ++j) {
    const int e = e0 + j;
    if (e < E) s.start[e] = run;
    run += cnt[j];
  }
  int total = 0;
#pragma unroll
  for (int w = 0; w < kThreads / kWave; ++w) total += s.wave_sum[w];
  if (tid == 0) s.start[E] = total;
  __syncthreads();
  return total;
}

// Decode tile id t (0 <= t < total) into its descriptor.
__device__ __forceinline__ Tile decode_tile(const SchedLds &s, int t, int E, int NT, int bm_fixed) {
  int lo = 0, hi = E;  // start[lo] <= t < start[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s.start[mid] <= t) lo = mid; else hi = mid;
  }
  Tile tl;
  const int m = s.off[lo + 1] - s.off[lo];
  const int b = bm_fixed ? bm_fixed : adaptive_bm(m);
  const int local = t - s.start[lo];
  const int mt = local / NT;
  const int nt = local - mt * NT;
  tl.expert = lo;
  tl.bm = b;
  tl.row0 = s.off[lo] + mt * b;
  tl.rows = min(b, m - mt * b);
  tl.col0 = nt * kBN;
  return tl;
}

}  // namespace gg
