// moe_align on the device: histogram -> pad to block_m -> exclusive scan -> stable
// scatter ("Mixture-of-Experts Kernels: Routing, Permutation, and Grouped GEMM",
// section 5; the argsort-free counting form of its section 11 exercise).
//
// Determinism: the position of a row inside its expert's run is its rank among the
// rows with the same expert in ascending flat-row order.  No rank comes from an
// atomic: rows are split into contiguous segments (one wave each); a segment's
// histogram gives each (segment, expert) a base offset through a column prefix
// over segments, and inside a segment a wave walks its rows 64 at a time, ranking
// equal experts with a ballot match loop (leader = first remaining lane, mask =
// ballot(expert == leader's), rank = popcount(mask & lanes-below)).
//
//   small R: one work-group does all three phases with the histogram in LDS;
//   large R: three launches (segment histograms -> one-WG scan -> segment scatter).
#include "common.hpp"
#include "launch.hpp"

#include "align_dev.hpp"

namespace moe {

namespace {

using namespace alignd;

__global__ void __launch_bounds__(kAlignThreads)
align_small_kernel(const int32_t* __restrict__ ids, int R, int E, int bm, int64_t cap,
                   int32_t* __restrict__ sorted_ids, int32_t* __restrict__ expert_ids,
                   int32_t* __restrict__ ntpp, int32_t* __restrict__ counts,
                   const int32_t* __restrict__ emap, int2* __restrict__ tile_run) {
  align_small_body(ids, R, E, bm, cap, sorted_ids, expert_ids, ntpp, counts, emap, tile_run);
}

// ---------------------------------------------------------------- multi-launch path
// Phase 1: one wave per segment of kSegRows rows -> hist[seg][e] (global, all E written);
// the grid also fills sorted_ids [0, cap) with the sentinel R, which the scatter of
// phase 3 then overwrites at the routed rows.
__global__ void __launch_bounds__(256)
align_hist_kernel(const int32_t* __restrict__ ids, int R, int E, int nseg, int64_t cap,
                  int32_t* __restrict__ hist, int32_t* __restrict__ sorted_ids) {
  __shared__ int cnt[4][kMaxE];
  const int w = wave_id();
  const int seg = blockIdx.x * 4 + w;
  const int64_t nthreads = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t p = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; p < cap;
       p += nthreads)
    sorted_ids[p] = R;
  for (int e = lane_id(); e < E; e += kWave) cnt[w][e] = 0;
  __builtin_amdgcn_wave_barrier();
  if (seg < nseg) {
    const int r0 = seg * kSegRows, r1 = min(R, r0 + kSegRows);
    segment_histogram(ids, r0, r1, E, cnt[w]);
    __builtin_amdgcn_wave_barrier();
    for (int e = lane_id(); e < E; e += kWave) hist[static_cast<int64_t>(seg) * E + e] = cnt[w][e];
  }
}

// Phase 2 (one work-group): totals, scan, expert_ids; hist[seg][e] becomes the run
// base of expert e in segment seg.  The [nseg x E] matrix is walked by every thread:
// thread (g, e) owns expert e and the contiguous segments [q0, q1) of group g (G groups,
// threads of one group read adjacent experts, so each row of hist is read coalesced), with
// loads issued eight at a time; the groups' partial counts are combined in LDS.
__global__ void __launch_bounds__(kAlignThreads)
align_scan_kernel(int R, int E, int bm, int64_t cap, int nseg, int32_t* __restrict__ hist,
                  int32_t* __restrict__ expert_ids, int32_t* __restrict__ ntpp,
                  int32_t* __restrict__ counts, const int32_t* __restrict__ emap,
                  int2* __restrict__ tile_run) {
  constexpr int kB = 8;                         // loads in flight per thread
  __shared__ int part[kAlignThreads];           // [g][e]: count, then the group's base
  __shared__ int cnt[kMaxE], start[kMaxE];
  __shared__ int total_s;
  int ep = 1;                                   // E rounded up to a power of two
  while (ep < E) ep <<= 1;
  const int G = kAlignThreads / ep;             // >= 2 (E <= 512)
  const int e = threadIdx.x % ep, g = threadIdx.x / ep;
  const int per = (nseg + G - 1) / G;
  const int q0 = min(nseg, g * per), q1 = min(nseg, q0 + per);
  const bool mine = e < E;
  int s = 0;
  if (mine) {
    for (int q = q0; q < q1; q += kB) {
      int v[kB];
#pragma unroll
      for (int b = 0; b < kB; ++b)
        v[b] = q + b < q1 ? hist[static_cast<int64_t>(q + b) * E + e] : 0;
#pragma unroll
      for (int b = 0; b < kB; ++b) s += v[b];
    }
  }
  part[threadIdx.x] = s;
  __syncthreads();
  // per expert: total count, and each group's base inside the expert's run (groups in
  // ascending segment order)
  if (g == 0 && mine) {
    int run = 0;
    for (int h = 0; h < G; ++h) {
      const int c = part[h * ep + e];
      part[h * ep + e] = run;
      run += c;
    }
    cnt[e] = run;
  }
  __syncthreads();
  scan_padded(cnt, E, bm, start, &total_s);
  __syncthreads();
  const int total = total_s;
  if (mine) {
    int run = start[e] + part[threadIdx.x];
    for (int q = q0; q < q1; q += kB) {
      int v[kB];
#pragma unroll
      for (int b = 0; b < kB; ++b)
        v[b] = q + b < q1 ? hist[static_cast<int64_t>(q + b) * E + e] : 0;
#pragma unroll
      for (int b = 0; b < kB; ++b) {
        if (q + b < q1) hist[static_cast<int64_t>(q + b) * E + e] = run;
        run += v[b];
      }
    }
    if (counts && g == 0) counts[e] = cnt[e];
  }
  if (threadIdx.x == 0) *ntpp = total;
  fill_expert_ids(cnt, start, E, bm, total, cap, expert_ids, emap, tile_run);
}

// Phase 3: one wave per segment, stable scatter from the segment's run bases.
__global__ void __launch_bounds__(256)
align_scatter_kernel(const int32_t* __restrict__ ids, int R, int E, int nseg,
                     const int32_t* __restrict__ hist, int32_t* __restrict__ sorted_ids) {
  __shared__ int run[4][kMaxE];
  const int w = wave_id();
  const int seg = blockIdx.x * 4 + w;
  if (seg >= nseg) return;                      // whole wave exits together
  for (int e = lane_id(); e < E; e += kWave) run[w][e] = hist[static_cast<int64_t>(seg) * E + e];
  __builtin_amdgcn_wave_barrier();
  const int r0 = seg * kSegRows, r1 = min(R, r0 + kSegRows);
  segment_scatter(ids, r0, r1, E, run[w], sorted_ids);
}

}  // namespace

constexpr int kAlignSmallMaxRows = 8192;

size_t align_ws_bytes(int R, int E) {
  if (R <= kAlignSmallMaxRows) return 0;
  const size_t nseg = (static_cast<size_t>(R) + kSegRows - 1) / kSegRows;
  return nseg * static_cast<size_t>(E) * sizeof(int32_t);
}

hipError_t launch_align(const int32_t* ids, int R, int E, int bm, int64_t cap,
                        int32_t* sorted_ids, int32_t* expert_ids, int32_t* ntpp,
                        int32_t* counts, int32_t* ws_hist, const int32_t* emap, hipStream_t s,
                        int2* tile_run) {
  if (R <= kAlignSmallMaxRows) {
    hipLaunchKernelGGL(align_small_kernel, dim3(1), dim3(kAlignThreads), 0, s, ids, R, E, bm,
                       cap, sorted_ids, expert_ids, ntpp, counts, emap, tile_run);
    return hipGetLastError();
  }
  const int nseg = (R + kSegRows - 1) / kSegRows;
  const int blocks = (nseg + 3) / 4;
  hipLaunchKernelGGL(align_hist_kernel, dim3(blocks), dim3(256), 0, s, ids, R, E, nseg, cap,
                     ws_hist, sorted_ids);
  hipLaunchKernelGGL(align_scan_kernel, dim3(1), dim3(kAlignThreads), 0, s, R, E, bm, cap, nseg,
                     ws_hist, expert_ids, ntpp, counts, emap, tile_run);
  hipLaunchKernelGGL(align_scatter_kernel, dim3(blocks), dim3(256), 0, s, ids, R, E, nseg,
                     ws_hist, sorted_ids);
  return hipGetLastError();
}

}  // namespace moe
