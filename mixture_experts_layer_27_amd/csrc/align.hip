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

namespace moe {

namespace {

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / kWave;
constexpr int kSegRows = 256;        // rows per segment in the multi-launch path
constexpr int kMaxE = 512;

// Histogram of one segment into hist[0..E) (LDS or global through LDS staging).
__device__ void segment_histogram(const int32_t* __restrict__ ids, int r0, int r1,
                                  int* __restrict__ lds_cnt) {
  const int lane = lane_id();
  for (int r = r0 + lane; r < r1; r += kWave) atomicAdd(&lds_cnt[ids[r]], 1);
}

// Stable scatter of one segment; run[e] holds the next free position of expert e
// for this segment (LDS, owned by this wave).
__device__ void segment_scatter(const int32_t* __restrict__ ids, int r0, int r1,
                                int* __restrict__ run, int32_t* __restrict__ sorted_ids) {
  const int lane = lane_id();
  const uint64_t lt = lanemask_lt();
  for (int base = r0; base < r1; base += kWave) {
    const int r = base + lane;
    const bool valid = r < r1;
    const int e = valid ? ids[r] : -1;
    uint64_t remaining = __ballot(valid);
    while (remaining) {
      const int leader = __ffsll(static_cast<unsigned long long>(remaining)) - 1;
      const int le = __shfl(e, leader, kWave);
      const uint64_t m = __ballot(e == le);
      const int start = run[le];                       // every lane reads before the leader writes
      if (e == le) sorted_ids[start + __popcll(m & lt)] = r;
      __builtin_amdgcn_wave_barrier();
      if (lane == leader) run[le] = start + __popcll(m);
      __builtin_amdgcn_wave_barrier();
      remaining &= ~m;
    }
  }
}

// Block-wide (first wave) exclusive scan over E padded counts held in LDS.
// Writes start[e] (rows) and returns total via *total_out; cnt[e] must be final.
__device__ void scan_padded(const int* __restrict__ cnt, int E, int bm, int* __restrict__ start,
                            int* __restrict__ tile_end, int* __restrict__ total_out) {
  if (wave_id() != 0) return;
  const int lane = lane_id();
  int carry = 0;
  for (int e0 = 0; e0 < E; e0 += kWave) {
    const int e = e0 + lane;
    const int n = e < E ? cnt[e] : 0;
    const int padded = (n + bm - 1) / bm * bm;
    int incl = padded;
    for (int d = 1; d < kWave; d <<= 1) {
      const int v = __shfl_up(incl, d, kWave);
      if (lane >= d) incl += v;
    }
    if (e < E) {
      start[e] = carry + incl - padded;
      tile_end[e] = (carry + incl) / bm;          // exclusive end tile of expert e
    }
    carry += __shfl(incl, kWave - 1, kWave);
  }
  if (lane == 0) *total_out = carry;
}

// expert_ids[p] for every p < cap/bm, and the sentinel on the padding positions and
// the tail of sorted_ids.  Uses start[], tile_end[] and cnt[] from LDS.
__device__ void fill_tables(const int* __restrict__ cnt, const int* __restrict__ start,
                            const int* __restrict__ tile_end, int E, int bm, int total,
                            int64_t cap, int R, int32_t* __restrict__ sorted_ids,
                            int32_t* __restrict__ expert_ids) {
  const int ntiles_cap = static_cast<int>(cap / bm);
  const int ntiles = total / bm;
  for (int p = threadIdx.x; p < ntiles_cap; p += blockDim.x) {
    int e = -1;
    if (p < ntiles) {                       // first e with tile_end[e] > p
      int lo = 0, hi = E - 1;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (tile_end[mid] > p) hi = mid; else lo = mid + 1;
      }
      e = lo;
    }
    expert_ids[p] = e;
  }
  // padding positions [start_e + n_e, start_e + padded_e): one thread per (e, slot)
  for (int i = threadIdx.x; i < E * bm; i += blockDim.x) {
    const int e = i / bm, j = i % bm;
    const int n = cnt[e];
    const int padded = (n + bm - 1) / bm * bm;
    if (n + j < padded) sorted_ids[start[e] + n + j] = R;
  }
  for (int64_t p = total + threadIdx.x; p < cap; p += blockDim.x) sorted_ids[p] = R;
}

// ---------------------------------------------------------------- single work-group path
__global__ void __launch_bounds__(kAlignThreads)
align_small_kernel(const int32_t* __restrict__ ids, int R, int E, int bm, int64_t cap,
                   int32_t* __restrict__ sorted_ids, int32_t* __restrict__ expert_ids,
                   int32_t* __restrict__ ntpp, int32_t* __restrict__ counts) {
  __shared__ int hist[kAlignWaves][kMaxE];   // per-wave segment histogram, later run cursors
  __shared__ int cnt[kMaxE], start[kMaxE], tile_end[kMaxE];
  __shared__ int total_s;
  const int w = wave_id();
  // segments: contiguous, multiple of 64 rows, one per wave
  const int per = ((R + kAlignWaves - 1) / kAlignWaves + kWave - 1) / kWave * kWave;
  const int r0 = min(R, w * per), r1 = min(R, r0 + per);
  for (int i = threadIdx.x; i < kAlignWaves * kMaxE; i += blockDim.x) (&hist[0][0])[i] = 0;
  __syncthreads();
  segment_histogram(ids, r0, r1, hist[w]);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int s = 0;
    for (int q = 0; q < kAlignWaves; ++q) s += hist[q][e];
    cnt[e] = s;
  }
  __syncthreads();
  scan_padded(cnt, E, bm, start, tile_end, &total_s);
  __syncthreads();
  const int total = total_s;
  // per-wave run cursors: start_e + rows of expert e in earlier segments
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = start[e];
    for (int q = 0; q < kAlignWaves; ++q) {
      const int c = hist[q][e];
      hist[q][e] = run;
      run += c;
    }
    if (counts) counts[e] = cnt[e];
  }
  if (threadIdx.x == 0) *ntpp = total;
  __syncthreads();
  fill_tables(cnt, start, tile_end, E, bm, total, cap, R, sorted_ids, expert_ids);
  segment_scatter(ids, r0, r1, hist[w], sorted_ids);
}

// ---------------------------------------------------------------- multi-launch path
// Phase 1: one wave per segment of kSegRows rows -> hist[seg][e] (global, all E written).
__global__ void __launch_bounds__(256)
align_hist_kernel(const int32_t* __restrict__ ids, int R, int E, int nseg,
                  int32_t* __restrict__ hist) {
  __shared__ int cnt[4][kMaxE];
  const int w = wave_id();
  const int seg = blockIdx.x * 4 + w;
  for (int e = lane_id(); e < E; e += kWave) cnt[w][e] = 0;
  __builtin_amdgcn_wave_barrier();
  if (seg < nseg) {
    const int r0 = seg * kSegRows, r1 = min(R, r0 + kSegRows);
    segment_histogram(ids, r0, r1, cnt[w]);
    __builtin_amdgcn_wave_barrier();
    for (int e = lane_id(); e < E; e += kWave) hist[static_cast<int64_t>(seg) * E + e] = cnt[w][e];
  }
}

// Phase 2 (one work-group): totals, scan, tables; hist[seg][e] becomes the run base
// of expert e in segment seg.
__global__ void __launch_bounds__(kAlignThreads)
align_scan_kernel(int R, int E, int bm, int64_t cap, int nseg, int32_t* __restrict__ hist,
                  int32_t* __restrict__ sorted_ids, int32_t* __restrict__ expert_ids,
                  int32_t* __restrict__ ntpp, int32_t* __restrict__ counts) {
  __shared__ int cnt[kMaxE], start[kMaxE], tile_end[kMaxE];
  __shared__ int total_s;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int s = 0;
    for (int q = 0; q < nseg; ++q) s += hist[static_cast<int64_t>(q) * E + e];
    cnt[e] = s;
  }
  __syncthreads();
  scan_padded(cnt, E, bm, start, tile_end, &total_s);
  __syncthreads();
  const int total = total_s;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = start[e];
    for (int q = 0; q < nseg; ++q) {
      const int64_t i = static_cast<int64_t>(q) * E + e;
      const int c = hist[i];
      hist[i] = run;
      run += c;
    }
    if (counts) counts[e] = cnt[e];
  }
  if (threadIdx.x == 0) *ntpp = total;
  fill_tables(cnt, start, tile_end, E, bm, total, cap, R, sorted_ids, expert_ids);
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
  segment_scatter(ids, r0, r1, run[w], sorted_ids);
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
                        int32_t* counts, int32_t* ws_hist, hipStream_t s) {
  if (R <= kAlignSmallMaxRows) {
    hipLaunchKernelGGL(align_small_kernel, dim3(1), dim3(kAlignThreads), 0, s, ids, R, E, bm,
                       cap, sorted_ids, expert_ids, ntpp, counts);
    return hipGetLastError();
  }
  const int nseg = (R + kSegRows - 1) / kSegRows;
  const int blocks = (nseg + 3) / 4;
  hipLaunchKernelGGL(align_hist_kernel, dim3(blocks), dim3(256), 0, s, ids, R, E, nseg, ws_hist);
  hipLaunchKernelGGL(align_scan_kernel, dim3(1), dim3(kAlignThreads), 0, s, R, E, bm, cap, nseg,
                     ws_hist, sorted_ids, expert_ids, ntpp, counts);
  hipLaunchKernelGGL(align_scatter_kernel, dim3(blocks), dim3(256), 0, s, ids, R, E, nseg,
                     ws_hist, sorted_ids);
  return hipGetLastError();
}

}  // namespace moe
