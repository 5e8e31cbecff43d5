// Device-side building blocks of moe_align (histogram -> pad -> scan -> stable scatter),
// shared by the align kernels and the fused small-batch routing kernel.
// ("Mixture-of-Experts Kernels: Routing, Permutation, and Grouped GEMM", section 5.)
//
// Written for latency: at decode batch sizes the whole table is a few hundred rows,
// so the cost is the number of dependent LDS / memory round trips, not bandwidth.
// Every phase is one pass of independent accesses per thread (no per-element search,
// no runtime division: block_m is a power of two).
#pragma once
#include "common.hpp"

namespace moe {
namespace alignd {

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / kWave;
constexpr int kSegRows = 256;        // rows per segment in the multi-launch path
constexpr int kMaxE = 512;

__device__ __forceinline__ int log2_pow2(int v) { return __builtin_ctz(static_cast<unsigned>(v)); }

// Histogram of rows [r0, r1) into lds_cnt[0..E) (LDS atomics).  An id outside [0, E)
// (possible only for ids the caller supplies) is skipped: it is counted nowhere, so the
// table stays consistent for the other rows and the counts sum to less than the rows.
__device__ inline void segment_histogram(const int32_t* __restrict__ ids, int r0, int r1, int E,
                                         int* __restrict__ lds_cnt) {
  const int lane = lane_id();
  for (int r = r0 + lane; r < r1; r += kWave) {
    const int e = ids[r];
    if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) atomicAdd(&lds_cnt[e], 1);
  }
}

// Stable scatter of rows [r0, r1) by the calling wave; run[e] holds the next free
// position of expert e for this segment (LDS, owned by this wave).  Rows of equal
// expert inside a 64-row chunk are ranked with a ballot match loop.  Rows whose id is
// outside [0, E) are skipped, as in the histogram.
__device__ inline void segment_scatter(const int32_t* __restrict__ ids, int r0, int r1, int E,
                                       int* __restrict__ run, int32_t* __restrict__ sorted_ids) {
  const int lane = lane_id();
  const uint64_t lt = lanemask_lt();
  for (int base = r0; base < r1; base += kWave) {
    const int r = base + lane;
    const int id = r < r1 ? ids[r] : -1;
    const bool valid = static_cast<unsigned>(id) < static_cast<unsigned>(E);
    const int e = valid ? id : -1;
    uint64_t remaining = __ballot(valid);
    while (remaining) {
      const int leader = __ffsll(static_cast<unsigned long long>(remaining)) - 1;
      const int le = read_lane(e, leader);
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

// Register-resident forms for the single work-group path, where a wave's segment is at
// most NC chunks of 64 rows: the ids are loaded once, all at the same time (row
// r0 + 64 c + lane in idr[c], -1 past r1), and both passes read them from registers
// instead of walking the segment twice with a memory round trip per chunk.
template <int NC>
__device__ __forceinline__ void load_segment(const int32_t* __restrict__ ids, int r0, int r1,
                                             int (&idr)[NC]) {
  const int lane = lane_id();
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int r = r0 + c * kWave + lane;
    idr[c] = r < r1 ? ids[r] : -1;
  }
}

template <int NC>
__device__ __forceinline__ void histogram_regs(const int (&idr)[NC], int E,
                                               int* __restrict__ lds_cnt) {
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (static_cast<unsigned>(idr[c]) < static_cast<unsigned>(E)) atomicAdd(&lds_cnt[idr[c]], 1);
}

// The stable scatter of segment_scatter over register-resident ids.  With E <= 64 the
// cursor of expert e lives in lane e and a chunk takes one ballot per expert, all
// independent of each other (a row's position: its expert's cursor plus the rows of that
// expert in lower lanes), then one store, instead of a serial match loop over the experts
// present; the ranks are the same.
template <int NC>
__device__ inline void scatter_regs(const int (&idr)[NC], int r0, int r1, int E,
                                    int* __restrict__ run, int32_t* __restrict__ sorted_ids) {
  const int lane = lane_id();
  const uint64_t lt = lanemask_lt();
  const bool in_lanes = E <= kWave;
  int cur = in_lanes && lane < E ? run[lane] : 0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int base = r0 + c * kWave;
    if (base >= r1) break;
    const int r = base + lane;
    const bool valid = static_cast<unsigned>(idr[c]) < static_cast<unsigned>(E);
    const int e = valid ? idr[c] : -1;
    if (in_lanes) {
      int pos = 0;
      for (int x = 0; x < E; ++x) {
        const uint64_t m = __ballot(e == x);
        if (m == 0) continue;
        const int start = read_lane(cur, x);
        if (e == x) pos = start + __popcll(m & lt);
        if (lane == x) cur = start + __popcll(m);
      }
      if (valid) sorted_ids[pos] = r;
      continue;
    }
    uint64_t remaining = __ballot(valid);
    while (remaining) {
      const int leader = __ffsll(static_cast<unsigned long long>(remaining)) - 1;
      const int le = read_lane(e, leader);
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

// Exclusive scan of the padded counts by the first wave: start[e] for every e and
// *total_out = sum of padded counts.  cnt[e] must be final.
__device__ inline void scan_padded(const int* __restrict__ cnt, int E, int bm,
                                   int* __restrict__ start, int* __restrict__ total_out) {
  if (wave_id() != 0) return;
  const int lane = lane_id();
  int carry = 0;
  for (int e0 = 0; e0 < E; e0 += kWave) {
    const int e = e0 + lane;
    const int n = e < E ? cnt[e] : 0;
    const int padded = (n + bm - 1) & -bm;
    const int incl = wave_incl_scan(padded);
    if (e < E) start[e] = carry + incl - padded;
    carry += read_lane(incl, kWave - 1);
  }
  if (lane == 0) *total_out = carry;
}

// expert_ids: thread e writes the tiles of expert e ([start_e, start_e + padded_e) / bm)
// with its owner: e, or emap[e] when an expert map is given (expert parallelism: the
// expert's index among this GPU's experts, -1 for an expert held elsewhere); the rest
// of the first cap/bm entries gets -1.  tile_run (optional, cap/bm + 1 entries): each of
// those tiles gets (first tile, number of tiles) of its expert's run, and entry cap/bm
// gets (longest run, 0).  Called by every thread of the work-group.
__device__ inline void fill_expert_ids(const int* __restrict__ cnt, const int* __restrict__ start,
                                       int E, int bm, int total, int64_t cap,
                                       int32_t* __restrict__ expert_ids,
                                       const int32_t* __restrict__ emap,
                                       int2* __restrict__ tile_run = nullptr) {
  const int lg = log2_pow2(bm);
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const int n = cnt[e];
    const int s = start[e];
    const int p1 = (s + n + bm - 1) >> lg;
    const int owner = emap ? emap[e] : e;
    for (int p = s >> lg; p < p1; ++p) expert_ids[p] = owner;
    if (tile_run)
      for (int p = s >> lg; p < p1; ++p) tile_run[p] = make_int2(s >> lg, p1 - (s >> lg));
  }
  if (tile_run) {
    __shared__ int longest;
    if (threadIdx.x == 0) longest = 0;
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x)
      atomicMax(&longest, (cnt[e] + bm - 1) >> lg);
    __syncthreads();
    if (threadIdx.x == 0) tile_run[cap >> lg] = make_int2(longest, 0);
  }
  const int ntiles_cap = static_cast<int>(cap >> lg);
  for (int p = (total >> lg) + threadIdx.x; p < ntiles_cap; p += blockDim.x) expert_ids[p] = -1;
}

// ---------------------------------------------------------------- single work-group path
// The whole table in one work-group of kAlignThreads threads (ids may live in LDS).
// sorted_ids is first filled with the sentinel R, then the scatter overwrites the
// routed rows (the barrier between the two waits for the stores to complete).
__device__ inline void align_small_body(const int32_t* ids, int R, int E, int bm, int64_t cap,
                                        int32_t* __restrict__ sorted_ids,
                                        int32_t* __restrict__ expert_ids,
                                        int32_t* __restrict__ ntpp, int32_t* __restrict__ counts,
                                        const int32_t* __restrict__ emap,
                                        int2* __restrict__ tile_run = nullptr) {
  __shared__ int hist[kAlignWaves][kMaxE];   // per-wave segment histogram, later run cursors
  __shared__ int cnt[kMaxE], start[kMaxE];
  __shared__ int total_s;
  const int w = wave_id();
  // contiguous segments, one per wave, in ascending row order
  const int per = (R + kAlignWaves - 1) / kAlignWaves;
  const int r0 = min(R, w * per), r1 = min(R, r0 + per);
  // the callers keep R <= 8192, so a segment fits in registers; the loads are issued
  // first and complete under the clearing below
  constexpr int kChunks = 8;
  const bool regs = per <= kChunks * kWave;
  int idr[kChunks];
  if (regs) load_segment(ids, r0, r1, idr);
  for (int i = threadIdx.x; i < kAlignWaves * kMaxE; i += blockDim.x) {
    if ((i & (kMaxE - 1)) < E) (&hist[0][0])[i] = 0;
  }
  for (int64_t p = threadIdx.x; p < cap; p += blockDim.x) sorted_ids[p] = R;
  __syncthreads();
  if (regs) histogram_regs(idr, E, hist[w]);
  else segment_histogram(ids, r0, r1, E, hist[w]);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int s = 0;
#pragma unroll
    for (int q = 0; q < kAlignWaves; ++q) s += hist[q][e];
    cnt[e] = s;
  }
  __syncthreads();
  scan_padded(cnt, E, bm, start, &total_s);
  __syncthreads();
  const int total = total_s;
  // per-wave run cursors: start_e + rows of expert e in earlier segments
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = start[e];
#pragma unroll
    for (int q = 0; q < kAlignWaves; ++q) {
      const int c = hist[q][e];
      hist[q][e] = run;
      run += c;
    }
    if (counts) counts[e] = cnt[e];
  }
  if (threadIdx.x == 0) *ntpp = total;
  fill_expert_ids(cnt, start, E, bm, total, cap, expert_ids, emap, tile_run);
  __syncthreads();
  if (regs) scatter_regs(idr, r0, r1, E, hist[w], sorted_ids);
  else segment_scatter(ids, r0, r1, E, hist[w], sorted_ids);
}

}  // namespace alignd
}  // namespace moe
