// Small-M expert GEMMs for decode: stream each active expert's weights once at HBM rate
// ("Mixture-of-Experts Kernels: Routing, Permutation, and Grouped GEMM", section 7 (decode
// tiles) and section 8 (FLOP per weight byte ~ n_e: bandwidth-bound below hundreds of
// rows per expert)).
//
// Operand swap: the weights are the MFMA "A" side (16 weight rows per
// v_mfma_f32_16x16x32_bf16) and up to 16 routed token rows the "B" side, so a tile with
// a single routed row still feeds whole MFMAs from the weight stream.
//
// Weights are bf16, or OCP E4M3 bytes with one fp32 scale per weight row (FP8 weights:
// section 8 of the same page prices an expert at one byte per weight).  FP8 rows are
// streamed as bytes, expanded to bf16 after the LDS read (exact: every E4M3 value is a
// bf16 value) and fed to the same bf16 MFMA; the row scale multiplies the fp32
// accumulator in the epilogue.
//
// Every wave is an independent streaming unit (one-wave work-groups, persistent grid).
// Work item = (sub-tile of 16 routed rows, block of RB weight rows of its expert).
// For each K step of STEP elements the wave copies the item's RB weight rows and the 16
// token rows into a slot of its own LDS ring with global_load_lds: one load instruction
// moves 1 KB made of whole 256-byte (STEP 128) or 128-byte (STEP 64) row segments,
// the access pattern HBM serves fastest, and the MFMA register layout is recovered by
// the LDS reads.  The XOR swizzle that keeps those reads conflict-free is applied on the
// global side (lane i of a DMA fetches the chunk that belongs at LDS position i).
// P ring slots: while step g is consumed, steps g+1 .. g+P-1 are in flight, across
// item boundaries.  All loads of the loop are these DMAs (routing ids come through
// scalar loads), so a fixed s_waitcnt vmcnt tells exactly when step g has landed.
#include <algorithm>

#include "common.hpp"
#include "dma.hpp"
#include "launch.hpp"
#include "route_dev.hpp"

namespace moe {

namespace {

struct DArgs {
  const uint8_t* A;       // weights: W13 [E,2I,H] or W2 [E,H,I] (bf16 or E4M3 bytes)
  const uint16_t* X;      // token rows: x [T,H] (GEMM1) or a [R,I] (GEMM2)
  void* C;                // a [R,I] bf16 or y [R,H] f32
  int R, gather_div, K, I, H;
  int64_t a_expert_stride;   // weight elements per expert
  int block_m;            // >= 16: a tile holds block_m / 16 sub-tiles of 16 rows
  int nblk;               // weight-row blocks per expert
  int nsub_cap;           // sub-tiles in the table's capacity (cap / (16 * NTG))
  int bm_shift;           // log2(block_m): sub-tile u lies in align tile (u * SUB) >> bm_shift
};

// One K step of STEP elements: weight rows of WB bytes per element, token rows bf16.
template <int STEP, int WB>
struct DStep {
  static constexpr int WROWB = STEP * WB;   // weight bytes per row per step
  static constexpr int XROWB = STEP * 2;    // token bytes per row per step
  static constexpr int WCPR = WROWB / 16;   // 16-byte chunks per weight row
  static constexpr int XCPR = XROWB / 16;
  static constexpr int WRPI = kWave / WCPR; // weight rows per DMA instruction (1 KB)
  static constexpr int XRPI = kWave / XCPR;
  static constexpr int KSUB = STEP / 32;    // MFMA k-substeps per step
  static_assert(WROWB == 128 || WROWB == 256, "weight row segment");
  static_assert(XROWB >= 128 && XROWB <= 512, "token row segment");
};

// LDS position of logical 16-byte chunk c of row r: rows r..r+15 at one logical chunk
// land on 16 distinct 16-byte bank groups (rows of 256 bytes or more: c ^ r inside each
// 256-byte half; 128-byte rows: two rows share a bank window, so the low row bit
// selects the half and r>>1 the XOR)
template <int CPR>
__device__ __forceinline__ int dsw(int r, int c) {
  return CPR >= 16 ? (c ^ (r & 15)) : (c ^ ((r >> 1) & 7));
}

// the SUB routed rows of sub-tile u (uniform scalar loads); R marks an empty slot
template <int SUB>
__device__ __forceinline__ void load_ids(const int32_t* __restrict__ sorted_ids, int u,
                                         int (&ids)[SUB]) {
  const int32_t* sp = sorted_ids + static_cast<int64_t>(u) * SUB;
#pragma unroll
  for (int t = 0; t < SUB; ++t) ids[t] = sp[t];
}

// v[t] for a per-lane t in [0, N <= 64) of N wave-uniform values: lane q receives v[q]
// (v_writelane), then the lane crossbar (ds_bpermute) reads lane t.  (A select chain
// over constant indices gets turned into a private-memory table lookup, whose loads
// would disturb the DMA wait counts.)
template <int N>
__device__ __forceinline__ int spread(const int (&v)[N]) {
  static_assert(N <= kWave, "one value per lane");
  int lanes = 0;
#pragma unroll
  for (int q = 0; q < N; ++q)
    asm volatile("v_writelane_b32 %0, %1, %2" : "+v"(lanes) : "s"(v[q]), "n"(q));
  return lanes;
}
template <int N>
__device__ __forceinline__ int pick(const int (&v)[N], int t) {
  return __shfl(spread(v), t, kWave);
}

// 16 E4M3 bytes -> two runs of 8 bf16 (bytes 0..7, bytes 8..15), exact
__device__ __forceinline__ void fp8x16_to_bf16(const u32x4 q, bf16x8& lo, bf16x8& hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 p[8];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    p[2 * d] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[d], 1.0f, false);
    p[2 * d + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[d], 1.0f, true);
  }
  lo = bf16x8{p[0][0], p[0][1], p[1][0], p[1][1], p[2][0], p[2][1], p[3][0], p[3][1]};
  hi = bf16x8{p[4][0], p[4][1], p[5][0], p[5][1], p[6][0], p[6][1], p[7][0], p[7][1]};
}

// DMA sources of one work item: RB weight rows of one expert and the first XR of the
// SUB = 16*NTG token rows of one sub-tile.  XR < SUB when no expert can hold more than
// XR routed rows (T <= XR: top-k experts are distinct, so an expert holds at most one
// row per token, at the head of its table tile); the MFMA columns of the rows past XR
// then read rows of the XR (their results are padding and never stored).
template <int MODE, int RB, int NTG, int STEP, bool NT, int WB, int XR>
struct Stream {
  using S = DStep<STEP, WB>;
  static constexpr int SUB = 16 * NTG;
  static constexpr int NW = RB / S::WRPI;       // weight DMAs per step
  static constexpr int NX = XR / S::XRPI;       // token-row DMAs per step
  static_assert(XR % S::XRPI == 0 && XR <= SUB && (XR == SUB || NTG == 1), "token rows");

  // per-lane sources of an item's DMAs at k offset 0
  // item = (sub-tile of the align table, weight-row block blk); idsv: its routed row ids
  // held in lanes (lane t: row t of the sub-tile); e: its expert (index into the
  // weights), >= 0
  static __device__ __forceinline__ void setup(const DArgs& p, int idsv, int blk, int e,
                                               const uint8_t* (&wp)[NW],
                                               const uint16_t* (&xp)[NX]) {
    const int lane = lane_id();
    const uint8_t* wb = p.A + static_cast<int64_t>(e) * p.a_expert_stride * WB;
    const int rl = lane / S::WCPR, ch = lane % S::WCPR;
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      const int row = j * S::WRPI + rl;
      int wrow;
      if (MODE == 1)   // first half gate rows W1, second half the matching up rows W3
        wrow = row < RB / 2 ? blk * (RB / 2) + row : p.I + blk * (RB / 2) + (row - RB / 2);
      else
        wrow = blk * RB + row;
      wp[j] = wb + static_cast<int64_t>(wrow) * p.K * WB + dsw<S::WCPR>(row, ch) * 16;
    }
    // empty slots re-read the sub-tile's first row (row 0 if the whole sub-tile is
    // padding, which happens only when block_m > SUB)
    const int id0 = read_lane(idsv, 0);
    const int fb = id0 < p.R ? id0 : 0;
    const int xl = lane / S::XCPR, xch = lane % S::XCPR;
#pragma unroll
    for (int j = 0; j < NX; ++j) {
      const int t = j * S::XRPI + xl;
      int r = __shfl(idsv, t, kWave);
      r = r < p.R ? r : fb;
      const int xrow = r / p.gather_div;
      xp[j] = p.X + static_cast<int64_t>(xrow) * p.K + dsw<S::XCPR>(t & 15, xch) * 8;
    }
  }

  // k0: element offset of the step
  static __device__ __forceinline__ void issue(const uint8_t* const (&wp)[NW],
                                               const uint16_t* const (&xp)[NX], int k0,
                                               MOE_LDS uint8_t* slot) {
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      if (NT) dma16_nt(wp[j] + k0 * WB, slot + j * 1024);    // weights read once
      else dma16(wp[j] + k0 * WB, slot + j * 1024);
    }
#pragma unroll
    for (int j = 0; j < NX; ++j) dma16(xp[j] + k0, slot + RB * S::WROWB + j * 1024);
  }
};

// Expert parallelism: a tile whose expert is held by another GPU has expert_ids = -1.
// The persistent loop deals out the items of local sub-tiles only (so the waves stay
// balanced however the local experts are spread over the table); GEMM2 writes zeros
// into the rows of the other sub-tiles so the combine adds nothing for them.
//
// Local sub-tile table, held in lanes: lane l covers sub-tiles [l*B, l*B + B) (B <= 64,
// so at most 4096 sub-tiles): (lo, hi) = bitmask of its local ones, pre = number of
// local sub-tiles in lower lanes' blocks.  The q-th local sub-tile is found with one
// ballot and scalar bit arithmetic, no memory access.
struct LocalSubtiles {
  uint32_t lo, hi;
  int pre;
  int B;
  int count;       // local sub-tiles in the table
};

// The blocks cover the table's capacity (ncap sub-tiles), so the owner loads do not wait
// for the padded total; sub-tiles at or past nsub (the total's) count as not local.
template <int SUB>
__device__ __forceinline__ LocalSubtiles local_subtiles(const int32_t* __restrict__ expert_ids,
                                                        int ncap, int nsub, int bm_shift) {
  const int lane = lane_id();
  LocalSubtiles t;
  t.B = (ncap + kWave - 1) / kWave;
  uint64_t fl = 0;
  // per-lane loads, issued 8 at a time (before any DMA of the ring is in flight); they do
  // not depend on nsub, whose limit is applied to the bits afterwards
  for (int i0 = 0; i0 < t.B; i0 += 8) {
    int ow[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int u = min(lane * t.B + i0 + i, ncap - 1);
      ow[i] = expert_ids[(u * SUB) >> bm_shift];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i0 + i < t.B && ow[i] >= 0) fl |= 1ull << (i0 + i);
  }
  const int lim = nsub - lane * t.B;            // bits at or past lim are past the total
  fl &= lim >= 64 ? ~0ull : (lim <= 0 ? 0ull : (1ull << lim) - 1);
  const int cnt = __popcll(fl);
  const int incl = wave_incl_scan(cnt);
  t.pre = incl - cnt;
  t.count = read_lane(incl, kWave - 1);
  t.lo = static_cast<uint32_t>(fl);
  t.hi = static_cast<uint32_t>(fl >> 32);
  return t;
}

// position of the n-th (from 0) set bit of m (m has more than n set bits)
__device__ __forceinline__ int nth_set_bit(uint64_t m, int n) {
  int pos = 0;
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) {
    const int c = __popcll(m & ((1ull << w) - 1));
    if (n >= c) {
      n -= c;
      m >>= w;
      pos += w;
    }
  }
  return pos;
}

// sub-tile index of the q-th local sub-tile (q < count; whole wave active)
__device__ __forceinline__ int local_subtile(const LocalSubtiles& t, int q) {
  const uint64_t below = __ballot(t.pre <= q);
  const int l = 63 - __clzll(static_cast<long long>(below));
  const uint64_t m = (static_cast<uint64_t>(static_cast<uint32_t>(read_lane(static_cast<int>(t.hi), l))) << 32) |
                     static_cast<uint32_t>(read_lane(static_cast<int>(t.lo), l));
  return l * t.B + nth_set_bit(m, q - read_lane(t.pre, l));
}

__device__ __forceinline__ bool is_local(const LocalSubtiles& t, int u) {
  const int l = u / t.B, b = u - l * t.B;
  const uint32_t w = static_cast<uint32_t>(read_lane(static_cast<int>(b < 32 ? t.lo : t.hi), l));
  return (w >> (b & 31)) & 1u;
}

// GEMM2: zeros in y for the remote items among [i0, i1) of all nsub*nblk items
// (item = sub-tile * nblk + block).  RB/4 lanes write the RB floats of one row's block,
// 64/(RB/4) rows at a time.
template <int RB, int SUB>
__device__ __forceinline__ void zero_range(const DArgs& p, const int32_t* __restrict__ sorted_ids,
                                           const LocalSubtiles& lt, int i0, int i1) {
  constexpr int LPR = RB / 4, RPP = kWave / LPR;
  static_assert(RB % 4 == 0 && kWave % LPR == 0 && SUB % RPP == 0, "row split");
  const int lane = lane_id();
  int it = i0;
  while (it < i1) {
    const int u = it / p.nblk;
    const int end = min(i1, (u + 1) * p.nblk);
    if (!is_local(lt, u)) {
      int ids[SUB];
      load_ids<SUB>(sorted_ids, u, ids);
#pragma unroll
      for (int t0 = 0; t0 < SUB; t0 += RPP) {
        const int r = pick(ids, t0 + lane / LPR);
        if (r < p.R) {
          float* row = static_cast<float*>(p.C) + static_cast<int64_t>(r) * p.H;
          for (int b = it - u * p.nblk; b < end - u * p.nblk; ++b)
            *reinterpret_cast<float4*>(row + b * RB + 4 * (lane % LPR)) =
                make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
    }
    it = end;
  }
}

// Single-token decode with the routing folded into GEMM1 (ROUTE).  Every wave selects
// the token's experts itself (rdev::topk_select on the router's logit slabs) and ranks
// them by expert index, so that sub-tile u holds the one row of the u-th smallest selected
// expert: the table moe_align builds for these rows with block_m = 16, known to each wave
// without a launch in between.  Work-group 0 also writes the routing (ids, weights) and
// that table for GEMM2.  Ids outside [0, ES) (only where fewer than k experts are
// eligible) get no sub-tile, as in moe_align.
struct DRoute {
  rdev::TopkParams tp;     // T = 1; tp.ids / tp.w: the k + shared slots
  int32_t* sorted_ids;     // [cap]
  int32_t* expert_ids;     // [cap / 16]
  int32_t* ntpp;
  int32_t* counts;         // [ES] or null
  int ES;                  // experts of the table (E + shared)
  int cap;                 // 16 * (k + shared)
};

// lane u < nvalid returns sub-tile u's expert (e_sorted) and row (j_sorted)
__device__ __forceinline__ void route_single_token(const DRoute& r, rdev::TopkLds& tsh,
                                                   bool writer, int& e_sorted, int& j_sorted,
                                                   int& nvalid) {
  const int lane = lane_id();
  int id;
  float w;
  rdev::topk_select<4, 15>(r.tp, 0, tsh, id, w);
  const int K1 = r.tp.k + r.tp.shared;
  const bool valid = lane < K1 && static_cast<unsigned>(id) < static_cast<unsigned>(r.ES);
  const uint64_t vm = __ballot(valid);
  nvalid = __popcll(vm);
  // the selected experts are distinct: rank = number of smaller valid ones
  int rank = 0;
  for (int i = 0; i < K1; ++i) rank += (((vm >> i) & 1) && read_lane(id, i) < id) ? 1 : 0;
  const int dst = valid ? rank : kWave - 1;       // K1 < 64: lane 63 takes the rest
  e_sorted = __builtin_amdgcn_ds_permute(dst * 4, id);
  j_sorted = __builtin_amdgcn_ds_permute(dst * 4, lane);
  if (!writer) return;
  if (lane < K1) {
    r.tp.ids[lane] = id;
    r.tp.w[lane] = w;
  }
  // sorted_ids: the first entry of tile u is its row, the rest the sentinel K1
  for (int q0 = 0; q0 < r.cap; q0 += kWave) {
    const int q = q0 + lane, u = min(q >> 4, kWave - 1);
    const int ju = __shfl(j_sorted, u, kWave);
    if (q < r.cap) r.sorted_ids[q] = ((q & 15) == 0 && u < nvalid) ? ju : K1;
  }
  if (lane < (r.cap >> 4)) r.expert_ids[lane] = lane < nvalid ? e_sorted : -1;
  if (lane == 0) *r.ntpp = 16 * nvalid;
  if (r.counts) {
    for (int e = lane; e < r.ES; e += kWave) {
      int c = 0;
      for (int i = 0; i < K1; ++i) c += (((vm >> i) & 1) && read_lane(id, i) == e) ? 1 : 0;
      r.counts[e] = c;
    }
  }
}

// The routing tables are separate __restrict__ arguments: with them the compiler may
// read the (wave-uniform) entries with scalar loads, which count on lgkmcnt and leave
// the vmcnt accounting of the DMA ring untouched.
//
// Latency outside the stream.  Every wave starts at once, so the memory round trips
// before the first weight DMA and after the last MFMA are dead time for the whole GPU.
// The prologue therefore issues every load that does not depend on another before the
// first wait: the padded total, the owners of the table's whole capacity, and the routing
// ids and owner of the sub-tile that the wave's first item has when every sub-tile is
// local (one round trip to the first DMA instead of four; about 1 us of a one-token
// step).  CACHED (K / STEP >= P: the issue cursor is at most one item ahead of the
// compute): an item's routing ids (and GEMM2's router weights) are kept from its setup for
// its epilogue, and the next item's ids and owner are loaded one item ahead, so the item
// boundaries of the DMA stream and the epilogues do not wait on the routing tables (the
// FP8 epilogue still loads its row scales).
template <int MODE, int RB, int NTG, int STEP, int P, bool NT, int WB, bool CACHED, int XR,
          bool ROUTE = false>
__global__ void __launch_bounds__(64)
moe_decode_kernel(DArgs p, const int32_t* __restrict__ sorted_ids,
                  const int32_t* __restrict__ expert_ids, const int32_t* __restrict__ ntpp,
                  const float* __restrict__ topk_w, const float* __restrict__ wscale,
                  DRoute rt) {
  using S = DStep<STEP, WB>;
  using St = Stream<MODE, RB, NTG, STEP, NT, WB, XR>;
  constexpr int SUB = St::SUB;
  constexpr int NF = RB / 16;                   // 16-row weight fragments per item
  constexpr int NI = St::NW + St::NX;           // DMAs per step
  constexpr int SLOT = RB * S::WROWB + XR * S::XROWB;
  static_assert(RB <= kWave, "one scale per lane");
  static_assert(P >= 3 && (P - 2) * NI < 64, "ring depth");
  static_assert(MODE != 1 || NF % 2 == 0, "gate/up fragment pairs");
  static_assert(!ROUTE || (MODE == 1 && NTG == 1), "routing folds into single-token GEMM1");
  __shared__ __attribute__((aligned(1024))) uint8_t ring[P * SLOT];

  const int lane = lane_id();
  const int first = blockIdx.x;
  // independent loads first (see above); u0 < nsub_cap keeps them inside the table
  // (per-lane vector loads: no DMA is in flight yet, so their waits cost nothing, and the
  // compiler keeps them in one batch with the owner loads)
  const int u0 = min(first / p.nblk, p.nsub_cap - 1);
  int ids0v, e0v, nsub;
  LocalSubtiles lt;
  int re_sorted = 0, rj_sorted = 0;             // ROUTE: sub-tile (lane) -> expert, row
  if constexpr (ROUTE) {
    __shared__ rdev::TopkLds tsh;
    int nvalid;
    route_single_token(rt, tsh, first == 0, re_sorted, rj_sorted, nvalid);
    const int j0 = __shfl(rj_sorted, u0, kWave);
    ids0v = lane == 0 ? j0 : p.R;
    e0v = __shfl(re_sorted, u0, kWave);
    nsub = nvalid;
    lt.count = nsub;
  } else {
    ids0v = sorted_ids[static_cast<int64_t>(u0) * SUB + min(lane, SUB - 1)];
    e0v = expert_ids[(u0 * SUB) >> p.bm_shift];
    const int totalv = *ntpp;
    lt = local_subtiles<SUB>(expert_ids, p.nsub_cap, totalv / SUB, p.bm_shift);
    nsub = read_lane(totalv, 0) / SUB;
  }
  if (nsub == 0) return;
  const int nitems = lt.count * p.nblk;         // items of local sub-tiles
  const bool all_local = lt.count == nsub;
  // as many waves as give every wave the same number of items (the fewest waves that
  // reach the smallest per-wave count): a wave streams at a bounded rate, so a tail of
  // waves with one item more would run at a fraction of the bandwidth
  const int per = (nitems + gridDim.x - 1) / gridDim.x;
  const int G = per > 0 ? (nitems + per - 1) / per : 0;
  if (MODE == 2 && !all_local) {
    // zeros for the rows of remote sub-tiles: the waves left without local items share
    // them in contiguous ranges (the sub-tile's row ids are loaded once per sub-tile);
    // when every wave streams, each adds an equal share after its own items
    const int64_t nz = static_cast<int64_t>(nsub) * p.nblk;
    const int idle = gridDim.x - G;
    if (idle > 0 && first >= G) {
      const int w = first - G;
      zero_range<RB, SUB>(p, sorted_ids, lt, static_cast<int>(nz * w / idle),
                          static_cast<int>(nz * (w + 1) / idle));
      return;
    }
  }
  if (first >= G) return;
  const int nsteps = p.K / STEP;
  const int gtot = ((nitems - 1 - first) / G + 1) * nsteps;   // this wave's steps

  // local item j -> (sub-tile u, weight-row block blk)
  auto item_at = [&](int j, int& u, int& blk) {
    const int q = j / p.nblk;
    blk = j - q * p.nblk;
    u = all_local ? q : local_subtile(lt, q);
  };
  auto owner = [&](int u) {
    if constexpr (ROUTE) return read_lane(re_sorted, u);
    else return expert_ids[(u * SUB) >> p.bm_shift];
  };
  // the SUB routed rows of sub-tile u
  auto fetch_ids = [&](int u, int (&ids)[SUB]) {
    if constexpr (ROUTE) {
      ids[0] = read_lane(rj_sorted, u);
#pragma unroll
      for (int t = 1; t < SUB; ++t) ids[t] = p.R;
    } else {
      load_ids<SUB>(sorted_ids, u, ids);
    }
  };

  // issue item: routing ids (in lanes), block, expert
  int iidsv, ib, ie;
  if (all_local) {
    ib = first - u0 * p.nblk;
    ie = read_lane(e0v, 0);
    iidsv = ids0v;
  } else {
    int iu;
    item_at(first, iu, ib);
    ie = owner(iu);
    int ids[SUB];
    fetch_ids(iu, ids);
    iidsv = spread(ids);
  }
  // CACHED: the next issue item (loaded one item ahead), the issue item's ids held in
  // lanes and its GEMM2 router weights (loads in flight), the compute item's ones
  int nids[SUB], nb = 0, ne = 0;
  int bw[SUB];
  int c_idsv = 0, c_wv = 0, cb = 0, ce = 0;
  auto prefetch_next = [&](int j) {
    if (j < nitems) {
      int nu;
      item_at(j, nu, nb);
      ne = owner(nu);
      fetch_ids(nu, nids);
    }
  };
  // GEMM2: the router weights of the issue item's rows (uniform loads)
  auto load_issue_weights = [&]() {
    if (MODE == 2) {
#pragma unroll
      for (int t = 0; t < SUB; ++t) {
        const int r = read_lane(iidsv, t);
        bw[t] = __float_as_int(topk_w[r < p.R ? r : 0]);
      }
    }
  };

  // issue cursor: the step the next DMA batch belongs to (it stays on the last step
  // once everything is issued, so the ring tail re-reads it into unused slots)
  MOE_LDS uint8_t* lring = (MOE_LDS uint8_t*)ring;
  const uint8_t* wp[St::NW];
  const uint16_t* xp[St::NX];
  St::setup(p, iidsv, ib, ie, wp, xp);
  if (CACHED) {
    load_issue_weights();
    prefetch_next(first + G);
  }
  int gi = 0, iss_s = 0, iss_item = first;
  auto issue_next = [&]() {
    St::issue(wp, xp, iss_s * STEP, lring + (gi % P) * SLOT);
    ++gi;
    if (gi < gtot && ++iss_s == nsteps) {
      iss_s = 0;
      iss_item += G;
      if (CACHED) {
        ib = nb;
        ie = ne;
        iidsv = spread(nids);
        St::setup(p, iidsv, ib, ie, wp, xp);
        load_issue_weights();
        prefetch_next(iss_item + G);
      } else {
        int iu;
        item_at(iss_item, iu, ib);
        ie = owner(iu);
        int ids[SUB];
        fetch_ids(iu, ids);
        iidsv = spread(ids);
        St::setup(p, iidsv, ib, ie, wp, xp);
      }
    }
  };
#pragma unroll
  for (int q = 0; q < P - 1; ++q) issue_next();
  // CACHED: K / STEP >= P, so the prologue stayed inside the first item
  auto take_issue_item = [&]() {
    c_idsv = iidsv;
    if (MODE == 2) c_wv = spread(bw);
    cb = ib;
    ce = ie;
  };
  if (CACHED) take_issue_item();

  f32x4 acc[NTG][NF];
  int cs = 0, cmp_item = first;
  const int tr = lane & 15;
  const int xrow = XR < 16 ? (tr & (XR - 1)) : tr;   // token row the lane's column reads
  for (int g = 0; g < gtot; ++g) {
    wait_vm_c<(P - 2) * NI>();                  // step g's batch has landed in LDS
    asm volatile("" ::: "memory");
    issue_next();                               // into the slot step g-1 used
    if (cs == 0) {
#pragma unroll
      for (int q = 0; q < NTG; ++q)
#pragma unroll
        for (int f = 0; f < NF; ++f) acc[q][f] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const uint8_t* slot = ring + (g % P) * SLOT;
    const uint8_t* xs = slot + RB * S::WROWB;   // token rows of the step
    if (WB == 2) {
#pragma unroll
      for (int ks = 0; ks < S::KSUB; ++ks) {
        const int c = ks * 4 + (lane >> 4);     // 8 k-elements of lane group lane>>4
        bf16x8 b[NTG];
#pragma unroll
        for (int q = 0; q < NTG; ++q)
          b[q] = *reinterpret_cast<const bf16x8*>(xs + (16 * q + xrow) * S::XROWB +
                                                  dsw<S::XCPR>(xrow, c) * 16);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const int row = 16 * f + tr;
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(slot + row * S::WROWB +
                                                            dsw<S::WCPR>(row, c) * 16);
#pragma unroll
          for (int q = 0; q < NTG; ++q)
            acc[q][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[q], acc[q][f], 0, 0, 0);
        }
      }
    } else {
      // Two MFMAs per 64 k-elements.  The sum over k does not depend on how k is dealt
      // to lane groups, so lane group gq takes the 16 consecutive k-elements
      // 16*gq .. 16*gq+15 of the 64: one 16-byte chunk of each weight row (expanded to
      // two bf16x8), and the two matching bf16 chunks of each token row.
#pragma unroll
      for (int kp = 0; kp < S::KSUB / 2; ++kp) {
        const int gq = lane >> 4;
        const int cw = kp * 4 + gq;             // weight chunk (16 E4M3 values)
        const int cx = kp * 8 + 2 * gq;         // first of two token chunks
        bf16x8 b0[NTG], b1[NTG];
#pragma unroll
        for (int q = 0; q < NTG; ++q) {
          const uint8_t* xr = xs + (16 * q + xrow) * S::XROWB;
          b0[q] = *reinterpret_cast<const bf16x8*>(xr + dsw<S::XCPR>(xrow, cx) * 16);
          b1[q] = *reinterpret_cast<const bf16x8*>(xr + dsw<S::XCPR>(xrow, cx + 1) * 16);
        }
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const int row = 16 * f + tr;
          const u32x4 wq = *reinterpret_cast<const u32x4*>(slot + row * S::WROWB +
                                                           dsw<S::WCPR>(row, cw) * 16);
          bf16x8 a0, a1;
          fp8x16_to_bf16(wq, a0, a1);
#pragma unroll
          for (int q = 0; q < NTG; ++q) {
            acc[q][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b0[q], acc[q][f], 0, 0, 0);
            acc[q][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1[q], acc[q][f], 0, 0, 0);
          }
        }
      }
    }
    if (++cs == nsteps) {
      // epilogue.  D layout (16x16): lane holds token column (lane & 15), weight rows
      // 4*(lane>>4)+v of each fragment
      cs = 0;
      int blk, cmp_e, idsv, wv = 0;
      if (CACHED) {
        blk = cb;
        cmp_e = ce;
        idsv = c_idsv;
        wv = c_wv;
      } else {
        int u;
        item_at(cmp_item, u, blk);
        cmp_e = owner(u);
        int ids[SUB];
        fetch_ids(u, ids);
        idsv = spread(ids);
        if (MODE == 2) {
          int wts[SUB];                         // router weights (uniform loads)
#pragma unroll
          for (int t = 0; t < SUB; ++t)
            wts[t] = __float_as_int(topk_w[ids[t] < p.R ? ids[t] : 0]);
          wv = spread(wts);
        }
      }
      // FP8 weights: the row scales of this lane's accumulator rows 16f + 4(lane>>4) + v.
      // Lane j of stab holds the scale of the item's weight row j (uniform loads, in the
      // order of the DMA rows: gate rows then up rows for GEMM1); the lane-crossbar reads
      // run here, with the whole wave active (an inactive source lane reads as 0).
      float rs[NF][4];
      if (WB == 1) {
        const int nrows = MODE == 1 ? 2 * p.I : p.H;
        const float* sp = wscale + static_cast<int64_t>(cmp_e) * nrows;
        int sv[RB];
#pragma unroll
        for (int j = 0; j < RB; ++j) {
          const int wrow = MODE == 1 ? (j < RB / 2 ? blk * (RB / 2) + j
                                                   : p.I + blk * (RB / 2) + (j - RB / 2))
                                     : blk * RB + j;
          sv[j] = __float_as_int(sp[wrow]);
        }
        const int stab = spread(sv);
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            rs[f][v] = __int_as_float(__shfl(stab, 16 * f + 4 * (lane >> 4) + v, kWave));
      }
#pragma unroll
      for (int q = 0; q < NTG; ++q) {
        const int r = __shfl(idsv, 16 * q + tr, kWave);
        const float wr = MODE == 2 ? __int_as_float(__shfl(wv, 16 * q + tr, kWave)) : 0.f;
        if (r < p.R) {
          if (MODE == 1) {
#pragma unroll
            for (int f = 0; f < NF / 2; ++f) {
              f32x4 gt = acc[q][f], up = acc[q][f + NF / 2];
              if (WB == 1) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                  gt[v] *= rs[f][v];
                  up[v] *= rs[f + NF / 2][v];
                }
              }
              uint32_t pk[2];
#pragma unroll
              for (int v = 0; v < 4; v += 2)
                pk[v / 2] = pack_bf16x2(silu_mul_bf16path(gt[v], up[v]),
                                        silu_mul_bf16path(gt[v + 1], up[v + 1]));
              uint16_t* out = static_cast<uint16_t*>(p.C) + static_cast<int64_t>(r) * p.I +
                              blk * (RB / 2) + 16 * f + 4 * (lane >> 4);
              *reinterpret_cast<uint2*>(out) = make_uint2(pk[0], pk[1]);
            }
          } else {
#pragma unroll
            for (int f = 0; f < NF; ++f) {
              f32x4 v4 = acc[q][f];
              if (WB == 1) {
#pragma unroll
                for (int v = 0; v < 4; ++v) v4[v] *= rs[f][v];
              }
              float* out = static_cast<float*>(p.C) + static_cast<int64_t>(r) * p.H +
                           blk * RB + 16 * f + 4 * (lane >> 4);
              *reinterpret_cast<float4*>(out) =
                  make_float4(wr * v4[0], wr * v4[1], wr * v4[2], wr * v4[3]);
            }
          }
        }
      }
      cmp_item += G;
      // the issue cursor is on the next item by now (or still on this one, the last)
      if (CACHED) take_issue_item();
    }
  }
  if (MODE == 2 && !all_local && G == static_cast<int>(gridDim.x)) {
    const int64_t nz = static_cast<int64_t>(nsub) * p.nblk;
    zero_range<RB, SUB>(p, sorted_ids, lt, static_cast<int>(nz * first / G),
                        static_cast<int>(nz * (first + 1) / G));
  }
  wait_vm_c<0>();                                // no DMA may land after the wave exits
}

constexpr int kDecodeRB = 64;   // weight rows per work item (32 for bf16 16-row sub-tiles)

int decode_ntg(int block_m, int R, int E) {
  // 32-row sub-tiles once experts average more than one row: the popular experts then
  // fit one sub-tile and their weights are streamed once (measured +9 % at T=64 on the
  // DeepSeek-V3 layer); never more than one align tile
  const int want = R > E ? 2 : 1;
  return std::min(want, block_m / 16);
}

template <int MODE, int NTG, int STEP, bool NT, int WB, int P, int RB, int XR>
hipError_t launch_decode_x(const DArgs& p0, const GemmArgs& g, hipStream_t s, const DRoute* rt) {
  using S = DStep<STEP, WB>;
  DArgs p = p0;
  p.nblk = (MODE == 1 ? 2 * p.I : p.H) / RB;
  constexpr int kLds = P * (RB * S::WROWB + XR * S::XROWB);
  constexpr int kPerCU = std::max(1, (160 * 1024) / kLds);
  p.nsub_cap = static_cast<int>(g.cap / (16 * NTG));
  p.bm_shift = __builtin_ctz(static_cast<unsigned>(p.block_m));   // block_m: a power of two
  if (p.nsub_cap == 0) return hipSuccess;
  const int64_t max_items = static_cast<int64_t>(p.nsub_cap) * p.nblk;
  const unsigned grid = static_cast<unsigned>(std::min<int64_t>(max_items, 256 * kPerCU));
  if constexpr (MODE == 1 && NTG == 1 && NT && XR < 16) {
    if (rt) {
      if (p.K / STEP >= P)
        hipLaunchKernelGGL((moe_decode_kernel<MODE, RB, NTG, STEP, P, NT, WB, true, XR, true>),
                           dim3(grid), dim3(64), 0, s, p, g.sorted_ids, g.expert_ids, g.ntpp,
                           g.topk_w, g.w_scale, *rt);
      else
        hipLaunchKernelGGL((moe_decode_kernel<MODE, RB, NTG, STEP, P, NT, WB, false, XR, true>),
                           dim3(grid), dim3(64), 0, s, p, g.sorted_ids, g.expert_ids, g.ntpp,
                           g.topk_w, g.w_scale, *rt);
      return hipGetLastError();
    }
  }
  if (rt) return hipErrorInvalidValue;          // routing folds into single-token GEMM1 only
  const DRoute none{};
  if (p.K / STEP >= P)
    hipLaunchKernelGGL((moe_decode_kernel<MODE, RB, NTG, STEP, P, NT, WB, true, XR>),
                       dim3(grid), dim3(64), 0, s, p, g.sorted_ids, g.expert_ids, g.ntpp,
                       g.topk_w, g.w_scale, none);
  else
    hipLaunchKernelGGL((moe_decode_kernel<MODE, RB, NTG, STEP, P, NT, WB, false, XR>),
                       dim3(grid), dim3(64), 0, s, p, g.sorted_ids, g.expert_ids, g.ntpp,
                       g.topk_w, g.w_scale, none);
  return hipGetLastError();
}

// token rows per sub-tile that are streamed: one DMA's worth when no expert holds more
// rows than that (16-row sub-tiles only), else all of them
template <int MODE, int NTG, int STEP, bool NT, int WB, int P, int RB = kDecodeRB,
          int PF = P, int RBF = RB>
hipError_t launch_decode(const DArgs& p, const GemmArgs& g, hipStream_t s, const DRoute* rt) {
  constexpr int XRPI = DStep<STEP, WB>::XRPI;
  const int64_t bound = g.max_rows > 0 ? g.max_rows : static_cast<int64_t>(g.T) * g.k;
  if constexpr (NTG == 1)
    if (bound <= XRPI) return launch_decode_x<MODE, NTG, STEP, NT, WB, PF, RBF, XRPI>(p, g, s, rt);
  return launch_decode_x<MODE, NTG, STEP, NT, WB, P, RB, 16 * NTG>(p, g, s, rt);
}

// bf16 weights, 128-element steps (K % 128 != 0: 64).  GEMM1 with 16-row sub-tiles:
// 32-row work items with a 6-slot ring (two waves per CU); against 64-row items and a
// 4-slot ring it measured level at the DeepSeek-V3 shape's T = 1 and 20 % faster when
// the items just exceed the waves (Kimi K2 at T = 1: 9 experts, 576 items of 64 rows
// for 512 waves).  GEMM2 measured no better that way and keeps 64-row items; 32-row
// sub-tiles keep 64-row items and a 3-slot ring.
template <int MODE, int NTG, bool NT>
hipError_t launch_decode_bf16(const DArgs& p, const GemmArgs& g, hipStream_t s,
                              const DRoute* rt) {
  if (p.K % 128 != 0) return launch_decode<MODE, NTG, 64, NT, 2, NTG == 1 ? 4 : 3>(p, g, s, rt);
  if constexpr (NTG == 1 && MODE == 1) return launch_decode<MODE, NTG, 128, NT, 2, 6, 32>(p, g, s, rt);
  else return launch_decode<MODE, NTG, 128, NT, 2, NTG == 1 ? 4 : 3>(p, g, s, rt);
}

// FP8 weights: 128-element steps (128-byte weight rows, 256-byte token rows; K % 128 == 0
// is checked by the caller).  Measured on the DeepSeek-V3 layer: a 4-slot ring at three
// waves per CU streams faster than 256-element steps (which fit one or two waves per CU)
// at every batch size; 32-row sub-tiles need the 3-slot ring to keep three waves.
template <int MODE, int NTG, bool NT>
hipError_t launch_decode_fp8(const DArgs& p, const GemmArgs& g, hipStream_t s,
                              const DRoute* rt) {
  return launch_decode<MODE, NTG, 128, NT, 1, NTG == 1 ? 4 : 3>(p, g, s, rt);
}

template <int MODE, int NTG, bool NT>
hipError_t launch_decode_w(const DArgs& p, const GemmArgs& g, hipStream_t s, const DRoute* rt) {
  return g.w_scale ? launch_decode_fp8<MODE, NTG, NT>(p, g, s, rt)
                   : launch_decode_bf16<MODE, NTG, NT>(p, g, s, rt);
}

template <int MODE>
hipError_t run_decode(const GemmArgs& g, hipStream_t s, const DRoute* rt = nullptr) {
  DArgs p{};
  const bool g1 = MODE == 1;
  p.A = static_cast<const uint8_t*>(g.B);
  p.X = static_cast<const uint16_t*>(g.A);
  p.C = g.C;
  p.R = g.T * g.k;
  p.gather_div = g1 ? g.k : 1;
  p.K = g1 ? g.H : g.I;
  p.I = g.I;
  p.H = g.H;
  p.a_expert_stride = g1 ? static_cast<int64_t>(2) * g.I * g.H : static_cast<int64_t>(g.H) * g.I;
  p.block_m = g.block_m;
  if (g.cap == 0) return hipSuccess;
  const int ntg = decode_ntg(g.block_m, p.R, g.E);
  // non-temporal weight stream while almost every expert fits one sub-tile (each weight
  // block read once); otherwise the sub-tiles of one expert re-read its weights, and
  // those re-reads should hit in L2
  if (ntg == 2)
    return p.R <= 4 * g.E ? launch_decode_w<MODE, 2, true>(p, g, s, rt)
                          : launch_decode_w<MODE, 2, false>(p, g, s, rt);
  return p.R <= 2 * g.E ? launch_decode_w<MODE, 1, true>(p, g, s, rt)
                        : launch_decode_w<MODE, 1, false>(p, g, s, rt);
}

}  // namespace

int decode_block_m(int R, int E) { return 16 * decode_ntg(256, R, E); }

hipError_t launch_decode_gemm1(const GemmArgs& g, hipStream_t s) { return run_decode<1>(g, s); }

bool decode_route_ok(int T, int E, int k, int shared) {
  return T == 1 && E <= 4 * kWave && k + shared < kWave;
}

hipError_t launch_decode_gemm1_routed(const GemmArgs& g, const float* logits, int nz,
                                      const RouteArgs& a, int E, int k, int32_t* ids, float* w,
                                      int32_t* counts, hipStream_t s) {
  if (!decode_route_ok(g.T, E, k, a.shared) || g.k != k + a.shared || g.block_m != 16 ||
      g.cap != 16 * g.k)
    return hipErrorInvalidValue;
  DRoute r{};
  r.tp.logits = logits;
  r.tp.t0 = 0;
  r.tp.nz = nz;
  r.tp.logits_out = nullptr;
  r.tp.T = 1;
  r.tp.E = E;
  r.tp.k = k;
  r.tp.mode = a.mode;
  r.tp.offset = a.offset;
  r.tp.bias = a.bias;
  r.tp.n_group = a.n_group;
  r.tp.topk_group = a.topk_group;
  r.tp.scaling = a.scaling;
  r.tp.ids = ids;
  r.tp.w = w;
  r.tp.shared = a.shared;
  r.sorted_ids = const_cast<int32_t*>(g.sorted_ids);
  r.expert_ids = const_cast<int32_t*>(g.expert_ids);
  r.ntpp = const_cast<int32_t*>(g.ntpp);
  r.counts = counts;
  r.ES = g.E;
  r.cap = static_cast<int>(g.cap);
  GemmArgs g1 = g;
  g1.max_rows = 1;
  return run_decode<1>(g1, s, &r);
}
hipError_t launch_decode_gemm2(const GemmArgs& g, hipStream_t s) { return run_decode<2>(g, s); }

}  // namespace moe
