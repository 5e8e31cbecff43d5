// Large-tile gathered grouped GEMMs for prefill (GEMM1 + SwiGLU, GEMM2 x router weight):
// same contract as the kernels in gemm.hip ("Mixture-of-Experts Kernels: Routing,
// Permutation, and Grouped GEMM", section 6), with a deeper memory pipeline for gfx950:
//
// * Global -> LDS without registers: global_load_lds_dwordx4 writes each lane's 16 bytes
//   at (wave base + 16 * lane), so the LDS swizzle is applied on the global side: lane i
//   of an instruction fetches the logical chunk that belongs at physical slot i.
// * A ring of 64-element stages: 128-byte LDS rows (bf16; chunk c of row m at
//   c ^ ((m >> 1) & 7)) and 64-byte rows (FP8 B; c ^ sw4(m)); both swizzles are
//   conflict-free for the DMA writes and the 32-row MFMA operand reads.
// * v_mfma_f32_32x32x16_bf16, WM x WN waves each holding a (BM/WM) x (BN/WN) fp32
//   accumulator tile; GEMM1 B tiles interleave 32-row gate and up blocks so that SwiGLU
//   runs in registers.
// * 2 x 4 waves (two per SIMD, 128 x 64 or 64 x 64 each) in a ping-pong schedule over
//   two 64-element stages (bf16 256-row tiles) or three (the other tiles): the two waves
//   of a SIMD alternate between loading a half-stage of fragments from LDS and a burst of
//   MFMAs from registers, with a barrier at each turn and the DMAs between the MFMAs (see
//   the K loop).
// * GEMM2 splits a short last round of tiles in K over every CU (see split_plan).
// * FP8 expert weights (OCP E4M3 bytes, one fp32 scale per weight row; section 8 of the
//   same page prices an expert at one byte per weight): the B tile is staged as bytes
//   (64-byte LDS rows per 64-element stage, half the bf16 B tile, so the 256-row tile
//   fits a 3-stage ring), each 16-byte chunk is expanded to bf16 after the LDS read (exact,
//   in the load phase of the ping-pong) and feeds two bf16 MFMAs, and the row scales
//   (staged in LDS with the tile's rows) multiply the fp32 accumulators in the epilogue.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "common.hpp"
#include "dma.hpp"
#include "launch.hpp"

namespace moe {

namespace {

struct PArgs {
  const uint16_t* A;
  const uint8_t* B;        // bf16 or E4M3 bytes
  const float* B_scale;    // FP8 weights: per-row scales [E, 2I] or [E, H]
  void* C;
  const float* topk_w;
  const int32_t* sorted_ids;
  const int32_t* expert_ids;
  const int32_t* ntpp;
  int R, gather_div, K, N, I;
  int64_t b_expert_stride;
  int block_m;
  int mtiles, nblocks;
  int n_outer;             // raster order of the tile groups (see grouped_slot)
  // GEMM2: split of the last partial round (see split_plan); 1 = off
  int split_max;
  int ncu;                 // work-groups in flight: one round = ncu tiles (CUs x work-groups per CU)
  float* partial;          // [ncu][BM][BN] fp32 partial sums of the split tiles
  const int2* tile_run;    // nullable: (first tile, tiles) of each block_m tile's expert run,
                           // then (longest run, 0) at index mtiles / tile_div
  int tile_div;            // block_m / BM: BM-row tiles per align tile
};

template <int MODE, int BM, int BN, int WM, int WN, int BK_, int NSTAGE, int WB = 2>
struct PCfg {
  static constexpr int NW = WM * WN;
  static constexpr int NT = NW * kWave;
  static constexpr int BK = BK_;                      // K elements per stage (64)
  static constexpr int ROWA = BK * 2;                 // bytes per LDS row of A (bf16)
  static constexpr int ROWB = BK * WB;                // bytes per LDS row of B (bf16 / E4M3)
  static constexpr int CPRA = ROWA / 16, CPRB = ROWB / 16;   // 16-byte chunks per row
  static constexpr int RPIA = kWave / CPRA;           // rows per DMA instruction (1 KB)
  static constexpr int RPIB = kWave / CPRB;
  static constexpr int KS = BK / 16;                  // k16 MFMA steps per stage
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int LA = BM / RPIA / NW;           // DMA instructions per wave per stage (A)
  static constexpr int LB = BN / RPIB / NW;           // (B)
  static constexpr int L = LA + LB;
  static constexpr int SA = BM * ROWA, SB = BN * ROWB;
  static constexpr int STAGE = SA + SB;
  static constexpr int EXTRA = BM * 4 + (MODE == 2 ? BM * 4 : 0) + (WB == 1 ? BN * 4 : 0);
  static_assert(BK == 64, "64-element stages");
  static_assert(BM % (RPIA * NW) == 0 && BN % (RPIB * NW) == 0, "DMA rows per wave");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  static_assert(MODE != 1 || WTN % 64 == 0, "GEMM1 wave tile holds gate/up pairs");
  static_assert(NSTAGE >= 2 && NSTAGE * STAGE + EXTRA <= 160 * 1024, "LDS");
};

// LDS swizzles (chunk c of row m lives at physical chunk c ^ sw(m)).  64-byte rows:
// sw = (m >> 2) & 3; 128-byte rows: sw = (m >> 1) & 7.  Both spread the MFMA operand
// reads (rows m..m+31 at one logical chunk) over all banks: measured with
// SQ_LDS_BANK_CONFLICT on 64-byte rows (Qwen3 shape, then in bf16 tiles of 32-element
// stages), (m >> 2) & 3 takes the conflict cycles from half of the LDS-active cycles to
// none, where ((m >> 1) ^ (m >> 3)) & 3 left them.
__device__ __forceinline__ int sw4(int row) { return (row >> 2) & 3; }
template <int ROWB>
__device__ __forceinline__ int swz(int row) { return ROWB == 64 ? sw4(row) : ((row >> 1) & 7); }
template <int ROWB>
__device__ __forceinline__ int pswz(int row, int chunk) {
  return row * ROWB + ((chunk ^ swz<ROWB>(row)) << 4);
}

// 16 E4M3 bytes -> two runs of 8 bf16 (bytes 0..7, bytes 8..15), exact
__device__ __forceinline__ void fp8x16_to_bf16x2(const u32x4 q, bf16x8& lo, bf16x8& hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 h[8];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    h[2 * d] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[d], 1.0f, false);
    h[2 * d + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[d], 1.0f, true);
  }
  lo = bf16x8{h[0][0], h[0][1], h[1][0], h[1][1], h[2][0], h[2][1], h[3][0], h[3][1]};
  hi = bf16x8{h[4][0], h[4][1], h[5][0], h[5][1], h[6][0], h[6][1], h[7][0], h[7][1]};
}

// Register fragments of one MFMA step group: bf16 weights use one k16 step (A and B
// chunk per lane); FP8 weights use two k16 steps per B chunk (16 E4M3 values per lane).
template <int FM, int FN, int WB>
struct Frags;
template <int FM, int FN>
struct Frags<FM, FN, 2> {
  bf16x8 a[FM], b[FN];
};
template <int FM, int FN>
struct Frags<FM, FN, 1> {
  bf16x8 a0[FM], a1[FM];
  u32x4 q[FN];
};

// Work-group -> (m-tile, n-block).  Work-groups are dealt round-robin over the 8 XCDs
// (bid % 8) and each XCD runs its share in bid order, so bid = 8*j + xcd is the j-th
// work-group of that XCD.  Slots are cut into groups of GM m-tiles x GN n-blocks; group
// g runs on XCD g % 8, its GM*GN tiles back to back, so the tiles running together on
// one XCD share GM A tiles (token rows) and GN B tiles (expert weight blocks) through
// that XCD's L2.  Group order: with n_outer, n-groups outer and m-groups inner (the
// groups in flight at once on the 8 XCDs cover many m-tiles of the same weight
// columns); otherwise m-groups outer (an XCD's consecutive groups reuse the same token
// rows while the weight columns advance).  The host picks n_outer when there are more
// m-tiles than n-blocks.  Returns false for the slots past the last group.
template <int GM, int GN>
__device__ __forceinline__ bool grouped_slot(int bid, int mtiles, int nblocks, bool n_outer,
                                             int& mt, int& nb) {
  constexpr int GS = GM * GN;
  const int xcd = bid & 7, j = bid >> 3;
  const int g = (j / GS) * 8 + xcd, pos = j % GS;
  int gm, gn;
  if (n_outer) {
    const int ngroups_m = (mtiles + GM - 1) / GM;
    gn = g / ngroups_m;
    gm = g % ngroups_m;
  } else {
    const int ngroups_n = (nblocks + GN - 1) / GN;
    gm = g / ngroups_n;
    gn = g % ngroups_n;
  }
  mt = gm * GM + pos % GM;
  nb = gn * GN + pos / GM;
  return mt < mtiles && nb < nblocks;
}
constexpr int kGroupM = 4, kGroupN = 4;

// GEMM2: balanced rounds with a split last round.  GEMM2's tiles are few
// and long (K = I), so the rounds of ncu tiles (the work-groups in flight) quantise: at the
// Mixtral-8x7B shape 592 tiles make 2.3 rounds but take 3, with the grouped raster above
// dealing 96 tiles to some XCDs and 64 to others.  Here the real tile count N (from the
// padded total on the device) is split into N - rem whole tiles, rem = N mod ncu, and the
// rem tiles of the last round, each cut into `parts` K ranges (parts <= split_max, parts *
// rem <= ncu), so the last round is a few partial-sum work-groups spread over every CU.
// Whole tiles: XCD x (= bid % 8) takes the contiguous tile range [x N'/8, (x+1) N'/8) in
// order; tiles are in the expert-ordered raster when align supplied the run table (see
// expert_tile), else in strips of 8 n-blocks with the m-tiles inside, so the 32 tiles an
// XCD runs at once are 4 m-tiles x 8 n-blocks, as with the grouped raster.  Split
// parts write raw fp32 sums to `partial`; a fix-up launch adds them in part order and
// applies the row scale (FP8 weights) and the router weight.  When the plan splits nothing (rem = 0, or too many tiles
// left over for a short round) the grouped raster above is kept.
struct SplitPlan {
  int mreal, full, rem, parts;
};
__device__ __forceinline__ SplitPlan split_plan(int total, int bm, int nblocks, int ncu,
                                                int split_max, int nk) {
  SplitPlan s;
  s.mreal = total / bm;
  const int nreal = s.mreal * nblocks;
  s.rem = nreal % ncu;
  s.parts = s.rem > 0 ? min(min(split_max, ncu / s.rem), nk) : 1;
  if (s.parts < 2) {
    s.rem = 0;
    s.parts = 1;
  }
  s.full = nreal - s.rem;
  return s;
}
// Expert-ordered raster (when align supplied the run table): items (m-tile, n-block) in
// order of expert run, and XCD x takes the contiguous item range [x N / 8, (x + 1) N / 8).
// Inside a run the m-tiles go in chunks of up to kRunChunk, each chunk n-block major and
// m-tile minor.  The ~32 tiles an XCD runs together are then the m-tiles of one chunk
// times a few n-blocks: each weight block crosses that XCD's L2 once per chunk (once per
// expert at the Mixtral-8x7B shape, 4-5 m-tiles of 256 rows per expert, instead of once
// per group of 4 m-tiles), and a long run (a hot expert) still reuses its token rows
// across the chunk's n-blocks.  An expert's items are [first * nblocks, (first + tiles)
// * nblocks), so item q belongs to the run of BM-tile q / nblocks.
constexpr int kRunChunk = 8;
// longest expert run (in BM-row tiles) for which the expert order is used: with longer
// runs (a few hot experts holding most rows) the grouped raster measured faster (Qwen3
// skewed routing: 3.58 against 3.80 ms for the layer)
constexpr int kRunOrderMax = 32;
// stands in for the longest-run entry when align supplied no run table, so that the
// kernel's first loads (padded total, longest run) issue together without a branch
__device__ const int2 kNoRunTable = {1 << 29, 0};
template <typename Args>
__device__ __forceinline__ const int2* longest_run_entry(const Args& p) {
  return p.tile_run ? p.tile_run + p.mtiles / p.tile_div : &kNoRunTable;
}
template <typename Args>
__device__ __forceinline__ bool use_run_order(const Args& p, int longest) {
  return p.tile_run && longest * p.tile_div <= kRunOrderMax;
}
template <typename Args>
__device__ __forceinline__ bool use_run_order(const Args& p) {
  return use_run_order(p, longest_run_entry(p)->x);
}
template <typename Args>
__device__ __forceinline__ void expert_tile(int64_t q, const Args& p, int& mt, int& nb) {
  const int t = static_cast<int>(q / p.nblocks);
  const int2 run = p.tile_run[t / p.tile_div];
  const int first = run.x * p.tile_div, tiles = run.y * p.tile_div;
  const int64_t local = q - static_cast<int64_t>(first) * p.nblocks;
  const int64_t span = static_cast<int64_t>(kRunChunk) * p.nblocks;   // items of a full chunk
  const int k = static_cast<int>(local / span);
  const int rest = static_cast<int>(local - k * span);
  const int ck = min(kRunChunk, tiles - k * kRunChunk);               // m-tiles of chunk k
  nb = rest / ck;
  mt = first + k * kRunChunk + (rest - nb * ck);
}

// tile q of the strip order -> (m-tile, n-block)
__device__ __forceinline__ void strip_tile(int q, int mreal, int nblocks, int& mt, int& nb) {
  const int nfs = nblocks / 8, span = mreal * 8;
  if (q < nfs * span) {
    const int st = q / span, r = q - st * span;
    mt = r / 8;
    nb = st * 8 + r % 8;
  } else {
    const int wl = nblocks - nfs * 8, r = q - nfs * span;
    mt = r / wl;
    nb = nfs * 8 + r % wl;
  }
}

// Two waves per SIMD with 8-wave work-groups (the ping-pong tiles: the two waves of a SIMD
// take turns at the MFMA pipe, see the K loop); the register budget is held to that.  One
// work-group per CU in every configuration (its ring takes 96 to 144 KB of LDS).
template <int MODE, int BM, int BN, int WM, int WN, int BK, int NSTAGE, int WB>
__global__ void __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(WM * WN == 8 ? 2 : 1)))
moe_gemm_pipe_kernel(PArgs p) {
  using C = PCfg<MODE, BM, BN, WM, WN, BK, NSTAGE, WB>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NSTAGE * C::STAGE];
  __shared__ int srow[BM];
  __shared__ float swt[MODE == 2 ? BM : 1];       // GEMM2: router weight of each tile row
  __shared__ float sscale[WB == 1 ? BN : 1];      // FP8: scale of each B tile row

  // the two independent loads that every tile's mapping starts from, issued together (the
  // mapping, the tile's expert and its row ids follow: three round trips in all)
  const int total = *p.ntpp;                      // padded total
  const int longest = longest_run_entry(p)->x;
  int mt, nb;
  int kb = 0, ke = p.K / C::BK;   // the K stages of this work-group
  int unit = -1;                  // >= 0: a K range of a split tile (writes partial sums)
  SplitPlan sp{0, 0, 0, 1};
  if (MODE == 2 && p.split_max > 1)
    sp = split_plan(total, BM, p.nblocks, p.ncu, p.split_max, ke);
  const bool run_order = use_run_order(p, longest);
  if (sp.parts > 1) {
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int x0 = static_cast<int>(static_cast<int64_t>(sp.full) * xcd / 8);
    const int x1 = static_cast<int>(static_cast<int64_t>(sp.full) * (xcd + 1) / 8);
    const int jmax = (sp.full + 7) / 8;
    int q;
    if (j < x1 - x0) {
      q = x0 + j;
    } else if (j >= jmax) {
      const int v = (j - jmax) * 8 + xcd;
      if (v >= sp.rem * sp.parts) return;
      q = sp.full + v / sp.parts;
      const int part = v % sp.parts, nk0 = ke;
      unit = v;
      kb = part * nk0 / sp.parts;
      ke = (part + 1) * nk0 / sp.parts;
    } else {
      return;
    }
    if (run_order) expert_tile(q, p, mt, nb);
    else strip_tile(q, sp.mreal, p.nblocks, mt, nb);
  } else if (run_order) {
    const int64_t n = static_cast<int64_t>(total / BM) * p.nblocks;
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int64_t q = n * xcd / 8 + j;
    if (q >= n * (xcd + 1) / 8) return;
    expert_tile(q, p, mt, nb);
  } else {
    // groups over the m-tiles that hold routed rows (from the padded total), not over the
    // table's capacity: the slots past them then come last in every XCD's order instead
    // of interleaving empty work-groups with the real ones
    const int mreal = min(p.mtiles, (total + BM - 1) / BM);
    if (!grouped_slot<kGroupM, kGroupN>(blockIdx.x, mreal, p.nblocks, p.n_outer, mt, nb)) return;
  }
  if (mt * BM >= total) return;
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  const int K = p.K;
  // the tile's expert and its row ids are independent loads, issued together
  static_assert(C::NT >= BM, "one tile row per thread");
  const int e = p.expert_ids[(mt * BM) / p.block_m];
  const int rid = tid < BM ? p.sorted_ids[static_cast<int64_t>(mt) * BM + tid] : p.R;
  if (MODE == 1 && e < 0) return;       // expert held by another GPU: nothing to compute

  // rows of the tile (sentinels read row 0 and are never stored).  GEMM2 also stages the
  // router weights in LDS, so its epilogue issues no dependent global loads; with bf16
  // weights they are stored there after the K loop, under which their loads complete (the
  // FP8 tiles, at the register limit, store them now)
  const float wrow = (MODE == 2 && rid < p.R) ? p.topk_w[rid] : 0.f;
  if (tid < BM) srow[tid] = rid;
  if (MODE == 2 && WB == 1 && tid < BM) swt[tid] = wrow;
  const int valid = rid < p.R;
  if (MODE == 2 && e < 0) {
    // expert held by another GPU: zeros in this tile's slice of y, so the combine adds
    // nothing for these rows (the fix-up writes them for a split tile)
    if (unit >= 0) return;
    __syncthreads();
    float* out = static_cast<float*>(p.C);
    for (int idx = tid; idx < BM * (BN / 4); idx += C::NT) {
      const int m = idx / (BN / 4), col = nb * BN + (idx % (BN / 4)) * 4;
      const int r = srow[m];
      if (r < p.R && col < p.N)
        *reinterpret_cast<float4*>(out + static_cast<int64_t>(r) * p.N + col) =
            make_float4(0.f, 0.f, 0.f, 0.f);
    }
    return;
  }
  // B tile row n -> weight row of the expert (GEMM1: 32-row gate and up blocks
  // interleaved, so each wave's accumulators hold matching gate/up pairs); columns past
  // N read row 0 and are never stored
  auto b_row = [&](int n) {
    if (MODE == 1) {
      const int blk = n >> 5;
      int col = nb * (BN / 2) + (blk >> 1) * 32 + (n & 31);
      if (col >= p.N) col = 0;
      return (blk & 1) ? p.I + col : col;
    }
    int col = nb * BN + n;
    if (col >= p.N) col = 0;
    return col;
  };
  if (WB == 1) {
    const int nrows = MODE == 1 ? 2 * p.I : p.N;
    for (int n = tid; n < BN; n += C::NT)
      sscale[n] = p.B_scale[static_cast<int64_t>(e) * nrows + b_row(n)];
  }
  // routed rows of the tile: a prefix (an expert's padding rows end its last tile)
  const int nv = __syncthreads_count(valid);

  // DMA sources: instruction j of wave w fills tile rows RPI*(w + NW*j) .. +RPI (1 KB);
  // lane -> row lane / CPR, physical chunk lane % CPR, logical chunk pch ^ swz(row)
  const int lrow = lane / C::CPRA, pch = lane % C::CPRA;
  const uint16_t* a_src[C::LA];
#pragma unroll
  for (int j = 0; j < C::LA; ++j) {
    const int m = C::RPIA * (w + C::NW * j) + lrow;
    const int r = srow[m];
    const int arow = r < p.R ? r / p.gather_div : 0;
    a_src[j] = p.A + static_cast<int64_t>(arow) * K + kb * C::BK + ((pch ^ swz<C::ROWA>(m)) << 3);
  }
  const uint8_t* b_base = p.B + static_cast<int64_t>(e) * p.b_expert_stride * WB;
  const uint8_t* b_src[C::LB];
  const int lrowb = lane / C::CPRB, pchb = lane % C::CPRB;
#pragma unroll
  for (int j = 0; j < C::LB; ++j) {
    const int n = C::RPIB * (w + C::NW * j) + lrowb;
    b_src[j] = b_base + static_cast<int64_t>(b_row(n)) * K * WB + kb * C::BK * WB +
               ((pchb ^ swz<C::ROWB>(n)) << 4);
  }

  auto issue = [&](int kt) {
    uint8_t* st = smem + (kt % NSTAGE) * C::STAGE;
    const int k0 = kt * C::BK;
#pragma unroll
    for (int j = 0; j < C::LA; ++j)
      dma16(a_src[j] + k0, (MOE_LDS void*)(st + 1024 * (w + C::NW * j)));
#pragma unroll
    for (int j = 0; j < C::LB; ++j)
      dma16(b_src[j] + k0 * WB, (MOE_LDS void*)(st + C::SA + 1024 * (w + C::NW * j)));
  };

  const int wm = w / WN, wn = w % WN;
  // The 32-row fragments holding routed rows (the rest of the tile is padding, whose
  // MFMAs and A-operand reads are skipped) are split evenly over the two wave rows, the
  // first row taking the odd one: an expert's last tile, partly padding, then keeps both
  // waves of every SIMD issuing MFMAs instead of leaving the second row idle.
  static_assert(WM == 2 && C::NW == 8, "two wave rows of four waves");
  const int nf = min(2 * C::FM, (nv + 31) >> 5);
  const int fa = min(C::FM, (nf + 1) >> 1);
  const int wr0 = wm == 0 ? 0 : 32 * fa;           // first tile row of this wave's fragments
  const int nown = wm == 0 ? fa : nf - fa;         // fragments owned
  const int na = __builtin_amdgcn_readfirstlane(nown);
  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk = ke - kb;
  // Fragments of step ks of stage kt: A rows of this wave's M slice, B rows of its N
  // slice.  bf16 weights: one k16 step per ks, lanes 0-31 take logical chunk 2*ks,
  // lanes 32-63 chunk 2*ks+1 of each row.  FP8 weights: two k16 steps per ks (32
  // k-elements); the sum over k does not depend on how k is dealt to the lanes, so lane
  // half h takes the 16 consecutive k-elements 32*ks + 16h .. +15: B chunk 2*ks + h (16
  // E4M3 values) and A chunks 4*ks + 2h (first MFMA) and 4*ks + 2h + 1 (second).
  constexpr int NSTEP = WB == 2 ? C::KS : C::KS / 2;
  using Fr = Frags<C::FM, C::FN, WB>;
  auto read_frags = [&](auto full, int kt, int ks, Fr& f) {
    const uint8_t* sa = smem + (kt % NSTAGE) * C::STAGE;
    const uint8_t* sb = sa + C::SA;
    if constexpr (WB == 2) {
      const int ch = 2 * ks + (lane >> 5);
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        const int row = wr0 + i * 32 + (lane & 31);
        if (decltype(full)::value || i < na) f.a[i] = *reinterpret_cast<const bf16x8*>(sa + pswz<C::ROWA>(row, ch));
      }
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const int row = wn * C::WTN + j * 32 + (lane & 31);
        f.b[j] = *reinterpret_cast<const bf16x8*>(sb + pswz<C::ROWB>(row, ch));
      }
    } else {
      const int h = lane >> 5;
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        const int row = wr0 + i * 32 + (lane & 31);
        if (decltype(full)::value || i < na) {
          f.a0[i] = *reinterpret_cast<const bf16x8*>(sa + pswz<C::ROWA>(row, 4 * ks + 2 * h));
          f.a1[i] = *reinterpret_cast<const bf16x8*>(sa + pswz<C::ROWA>(row, 4 * ks + 2 * h + 1));
        }
      }
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const int row = wn * C::WTN + j * 32 + (lane & 31);
        f.q[j] = *reinterpret_cast<const u32x4*>(sb + pswz<C::ROWB>(row, 2 * ks + h));
      }
    }
  };
  // the fragments of one half-stage (two k16 steps with bf16 weights, one Frags with FP8)
  Fr fr[2];
  using T_ = std::true_type;
  using F_ = std::false_type;

  // The K loop, instantiated for full tiles and for a tile whose last fragments are padding
  auto kloop = [&](auto full) {

  if constexpr (NSTAGE == 3) {
    // Ping-pong over a three-stage ring of 64-element stages: the FP8 256-row tile (48 KB
    // stages: 128-byte A rows, 64-byte B rows of E4M3 bytes), the bf16 128-row tile (48 KB)
    // and the FP8 128-row tile (32 KB).  The
    // phases are those of the bf16 two-stage ring below: wave row 0 (waves 0-3) and row 1
    // (waves 4-7) put one wave of each row on every SIMD and run half a phase apart; a
    // load phase reads the fragments of a 32-element half-stage from LDS (and expands FP8
    // B bytes to bf16), a compute phase runs their MFMAs, a barrier ends each phase and
    // row 1 starts one barrier late.
    // With three stages each wave keeps its usual share of every stage's DMAs: stage S is
    // read out at barrier 4S+4 and its slot takes stage S+3, whose share row 1 issues in
    // its next compute phase (half-stage 2S+1) and row 0 in its (half-stage 2S+2); stage
    // S+3 is first read after barrier 4S+12, so both have about seven phases of latency to
    // cover.  Before barrier 4X (stage X first read) a wave has issued its share up to
    // stage X+1, which may stay in flight.  Every wave passes 4 nk + 1 barriers here.
    static_assert(C::KS == 4 && NSTEP == (WB == 1 ? 2 : 4), "64-element stages");
    constexpr int NM = 2 * C::FM * C::FN;               // MFMAs per compute phase
    const int grp = __builtin_amdgcn_readfirstlane(wm);
    bf16x8 bq0[C::FN], bq1[C::FN];                      // FP8: the half-stage's B, expanded
    auto load = [&](int S, int h) {
      if constexpr (WB == 1) {
        read_frags(full, S, h, fr[0]);
        wait_lgkm0();
#pragma unroll
        for (int j = 0; j < C::FN; ++j) fp8x16_to_bf16x2(fr[0].q[j], bq0[j], bq1[j]);
        __builtin_amdgcn_sched_barrier(0);   // the expansion stays in the load phase
      } else {
        read_frags(full, S, 2 * h, fr[0]);
        read_frags(full, S, 2 * h + 1, fr[1]);
        wait_lgkm0();
      }
    };
    // all first-k16 MFMAs, then all second-k16 ones (dependent MFMAs FM x FN apart); with
    // refill, DMA d of this wave's share of stage S2 after MFMA (NM d) / L
    auto compute = [&](auto refill, int S2) {
      uint8_t* st = smem + (S2 % NSTAGE) * C::STAGE;
      const int k0 = S2 * C::BK;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < NM; ++q) {
        const int half = q / (C::FM * C::FN), i = (q / C::FN) % C::FM, j = q % C::FN;
        if (decltype(full)::value || i < na) {
          if constexpr (WB == 1)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(half ? fr[0].a1[i] : fr[0].a0[i],
                                                                half ? bq1[j] : bq0[j], acc[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[half].a[i], fr[half].b[j], acc[i][j], 0, 0, 0);
        }
        if constexpr (decltype(refill)::value) {
#pragma unroll
          for (int d = 0; d < C::L; ++d) {
            if ((d * NM) / C::L == q) {
              __builtin_amdgcn_sched_barrier(0);
              if (d < C::LA) dma16(a_src[d] + k0, (MOE_LDS void*)(st + 1024 * (w + C::NW * d)));
              else dma16(b_src[d - C::LA] + k0 * WB, (MOE_LDS void*)(st + C::SA + 1024 * (w + C::NW * (d - C::LA))));
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    // stages after X = S+1 that this wave may still have in flight at barrier 4S+4
    auto allow = [&](int S) { return max(0, min(S + 2, nk - 1) - (S + 1)) * C::L; };
#pragma unroll
    for (int s = 0; s < NSTAGE; ++s)
      if (s < nk) issue(s);
    wait_vm(min(NSTAGE - 1, nk - 1) * C::L);
    barrier_keep_vm();
    if (grp == 0) {
      // half-stage 2S refills this row's share of stage S+2 for 1 <= S < nk-2
      auto iter = [&](auto refill, auto steady, int S) {
        load(S, 0);
        barrier_keep_vm();
        compute(refill, S + 2);
        barrier_keep_vm();
        load(S, 1);
        barrier_keep_vm();
        compute(F_{}, 0);
        if constexpr (decltype(steady)::value) wait_vm_c<C::L>();
        else wait_vm(allow(S));
        barrier_keep_vm();
      };
      int S = 0;
      if (nk > 0) iter(F_{}, F_{}, S++);
      for (; S + 2 < nk; ++S) iter(T_{}, T_{}, S);
      for (; S < nk; ++S) iter(F_{}, F_{}, S);
      barrier_keep_vm();
    } else {
      barrier_keep_vm();
      // half-stage 2S+1 refills this row's share of stage S+3 for S < nk-3
      auto iter = [&](auto refill, auto steady, int S) {
        load(S, 0);
        barrier_keep_vm();
        compute(F_{}, 0);
        barrier_keep_vm();
        load(S, 1);
        if constexpr (decltype(steady)::value) wait_vm_c<C::L>();
        else wait_vm(allow(S));
        barrier_keep_vm();
        compute(refill, S + 3);
        barrier_keep_vm();
      };
      int S = 0;
      for (; S + 3 < nk; ++S) iter(T_{}, T_{}, S);
      for (; S < nk; ++S) iter(F_{}, F_{}, S);
    }
    wait_vm_c<0>();
  } else if constexpr (NSTAGE == 2) {
    // Ping-pong over a two-stage ring of 64-element stages (128-byte LDS rows, so each DMA
    // request fetches whole 128-byte lines), consumed in 32-element half-stages.  Wave row 0
    // (waves 0-3) and wave row 1 (waves 4-7) put one wave of each row on every SIMD and run
    // half a phase apart: a wave alternates a load phase (the fragments of half-stage u from
    // LDS into registers, awaited) and a compute phase (the MFMAs of half-stage u from
    // registers); a barrier ends each phase and row 1 starts one barrier late, so on each
    // SIMD one wave's MFMA burst runs while the other loads.  Barrier b ends phase b of row
    // 0 and phase b-1 of row 1, so half-stage u is read after barrier 2u (row 0) and 2u+1
    // (row 1).  Row 0 reads A rows 0-127 (in a tile that is partly padding, row 1 may start
    // below 128), row 1 the rest, both all of B.
    //
    // Refills.  Stage S is read out once row 1 passes barrier 4S+4; stage S+2 then goes into
    // its slot, and is first read after barrier 4S+8 (A rows 0-127 and B, by row 0) and
    // 4S+9 (A rows 128-255, by row 1).  Row 1 fetches what is needed first, A rows 0-127
    // and all of B (12 DMAs per wave), during its compute phase of half-stage 2S+1 right
    // after barrier 4S+4, and waits for them before barrier 4S+8; row 0 fetches A rows
    // 128-255 (4 per wave) during its compute phase of half-stage 2S+2 and waits for them
    // before barrier 4S+9.  Each row thus has about three and a half phases of latency to
    // cover.  The DMAs sit between the MFMAs at fixed positions (a branch around an MFMA
    // costs more issue time than the DMA it would spread).  Every wave passes 4 nk + 1
    // barriers here.
    static_assert(NSTAGE == 2 && C::KS == 4 && WB == 2, "two 64-element bf16 stages");
    static_assert(C::RPIA == 8 && C::RPIB == 8 && BM == 256 && BN == 256 && C::NW == 8, "tile");
    constexpr int NM = 2 * C::FM * C::FN;               // MFMAs per compute phase (16)
    constexpr int ND1 = 12, ND0 = 4;                    // DMAs per wave and stage (rows 1, 0)
    const int grp = __builtin_amdgcn_readfirstlane(wm);
    const int v = __builtin_amdgcn_readfirstlane(w & 3);          // wave within its row
    // DMA j of this wave: j < 4 A rows (row 1: 8 (v + 4 j) .. +7; row 0: 128 + the same),
    // j >= 4 (row 1 only) B rows 8 (v + 4 (j - 4)) .. +7; lanes as in issue()
    const uint8_t* src[ND1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = (grp ? 0 : 128) + 8 * (v + 4 * j) + lrow;
      const int r = srow[m];
      const int arow = r < p.R ? r / p.gather_div : 0;
      src[j] = reinterpret_cast<const uint8_t*>(p.A + static_cast<int64_t>(arow) * K + kb * C::BK +
                                                ((pch ^ swz<C::ROWA>(m)) << 3));
    }
#pragma unroll
    for (int j = 4; j < ND1; ++j) {
      const int n = 8 * (v + 4 * (j - 4)) + lrowb;
      src[j] = b_base + static_cast<int64_t>(b_row(n)) * K * WB + kb * C::BK * WB +
               ((pchb ^ swz<C::ROWB>(n)) << 4);
    }
    const int aofs = __builtin_amdgcn_readfirstlane((grp ? 0 : 128 * C::ROWA) + 1024 * v);
    const int bofs = __builtin_amdgcn_readfirstlane(C::SA + 1024 * v);
    auto dma_j = [&](int j, uint8_t* st, int kbytes) {
      if (j < 4) dma16(src[j] + kbytes, (MOE_LDS void*)(st + aofs + 4096 * j));
      else dma16(src[j] + kbytes, (MOE_LDS void*)(st + bofs + 4096 * (j - 4)));
    };
    auto issue_pp = [&](int S2) {
      uint8_t* st = smem + (S2 % NSTAGE) * C::STAGE;
      if (grp) {
#pragma unroll
        for (int j = 0; j < ND1; ++j) dma_j(j, st, S2 * C::BK * 2);
      } else {
#pragma unroll
        for (int j = 0; j < ND0; ++j) dma_j(j, st, S2 * C::BK * 2);
      }
    };
    auto load = [&](int S, int h) {
      read_frags(full, S, 2 * h, fr[0]);
      read_frags(full, S, 2 * h + 1, fr[1]);
      wait_lgkm0();
    };
    // the MFMAs of the registers' half-stage; with ndma > 0, DMA d of stage S2 after MFMA
    // d + d / 3 (12 DMAs) or 4 d (4 DMAs)
    auto compute = [&](auto ndma, int S2) {
      constexpr int ND = decltype(ndma)::value;
      static_assert(ND == 0 || ND == ND0 || ND == ND1, "DMA count");
      uint8_t* st = smem + (S2 % NSTAGE) * C::STAGE;
      const int kbytes = S2 * C::BK * 2;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < NM; ++q) {
        const int ks = q / (C::FM * C::FN), i = (q / C::FN) % C::FM, j = q % C::FN;
        if (decltype(full)::value || i < na)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[ks].a[i], fr[ks].b[j], acc[i][j], 0, 0, 0);
        const bool has = ND == ND1 ? (q % 4 != 3) : (ND == ND0 ? q % 4 == 0 : false);
        if (has) {
          const int d = ND == ND1 ? q - q / 4 : q / 4;
          __builtin_amdgcn_sched_barrier(0);     // the DMA stays between these MFMAs
          dma_j(d, st, kbytes);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    using N0 = std::integral_constant<int, 0>;
    using NR0 = std::integral_constant<int, ND0>;
    using NR1 = std::integral_constant<int, ND1>;
    // Each row runs its own loop, peeled so that whether a compute phase refills is known
    // at compile time (a runtime choice between the two forms makes the register
    // allocation spill).
    issue_pp(0);
    if (nk > 1) issue_pp(1);
    wait_vm(nk > 1 ? (grp ? ND1 : ND0) : 0);
    barrier_keep_vm();
    if (grp == 0) {
      // half-stage 2S (after a wait for this row's part of stage S, S >= 1), refilling stage
      // S+1 for 1 <= S < nk-1; half-stage 2S+1
      auto iter = [&](auto nd, int S) {
        load(S, 0);
        if (S > 0) wait_vm_c<0>();
        barrier_keep_vm();
        compute(nd, S + 1);
        barrier_keep_vm();
        load(S, 1);
        barrier_keep_vm();
        compute(N0{}, 0);
        barrier_keep_vm();
      };
      int S = 0;
      for (; S < nk && (S == 0 || S + 1 >= nk); ++S) iter(N0{}, S);
      for (; S + 1 < nk; ++S) iter(NR0{}, S);
      for (; S < nk; ++S) iter(N0{}, S);
      barrier_keep_vm();
    } else {
      barrier_keep_vm();
      // half-stage 2S; half-stage 2S+1 (after a wait for this row's part of stage S+1),
      // refilling stage S+2 for S < nk-2
      auto iter = [&](auto nd, int S) {
        load(S, 0);
        barrier_keep_vm();
        compute(N0{}, 0);
        barrier_keep_vm();
        load(S, 1);
        wait_vm_c<0>();
        barrier_keep_vm();
        compute(nd, S + 2);
        barrier_keep_vm();
      };
      int S = 0;
      for (; S + 2 < nk; ++S) iter(NR1{}, S);
      for (; S < nk; ++S) iter(N0{}, S);
    }
    wait_vm_c<0>();
  }

  };
  if (na == C::FM) kloop(T_{});
  else kloop(F_{});
  if (MODE == 2 && WB == 2 && unit < 0) {
    if (tid < BM) swt[tid] = wrow;
    __syncthreads();
  }

  // ---- epilogue.  D layout (32x32): lane holds column (lane & 31),
  //      rows 8*(v/4) + 4*(lane/32) + (v%4), v = 0..15.
  if (MODE == 1) {
    // SwiGLU in registers, bf16 tile staged in LDS (the ring is free once every wave is
    // past its last stage), then written as 16-byte row chunks: one 256-byte row
    // segment per 16 lanes instead of 2-byte scattered stores.
    constexpr int NA = BN / 2;                          // a-columns of the tile
    constexpr int ROWS = NA * 2 + 16;                   // padded row stride (bytes)
    static_assert(BM * ROWS <= NSTAGE * C::STAGE, "epilogue tile fits the ring");
    __syncthreads();
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
      if (i >= nown) continue;                     // rows of the other wave row, or padding
#pragma unroll
      for (int q = 0; q < C::FN / 2; ++q) {
        const int lc = (wn * C::WTN) / 2 + q * 32 + (lane & 31);
        // FP8: scales of this lane's gate and up weight rows (tile rows of fragments 2q
        // and 2q+1)
        const float sg = WB == 1 ? sscale[wn * C::WTN + 2 * q * 32 + (lane & 31)] : 1.f;
        const float su = WB == 1 ? sscale[wn * C::WTN + (2 * q + 1) * 32 + (lane & 31)] : 1.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = wr0 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          float g = acc[i][2 * q][v], u = acc[i][2 * q + 1][v];
          if (WB == 1) {
            g *= sg;
            u *= su;
          }
          *reinterpret_cast<uint16_t*>(smem + m * ROWS + lc * 2) = f32_to_bf16(silu_mul_bf16path(g, u));
        }
      }
    }
    __syncthreads();
    uint16_t* out = static_cast<uint16_t*>(p.C);
    constexpr int CPR = NA / 8;                          // 16-byte chunks per row
    for (int idx = tid; idx < BM * CPR; idx += C::NT) {
      const int m = idx / CPR, c = idx % CPR;
      const int r = srow[m];
      const int col = nb * NA + c * 8;
      if (r >= p.R || col >= p.N) continue;
      *reinterpret_cast<u32x4*>(out + static_cast<int64_t>(r) * p.N + col) =
          *reinterpret_cast<const u32x4*>(smem + m * ROWS + c * 16);
    }
  } else if (unit >= 0) {
    // split tile: raw fp32 sums of this K range, [BM][BN] per part
    float* part = p.partial + static_cast<int64_t>(unit) * BM * BN;
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
      if (i >= nown) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = wr0 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          part[m * BN + wn * C::WTN + j * 32 + (lane & 31)] = acc[i][j][v];
      }
    }
  } else {
    float* out = static_cast<float*>(p.C);
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
      if (i >= nown) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = wr0 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const int r = srow[m];
        if (r >= p.R) continue;
        const float wr = swt[m];
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
          const int col = nb * BN + wn * C::WTN + j * 32 + (lane & 31);
          const float a = WB == 1 ? acc[i][j][v] * sscale[wn * C::WTN + j * 32 + (lane & 31)]
                                  : acc[i][j][v];
          if (col < p.N) out[static_cast<int64_t>(r) * p.N + col] = wr * a;
        }
      }
    }
  }
}

// Fix-up of the split GEMM2 tiles: y = w * (sum of the parts in part order); rows of a
// tile whose expert is held by another GPU get zeros.  Block (i, b): split tile i,
// elements 1024 b .. 1024 b + 1023 of its BM x BN slice, four per thread.
template <int BM, int BN, int BK>
__global__ void __launch_bounds__(256)
gemm2_split_fixup_kernel(PArgs p) {
  const int total = *p.ntpp;
  const SplitPlan sp = split_plan(total, BM, p.nblocks, p.ncu, p.split_max, p.K / BK);
  const int i = blockIdx.x;
  if (i >= sp.rem) return;
  int mt, nb;
  if (use_run_order(p)) expert_tile(sp.full + i, p, mt, nb);
  else strip_tile(sp.full + i, sp.mreal, p.nblocks, mt, nb);
  const int idx = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (idx >= BM * BN) return;
  const int m = idx / BN, c = idx % BN;
  const int r = p.sorted_ids[static_cast<int64_t>(mt) * BM + m];
  const int col = nb * BN + c;
  if (r >= p.R || col >= p.N) return;                // N % 4 == 0: the 4 columns are in
  float* out = static_cast<float*>(p.C) + static_cast<int64_t>(r) * p.N + col;
  const int e = p.expert_ids[(mt * BM) / p.block_m];
  if (e < 0) {
    *reinterpret_cast<float4*>(out) = make_float4(0.f, 0.f, 0.f, 0.f);
    return;
  }
  const float* src = p.partial + static_cast<int64_t>(i) * sp.parts * BM * BN + idx;
  float4 a = *reinterpret_cast<const float4*>(src);
  for (int q = 1; q < sp.parts; ++q) {
    const float4 b = *reinterpret_cast<const float4*>(src + static_cast<int64_t>(q) * BM * BN);
    a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
  }
  if (p.B_scale) {   // FP8 weights: the row scale of each output column, as the epilogue
    const float4 sc = *reinterpret_cast<const float4*>(p.B_scale + static_cast<int64_t>(e) * p.N + col);
    a.x *= sc.x; a.y *= sc.y; a.z *= sc.z; a.w *= sc.w;
  }
  const float wr = p.topk_w[r];
  *reinterpret_cast<float4*>(out) = make_float4(wr * a.x, wr * a.y, wr * a.z, wr * a.w);
}

int device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

template <int MODE, int BM, int BN, int WM, int WN, int BK, int NSTAGE, int WB = 2>
hipError_t run_pipe(const GemmArgs& g, hipStream_t s) {
  PArgs p{};
  const bool g1 = MODE == 1;
  p.A = static_cast<const uint16_t*>(g.A);
  p.B = static_cast<const uint8_t*>(g.B);
  p.B_scale = g.w_scale;
  p.C = g.C;
  p.topk_w = g.topk_w;
  p.sorted_ids = g.sorted_ids;
  p.expert_ids = g.expert_ids;
  p.ntpp = g.ntpp;
  p.R = g.T * g.k;
  p.gather_div = g1 ? g.k : 1;
  p.K = g1 ? g.H : g.I;
  p.N = g1 ? g.I : g.H;
  p.I = g.I;
  p.b_expert_stride = g1 ? static_cast<int64_t>(2) * g.I * g.H : static_cast<int64_t>(g.H) * g.I;
  p.block_m = g.block_m;
  p.tile_run = g.block_m % BM == 0 ? g.tile_run : nullptr;
  p.tile_div = g.block_m / BM;
  p.mtiles = static_cast<int>(g.cap / BM);
  const int ncols = g1 ? BN / 2 : BN;
  p.nblocks = (p.N + ncols - 1) / ncols;
  p.n_outer = p.mtiles > p.nblocks;
  // every (group, position) slot: ceil over groups of kGroupM x kGroupN, 8 XCDs at a time
  const int64_t groups = static_cast<int64_t>((p.mtiles + kGroupM - 1) / kGroupM) *
                         ((p.nblocks + kGroupN - 1) / kGroupN);
  int64_t G = (groups + 7) / 8 * 8 * kGroupM * kGroupN;
  if (G == 0) return hipSuccess;
  p.split_max = 1;
  if (MODE == 2 && g.split_ws) {
    const int ncu = device_cu_count();              // one work-group per CU
    if (ncu > 0 && g.split_ws_bytes >= static_cast<size_t>(ncu) * BM * BN * sizeof(float)) {
      p.split_max = 4;
      p.ncu = ncu;
      p.partial = g.split_ws;
      // whole tiles (<= every real tile) + one round of parts + the XCD rounding, or the
      // grouped raster's slots when the plan does not split
      G = std::max<int64_t>(G, (static_cast<int64_t>(p.mtiles) * p.nblocks + ncu + 16 + 7) / 8 * 8);
    }
  }
  hipLaunchKernelGGL((moe_gemm_pipe_kernel<MODE, BM, BN, WM, WN, BK, NSTAGE, WB>),
                     dim3(static_cast<unsigned>(G)), dim3(WM * WN * 64), 0, s, p);
  if (MODE == 2 && p.split_max > 1)
    hipLaunchKernelGGL((gemm2_split_fixup_kernel<BM, BN, BK>),
                       dim3(static_cast<unsigned>(p.ncu), (BM * BN) / 1024), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

// Tile choice for the pipelined prefill kernels; returns hipErrorInvalidValue when
// block_m does not allow a 128/256-row tile (callers fall back to gemm.hip's tiles).
hipError_t launch_pipe_gemm1(const GemmArgs& g, int tile_m, hipStream_t s) {
  if (g.w_scale) {     // FP8 weights: the half-size B tile leaves room for a deeper ring
    // 256-row tile: 8 waves in the ping-pong schedule over three stages (Mixtral-8x7B
    // shape: 1.63 ms against 1.87 ms for 4 waves, one per SIMD; the 128-row tile likewise,
    // DeepSeek-V3-shaped FP8 layer at T = 1024: 1.50 against 1.65 ms)
    if (tile_m == 256) return run_pipe<1, 256, 256, 2, 4, 64, 3, 1>(g, s);
    if (tile_m == 128) return run_pipe<1, 128, 256, 2, 4, 64, 3, 1>(g, s);
    return hipErrorInvalidValue;
  }
  // 8 waves (2 x 4, two per SIMD) in the ping-pong schedule for the 256-row tile
  // (Mixtral-8x7B shape: 1.70 ms against 1.84 ms for the same 8 waves with the operand
  // reads and DMAs spread between the MFMAs of every wave)
  if (tile_m == 256) return run_pipe<1, 256, 256, 2, 4, 64, 2>(g, s);
  // 128-row tile: the same 8 waves over three 64-element stages (Qwen3 shape, T = 1024:
  // layer 1.12 ms against 1.17 ms for 4 waves over 32-element stages, two work-groups a CU)
  if (tile_m == 128) return run_pipe<1, 128, 256, 2, 4, 64, 3>(g, s);
  return hipErrorInvalidValue;
}

hipError_t launch_pipe_gemm2(const GemmArgs& g, int tile_m, hipStream_t s) {
  if (g.w_scale) {
    if (tile_m == 256) return run_pipe<2, 256, 256, 2, 4, 64, 3, 1>(g, s);   // 0.95 against 1.15 ms
    if (tile_m == 128) return run_pipe<2, 128, 256, 2, 4, 64, 3, 1>(g, s);
    return hipErrorInvalidValue;
  }
  // the ping-pong schedule as GEMM1 (Mixtral-8x7B shape: 1.00 ms against 1.08 ms)
  if (tile_m == 256) return run_pipe<2, 256, 256, 2, 4, 64, 2>(g, s);
  if (tile_m == 128) return run_pipe<2, 128, 256, 2, 4, 64, 3>(g, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
