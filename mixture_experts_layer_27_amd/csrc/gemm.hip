// Gathered grouped GEMMs of the expert FFN ("Mixture-of-Experts Kernels: Routing,
// Permutation, and Grouped GEMM", section 6): every BM-row tile belongs to one expert
// (expert_ids), reads its A rows through sorted_ids (GEMM1: token r / k of x; GEMM2:
// row r of a), multiplies by that expert's weights and stores at row r.
//
//   GEMM1 + SwiGLU:  a[r, n] = silu(x[r/k] . W13[e, n]) * (x[r/k] . W13[e, I + n])
//   GEMM2 x weight:  y[r, n] = topk_w[r] * (a[r] . W2[e, n])
//
// bf16 kernel (gfx950): v_mfma_f32_32x32x16_bf16, fp32 accumulators.  A work-group
// computes a BM x BN tile with WM x WN waves; K advances 64 elements per stage through
// a double-buffered LDS tile (register staging).  LDS rows are 128 bytes (64 bf16);
// the 16-byte chunk c of row m is stored at chunk position c ^ (m & 7) so that the
// MFMA operand reads (32 rows at one chunk) and the row-wise stores both spread over
// all banks.  For GEMM1 the B tile interleaves 32-row blocks of gate rows and up rows
// of the same 32 output columns, so one wave holds gate and up accumulators of the
// same (row, column) in identical register layouts and applies silu(g)*u in registers.
//
// The grid covers every (m-tile, n-block) slot of the worst-case table; slots past
// the device-side padded total exit at once.  Work-group ids are remapped so that
// each XCD (work-groups are dealt round-robin over 8 XCDs) receives a contiguous
// range of slots, m-tile fastest: the tiles that share an expert's weight block run
// at the same time on the same XCD and share its L2.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

struct KArgs {
  const uint16_t* A;
  const uint16_t* B;
  void* C;
  const float* topk_w;
  const int32_t* sorted_ids;
  const int32_t* expert_ids;
  const int32_t* ntpp;
  int R;          // T * k (sentinel)
  int gather_div; // k for GEMM1, 1 for GEMM2
  int K;          // reduction length (H or I)
  int N;          // output columns (I or H)
  int I;          // GEMM1: offset of the up rows in W13
  int64_t b_expert_stride;
  int block_m;
  int mtiles, nblocks;
};

template <int MODE, int BM, int BN, int WM, int WN>
struct Cfg {
  static constexpr int NT = WM * WN * kWave;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int BK = 64;
  static constexpr int A_PER_T = BM * 8 / NT, B_PER_T = BN * 8 / NT;
  static constexpr int LDS_A = BM * 128, LDS_B = BN * 128;
  static constexpr int STAGE = LDS_A + LDS_B;
  static_assert(BM * 8 % NT == 0 && BN * 8 % NT == 0, "tile/thread mismatch");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  static_assert(MODE != 1 || WTN % 64 == 0, "GEMM1 wave tile must hold gate/up pairs");
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

__device__ __forceinline__ int xcd_remap(int bid, int G) {
  const int xcd = bid & 7, j = bid >> 3, q = G >> 3, rmd = G & 7;
  return (xcd < rmd ? xcd * (q + 1) : rmd * (q + 1) + (xcd - rmd) * q) + j;
}

template <int MODE, int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(WM * WN * 64)
moe_gemm_bf16_kernel(KArgs p) {
  using C = Cfg<MODE, BM, BN, WM, WN>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * C::STAGE];
  __shared__ int srow[BM];

  const int G = p.mtiles * p.nblocks;
  const int logical = xcd_remap(blockIdx.x, G);
  const int mt = logical % p.mtiles, nb = logical / p.mtiles;
  const int total = *p.ntpp;
  if (mt * BM >= total) return;
  const int e = p.expert_ids[(mt * BM) / p.block_m];
  if (e < 0) {
    // expert held by another GPU: GEMM1 skips the tile, GEMM2 writes zeros into its
    // slice of y so the combine adds nothing for these rows
    if (MODE == 2) {
      float* out = static_cast<float*>(p.C);
      for (int idx = threadIdx.x; idx < BM * BN; idx += blockDim.x) {
        const int r = p.sorted_ids[static_cast<int64_t>(mt) * BM + idx / BN];
        const int col = nb * BN + idx % BN;
        if (r < p.R && col < p.N) out[static_cast<int64_t>(r) * p.N + col] = 0.f;
      }
    }
    return;
  }

  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  const int kc = tid & 7;
  const int K = p.K;

  // ---- per-thread global source rows
  const uint16_t* a_src[C::A_PER_T];
#pragma unroll
  for (int i = 0; i < C::A_PER_T; ++i) {
    const int m = (tid >> 3) + i * (C::NT / 8);
    const int r = p.sorted_ids[static_cast<int64_t>(mt) * BM + m];
    const bool ok = r < p.R;
    const int arow = ok ? r / p.gather_div : 0;      // sentinel rows read row 0, never stored
    a_src[i] = p.A + static_cast<int64_t>(arow) * K + kc * 8;
    if (kc == 0) srow[m] = r;
  }
  const uint16_t* b_base = p.B + static_cast<int64_t>(e) * p.b_expert_stride;
  const uint16_t* b_src[C::B_PER_T];
#pragma unroll
  for (int i = 0; i < C::B_PER_T; ++i) {
    const int n = (tid >> 3) + i * (C::NT / 8);
    int brow;
    if (MODE == 1) {
      const int blk = n >> 5;
      int col = nb * (BN / 2) + (blk >> 1) * 32 + (n & 31);
      if (col >= p.N) col = 0;                       // column tail: any valid row, not stored
      brow = (blk & 1) ? p.I + col : col;
    } else {
      int col = nb * BN + n;
      if (col >= p.N) col = 0;
      brow = col;
    }
    b_src[i] = b_base + static_cast<int64_t>(brow) * K + kc * 8;
  }

  u32x4 ra[C::A_PER_T], rb[C::B_PER_T];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) ra[i] = *reinterpret_cast<const u32x4*>(a_src[i] + k0);
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) rb[i] = *reinterpret_cast<const u32x4*>(b_src[i] + k0);
  };
  auto lstore = [&](int stage) {
    uint8_t* sa = smem + stage * C::STAGE;
    uint8_t* sb = sa + C::LDS_A;
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
      const int m = (tid >> 3) + i * (C::NT / 8);
      *reinterpret_cast<u32x4*>(sa + swz(m, kc)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) {
      const int n = (tid >> 3) + i * (C::NT / 8);
      *reinterpret_cast<u32x4*>(sb + swz(n, kc)) = rb[i];
    }
  };

  const int wm = w / WN, wn = w % WN;
  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk = K / C::BK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * C::BK);
    const uint8_t* sa = smem + cur * C::STAGE;
    const uint8_t* sb = sa + C::LDS_A;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int ch = 2 * ks + (lane >> 5);
      bf16x8 af[C::FM], bfr[C::FN];
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        const int row = wm * C::WTM + i * 32 + (lane & 31);
        af[i] = *reinterpret_cast<const bf16x8*>(sa + swz(row, ch));
      }
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const int row = wn * C::WTN + j * 32 + (lane & 31);
        bfr[j] = *reinterpret_cast<const bf16x8*>(sb + swz(row, ch));
      }
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue.  D layout (32x32): lane holds column (lane & 31),
  //      rows 8*(v/4) + 4*(lane/32) + (v%4), v = 0..15.
  if (MODE == 1) {
    uint16_t* out = static_cast<uint16_t*>(p.C);
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
#pragma unroll
      for (int q = 0; q < C::FN / 2; ++q) {
        const int col = nb * (BN / 2) + (wn * C::WTN) / 2 + q * 32 + (lane & 31);
        if (col >= p.N) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = wm * C::WTM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          const int r = srow[m];
          if (r >= p.R) continue;
          const float g = acc[i][2 * q][v], u = acc[i][2 * q + 1][v];
          const float a = silu_mul_bf16path(g, u);
          out[static_cast<int64_t>(r) * p.N + col] = f32_to_bf16(a);
        }
      }
    }
  } else {
    float* out = static_cast<float*>(p.C);
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = wm * C::WTM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const int r = srow[m];
        if (r >= p.R) continue;
        const float wr = p.topk_w[r];
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
          const int col = nb * BN + wn * C::WTN + j * 32 + (lane & 31);
          if (col < p.N) out[static_cast<int64_t>(r) * p.N + col] = wr * acc[i][j][v];
        }
      }
    }
  }
}

// ------------------------------------------------------------------ fp32 path
// v_mfma_f32_16x16x4_f32 tiles for tables whose block_m is a multiple of 16 (every 16-row
// tile then lies in one expert's block): a work-group of 4 waves computes 16 table rows x
// 64 output columns (GEMM1: 64 gate columns and the matching 64 up columns), with K staged
// through LDS in 32-element chunks (rows padded by one word, so that the 16 rows a step
// reads fall in distinct banks).  Lane layout of one 16x16x4 step: lane i supplies
// A[i % 16][i / 16] and B[i / 16][i % 16]; accumulator element j of lane i is
// D[4 (i / 16) + j][i % 16].
constexpr int kF32M = 16, kF32N = 64, kF32K = 32;

template <int MODE>   // 1: GEMM1 + SwiGLU; 2: GEMM2 x router weight
__global__ void __launch_bounds__(256)
gemm_f32_mfma_kernel(const float* __restrict__ A, const float* __restrict__ W,
                     const float* __restrict__ topk_w, const int32_t* __restrict__ sorted_ids,
                     const int32_t* __restrict__ expert_ids, const int32_t* __restrict__ ntpp,
                     int R, int gather_div, int K, int N, int block_m, float* __restrict__ out) {
  constexpr int NB = MODE == 1 ? 2 : 1;          // weight blocks: gate and up, or W2 rows
  __shared__ float sa[kF32M][kF32K + 1];
  __shared__ float sb[NB * kF32N][kF32K + 1];
  __shared__ int srow[kF32M];
  const int m0 = blockIdx.x * kF32M, n0 = blockIdx.y * kF32N;
  if (m0 >= *ntpp) return;
  const int e = expert_ids[m0 / block_m];
  if (MODE == 1 && e < 0) return;                // expert held by another GPU
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid < kF32M) srow[tid] = sorted_ids[m0 + tid];
  __syncthreads();
  if (MODE == 2 && e < 0) {
    // zeros in this tile's slice of y, so the combine adds nothing for these rows
    for (int idx = tid; idx < kF32M * kF32N; idx += 256) {
      const int r = srow[idx / kF32N], col = n0 + idx % kF32N;
      if (r < R && col < N) out[static_cast<int64_t>(r) * N + col] = 0.f;
    }
    return;
  }
  const int64_t wrows = MODE == 1 ? 2 * static_cast<int64_t>(N) : N;   // weight rows per expert
  const float* we = W + static_cast<int64_t>(e) * wrows * K;
  f32x4 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < K; k0 += kF32K) {
    for (int idx = tid; idx < kF32M * kF32K; idx += 256) {
      const int m = idx / kF32K, kk = idx % kF32K, r = srow[m];
      sa[m][kk] = (r < R && k0 + kk < K)
                      ? A[static_cast<int64_t>(r / gather_div) * K + k0 + kk] : 0.f;
    }
    for (int idx = tid; idx < NB * kF32N * kF32K; idx += 256) {
      const int n = idx / kF32K, kk = idx % kF32K, col = n0 + n % kF32N;
      const int64_t wrow = (MODE == 1 && n >= kF32N) ? N + col : col;
      sb[n][kk] = (col < N && k0 + kk < K) ? we[wrow * K + k0 + kk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kF32K / 4; ++ks) {
      const float av = sa[lane & 15][4 * ks + (lane >> 4)];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float bv = sb[b * kF32N + 16 * w + (lane & 15)][4 * ks + (lane >> 4)];
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[b], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  const int col = n0 + 16 * w + (lane & 15);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = srow[4 * (lane >> 4) + j];
    if (r >= R || col >= N) continue;
    if (MODE == 1) {
      const float g = acc[0][j], u = acc[1][j];
      out[static_cast<int64_t>(r) * N + col] = g / (1.f + expf(-g)) * u;
    } else {
      out[static_cast<int64_t>(r) * N + col] = topk_w[r] * acc[0][j];
    }
  }
}

// Scalar kernels for tables with block_m not a multiple of 16 (a 16-row tile would span
// experts there): one thread per output, K walked in order.
__global__ void __launch_bounds__(256)
gemm1_f32_kernel(const float* __restrict__ x, const float* __restrict__ w13,
                 const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ expert_ids,
                 const int32_t* __restrict__ ntpp, int R, int k, int H, int I, int block_m,
                 int64_t cap, float* __restrict__ a) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= cap * I) return;
  const int64_t pos = i / I;
  const int n = static_cast<int>(i % I);
  if (pos >= *ntpp) return;
  const int r = sorted_ids[pos];
  if (r >= R) return;
  const int e = expert_ids[pos / block_m];
  if (e < 0) return;                              // expert held by another GPU
  const float* xr = x + static_cast<int64_t>(r / k) * H;
  const float* wgate = w13 + (static_cast<int64_t>(e) * 2 * I + n) * H;
  const float* wup = w13 + (static_cast<int64_t>(e) * 2 * I + I + n) * H;
  float g = 0.f, u = 0.f;
  for (int h = 0; h < H; ++h) {
    g = fmaf(xr[h], wgate[h], g);
    u = fmaf(xr[h], wup[h], u);
  }
  a[static_cast<int64_t>(r) * I + n] = g / (1.f + expf(-g)) * u;
}

__global__ void __launch_bounds__(256)
gemm2_f32_kernel(const float* __restrict__ a, const float* __restrict__ w2,
                 const float* __restrict__ topk_w, const int32_t* __restrict__ sorted_ids,
                 const int32_t* __restrict__ expert_ids, const int32_t* __restrict__ ntpp, int R,
                 int H, int I, int block_m, int64_t cap, float* __restrict__ y) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= cap * H) return;
  const int64_t pos = i / H;
  const int n = static_cast<int>(i % H);
  if (pos >= *ntpp) return;
  const int r = sorted_ids[pos];
  if (r >= R) return;
  const int e = expert_ids[pos / block_m];
  if (e < 0) {                                    // expert held by another GPU
    y[static_cast<int64_t>(r) * H + n] = 0.f;
    return;
  }
  const float* ar = a + static_cast<int64_t>(r) * I;
  const float* wr = w2 + (static_cast<int64_t>(e) * H + n) * I;
  float acc = 0.f;
  for (int q = 0; q < I; ++q) acc = fmaf(ar[q], wr[q], acc);
  y[static_cast<int64_t>(r) * H + n] = topk_w[r] * acc;
}

// ------------------------------------------------------------------ combine
// out[t, h] = sum_j y[t*k + j, h] in slot order, one rounding.
// Vector path: 8 consecutive h per thread (two 16-byte loads per source row, one 16-byte
// bf16 or two 16-byte fp32 stores), token rows on grid.y.
template <bool BF16>
__global__ void __launch_bounds__(256)
combine_vec_kernel(const float* __restrict__ y, int T, int H, int k, void* __restrict__ out) {
  const int h0 = (blockIdx.x * 256 + threadIdx.x) * 8;
  if (h0 >= H) return;
  for (int t = blockIdx.y; t < T; t += gridDim.y) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // the rows of up to 8 slots are loaded before any is added (one round trip per 8
    // slots; slots past k re-read slot k-1 and are not added), then added in slot order
    for (int j0 = 0; j0 < k; j0 += 8) {
      float4 a[8], b[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float* row = y + (static_cast<int64_t>(t) * k + min(j0 + q, k - 1)) * H + h0;
        a[q] = *reinterpret_cast<const float4*>(row);
        b[q] = *reinterpret_cast<const float4*>(row + 4);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (j0 + q < k) {
          acc[0] += a[q].x; acc[1] += a[q].y; acc[2] += a[q].z; acc[3] += a[q].w;
          acc[4] += b[q].x; acc[5] += b[q].y; acc[6] += b[q].z; acc[7] += b[q].w;
        }
      }
    }
    if (BF16) {
      u32x4 v;
      v[0] = pack_bf16x2(acc[0], acc[1]);
      v[1] = pack_bf16x2(acc[2], acc[3]);
      v[2] = pack_bf16x2(acc[4], acc[5]);
      v[3] = pack_bf16x2(acc[6], acc[7]);
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + static_cast<int64_t>(t) * H + h0) = v;
    } else {
      float* o = static_cast<float*>(out) + static_cast<int64_t>(t) * H + h0;
      *reinterpret_cast<float4*>(o) = make_float4(acc[0], acc[1], acc[2], acc[3]);
      *reinterpret_cast<float4*>(o + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
}

// any H or alignment: one element per thread
template <bool BF16>
__global__ void __launch_bounds__(256)
combine_kernel(const float* __restrict__ y, int T, int H, int k, void* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(T) * H) return;
  const int64_t t = i / H, h = i % H;
  float s = 0.f;
  for (int j = 0; j < k; ++j) s += y[(t * k + j) * H + h];
  if (BF16) static_cast<uint16_t*>(out)[i] = f32_to_bf16(s);
  else static_cast<float*>(out)[i] = s;
}

template <int MODE, int BM, int BN, int WM, int WN>
hipError_t run_bf16(const GemmArgs& g, hipStream_t s) {
  KArgs p{};
  const bool g1 = MODE == 1;
  p.A = static_cast<const uint16_t*>(g.A);
  p.B = static_cast<const uint16_t*>(g.B);
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
  p.mtiles = static_cast<int>(g.cap / BM);
  const int ncols = g1 ? BN / 2 : BN;
  p.nblocks = (p.N + ncols - 1) / ncols;
  const int64_t G = static_cast<int64_t>(p.mtiles) * p.nblocks;
  if (G == 0) return hipSuccess;
  hipLaunchKernelGGL((moe_gemm_bf16_kernel<MODE, BM, BN, WM, WN>), dim3(static_cast<unsigned>(G)),
                     dim3(WM * WN * 64), 0, s, p);
  return hipGetLastError();
}

template <int MODE>
hipError_t dispatch_bf16(const GemmArgs& g, int variant, hipStream_t s) {
  const int bm = g.block_m;
  if (variant == 2) return MODE == 1 ? launch_decode_gemm1(g, s) : launch_decode_gemm2(g, s);
  if (g.w_scale && bm % 128 != 0) return hipErrorInvalidValue;   // FP8: pipelined tiles only
  if (bm % 256 == 0) return MODE == 1 ? launch_pipe_gemm1(g, 256, s) : launch_pipe_gemm2(g, 256, s);
  if (bm % 128 == 0) return MODE == 1 ? launch_pipe_gemm1(g, 128, s) : launch_pipe_gemm2(g, 128, s);
  if (bm % 64 == 0) return run_bf16<MODE, 64, 128, 1, 2>(g, s);
  if (bm % 32 == 0) return run_bf16<MODE, 32, 128, 1, 2>(g, s);
  return hipErrorInvalidValue;
}

}  // namespace

int prefill_tile_m(int block_m) {
  if (block_m % 128 == 0) return 128;
  if (block_m % 64 == 0) return 64;
  if (block_m % 32 == 0) return 32;
  return 0;
}

hipError_t launch_gemm1(const GemmArgs& g, bool bf16, int variant, hipStream_t s) {
  if (g.T == 0 || g.cap == 0) return hipSuccess;
  if (bf16) return dispatch_bf16<1>(g, variant, s);
  if (g.block_m % kF32M == 0) {
    hipLaunchKernelGGL(gemm_f32_mfma_kernel<1>,
                       dim3(static_cast<unsigned>(g.cap / kF32M), static_cast<unsigned>((g.I + kF32N - 1) / kF32N)),
                       dim3(256), 0, s, static_cast<const float*>(g.A), static_cast<const float*>(g.B),
                       nullptr, g.sorted_ids, g.expert_ids, g.ntpp, g.T * g.k, g.k, g.H, g.I,
                       g.block_m, static_cast<float*>(g.C));
    return hipGetLastError();
  }
  const int64_t n = g.cap * g.I;
  hipLaunchKernelGGL(gemm1_f32_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                     s, static_cast<const float*>(g.A), static_cast<const float*>(g.B),
                     g.sorted_ids, g.expert_ids, g.ntpp, g.T * g.k, g.k, g.H, g.I, g.block_m,
                     g.cap, static_cast<float*>(g.C));
  return hipGetLastError();
}

hipError_t launch_gemm2(const GemmArgs& g, bool bf16, int variant, hipStream_t s) {
  if (g.T == 0 || g.cap == 0) return hipSuccess;
  if (bf16) return dispatch_bf16<2>(g, variant, s);
  if (g.block_m % kF32M == 0) {
    hipLaunchKernelGGL(gemm_f32_mfma_kernel<2>,
                       dim3(static_cast<unsigned>(g.cap / kF32M), static_cast<unsigned>((g.H + kF32N - 1) / kF32N)),
                       dim3(256), 0, s, static_cast<const float*>(g.A), static_cast<const float*>(g.B),
                       g.topk_w, g.sorted_ids, g.expert_ids, g.ntpp, g.T * g.k, 1, g.I, g.H,
                       g.block_m, static_cast<float*>(g.C));
    return hipGetLastError();
  }
  const int64_t n = g.cap * g.H;
  hipLaunchKernelGGL(gemm2_f32_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                     s, static_cast<const float*>(g.A), static_cast<const float*>(g.B), g.topk_w,
                     g.sorted_ids, g.expert_ids, g.ntpp, g.T * g.k, g.H, g.I, g.block_m, g.cap,
                     static_cast<float*>(g.C));
  return hipGetLastError();
}

hipError_t launch_combine(const float* y, int T, int H, int k, bool bf16, void* out,
                          hipStream_t s) {
  const int64_t n = static_cast<int64_t>(T) * H;
  if (n == 0) return hipSuccess;
  const bool vec = H % 8 == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(out) & 15) == 0;
  if (vec) {
    const dim3 grid(static_cast<unsigned>((H / 8 + 255) / 256),
                    static_cast<unsigned>(std::min(T, 65535)));
    if (bf16) hipLaunchKernelGGL(combine_vec_kernel<true>, grid, dim3(256), 0, s, y, T, H, k, out);
    else hipLaunchKernelGGL(combine_vec_kernel<false>, grid, dim3(256), 0, s, y, T, H, k, out);
    return hipGetLastError();
  }
  const dim3 grid(static_cast<unsigned>((n + 255) / 256));
  if (bf16) hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(256), 0, s, y, T, H, k, out);
  else hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(256), 0, s, y, T, H, k, out);
  return hipGetLastError();
}

}  // namespace moe
