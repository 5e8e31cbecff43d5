// Small-M expert GEMMs for decode: stream each active expert's weights once at HBM rate
// ("Mixture-of-Experts Kernels: Routing, Permutation, and Grouped GEMM", section 7 (decode
// tiles) and section 8 (FLOP per weight byte ~ n_e: bandwidth-bound below hundreds of
// rows per expert)).
//
// Operand swap: the weights are the MFMA "A" side (16 weight rows per v_mfma_f32_16x16x32_bf16)
// and the few routed token rows are the "B" side (16 tokens per MFMA), so a tile with a
// single routed row still feeds whole MFMAs from the weight stream.  Weights go straight
// from HBM to registers: lane l owns weight row (l & 15); in each K step of 32*CH elements
// the four lanes of a row read 64 contiguous bytes per load instruction (16 rows per
// instruction), in the natural MFMA k order, and the token rows are read the same way.
//
// Work item = (align tile of block_m <= 64 rows, block of weight rows).  GEMM1 items hold
// 16 gate rows + the 16 matching up rows (16 output columns of a, SwiGLU in the epilogue);
// GEMM2 items hold 32 rows of W2 (32 output columns of y, router weight in the epilogue).
// The four waves of a work-group take K steps round-robin (adjacent 64*CH-byte pieces of the
// same rows at the same time) and reduce through LDS.  The grid is persistent: the item
// count comes from the device-side padded total, so no work-group is launched for padding.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kDecWaves = 4;
constexpr int kMaxTG = 4;   // token groups of 16 per pass (64 rows)

struct DArgs {
  const uint16_t* A;      // weights: W13 [E,2I,H] or W2 [E,H,I]
  const uint16_t* X;      // token rows: x [T,H] (GEMM1) or a [R,I] (GEMM2)
  void* C;                // a [R,I] bf16 or y [R,H] f32
  const float* topk_w;
  const int32_t* sorted_ids;
  const int32_t* expert_ids;
  const int32_t* ntpp;
  int R, gather_div, K, I, H;
  int64_t a_expert_stride;
  int block_m;
  int nblk;               // weight-row blocks per expert
};

template <int MODE, int CH>
__global__ void __launch_bounds__(256)
moe_decode_kernel(DArgs p) {
  __shared__ f32x4 red[kDecWaves][kMaxTG][2][kWave];
  __shared__ int rows_s[64];
  const int lane = lane_id(), w = wave_id();
  const int total = *p.ntpp;
  const int ntiles = total / p.block_m;
  const int nitems = ntiles * p.nblk;
  const int row16 = lane & 15, g = lane >> 4;
  const int K = p.K;
  constexpr int STEP = 32 * CH;            // K elements per step
  const int nsteps = K / STEP;

  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    const int tile = item / p.nblk, blk = item % p.nblk;
    const int e = p.expert_ids[tile];
    // weight rows of the two 16-row fragments
    int wrow0, wrow1;
    if (MODE == 1) { wrow0 = blk * 16 + row16; wrow1 = p.I + blk * 16 + row16; }
    else { wrow0 = blk * 32 + row16; wrow1 = blk * 32 + 16 + row16; }
    const uint16_t* wb = p.A + static_cast<int64_t>(e) * p.a_expert_stride;
    // step layout: MFMA substep c (k32 slice c of the step) takes, in lane group g, the
    // 8 elements at c*32 + g*8, so one load instruction reads 64 contiguous bytes of each
    // of the 16 rows (four lanes per row)
    const uint16_t* w0 = wb + static_cast<int64_t>(wrow0) * K + g * 8;
    const uint16_t* w1 = wb + static_cast<int64_t>(wrow1) * K + g * 8;

    for (int m0 = 0; m0 < p.block_m; m0 += 16 * kMaxTG) {
      // rows of this pass (up to 64) and how many 16-row groups hold a routed row
      __syncthreads();
      if (threadIdx.x < 64) {
        const int m = m0 + threadIdx.x;
        rows_s[threadIdx.x] = m < p.block_m ? p.sorted_ids[static_cast<int64_t>(tile) * p.block_m + m]
                                            : p.R;
      }
      __syncthreads();
      int ntg = 0;
#pragma unroll
      for (int q = 0; q < kMaxTG; ++q)
        if (rows_s[q * 16] < p.R) ntg = q + 1;   // valid rows come first in a tile
      if (ntg == 0) break;

      const uint16_t* xr[kMaxTG];
#pragma unroll
      for (int q = 0; q < kMaxTG; ++q) {
        const int r = rows_s[q * 16 + row16];
        const int xrow = r < p.R ? r / p.gather_div : 0;
        xr[q] = p.X + static_cast<int64_t>(xrow) * K + g * 8;
      }
      f32x4 acc[kMaxTG][2];
#pragma unroll
      for (int q = 0; q < kMaxTG; ++q)
#pragma unroll
        for (int f = 0; f < 2; ++f) acc[q][f] = f32x4{0.f, 0.f, 0.f, 0.f};

      for (int s = w; s < nsteps; s += kDecWaves) {
        const int k0 = s * STEP;
        bf16x8 a0[CH], a1[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          a0[c] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(w0 + k0 + c * 32));
          a1[c] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(w1 + k0 + c * 32));
        }
#pragma unroll
        for (int q = 0; q < kMaxTG; ++q) {
          if (q < ntg) {
            bf16x8 b[CH];
#pragma unroll
            for (int c = 0; c < CH; ++c) b[c] = *reinterpret_cast<const bf16x8*>(xr[q] + k0 + c * 32);
#pragma unroll
            for (int c = 0; c < CH; ++c) {
              acc[q][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[c], b[c], acc[q][0], 0, 0, 0);
              acc[q][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[c], b[c], acc[q][1], 0, 0, 0);
            }
          }
        }
      }
      // cross-wave reduction; wave q finishes token group q
#pragma unroll
      for (int q = 0; q < kMaxTG; ++q) {
        if (q < ntg) {
          red[w][q][0][lane] = acc[q][0];
          red[w][q][1][lane] = acc[q][1];
        }
      }
      __syncthreads();
      if (w < ntg) {
        const int q = w;
        f32x4 s0 = red[0][q][0][lane], s1 = red[0][q][1][lane];
#pragma unroll
        for (int ww = 1; ww < kDecWaves; ++ww) {
          const f32x4 o0 = red[ww][q][0][lane], o1 = red[ww][q][1][lane];
#pragma unroll
          for (int v = 0; v < 4; ++v) { s0[v] += o0[v]; s1[v] += o1[v]; }
        }
        // D layout (16x16): lane holds token column (lane & 15), weight rows 4*(lane>>4)+v
        const int r = rows_s[q * 16 + row16];
        if (r < p.R) {
          if (MODE == 1) {
            uint32_t pk[2];
#pragma unroll
            for (int v = 0; v < 4; v += 2) {
              const float ga = s0[v], ua = s1[v], gb = s0[v + 1], ub = s1[v + 1];
              pk[v / 2] = pack_bf16x2(ga / (1.f + __expf(-ga)) * ua, gb / (1.f + __expf(-gb)) * ub);
            }
            uint16_t* out = static_cast<uint16_t*>(p.C) + static_cast<int64_t>(r) * p.I + blk * 16 + 4 * g;
            *reinterpret_cast<uint2*>(out) = make_uint2(pk[0], pk[1]);
          } else {
            const float wr = p.topk_w[r];
            float* out = static_cast<float*>(p.C) + static_cast<int64_t>(r) * p.H + blk * 32 + 4 * g;
            *reinterpret_cast<float4*>(out) = make_float4(wr * s0[0], wr * s0[1], wr * s0[2], wr * s0[3]);
            *reinterpret_cast<float4*>(out + 16) = make_float4(wr * s1[0], wr * s1[1], wr * s1[2], wr * s1[3]);
          }
        }
      }
    }
  }
}

template <int MODE>
hipError_t run_decode(const GemmArgs& g, hipStream_t s) {
  DArgs p{};
  const bool g1 = MODE == 1;
  p.A = static_cast<const uint16_t*>(g.B);
  p.X = static_cast<const uint16_t*>(g.A);
  p.C = g.C;
  p.topk_w = g.topk_w;
  p.sorted_ids = g.sorted_ids;
  p.expert_ids = g.expert_ids;
  p.ntpp = g.ntpp;
  p.R = g.T * g.k;
  p.gather_div = g1 ? g.k : 1;
  p.K = g1 ? g.H : g.I;
  p.I = g.I;
  p.H = g.H;
  p.a_expert_stride = g1 ? static_cast<int64_t>(2) * g.I * g.H : static_cast<int64_t>(g.H) * g.I;
  p.block_m = g.block_m;
  p.nblk = g1 ? g.I / 16 : g.H / 32;
  const int64_t max_items = (g.cap / g.block_m) * p.nblk;
  if (max_items == 0) return hipSuccess;
  const unsigned grid = static_cast<unsigned>(std::min<int64_t>(max_items, 256 * 8));
  if (p.K % 128 == 0)
    hipLaunchKernelGGL((moe_decode_kernel<MODE, 4>), dim3(grid), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((moe_decode_kernel<MODE, 2>), dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_gemm1(const GemmArgs& g, hipStream_t s) { return run_decode<1>(g, s); }
hipError_t launch_decode_gemm2(const GemmArgs& g, hipStream_t s) { return run_decode<2>(g, s); }

}  // namespace moe
