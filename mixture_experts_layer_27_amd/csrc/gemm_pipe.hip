// Large-tile gathered grouped GEMMs for prefill (GEMM1 + SwiGLU, GEMM2 x router weight):
// same contract as the kernels in gemm.hip ("Mixture-of-Experts Kernels: Routing,
// Permutation, and Grouped GEMM", section 6), with a deeper memory pipeline for gfx950:
//
// * Global -> LDS without registers: global_load_lds_dwordx4 writes each lane's 16 bytes
//   at (wave base + 16 * lane), so the LDS swizzle is applied on the global side: lane i
//   of an instruction fetches the logical chunk that belongs at physical slot i.
// * NSTAGE-deep ring of BK=32 stages (64-byte LDS rows; chunk c of row m lives at
//   c ^ sw4(m), conflict-free for both the 16-row DMA writes and the 32-row MFMA
//   operand reads).  Stage kt+NSTAGE-1 is issued while stage kt is consumed; one
//   barrier per stage, preceded by an explicit vmcnt wait for this wave's own loads.
// * v_mfma_f32_32x32x16_bf16, WM x WN waves, each holding (BM/WM) x (BN/WN) fp32
//   accumulators; GEMM1 B tiles interleave 32-row gate and up blocks so that SwiGLU
//   runs in registers.
#include "common.hpp"
#include "launch.hpp"

#define MOE_LDS __attribute__((address_space(3)))

namespace moe {

namespace {

struct PArgs {
  const uint16_t* A;
  const uint16_t* B;
  void* C;
  const float* topk_w;
  const int32_t* sorted_ids;
  const int32_t* expert_ids;
  const int32_t* ntpp;
  int R, gather_div, K, N, I;
  int64_t b_expert_stride;
  int block_m;
  int mtiles, nblocks;
};

template <int MODE, int BM, int BN, int WM, int WN, int NSTAGE>
struct PCfg {
  static constexpr int NW = WM * WN;
  static constexpr int NT = NW * kWave;
  static constexpr int BK = 32;
  static constexpr int ROWB = BK * 2;                 // 64 bytes per LDS row
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int LA = BM / 16 / NW;             // DMA instructions per wave per stage (A)
  static constexpr int LB = BN / 16 / NW;             // (B)
  static constexpr int L = LA + LB;
  static constexpr int SA = BM * ROWB, SB = BN * ROWB;
  static constexpr int STAGE = SA + SB;
  static_assert(BM % (16 * NW) == 0 && BN % (16 * NW) == 0, "DMA rows per wave");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  static_assert(MODE != 1 || WTN % 64 == 0, "GEMM1 wave tile holds gate/up pairs");
  static_assert(NSTAGE * STAGE <= 160 * 1024, "LDS");
};

// LDS swizzle of 64-byte rows: chunk c of row m sits at c ^ sw(m).  sw(m) =
// ((m >> 1) ^ (m >> 3)) & 3 keeps the MFMA operand reads (rows m..m+31, one chunk)
// conflict-free whether the LDS serves 8 lanes x 16 B per cycle over 32 banks or
// 16 lanes x 16 B over 64 banks.
__device__ __forceinline__ int sw4(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }
__device__ __forceinline__ int pswz(int row, int chunk) {
  return row * 64 + ((chunk ^ sw4(row)) << 4);
}

__device__ __forceinline__ int xcd_remap(int bid, int G) {
  const int xcd = bid & 7, j = bid >> 3, q = G >> 3, rmd = G & 7;
  return (xcd < rmd ? xcd * (q + 1) : rmd * (q + 1) + (xcd - rmd) * q) + j;
}

// 16-byte global -> LDS DMA (global_load_lds_dwordx4): lane i writes lds_base + 16*i.
// Issued from inline assembly so that the compiler's wait-count insertion does not treat
// it as an LDS store that every later LDS read must wait for (which would force
// vmcnt(0) before each stage and collapse the ring); completion of this wave's DMAs is
// awaited explicitly with wait_vm() before the barrier that publishes a stage.
__device__ __forceinline__ void dma16(const void* gptr, const MOE_LDS void* lds_base) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_base)));   // wave-uniform
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(gptr), "s"(l) : "memory", "m0");
}

// work-group barrier that also keeps the compiler from moving LDS accesses across it,
// without the vmcnt(0) that __syncthreads() implies (the DMA ring stays in flight)
__device__ __forceinline__ void barrier_keep_vm() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// wait until at most n of this wave's vector-memory ops are outstanding (n <= 63)
__device__ __forceinline__ void wait_vm(int n) {
  // s_waitcnt immediate for gfx9: vmcnt[3:0] | expcnt(7)<<4 | lgkmcnt(15)<<8 | vmcnt[5:4]<<14
#define MOE_VMW(N) __builtin_amdgcn_s_waitcnt(((N) & 15) | (7 << 4) | (15 << 8) | (((N) >> 4) << 14))
  switch (n) {
    case 0: MOE_VMW(0); break;
    case 1: MOE_VMW(1); break;
    case 2: MOE_VMW(2); break;
    case 3: MOE_VMW(3); break;
    case 4: MOE_VMW(4); break;
    case 5: MOE_VMW(5); break;
    case 6: MOE_VMW(6); break;
    case 7: MOE_VMW(7); break;
    case 8: MOE_VMW(8); break;
    case 9: MOE_VMW(9); break;
    case 10: MOE_VMW(10); break;
    case 11: MOE_VMW(11); break;
    case 12: MOE_VMW(12); break;
    case 13: MOE_VMW(13); break;
    case 14: MOE_VMW(14); break;
    case 15: MOE_VMW(15); break;
    case 16: MOE_VMW(16); break;
    case 18: MOE_VMW(18); break;
    case 20: MOE_VMW(20); break;
    case 24: MOE_VMW(24); break;
    case 32: MOE_VMW(32); break;
    default: MOE_VMW(0); break;
  }
#undef MOE_VMW
}

template <int MODE, int BM, int BN, int WM, int WN, int NSTAGE>
__global__ void __launch_bounds__(WM * WN * 64)
moe_gemm_pipe_kernel(PArgs p) {
  using C = PCfg<MODE, BM, BN, WM, WN, NSTAGE>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NSTAGE * C::STAGE];
  __shared__ int srow[BM];

  const int G = p.mtiles * p.nblocks;
  const int logical = xcd_remap(blockIdx.x, G);
  const int mt = logical % p.mtiles, nb = logical / p.mtiles;
  const int total = *p.ntpp;
  if (mt * BM >= total) return;
  const int e = p.expert_ids[(mt * BM) / p.block_m];

  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  const int K = p.K;

  // rows of the tile (sentinels read row 0 and are never stored)
  for (int m = tid; m < BM; m += C::NT) srow[m] = p.sorted_ids[static_cast<int64_t>(mt) * BM + m];
  __syncthreads();

  // DMA sources: instruction j of wave w covers tile rows 16*(w + NW*j) .. +16;
  // lane -> row (lane >> 2), physical chunk (lane & 3), logical chunk pc ^ ((row>>1)&3)
  const int lrow = lane >> 2, pch = lane & 3;
  const uint16_t* a_src[C::LA];
#pragma unroll
  for (int j = 0; j < C::LA; ++j) {
    const int m = 16 * (w + C::NW * j) + lrow;
    const int r = srow[m];
    const int arow = r < p.R ? r / p.gather_div : 0;
    a_src[j] = p.A + static_cast<int64_t>(arow) * K + ((pch ^ sw4(m)) << 3);
  }
  const uint16_t* b_base = p.B + static_cast<int64_t>(e) * p.b_expert_stride;
  const uint16_t* b_src[C::LB];
#pragma unroll
  for (int j = 0; j < C::LB; ++j) {
    const int n = 16 * (w + C::NW * j) + lrow;
    int brow;
    if (MODE == 1) {
      const int blk = n >> 5;
      int col = nb * (BN / 2) + (blk >> 1) * 32 + (n & 31);
      if (col >= p.N) col = 0;
      brow = (blk & 1) ? p.I + col : col;
    } else {
      int col = nb * BN + n;
      if (col >= p.N) col = 0;
      brow = col;
    }
    b_src[j] = b_base + static_cast<int64_t>(brow) * K + ((pch ^ sw4(n)) << 3);
  }

  auto issue = [&](int kt) {
    uint8_t* st = smem + (kt % NSTAGE) * C::STAGE;
    const int k0 = kt * C::BK;
#pragma unroll
    for (int j = 0; j < C::LA; ++j)
      dma16(a_src[j] + k0, (MOE_LDS void*)(st + 1024 * (w + C::NW * j)));
#pragma unroll
    for (int j = 0; j < C::LB; ++j)
      dma16(b_src[j] + k0, (MOE_LDS void*)(st + C::SA + 1024 * (w + C::NW * j)));
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
#pragma unroll
  for (int s = 0; s < NSTAGE - 1; ++s)
    if (s < nk) issue(s);

  for (int kt = 0; kt < nk; ++kt) {
    // stages issued after kt and still allowed in flight
    const int ahead = min(NSTAGE - 2, nk - 1 - kt);
    wait_vm(ahead * C::L);
    barrier_keep_vm();
    if (kt + NSTAGE - 1 < nk) issue(kt + NSTAGE - 1);
    const uint8_t* sa = smem + (kt % NSTAGE) * C::STAGE;
    const uint8_t* sb = sa + C::SA;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int ch = 2 * ks + (lane >> 5);
      bf16x8 af[C::FM], bfr[C::FN];
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        const int row = wm * C::WTM + i * 32 + (lane & 31);
        af[i] = *reinterpret_cast<const bf16x8*>(sa + pswz(row, ch));
      }
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const int row = wn * C::WTN + j * 32 + (lane & 31);
        bfr[j] = *reinterpret_cast<const bf16x8*>(sb + pswz(row, ch));
      }
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
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
          out[static_cast<int64_t>(r) * p.N + col] = f32_to_bf16(g / (1.f + __expf(-g)) * u);
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

template <int MODE, int BM, int BN, int WM, int WN, int NSTAGE>
hipError_t run_pipe(const GemmArgs& g, hipStream_t s) {
  PArgs p{};
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
  hipLaunchKernelGGL((moe_gemm_pipe_kernel<MODE, BM, BN, WM, WN, NSTAGE>),
                     dim3(static_cast<unsigned>(G)), dim3(WM * WN * 64), 0, s, p);
  return hipGetLastError();
}

}  // namespace

// Tile choice for the pipelined prefill kernels; returns hipErrorInvalidValue when
// block_m does not allow a 128/256-row tile (callers fall back to gemm.hip's tiles).
hipError_t launch_pipe_gemm1(const GemmArgs& g, int tile_m, hipStream_t s) {
  if (tile_m == 256) return run_pipe<1, 256, 256, 2, 4, 4>(g, s);
  if (tile_m == 128) return run_pipe<1, 128, 256, 2, 4, 4>(g, s);
  return hipErrorInvalidValue;
}

hipError_t launch_pipe_gemm2(const GemmArgs& g, int tile_m, hipStream_t s) {
  if (tile_m == 256) return run_pipe<2, 256, 256, 2, 4, 4>(g, s);
  if (tile_m == 128) return run_pipe<2, 128, 256, 2, 4, 4>(g, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
