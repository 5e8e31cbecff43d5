// Router: logits = x . Wg^T (fp32 accumulate) and the top-k rules
// ("Mixture-of-Experts Kernels: Routing, Permutation, and Grouped GEMM", section 1
// model table, section 3 `route`, section 4 grouped sigmoid router).
//
// Logits (bf16): MFMA 16x16x32 bf16 with operands read straight from global memory
// in MFMA register layout: lane group g = lane>>4 of a row reads elements g*8..g*8+7
// of each 32-element half of a 64-element chunk, so the k order is the natural one and
// one load instruction covers 64 contiguous bytes of each of 16 rows.  A work-group
// covers 16 tokens x 16*(4/KSPLIT) experts; KSPLIT waves split its K range and reduce
// through LDS.  At decode batch sizes the K range is further split over NZ work-groups
// (slabs), each writing partial logits [NZ][T][E]; the top-k stage adds the slabs in
// ascending slab order, so the result does not depend on scheduling.  This spreads
// the Wg stream (3.7 MB for E=256, H=7168) over a few hundred work-groups.  Larger
// batches with more than 32 experts use 64 x 64 work-group tiles staged in LDS
// (router_logits_tile_kernel).
//
// Top-k: one wave per token; lane l owns experts l, l+64, ...; each of the k
// selections is a wave arg-max on (value desc, index asc) over the heads of per-lane
// sorted candidate lists.  For small batches a
// single work-group routes every token and then builds the align table in the same
// launch (the ids never leave LDS before the align step reads them).
#include "align_dev.hpp"
#include "common.hpp"
#include "launch.hpp"
#include "route_dev.hpp"

namespace moe {

namespace {

using namespace rdev;

constexpr int kMaxSlabs = 16;

template <int KSPLIT>
__global__ void __launch_bounds__(256)
router_logits_bf16_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg,
                          int T, int H, int E, int kz, float* __restrict__ logits) {
  constexpr int kExpWaves = 4 / KSPLIT;            // expert sub-blocks per WG
  __shared__ f32x4 red[4][kWave];
  const int lane = lane_id(), w = wave_id();
  const int eblk = w / KSPLIT, ks = w % KSPLIT;
  const int t0 = blockIdx.x * 16;
  const int e0 = (blockIdx.y * kExpWaves + eblk) * 16;
  const int z = blockIdx.z;                         // K slab of this work-group
  const int row = lane & 15, grp = lane >> 4;
  const int t = min(t0 + row, T - 1);
  const int e = min(e0 + row, E - 1);
  const uint16_t* xa = x + static_cast<int64_t>(t) * H + grp * 8;
  const uint16_t* wb = wg + static_cast<int64_t>(e) * H + grp * 8;
  const int klo = z * kz, khi = min(H, klo + kz);   // kz and H are multiples of 64
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = klo + ks * 64; k0 < khi; k0 += 64 * KSPLIT) {
    const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(xa + k0);
    const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(xa + k0 + 32);
    const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(wb + k0);
    const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(wb + k0 + 32);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b0, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1, acc, 0, 0, 0);
  }
  if (KSPLIT > 1) {
    red[w][lane] = acc;
    __syncthreads();
    if (ks != 0) return;
    for (int q = 1; q < KSPLIT; ++q) {
      const f32x4 o = red[w + q][lane];
      acc[0] += o[0]; acc[1] += o[1]; acc[2] += o[2]; acc[3] += o[3];
    }
  }
  // D layout (16x16): lane holds column (lane & 15) = expert, rows 4*(lane>>4)+v = tokens
  const int ec = e0 + (lane & 15);
  if (ec >= E) return;
  float* slab = logits + static_cast<int64_t>(z) * T * E;
  for (int v = 0; v < 4; ++v) {
    const int tr = t0 + 4 * (lane >> 4) + v;
    if (tr < T) slab[static_cast<int64_t>(tr) * E + ec] = acc[v];
  }
}

// Large batches (many experts): a work-group computes a 64-token x 64-expert tile, its
// 4 waves 32 x 32 each (2 x 2 MFMA 16x16 blocks).  Per 64-element K chunk the x and Wg
// tiles (8 KB each) are staged in LDS, double-buffered, with the next chunk's global
// loads in flight during the current chunk's MFMAs; every wave then reads its fragments
// from LDS instead of from global memory, which cuts the L2 traffic per logit about
// fourfold against one-wave 16 x 16 tiles.  LDS rows are 128 bytes; 16-byte chunk c of
// row r sits at c ^ ((r >> 1) & 7), so the 16 rows an MFMA operand read touches at one
// logical chunk land on distinct bank groups.  The MFMAs run over k in ascending order,
// as in the kernels above.
constexpr int kRt = 64;                            // tile rows (tokens) and columns (experts)

__global__ void __launch_bounds__(256)
router_logits_tile_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg, int T,
                          int H, int E, float* __restrict__ logits) {
  __shared__ __attribute__((aligned(16))) uint8_t sm[2][2][kRt * 128];   // [buf][x|wg]
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  const int t0 = blockIdx.x * kRt, e0 = blockIdx.y * kRt;
  // staging: thread tid moves 16-byte chunks (row, c) = (tid / 8 + 32 * h, tid % 8), h = 0, 1
  const int sr = tid / 8, sc = tid % 8;
  const uint16_t* xs[2];
  const uint16_t* ws[2];
  int so[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = sr + 32 * h;
    xs[h] = x + static_cast<int64_t>(min(t0 + r, T - 1)) * H + sc * 8;
    ws[h] = wg + static_cast<int64_t>(min(e0 + r, E - 1)) * H + sc * 8;
    so[h] = r * 128 + ((sc ^ ((r >> 1) & 7)) * 16);
  }
  const int wt = (w >> 1) * 32, we = (w & 1) * 32;   // this wave's 32 x 32 sub-tile
  const int fr = lane & 15, fg = lane >> 4;          // MFMA operand row, k group
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 px[2], pw[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    px[h] = *reinterpret_cast<const u32x4*>(xs[h]);
    pw[h] = *reinterpret_cast<const u32x4*>(ws[h]);
  }
  const int nchunk = H / 64;
  for (int c = 0; c < nchunk; ++c) {
    uint8_t* bx = sm[c & 1][0];
    uint8_t* bw = sm[c & 1][1];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      *reinterpret_cast<u32x4*>(bx + so[h]) = px[h];
      *reinterpret_cast<u32x4*>(bw + so[h]) = pw[h];
    }
    __syncthreads();
    if (c + 1 < nchunk) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        px[h] = *reinterpret_cast<const u32x4*>(xs[h] + (c + 1) * 64);
        pw[h] = *reinterpret_cast<const u32x4*>(ws[h] + (c + 1) * 64);
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int ch = ks * 4 + fg;                    // logical 16-byte chunk of the row
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wt + 16 * i + fr;
        a[i] = *reinterpret_cast<const bf16x8*>(bx + r * 128 + ((ch ^ ((r >> 1) & 7)) * 16));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = we + 16 * j + fr;
        b[j] = *reinterpret_cast<const bf16x8*>(bw + r * 128 + ((ch ^ ((r >> 1) & 7)) * 16));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    // the buffer written next iteration (the other one) was last read one iteration ago,
    // before this iteration's barrier: no second barrier needed
  }
  // D layout (16x16): lane holds column (lane & 15) = expert, rows 4*(lane>>4)+v = tokens
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int ec = e0 + we + 16 * j + (lane & 15);
    if (ec >= E) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int tr = t0 + wt + 16 * i + 4 * (lane >> 4) + v;
        if (tr < T) logits[static_cast<int64_t>(tr) * E + ec] = acc[i][j][v];
      }
  }
}

__global__ void __launch_bounds__(256)
router_logits_f32_kernel(const float* __restrict__ x, const float* __restrict__ wg, int T,
                         int H, int E, float* __restrict__ logits) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(T) * E) return;
  const int t = static_cast<int>(i / E), e = static_cast<int>(i % E);
  const float* xr = x + static_cast<int64_t>(t) * H;
  const float* wr = wg + static_cast<int64_t>(e) * H;
  float acc = 0.f;
  for (int h = 0; h < H; ++h) acc = fmaf(xr[h], wr[h], acc);
  logits[i] = acc;
}

template <int NSLOT>
__global__ void __launch_bounds__(256)
topk_kernel(TopkParams p) {
  __shared__ TopkLds sh[4];
  const int w = wave_id();
  const int t = blockIdx.x * 4 + w;
  if (t >= p.T) return;                            // whole wave leaves together
  topk_token<NSLOT, 60 / NSLOT>(p, t, sh[w], nullptr);
}

// Small batches: one work-group of 1024 threads routes all T tokens (wave w takes
// tokens w, w+16, ...) and then builds the align table from the ids held in LDS.
constexpr int kFusedMaxT = 32;
constexpr int kFusedMaxRows = kFusedMaxT * 16;
static_assert(alignd::kAlignThreads == 1024, "fused kernel runs the align body with 1024 threads");

template <int NSLOT>
__global__ void __launch_bounds__(1024)
route_align_small_kernel(TopkParams p, int bm, int64_t cap, int32_t* __restrict__ sorted_ids,
                         int32_t* __restrict__ expert_ids, int32_t* __restrict__ ntpp,
                         int32_t* __restrict__ counts, const int32_t* __restrict__ emap) {
  __shared__ TopkLds sh[16];
  __shared__ int32_t ids_lds[kFusedMaxRows];
  __shared__ float lg[kFusedMaxT * 4 * kWave];   // summed logits [T][E], E <= 256
  __shared__ float soff[4 * kWave], sbias[4 * kWave];
  const int w = wave_id();
  // the per-expert offsets and biases are staged in LDS beside the logits, their loads in
  // flight together with the slab loads below
  for (int i = threadIdx.x; i < p.E; i += blockDim.x) {
    if (p.offset) soff[i] = p.offset[i];
    if (p.bias) sbias[i] = p.bias[i];
  }
  // every thread sums the K slabs of some (token, expert) pairs, all slab loads in flight
  // at once (slabs added in ascending order, as in the one-wave path), so the per-token
  // selection below reads its logits from LDS instead of waiting on global round trips
  const int TE = p.T * p.E;
  const int64_t slab = static_cast<int64_t>(TE);
  for (int i = threadIdx.x; i < TE; i += blockDim.x) {
    float part[kMaxSlabs];
#pragma unroll
    for (int z = 0; z < kMaxSlabs; ++z) part[z] = p.logits[min(z, p.nz - 1) * slab + i];
    float l = part[0];
#pragma unroll
    for (int z = 1; z < kMaxSlabs; ++z) l = z < p.nz ? l + part[z] : l;
    lg[i] = l;
    if (p.logits_out) p.logits_out[i] = l;
  }
  __syncthreads();
  TopkParams q = p;
  q.logits = lg;
  q.nz = 1;
  q.logits_out = nullptr;
  q.offset = p.offset ? soff : nullptr;
  q.bias = p.bias ? sbias : nullptr;
  for (int t = w; t < p.T; t += 16) topk_token<NSLOT, 1>(q, t, sh[w], ids_lds);
  __syncthreads();
  alignd::align_small_body(ids_lds, p.T * (p.k + p.shared), p.E + p.shared, bm, cap, sorted_ids,
                           expert_ids, ntpp, counts, emap);
}

// Prefill with few experts (E <= 32), one launch: a work-group of 16 waves routes 16
// tokens.  The 16 x E logits are computed with MFMA 16x16x32 (operands read from global
// memory in MFMA register layout, as in router_logits_bf16_kernel): each wave takes a
// (16-expert block, K slice) pair, KS = 16 / blocks slices per block, and the KS partial
// sums of a block are added in slice order through LDS.  The logits stay in LDS and each
// wave then routes one token with the same per-token selection as topk_kernel.  With many
// experts the gate matrix a work-group reads would outgrow the 16 tokens' activations
// (at E = 128 eight times over), so those keep the two-launch path.
template <int KS>
__global__ void __launch_bounds__(1024)
route_fused_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg, int H,
                   TopkParams p) {
  constexpr int kSlots = 4;                        // topk_token's slots per lane (E <= 256)
  __shared__ TopkLds sh[16];
  __shared__ float lg[16 * 32];
  __shared__ f32x4 red[16][kWave];
  const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(wave_id());
  const int T = p.T, E = p.E;
  const int t0 = blockIdx.x * 16;
  const int row = lane & 15, grp = lane >> 4;
  const uint16_t* xa = x + static_cast<int64_t>(min(t0 + row, T - 1)) * H + grp * 8;
  const int blk = w / KS, ks = w % KS;
  const uint16_t* wb = wg + static_cast<int64_t>(min(blk * 16 + row, E - 1)) * H + grp * 8;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  // this wave's 64-element chunks k0 = ks*64 + c*64*KS, c < nc; the operands of D chunks
  // are in flight at once (the first window may load the last chunk again in place of
  // chunks past the end; those are not used)
  constexpr int D = 4;
  const int nc = (H / 64 - ks + KS - 1) / KS;
  const int klast = H - 64;
  bf16x8 fa[D][2], fb[D][2];
  auto load = [&](int d, int c) {
    const int k0 = min(ks * 64 + c * 64 * KS, klast);
    fa[d][0] = *reinterpret_cast<const bf16x8*>(xa + k0);
    fa[d][1] = *reinterpret_cast<const bf16x8*>(xa + k0 + 32);
    fb[d][0] = *reinterpret_cast<const bf16x8*>(wb + k0);
    fb[d][1] = *reinterpret_cast<const bf16x8*>(wb + k0 + 32);
  };
#pragma unroll
  for (int d = 0; d < D; ++d) load(d, d);
  for (int c = 0; c < nc; c += D) {                // nc is wave-uniform: no masked MFMA
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (c + d < nc) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[d][0], fb[d][0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[d][1], fb[d][1], acc, 0, 0, 0);
      }
      if (c + d + D < nc) load(d, c + d + D);
    }
  }
  red[w][lane] = acc;
  __syncthreads();
  // D layout (16x16): lane holds column (lane & 15) = expert, rows 4*(lane>>4)+v = tokens
  if (ks == 0) {
    for (int q = 1; q < KS; ++q) {
      const f32x4 o = red[w + q][lane];
      acc[0] += o[0]; acc[1] += o[1]; acc[2] += o[2]; acc[3] += o[3];
    }
    const int ec = blk * 16 + (lane & 15);
    if (ec < E)
      for (int v = 0; v < 4; ++v) lg[(4 * (lane >> 4) + v) * E + ec] = acc[v];
  }
  __syncthreads();
  if (t0 + w < T) {
    TopkParams q = p;
    q.logits = lg;
    q.t0 = t0;
    q.nz = 1;
    topk_token<kSlots, 1>(q, t0 + w, sh[w], nullptr);
  }
}

// One token, bf16: one one-wave work-group per expert (spread over every CU) computes the
// whole dot product x . Wg[e] (lane l
// takes the 8 elements at 512 c + 8 l of each 512-element chunk c, all chunks' loads in
// flight together, fp32 FMAs in chunk order, then a fixed butterfly over the lanes), so
// the logits come out whole and the selection reads one value per expert instead of
// summing K slabs.
__global__ void __launch_bounds__(64)
router_logits_gemv_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg,
                          int H, int E, float* __restrict__ logits) {
  constexpr int kB = 16;                           // chunks loaded per round trip (H <= 8192: one)
  const int lane = lane_id();
  const int e = blockIdx.x;
  const uint16_t* wr = wg + static_cast<int64_t>(e) * H;
  const int nch = (H + 511) / 512;
  float acc = 0.f;
  for (int c0 = 0; c0 < nch; c0 += kB) {
    u32x4 a[kB], b[kB];
#pragma unroll
    for (int q = 0; q < kB; ++q) {
      const int k = min((c0 + q) * 512 + lane * 8, H - 8);   // H % 8 == 0
      a[q] = *reinterpret_cast<const u32x4*>(x + k);
      b[q] = *reinterpret_cast<const u32x4*>(wr + k);
    }
#pragma unroll
    for (int q = 0; q < kB; ++q) {
      if (c0 + q < nch && (c0 + q) * 512 + lane * 8 < H) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          acc = fmaf(__uint_as_float(a[q][d] << 16), __uint_as_float(b[q][d] << 16), acc);
          acc = fmaf(__uint_as_float(a[q][d] & 0xffff0000u), __uint_as_float(b[q][d] & 0xffff0000u), acc);
        }
      }
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, kWave);
  if (lane == 0) logits[e] = acc;
}

// K slabs of the bf16 logits: at decode batch sizes enough work-groups to stream Wg
// from many CUs, each slab a multiple of 256 columns (64 per wave).
int slab_cols(int T, int H) {
  if (T > 64 || H % 256) return H;
  int nz = H / 512;
  nz = nz < 1 ? 1 : (nz > kMaxSlabs ? kMaxSlabs : nz);
  return (H / nz + 255) / 256 * 256;
}

TopkParams topk_params(const float* logits, int nz, float* logits_out, int T, int E, int k,
                       const RouteArgs& a, int32_t* ids, float* w) {
  TopkParams p;
  p.logits = logits;
  p.t0 = 0;
  p.nz = nz;
  p.logits_out = logits_out;
  p.T = T;
  p.E = E;
  p.k = k;
  p.mode = a.mode;
  p.offset = a.offset;
  p.bias = a.bias;
  p.n_group = a.n_group;
  p.topk_group = a.topk_group;
  p.scaling = a.scaling;
  p.ids = ids;
  p.w = w;
  p.shared = a.shared;
  return p;
}

}  // namespace

int router_slabs(int T, int H, bool bf16) {
  if (!bf16 || T <= 0) return 1;
  const int kz = slab_cols(T, H);
  return (H + kz - 1) / kz;
}

bool route_align_fusable(int T, int k, int E, int shared) {
  return T <= kFusedMaxT && T * (k + shared) <= kFusedMaxRows && E <= 4 * kWave;
}

hipError_t launch_router_logits(const void* x, const void* wg, int T, int H, int E, bool bf16,
                                float* logits, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (!bf16) {
    const int64_t n = static_cast<int64_t>(T) * E;
    hipLaunchKernelGGL(router_logits_f32_kernel, dim3(static_cast<unsigned>((n + 255) / 256)),
                       dim3(256), 0, s, static_cast<const float*>(x),
                       static_cast<const float*>(wg), T, H, E, logits);
    return hipGetLastError();
  }
  const unsigned tb = static_cast<unsigned>((T + 15) / 16);
  const int nz = router_slabs(T, H, true);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const uint16_t* wb = static_cast<const uint16_t*>(wg);
  if (T <= 64 && H % 256 == 0) {
    // decode: 16 experts per work-group, each slab's K range split over 4 waves
    hipLaunchKernelGGL(router_logits_bf16_kernel<4>, dim3(tb, (E + 15) / 16, nz), dim3(256), 0,
                       s, xb, wb, T, H, E, slab_cols(T, H), logits);
  } else if (E <= 16) {
    // few experts: one 16-expert block per work-group, K split over its 4 waves
    hipLaunchKernelGGL(router_logits_bf16_kernel<4>, dim3(tb, 1, 1), dim3(256), 0, s, xb, wb, T,
                       H, E, H, logits);
  } else if (E <= 32) {
    hipLaunchKernelGGL(router_logits_bf16_kernel<2>, dim3(tb, 1, 1), dim3(256), 0, s, xb, wb, T,
                       H, E, H, logits);
  } else {
    hipLaunchKernelGGL(router_logits_tile_kernel,
                       dim3(static_cast<unsigned>((T + kRt - 1) / kRt), (E + kRt - 1) / kRt),
                       dim3(256), 0, s, xb, wb, T, H, E, logits);
  }
  return hipGetLastError();
}

hipError_t launch_router_logits_gemv(const void* x, const void* wg, int H, int E,
                                     float* logits, hipStream_t s) {
  if (H % 8) return hipErrorInvalidValue;
  hipLaunchKernelGGL(router_logits_gemv_kernel, dim3(static_cast<unsigned>(E)),
                     dim3(64), 0, s, static_cast<const uint16_t*>(x),
                     static_cast<const uint16_t*>(wg), H, E, logits);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int nz, float* logits_out, int T, int E, int k,
                       const RouteArgs& a, int32_t* ids, float* w, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const TopkParams p = topk_params(logits, nz, logits_out, T, E, k, a, ids, w);
  if (E <= 4 * kWave)
    hipLaunchKernelGGL(topk_kernel<4>, dim3((T + 3) / 4), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(topk_kernel<8>, dim3((T + 3) / 4), dim3(256), 0, s, p);
  return hipGetLastError();
}

bool route_fused_ok(int T, int H, int E, bool bf16) {
  return bf16 && T > 64 && H % 64 == 0 && E <= 32;
}

hipError_t launch_route_fused(const void* x, const void* wg, int T, int H, int E, int k,
                              const RouteArgs& a, int32_t* ids, float* w, float* logits_out,
                              hipStream_t s) {
  const TopkParams p = topk_params(nullptr, 1, logits_out, T, E, k, a, ids, w);
  const dim3 grid(static_cast<unsigned>((T + 15) / 16));
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const uint16_t* wb = static_cast<const uint16_t*>(wg);
  // 16 waves over (expert block, K slice) pairs, 16 / blocks slices per block
  if (E <= 16)
    hipLaunchKernelGGL(route_fused_kernel<16>, grid, dim3(1024), 0, s, xb, wb, H, p);
  else if (E <= 32)
    hipLaunchKernelGGL(route_fused_kernel<8>, grid, dim3(1024), 0, s, xb, wb, H, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_route_align_small(const float* logits, int nz, float* logits_out, int T, int E,
                                    int k, const RouteArgs& a, int32_t* ids, float* w, int bm,
                                    int64_t cap, int32_t* sorted_ids, int32_t* expert_ids,
                                    int32_t* ntpp, int32_t* counts, const int32_t* emap,
                                    hipStream_t s) {
  // E <= 256 (route_align_fusable): four experts per lane
  const TopkParams p = topk_params(logits, nz, logits_out, T, E, k, a, ids, w);
  hipLaunchKernelGGL(route_align_small_kernel<4>, dim3(1), dim3(1024), 0, s, p, bm, cap,
                     sorted_ids, expert_ids, ntpp, counts, emap);
  return hipGetLastError();
}

}  // namespace moe
