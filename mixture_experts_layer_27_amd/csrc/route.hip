// Router: logits = x . Wg^T (fp32 accumulate) and the top-k rules
// ("Mixture-of-Experts Kernels: Routing, Permutation, and Grouped GEMM", section 1
// model table, section 3 `route`, section 4 grouped sigmoid router).
//
// Logits (bf16): MFMA 16x16x32 bf16 with operands read straight from global memory
// in MFMA register layout (each lane owns one row of A or B and 32 contiguous bytes
// of K; the same k permutation is applied to both operands, so the dot products are
// unchanged).  A work-group covers 16 tokens x 16*(4/KSPLIT) experts; KSPLIT waves
// split K and reduce through LDS, which spreads the Wg stream over more CUs when T
// is small (decode).
//
// Top-k: one wave per token; lane l owns experts l, l+64, ...; each of the k
// selections is a wave arg-max on (value desc, index asc).
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kMaxPerLane = 8;   // E <= 512

template <int KSPLIT>
__global__ void __launch_bounds__(256)
router_logits_bf16_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg,
                          int T, int H, int E, float* __restrict__ logits) {
  constexpr int kExpWaves = 4 / KSPLIT;            // expert sub-blocks per WG
  __shared__ f32x4 red[4][kWave];
  const int lane = lane_id(), w = wave_id();
  const int eblk = w / KSPLIT, ks = w % KSPLIT;
  const int t0 = blockIdx.x * 16;
  const int e0 = (blockIdx.y * kExpWaves + eblk) * 16;
  const int row = lane & 15, grp = lane >> 4;
  const int t = min(t0 + row, T - 1);
  const int e = min(e0 + row, E - 1);
  const uint16_t* xa = x + static_cast<int64_t>(t) * H + grp * 16;
  const uint16_t* wb = wg + static_cast<int64_t>(e) * H + grp * 16;
  const int kper = H / KSPLIT;                      // H % (64*KSPLIT) == 0 (host-checked)
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = ks * kper; k0 < (ks + 1) * kper; k0 += 64) {
    const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(xa + k0);
    const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(xa + k0 + 8);
    const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(wb + k0);
    const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(wb + k0 + 8);
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
  for (int v = 0; v < 4; ++v) {
    const int tr = t0 + 4 * (lane >> 4) + v;
    if (tr < T) logits[static_cast<int64_t>(tr) * E + ec] = acc[v];
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

// (value, index) arg-max across the wave: better = larger value, then smaller index.
__device__ __forceinline__ void wave_argmax(float& v, int& idx) {
  for (int d = 32; d >= 1; d >>= 1) {
    const float ov = __shfl_xor(v, d, kWave);
    const int oi = __shfl_xor(idx, d, kWave);
    if (ov > v || (ov == v && oi < idx)) { v = ov; idx = oi; }
  }
}

__device__ __forceinline__ float sigmoid_rn(float l) {
  // sigma(l) evaluated in double and rounded once to the nearest float
  return static_cast<float>(1.0 / (1.0 + exp(-static_cast<double>(l))));
}

__global__ void __launch_bounds__(256)
topk_kernel(const float* __restrict__ logits, int T, int E, int k, int mode,
            const float* __restrict__ offset, const float* __restrict__ bias, int n_group,
            int topk_group, float scaling, int32_t* __restrict__ ids, float* __restrict__ wout) {
  __shared__ float cval[4][512];
  __shared__ int keep_grp[4][64];
  __shared__ int chosen_id[4][16];
  __shared__ float chosen_src[4][16];
  const int lane = lane_id(), w = wave_id();
  const int t = blockIdx.x * 4 + w;
  if (t >= T) return;                              // whole wave leaves together
  const float* lrow = logits + static_cast<int64_t>(t) * E;
  const float kNegInf = -__builtin_inff();
  float sel[kMaxPerLane];    // selection value (-inf = not eligible / taken)
  float wsrc[kMaxPerLane];   // weight source: logit (modes 0,1) or unbiased sigmoid (2)
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = lane + kWave * i;
    float v = kNegInf, ws = 0.f;
    if (e < E) {
      float l = lrow[e];
      if (offset) l = l + offset[e];
      if (mode == 2) {
        const float s = sigmoid_rn(l);
        v = bias ? s + bias[e] : s;
        ws = s;
      } else {
        v = l;
        ws = l;
      }
    }
    sel[i] = v;
    wsrc[i] = ws;
  }
  if (mode == 2 && n_group > 0 && topk_group > 0) {
    // group scores: sum of the two largest biased scores of each contiguous group
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + kWave * i;
      if (e < E) cval[w][e] = sel[i];
    }
    wave_sync();
    const int gsz = E / n_group;
    float gscore = kNegInf;
    int gidx = lane;
    if (lane < n_group) {
      float m1 = kNegInf, m2 = kNegInf;
      for (int q = 0; q < gsz; ++q) {              // ascending index: ties keep the first
        const float c = cval[w][lane * gsz + q];
        if (c > m1) { m2 = m1; m1 = c; } else if (c > m2) { m2 = c; }
      }
      gscore = m1 + m2;
    }
    keep_grp[w][lane] = 0;
    wave_sync();
    for (int j = 0; j < topk_group; ++j) {
      float v = gscore;
      int idx = gidx;
      if (lane >= n_group) { v = kNegInf; idx = 0x7fffffff; }
      wave_argmax(v, idx);
      if (lane == idx) { keep_grp[w][lane] = 1; gscore = kNegInf; gidx = 0x7fffffff; }
      wave_sync();
    }
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + kWave * i;
      if (e < E && !keep_grp[w][e / gsz]) sel[i] = kNegInf;
    }
  }
  // k selections; lane 0 keeps the chosen (id, weight source) pairs in LDS
  for (int j = 0; j < k; ++j) {
    float bv = kNegInf;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {       // within a lane, larger i = larger index
      const int e = lane + kWave * i;
      if (e < E && (sel[i] > bv || (sel[i] == bv && e < bi))) {
        bv = sel[i];
        bi = e;
      }
    }
    wave_argmax(bv, bi);
    float src = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      if (lane + kWave * i == bi) { src = wsrc[i]; sel[i] = kNegInf; }
    }
    src = __shfl(src, bi & (kWave - 1), kWave);   // the owner lane broadcasts
    if (lane == 0) {
      chosen_id[w][j] = bi;
      chosen_src[w][j] = src;
    }
  }
  wave_sync();
  if (lane == 0) {
    double sum = 0.0;
    const double l0 = chosen_src[w][0];
    for (int j = 0; j < k; ++j) {
      const double v = mode == 2 ? static_cast<double>(chosen_src[w][j])
                                 : exp(static_cast<double>(chosen_src[w][j]) - l0);
      sum += v;
    }
    for (int j = 0; j < k; ++j) {
      const double v = mode == 2 ? static_cast<double>(chosen_src[w][j])
                                 : exp(static_cast<double>(chosen_src[w][j]) - l0);
      const double wt = mode == 2 ? static_cast<double>(scaling) * v / sum : v / sum;
      ids[static_cast<int64_t>(t) * k + j] = chosen_id[w][j];
      wout[static_cast<int64_t>(t) * k + j] = static_cast<float>(wt);
    }
  }
}

}  // namespace

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
  if (T <= 64 && H % 256 == 0) {
    // decode: 16 experts per WG, K split over 4 waves
    hipLaunchKernelGGL(router_logits_bf16_kernel<4>, dim3(tb, (E + 15) / 16), dim3(256), 0, s,
                       static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(wg), T, H,
                       E, logits);
  } else {
    hipLaunchKernelGGL(router_logits_bf16_kernel<1>, dim3(tb, (E + 63) / 64), dim3(256), 0, s,
                       static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(wg), T, H,
                       E, logits);
  }
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int T, int E, int k, const RouteArgs& a,
                       int32_t* ids, float* w, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, a.mode,
                     a.offset, a.bias, a.n_group, a.topk_group, a.scaling, ids, w);
  return hipGetLastError();
}

}  // namespace moe
