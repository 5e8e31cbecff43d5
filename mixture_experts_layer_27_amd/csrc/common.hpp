// Shared device helpers for the gfx950 MoE kernels (wave64, MFMA, bf16).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// bf16 <-> fp32.  The conversion to bf16 rounds to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// SiLU(g) * u for the bf16 SwiGLU epilogues: x * (1 / (1 + e^-x)) with the hardware
// reciprocal (v_rcp_f32, about 1 ulp), ample for a result rounded to bf16 next.
// e^-x overflowing to +inf gives rcp = 0 and SiLU = -0 for large negative x.
__device__ __forceinline__ float silu_mul_bf16path(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.f + __expf(-g)) * u;
}

// Orders LDS traffic between the lanes of one wave (no work-group barrier).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename T>
__device__ __forceinline__ T wave_shfl(T v, int src) { return __shfl(v, src, kWave); }

// ---------------------------------------------------------------- DPP lane moves
// Data-parallel-primitive moves stay in the VALU (no LDS round trip, unlike the
// ds_bpermute behind __shfl).  gfx9 control codes; every call must run with the
// whole wave active.
namespace dpp {
constexpr int kQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;  // lane i <- lane 7-i within each 8 lanes
constexpr int kRowMirror = 0x140;      // lane i <- lane 15-i within each 16-lane row
constexpr int kRowShr = 0x110;         // + n: lane i <- lane i-n of the same row
constexpr int kRowBcast15 = 0x142;     // lane 15 of row r -> every lane of row r+1
constexpr int kRowBcast31 = 0x143;     // lane 31 -> every lane of rows 2 and 3
}  // namespace dpp

// Lanes not written by the move (no source lane, or row masked off) return 0.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_move(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp_move<dpp::kRowShr + 1>(v);
  v += dpp_move<dpp::kRowShr + 2>(v);
  v += dpp_move<dpp::kRowShr + 4>(v);
  v += dpp_move<dpp::kRowShr + 8>(v);
  v += dpp_move<dpp::kRowBcast15, 0xA>(v);
  v += dpp_move<dpp::kRowBcast31, 0xC>(v);
  return v;
}

__device__ __forceinline__ int read_lane(int v, int lane) {
  return __builtin_amdgcn_readlane(v, lane);
}
__device__ __forceinline__ float read_lane(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
__device__ __forceinline__ double read_lane(double v, int lane) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(b & 0xffffffffu), lane);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(b >> 32), lane);
  return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

}  // namespace moe
