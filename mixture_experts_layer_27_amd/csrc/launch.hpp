// Internal host-side launchers of the HIP kernels (not exported; moe_api.cpp is the
// only caller).  All sizes are validated by the caller.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

struct RouteArgs {
  int mode;
  const float* offset;   // [E] or null
  const float* bias;     // [E] or null
  int n_group, topk_group;
  float scaling;
  int shared;            // 1: the routing gets slot k = shared expert E with weight 1
};

// router
// bf16 logits at decode batch sizes are produced as router_slabs(T,H) partial slabs
// [nz][T][E] that the top-k stage adds in ascending order (nz == 1: plain logits).
int router_slabs(int T, int H, bool bf16);
// one token, bf16 (H % 8 == 0): the E logits whole ([E] fp32, one one-wave work-group per
// expert)
hipError_t launch_router_logits_gemv(const void* x, const void* wg, int H, int E,
                                     float* logits, hipStream_t s);
hipError_t launch_router_logits(const void* x, const void* wg, int T, int H, int E, bool bf16,
                                float* logits, hipStream_t s);
// logits_out (nullable) receives the summed logits when nz > 1; ids / w are [T][k + a.shared]
hipError_t launch_topk(const float* logits, int nz, float* logits_out, int T, int E, int k,
                       const RouteArgs& a, int32_t* ids, float* w, hipStream_t s);
// prefill with up to 32 experts: logits and top-k in one launch (16 tokens per work-group)
bool route_fused_ok(int T, int H, int E, bool bf16);
hipError_t launch_route_fused(const void* x, const void* wg, int T, int H, int E, int k,
                              const RouteArgs& a, int32_t* ids, float* w, float* logits_out,
                              hipStream_t s);
// top-k of every token and the align table in one single-work-group launch (k routed
// slots over E experts, plus the shared slot when shared = 1)
bool route_align_fusable(int T, int k, int E, int shared);
hipError_t launch_route_align_small(const float* logits, int nz, float* logits_out, int T, int E,
                                    int k, const RouteArgs& a, int32_t* ids, float* w, int bm,
                                    int64_t cap, int32_t* sorted_ids, int32_t* expert_ids,
                                    int32_t* ntpp, int32_t* counts, const int32_t* emap,
                                    hipStream_t s);

// align; emap (nullable, [E]): expert parallelism, tiles carry emap[e] (-1: remote);
// tile_run (nullable, [cap / bm + 1]): each table tile gets (first tile, tiles) of its
// expert's run and the last entry (longest run, 0), for the expert-ordered raster of the
// prefill GEMMs
size_t align_ws_bytes(int R, int E);
hipError_t launch_align(const int32_t* ids, int R, int E, int bm, int64_t cap,
                        int32_t* sorted_ids, int32_t* expert_ids, int32_t* ntpp,
                        int32_t* counts, int32_t* ws_hist, const int32_t* emap, hipStream_t s,
                        int2* tile_run = nullptr);

// expert GEMMs
struct GemmArgs {
  const void* A;             // GEMM1: x [T,H]; GEMM2: a [R,I]
  const void* B;             // GEMM1: W13 [E,2I,H]; GEMM2: W2 [E,H,I]
  void* C;                   // GEMM1: a [R,I] (bf16/f32); GEMM2: y [R,H] f32
  const float* topk_w;       // GEMM2 only
  const float* w_scale;      // FP8 weights: per-row scales of B ([E,2I] or [E,H]); else null
  const int32_t* sorted_ids;
  const int32_t* expert_ids;     // owner of each tile; -1: skipped (GEMM2 zero-fills its rows)
  const int32_t* ntpp;
  int T, H, I, E, k, block_m;
  int64_t cap;               // capacity of sorted_ids
  // bound on the routed rows any one expert holds (0: T * k).  The layer passes T: its
  // router picks k distinct experts per token.
  int max_rows = 0;
  // (first tile, tiles) of each block_m tile's expert run (nullable): the prefill GEMMs
  // then order their tiles by expert run (see moe_gemm_pipe_kernel)
  const int2* tile_run = nullptr;
  // GEMM2 prefill: room for the partial sums of a split last round of
  // tiles (used when it holds one [256 x 256] fp32 tile per compute unit; else unsplit)
  float* split_ws = nullptr;
  size_t split_ws_bytes = 0;
};

// workspace the split last round of GEMM2 may use (one fp32 tile per work-group in flight,
// one work-group per CU: 256 tiles of up to 256 x 256, i.e. up to 256 CUs)
constexpr size_t kSplitWsBytes = static_cast<size_t>(256) * 256 * 256 * sizeof(float);

// variant: 1 prefill, 2 decode
hipError_t launch_gemm1(const GemmArgs& g, bool bf16, int variant, hipStream_t s);
hipError_t launch_gemm2(const GemmArgs& g, bool bf16, int variant, hipStream_t s);
hipError_t launch_combine(const float* y, int T, int H, int k, bool bf16, void* out,
                          hipStream_t s);


// small-M weight-streaming variant (decode.hip); block_m >= 16.  decode_block_m: the
// block_m whose tiles match the kernel's sub-tile height for R routed rows over E experts
int decode_block_m(int R, int E);
hipError_t launch_decode_gemm1(const GemmArgs& g, hipStream_t s);
// one token (T = 1, E <= 256): GEMM1 that first routes the token from the router's nz
// logit slabs ([nz][1][E]) with the rules of `a`, writes ids / w (k + shared slots) and
// the align table of g (block_m 16, cap 16 * g.k) and counts ([g.E]), then streams the
// selected experts
bool decode_route_ok(int T, int E, int k, int shared);
hipError_t launch_decode_gemm1_routed(const GemmArgs& g, const float* logits, int nz,
                                      const RouteArgs& a, int E, int k, int32_t* ids, float* w,
                                      int32_t* counts, hipStream_t s);
hipError_t launch_decode_gemm2(const GemmArgs& g, hipStream_t s);

// pipelined large-tile prefill kernels (gemm_pipe.hip); tile_m 128 or 256
hipError_t launch_pipe_gemm1(const GemmArgs& g, int tile_m, hipStream_t s);
hipError_t launch_pipe_gemm2(const GemmArgs& g, int tile_m, hipStream_t s);

// which prefill tile height the MFMA kernels use for a given align block_m (0 = none)
int prefill_tile_m(int block_m);

}  // namespace moe
