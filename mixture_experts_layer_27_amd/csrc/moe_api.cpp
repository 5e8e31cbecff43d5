// Host side of the C ABI declared in include/moe_mi355x.h: argument validation,
// workspace sizing, variant choice from host-known sizes, kernel dispatch.
// Nothing here allocates, copies or synchronises; every call only enqueues work.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/moe_mi355x.h"
#include "launch.hpp"

namespace {

thread_local std::string g_err;

moe_status fail(moe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

moe_status ok() {
  g_err.clear();
  return MOE_OK;
}

moe_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
// activation types of the router and the combine (x, Wg, out)
bool valid_dt(int dt) { return dt == MOE_F32 || dt == MOE_BF16; }
// expert GEMMs and the layer also take bf16 activations with FP8 expert weights
bool valid_expert_dt(int dt) { return valid_dt(dt) || dt == MOE_BF16_FP8W; }
bool bf16_acts(int dt) { return dt == MOE_BF16 || dt == MOE_BF16_FP8W; }
size_t esize(moe_dtype dt) { return bf16_acts(dt) ? 2 : 4; }
size_t round_up(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }
bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

constexpr int kMaxE = 512;
constexpr int kMaxK = 16;
// the weight-streaming kernels keep a table of up to 4096 16-row sub-tiles in lanes
constexpr int64_t kMaxDecodeRows = 4096 * 16;

moe_status check_tke(int T, int k, int E) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T=%d must be >= 0", T);
  if (k < 1 || k > kMaxK) return fail(MOE_ERR_UNSUPPORTED, "k=%d outside [1, %d]", k, kMaxK);
  if (E < k) return fail(MOE_ERR_INVALID_ARG, "E=%d must be >= k=%d", E, k);
  if (E > kMaxE) return fail(MOE_ERR_UNSUPPORTED, "E=%d above %d", E, kMaxE);
  if (static_cast<int64_t>(T) * k >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED, "T*k=%lld does not fit int32",
                static_cast<long long>(T) * k);
  return MOE_OK;
}

int64_t capacity(int T, int k, int E, int bm) {
  const int64_t R = static_cast<int64_t>(T) * k;
  const int64_t bound = R + std::min<int64_t>(E, R) * (bm - 1);
  return bound / bm * bm;
}

moe_status check_route_cfg(const moe_route_cfg* cfg, int E, int k) {
  if (!cfg) return fail(MOE_ERR_INVALID_ARG, "cfg is NULL");
  if (cfg->mode < 0 || cfg->mode > 2) return fail(MOE_ERR_INVALID_ARG, "mode=%d", cfg->mode);
  if (cfg->mode != MOE_ROUTE_SIGMOID_BIAS_GROUPED) {
    if (cfg->select_bias)
      return fail(MOE_ERR_INVALID_ARG, "select_bias is only meaningful for the sigmoid router");
    return MOE_OK;
  }
  const int ng = cfg->n_group, tg = cfg->topk_group;
  if (ng == 0 && tg == 0) return MOE_OK;
  if (ng <= 0 || tg <= 0) return fail(MOE_ERR_INVALID_ARG, "n_group=%d topk_group=%d", ng, tg);
  if (ng > 64) return fail(MOE_ERR_UNSUPPORTED, "n_group=%d above 64", ng);
  if (E % ng != 0) return fail(MOE_ERR_INVALID_ARG, "n_group=%d does not divide E=%d", ng, E);
  if (E / ng < 2) return fail(MOE_ERR_INVALID_ARG, "groups need >= 2 experts (E/n_group=%d)", E / ng);
  if (tg > ng) return fail(MOE_ERR_INVALID_ARG, "topk_group=%d > n_group=%d", tg, ng);
  if (static_cast<int64_t>(tg) * (E / ng) < k)
    return fail(MOE_ERR_INVALID_ARG, "topk_group*E/n_group=%d < k=%d", tg * (E / ng), k);
  return MOE_OK;
}

moe_route_cfg default_cfg() {
  moe_route_cfg c;
  std::memset(&c, 0, sizeof(c));
  c.routed_scaling = 1.f;
  return c;
}

moe::RouteArgs route_args(const moe_route_cfg* cfg) {
  moe::RouteArgs a;
  a.mode = cfg->mode;
  a.offset = cfg->logit_offset;
  a.bias = cfg->select_bias;
  a.n_group = cfg->mode == 2 ? cfg->n_group : 0;
  a.topk_group = cfg->mode == 2 ? cfg->topk_group : 0;
  a.scaling = cfg->mode == 2 ? cfg->routed_scaling : 1.f;
  a.shared = 0;
  return a;
}

int auto_variant(int T, int H, int I, int E, int k, moe_dtype dt) {
  (void)H; (void)I;
  if (dt == MOE_F32) return MOE_VARIANT_PREFILL;
  const int64_t R = static_cast<int64_t>(T) * k;
  // decode when the average expert holds at most 8 routed rows
  return R <= 8 * static_cast<int64_t>(E) ? MOE_VARIANT_DECODE : MOE_VARIANT_PREFILL;
}

int preferred_bm(int T, int H, int I, int E, int k, moe_dtype dt) {
  if (dt == MOE_F32) return 16;
  if (auto_variant(T, H, I, E, k, dt) == MOE_VARIANT_DECODE)
    return moe::decode_block_m(static_cast<int>(static_cast<int64_t>(T) * k), E);
  // 256-row MFMA tiles halve the weight-tile reloads per row but pad each expert's last
  // tile further; both heights run the ping-pong schedule.  Measured crossovers (average
  // rows per expert, layer time with 128- vs 256-row tiles): with a few large experts
  // (E = 8, I = 14336) 128 rows win up to 128 (bf16 0.796 vs 0.824 ms, FP8 0.622 vs 0.677)
  // and lose at 256 (bf16 1.185 vs 1.047, FP8 0.957 vs 0.890); with E = 128 or 256 they
  // are level at 128 (Qwen3 1.354 vs 1.344, gpt-oss 1.805 vs 1.844, DeepSeek-V3 4.25 vs
  // 3.98, its FP8 form 3.775 vs 3.701) and lose from 192 (Qwen3 1.675 vs 1.501).
  (void)H;
  const int64_t avg = static_cast<int64_t>(T) * k / E;
  return avg >= (E <= 32 ? 256 : 128) ? 256 : 128;
}

int resolve_variant(int variant, int T, int H, int I, int E, int k, moe_dtype dt) {
  return variant == MOE_VARIANT_AUTO ? auto_variant(T, H, I, E, k, dt) : variant;
}

moe_status check_gemm_common(int T, int H, int I, int E, int k, int block_m, int dt,
                             int variant) {
  moe_status st = check_tke(T, k, E);
  if (st != MOE_OK) return st;
  if (!valid_expert_dt(dt)) return fail(MOE_ERR_INVALID_ARG, "dtype=%d", dt);
  if (H <= 0 || I <= 0) return fail(MOE_ERR_INVALID_ARG, "H=%d I=%d must be > 0", H, I);
  if (!is_pow2(block_m) || block_m > 256)
    return fail(MOE_ERR_INVALID_ARG, "block_m=%d must be a power of two <= 256", block_m);
  if (variant < 0 || variant > 2) return fail(MOE_ERR_INVALID_ARG, "variant=%d", variant);
  if (dt == MOE_BF16) {
    if (H % 64 || I % 64)
      return fail(MOE_ERR_UNSUPPORTED, "bf16 path needs H, I multiples of 64 (H=%d I=%d)", H, I);
    const int v = resolve_variant(variant, T, H, I, E, k, static_cast<moe_dtype>(dt));
    if (v == MOE_VARIANT_PREFILL && moe::prefill_tile_m(block_m) == 0)
      return fail(MOE_ERR_UNSUPPORTED, "bf16 prefill tiles need block_m >= 32 (got %d)", block_m);
    if (v == MOE_VARIANT_DECODE && block_m < 16)
      return fail(MOE_ERR_UNSUPPORTED, "bf16 decode tiles need block_m >= 16 (got %d)", block_m);
  }
  if (dt == MOE_BF16_FP8W) {
    if (H % 128 || I % 128)
      return fail(MOE_ERR_UNSUPPORTED, "FP8 weights need H, I multiples of 128 (H=%d I=%d)", H, I);
    const int v = resolve_variant(variant, T, H, I, E, k, static_cast<moe_dtype>(dt));
    if (v == MOE_VARIANT_PREFILL && block_m < 128)
      return fail(MOE_ERR_UNSUPPORTED, "FP8-weight prefill tiles need block_m >= 128 (got %d)", block_m);
    if (v == MOE_VARIANT_DECODE && block_m < 16)
      return fail(MOE_ERR_UNSUPPORTED, "FP8-weight decode tiles need block_m >= 16 (got %d)", block_m);
  }
  if (bf16_acts(dt) &&
      resolve_variant(variant, T, H, I, E, k, static_cast<moe_dtype>(dt)) == MOE_VARIANT_DECODE &&
      capacity(T, k, E, block_m) > kMaxDecodeRows)
    return fail(MOE_ERR_UNSUPPORTED, "the decode variant takes at most %d padded rows (use prefill)",
                kMaxDecodeRows);
  if (static_cast<int64_t>(T) * k * std::max(H, I) >= (int64_t(1) << 40))
    return fail(MOE_ERR_UNSUPPORTED, "tensor too large");
  return MOE_OK;
}

moe::GemmArgs gemm_args(const void* A, const void* B, const float* B_scale, void* C,
                        const float* topk_w, const int32_t* sorted_ids,
                        const int32_t* expert_ids, const int32_t* ntpp, int T, int H, int I,
                        int E, int k, int block_m) {
  moe::GemmArgs g;
  g.A = A; g.B = B; g.w_scale = B_scale; g.C = C; g.topk_w = topk_w;
  g.sorted_ids = sorted_ids; g.expert_ids = expert_ids; g.ntpp = ntpp;
  g.T = T; g.H = H; g.I = I; g.E = E; g.k = k; g.block_m = block_m;
  g.cap = capacity(T, k, E, block_m);
  return g;
}

size_t forward_ws(int T, int H, int I, int k, moe_dtype dt) {
  const size_t R = static_cast<size_t>(T) * k;
  return round_up(R * I * esize(dt)) + round_up(R * H * sizeof(float));
}

// the forward workspace with room for GEMM2's split last round when the layer's automatic
// variant is prefill (the GEMM runs unsplit in a smaller workspace)
size_t forward_ws_full(int T, int H, int I, int E, int k, moe_dtype dt) {
  const bool split = bf16_acts(dt) && auto_variant(T, H, I, E, k, dt) == MOE_VARIANT_PREFILL;
  return forward_ws(T, H, I, k, dt) + (split ? moe::kSplitWsBytes : 0);
}

}  // namespace

extern "C" {

const char* moe_version(void) { return "moe_mi355x 0.1 (gfx950)"; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_err.c_str(); }

// ------------------------------------------------------------------------------ route
size_t moe_route_workspace_size(int T, int H, int E, moe_dtype dt) {
  if (T <= 0 || H <= 0 || E <= 0 || !valid_dt(dt)) return 0;
  const size_t nz = static_cast<size_t>(moe::router_slabs(T, H, dt == MOE_BF16));
  return round_up(nz * static_cast<size_t>(T) * E * sizeof(float));
}

moe_status moe_route(const void* x, const void* wg, int T, int H, int E, int k, moe_dtype dt,
                     const moe_route_cfg* cfg, int32_t* topk_ids, float* topk_w,
                     float* logits_out, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_tke(T, k, E);
  if (st != MOE_OK) return st;
  if (!valid_dt(dt)) return fail(MOE_ERR_INVALID_ARG, "dtype=%d", dt);
  if (H <= 0) return fail(MOE_ERR_INVALID_ARG, "H=%d", H);
  if ((st = check_route_cfg(cfg, E, k)) != MOE_OK) return st;
  if (T == 0) return ok();
  if (!x || !wg || !topk_ids || !topk_w) return fail(MOE_ERR_INVALID_ARG, "NULL tensor pointer");
  if (dt == MOE_BF16) {
    if (H % 64) return fail(MOE_ERR_UNSUPPORTED, "bf16 router needs H %% 64 == 0 (H=%d)", H);
    if (!aligned16(x) || !aligned16(wg)) return fail(MOE_ERR_INVALID_ARG, "x/Wg not 16-byte aligned");
  }
  const size_t need = moe_route_workspace_size(T, H, E, dt);
  if (!ws || ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "route workspace needs %zu bytes", need);
  float* slabs = static_cast<float*>(ws);
  const int nz = moe::router_slabs(T, H, dt == MOE_BF16);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (moe::route_fused_ok(T, H, E, dt == MOE_BF16))   // prefill: logits and top-k in one launch
    return hip_status(moe::launch_route_fused(x, wg, T, H, E, k, route_args(cfg), topk_ids, topk_w,
                                              logits_out, s),
                      "router");
  hipError_t e = moe::launch_router_logits(x, wg, T, H, E, dt == MOE_BF16, slabs, s);
  if (e != hipSuccess) return hip_status(e, "router logits");
  e = moe::launch_topk(slabs, nz, logits_out, T, E, k, route_args(cfg), topk_ids, topk_w, s);
  return hip_status(e, "top-k");
}

moe_status moe_route_from_logits(const float* logits, int T, int E, int k,
                                 const moe_route_cfg* cfg, int32_t* topk_ids, float* topk_w,
                                 void* stream) {
  moe_status st = check_tke(T, k, E);
  if (st != MOE_OK) return st;
  if ((st = check_route_cfg(cfg, E, k)) != MOE_OK) return st;
  if (T == 0) return ok();
  if (!logits || !topk_ids || !topk_w) return fail(MOE_ERR_INVALID_ARG, "NULL tensor pointer");
  hipError_t e = moe::launch_topk(logits, 1, nullptr, T, E, k, route_args(cfg), topk_ids, topk_w,
                                  static_cast<hipStream_t>(stream));
  return hip_status(e, "top-k");
}

// ------------------------------------------------------------------------------ align
int64_t moe_align_capacity(int T, int k, int E, int block_m) {
  if (T < 0 || k < 1 || E < 1 || block_m < 1) return -1;
  return capacity(T, k, E, block_m);
}

size_t moe_align_workspace_size(int T, int k, int E, int block_m) {
  (void)block_m;
  if (T <= 0 || k < 1 || E < 1) return 0;
  return round_up(moe::align_ws_bytes(T * k, E));
}

}  // extern "C"

namespace {

moe_status align_impl(const int32_t* topk_ids, int T, int k, int E, int block_m,
                      const int32_t* expert_map, int32_t* sorted_ids, int32_t* expert_ids,
                      int32_t* num_tokens_post_padded, int32_t* expert_counts, void* ws,
                      size_t ws_bytes, void* stream) {
  moe_status st = check_tke(T, k, E);
  if (st != MOE_OK) return st;
  if (!is_pow2(block_m) || block_m > 256)
    return fail(MOE_ERR_INVALID_ARG, "block_m=%d must be a power of two <= 256", block_m);
  const int64_t cap = capacity(T, k, E, block_m);
  if (cap >= (int64_t(1) << 31)) return fail(MOE_ERR_UNSUPPORTED, "capacity %lld too large",
                                             static_cast<long long>(cap));
  if (!num_tokens_post_padded) return fail(MOE_ERR_INVALID_ARG, "num_tokens_post_padded is NULL");
  if (T > 0 && (!topk_ids || !sorted_ids || !expert_ids))
    return fail(MOE_ERR_INVALID_ARG, "NULL tensor pointer");
  const size_t need = moe_align_workspace_size(T, k, E, block_m);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(MOE_ERR_WORKSPACE, "align workspace needs %zu bytes", need);
  hipError_t e = moe::launch_align(topk_ids, T * k, E, block_m, cap, sorted_ids, expert_ids,
                                   num_tokens_post_padded, expert_counts,
                                   static_cast<int32_t*>(ws), expert_map,
                                   static_cast<hipStream_t>(stream));
  return hip_status(e, "align");
}

}  // namespace

extern "C" {

moe_status moe_align(const int32_t* topk_ids, int T, int k, int E, int block_m,
                     int32_t* sorted_ids, int32_t* expert_ids,
                     int32_t* num_tokens_post_padded, int32_t* expert_counts, void* ws,
                     size_t ws_bytes, void* stream) {
  return align_impl(topk_ids, T, k, E, block_m, nullptr, sorted_ids, expert_ids,
                    num_tokens_post_padded, expert_counts, ws, ws_bytes, stream);
}

moe_status moe_align_ep(const int32_t* topk_ids, int T, int k, int E, int block_m,
                        const int32_t* expert_map, int32_t* sorted_ids, int32_t* expert_ids,
                        int32_t* num_tokens_post_padded, int32_t* expert_counts, void* ws,
                        size_t ws_bytes, void* stream) {
  if (!expert_map) return fail(MOE_ERR_INVALID_ARG, "expert_map is NULL");
  return align_impl(topk_ids, T, k, E, block_m, expert_map, sorted_ids, expert_ids,
                    num_tokens_post_padded, expert_counts, ws, ws_bytes, stream);
}

// ------------------------------------------------------------------------------ forward
int moe_auto_variant(int T, int H, int I, int E, int k, moe_dtype dt) {
  if (T < 0 || E < 1 || k < 1 || !valid_expert_dt(dt)) return 0;
  return auto_variant(T, H, I, E, k, dt);
}

int moe_preferred_block_m(int T, int H, int I, int E, int k, moe_dtype dt) {
  if (T < 0 || E < 1 || k < 1 || !valid_expert_dt(dt)) return 0;
  return preferred_bm(T, H, I, E, k, dt);
}

}  // extern "C"

namespace {

// FP8 weights need both scale arrays (the *_fp8 entry points); other weights take none
moe_status check_scales(int dt, const float* s13, const float* s2) {
  if (dt == MOE_BF16_FP8W) {
    if (!s13 || !s2)
      return fail(MOE_ERR_INVALID_ARG, "FP8 weights need their per-row scales (the *_fp8 entry points)");
  } else if (s13 || s2) {
    return fail(MOE_ERR_INVALID_ARG, "weight scales are only taken with FP8 weights");
  }
  return MOE_OK;
}

moe_status gemm1_impl(const void* x, const void* w13, const float* w13_scale,
                      const int32_t* sorted_ids, const int32_t* expert_ids,
                      const int32_t* num_tokens_post_padded, int T, int H, int I, int E, int k,
                      int block_m, moe_dtype dt, int variant, void* a, void* stream) {
  moe_status st = check_gemm_common(T, H, I, E, k, block_m, dt, variant);
  if (st != MOE_OK) return st;
  if ((st = check_scales(dt, w13_scale, w13_scale)) != MOE_OK) return st;
  if (T == 0) return ok();
  if (!x || !w13 || !sorted_ids || !expert_ids || !num_tokens_post_padded || !a)
    return fail(MOE_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!aligned16(x) || !aligned16(w13) || !aligned16(a))
    return fail(MOE_ERR_INVALID_ARG, "x/W13/a not 16-byte aligned");
  const int v = resolve_variant(variant, T, H, I, E, k, dt);
  moe::GemmArgs g = gemm_args(x, w13, w13_scale, a, nullptr, sorted_ids, expert_ids,
                              num_tokens_post_padded, T, H, I, E, k, block_m);
  return hip_status(moe::launch_gemm1(g, bf16_acts(dt), v, static_cast<hipStream_t>(stream)),
                    "gemm1");
}

moe_status gemm2_impl(const void* a, const void* w2, const float* w2_scale, const float* topk_w,
                      const int32_t* sorted_ids, const int32_t* expert_ids,
                      const int32_t* num_tokens_post_padded, int T, int H, int I, int E, int k,
                      int block_m, moe_dtype dt, int variant, float* y, void* stream) {
  moe_status st = check_gemm_common(T, H, I, E, k, block_m, dt, variant);
  if (st != MOE_OK) return st;
  if ((st = check_scales(dt, w2_scale, w2_scale)) != MOE_OK) return st;
  if (T == 0) return ok();
  if (!a || !w2 || !topk_w || !sorted_ids || !expert_ids || !num_tokens_post_padded || !y)
    return fail(MOE_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!aligned16(a) || !aligned16(w2) || !aligned16(y))
    return fail(MOE_ERR_INVALID_ARG, "a/W2/y not 16-byte aligned");
  const int v = resolve_variant(variant, T, H, I, E, k, dt);
  moe::GemmArgs g = gemm_args(a, w2, w2_scale, y, topk_w, sorted_ids, expert_ids,
                              num_tokens_post_padded, T, H, I, E, k, block_m);
  return hip_status(moe::launch_gemm2(g, bf16_acts(dt), v, static_cast<hipStream_t>(stream)),
                    "gemm2");
}

}  // namespace

extern "C" {

moe_status moe_gemm1_swiglu(const void* x, const void* w13, const int32_t* sorted_ids,
                            const int32_t* expert_ids, const int32_t* num_tokens_post_padded,
                            int T, int H, int I, int E, int k, int block_m, moe_dtype dt,
                            int variant, void* a, void* stream) {
  return gemm1_impl(x, w13, nullptr, sorted_ids, expert_ids, num_tokens_post_padded, T, H, I, E,
                    k, block_m, dt, variant, a, stream);
}

moe_status moe_gemm1_swiglu_fp8(const void* x, const uint8_t* w13, const float* w13_scale,
                                const int32_t* sorted_ids, const int32_t* expert_ids,
                                const int32_t* num_tokens_post_padded, int T, int H, int I,
                                int E, int k, int block_m, int variant, void* a, void* stream) {
  if (!w13_scale) return fail(MOE_ERR_INVALID_ARG, "w13_scale is NULL");
  return gemm1_impl(x, w13, w13_scale, sorted_ids, expert_ids, num_tokens_post_padded, T, H, I,
                    E, k, block_m, MOE_BF16_FP8W, variant, a, stream);
}

moe_status moe_gemm2_weighted(const void* a, const void* w2, const float* topk_w,
                              const int32_t* sorted_ids, const int32_t* expert_ids,
                              const int32_t* num_tokens_post_padded, int T, int H, int I,
                              int E, int k, int block_m, moe_dtype dt, int variant, float* y,
                              void* stream) {
  return gemm2_impl(a, w2, nullptr, topk_w, sorted_ids, expert_ids, num_tokens_post_padded, T, H,
                    I, E, k, block_m, dt, variant, y, stream);
}

moe_status moe_gemm2_weighted_fp8(const void* a, const uint8_t* w2, const float* w2_scale,
                                  const float* topk_w, const int32_t* sorted_ids,
                                  const int32_t* expert_ids,
                                  const int32_t* num_tokens_post_padded, int T, int H, int I,
                                  int E, int k, int block_m, int variant, float* y,
                                  void* stream) {
  if (!w2_scale) return fail(MOE_ERR_INVALID_ARG, "w2_scale is NULL");
  return gemm2_impl(a, w2, w2_scale, topk_w, sorted_ids, expert_ids, num_tokens_post_padded, T,
                    H, I, E, k, block_m, MOE_BF16_FP8W, variant, y, stream);
}

moe_status moe_combine(const float* y, int T, int H, int k, moe_dtype dt, void* out,
                       void* stream) {
  if (T < 0 || H <= 0 || k < 1 || k > kMaxK) return fail(MOE_ERR_INVALID_ARG, "T/H/k out of range");
  if (!valid_dt(dt)) return fail(MOE_ERR_INVALID_ARG, "dtype=%d", dt);
  if (T == 0) return ok();
  if (!y || !out) return fail(MOE_ERR_INVALID_ARG, "NULL tensor pointer");
  return hip_status(moe::launch_combine(y, T, H, k, dt == MOE_BF16, out,
                                        static_cast<hipStream_t>(stream)),
                    "combine");
}

size_t moe_forward_workspace_size(int T, int H, int I, int E, int k, moe_dtype dt) {
  if (T <= 0 || H <= 0 || I <= 0 || E <= 0 || k < 1 || !valid_expert_dt(dt)) return 0;
  return forward_ws_full(T, H, I, E, k, dt);
}

}  // extern "C"

namespace {

moe_status forward_impl(const void* x, const void* w13, const float* w13_scale, const void* w2,
                        const float* w2_scale, const float* topk_w, const int32_t* sorted_ids,
                        const int32_t* expert_ids, const int32_t* num_tokens_post_padded, int T,
                        int H, int I, int E, int k, int block_m, moe_dtype dt, int variant,
                        void* out, void* ws, size_t ws_bytes, void* stream,
                        int max_rows = 0, const int2* tile_run = nullptr) {
  moe_status st = check_gemm_common(T, H, I, E, k, block_m, dt, variant);
  if (st != MOE_OK) return st;
  if ((st = check_scales(dt, w13_scale, w2_scale)) != MOE_OK) return st;
  if (T == 0) return ok();
  if (!x || !w13 || !w2 || !topk_w || !sorted_ids || !expert_ids || !num_tokens_post_padded ||
      !out)
    return fail(MOE_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!aligned16(x) || !aligned16(w13) || !aligned16(w2) || !aligned16(out))
    return fail(MOE_ERR_INVALID_ARG, "x/W13/W2/out not 16-byte aligned");
  const size_t need = forward_ws(T, H, I, k, dt);
  if (!ws || ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "forward workspace needs %zu bytes", need);
  if (!aligned16(ws)) return fail(MOE_ERR_INVALID_ARG, "workspace not 16-byte aligned");
  const size_t R = static_cast<size_t>(T) * k;
  uint8_t* base = static_cast<uint8_t*>(ws);
  void* a = base;
  float* y = reinterpret_cast<float*>(base + round_up(R * I * esize(dt)));
  const int v = resolve_variant(variant, T, H, I, E, k, dt);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf = bf16_acts(dt);
  moe::GemmArgs g1 = gemm_args(x, w13, w13_scale, a, nullptr, sorted_ids, expert_ids,
                               num_tokens_post_padded, T, H, I, E, k, block_m);
  g1.max_rows = max_rows;
  g1.tile_run = tile_run;
  hipError_t e = moe::launch_gemm1(g1, bf, v, s);
  if (e != hipSuccess) return hip_status(e, "gemm1");
  moe::GemmArgs g2 = gemm_args(a, w2, w2_scale, y, topk_w, sorted_ids, expert_ids,
                               num_tokens_post_padded, T, H, I, E, k, block_m);
  g2.max_rows = max_rows;
  g2.tile_run = tile_run;
  if (bf && v == MOE_VARIANT_PREFILL && ws_bytes >= need + moe::kSplitWsBytes) {
    g2.split_ws = reinterpret_cast<float*>(base + need);
    g2.split_ws_bytes = moe::kSplitWsBytes;
  }
  e = moe::launch_gemm2(g2, bf, v, s);
  if (e != hipSuccess) return hip_status(e, "gemm2");
  return hip_status(moe::launch_combine(y, T, H, k, bf, out, s), "combine");
}

}  // namespace

extern "C" {

moe_status moe_forward(const void* x, const void* w13, const void* w2, const float* topk_w,
                       const int32_t* sorted_ids, const int32_t* expert_ids,
                       const int32_t* num_tokens_post_padded, int T, int H, int I, int E,
                       int k, int block_m, moe_dtype dt, int variant, void* out, void* ws,
                       size_t ws_bytes, void* stream) {
  return forward_impl(x, w13, nullptr, w2, nullptr, topk_w, sorted_ids, expert_ids,
                      num_tokens_post_padded, T, H, I, E, k, block_m, dt, variant, out, ws,
                      ws_bytes, stream);
}

moe_status moe_forward_fp8(const void* x, const uint8_t* w13, const float* w13_scale,
                           const uint8_t* w2, const float* w2_scale, const float* topk_w,
                           const int32_t* sorted_ids, const int32_t* expert_ids,
                           const int32_t* num_tokens_post_padded, int T, int H, int I, int E,
                           int k, int block_m, int variant, void* out, void* ws,
                           size_t ws_bytes, void* stream) {
  if (!w13_scale || !w2_scale) return fail(MOE_ERR_INVALID_ARG, "NULL scale pointer");
  return forward_impl(x, w13, w13_scale, w2, w2_scale, topk_w, sorted_ids, expert_ids,
                      num_tokens_post_padded, T, H, I, E, k, block_m, MOE_BF16_FP8W, variant,
                      out, ws, ws_bytes, stream);
}

// ------------------------------------------------------------------------------ layer
namespace {
struct LayerPlan {
  int bm, nz;
  bool fused_route_align;
  bool route_in_gemm1;     // one token: GEMM1 selects the experts from the logit slabs
  int64_t cap;
  size_t off_logits, off_ids, off_w, off_sorted, off_eids, off_ntpp, off_counts, off_runs,
      off_align, off_fwd, total;
};

// shared = 1: the routing gets one more slot (the shared expert, index E), so the table,
// the GEMMs and the combine see k + 1 slots over E + 1 experts
LayerPlan plan_layer(int T, int H, int I, int E, int k, moe_dtype dt, int shared = 0) {
  LayerPlan p;
  const int ES = E + shared, KS = k + shared;
  p.bm = preferred_bm(T, H, I, ES, KS, dt);
  p.cap = capacity(T, KS, ES, p.bm);
  const size_t R = static_cast<size_t>(T) * KS;
  size_t off = 0;
  p.nz = moe::router_slabs(T, H, bf16_acts(dt));
  p.fused_route_align = moe::route_align_fusable(T, k, E, shared);
  p.route_in_gemm1 = bf16_acts(dt) && moe::decode_route_ok(T, E, k, shared) &&
                     auto_variant(T, H, I, ES, KS, dt) == MOE_VARIANT_DECODE && p.bm == 16 &&
                     p.cap == 16 * KS;
  p.off_logits = off; off += round_up(static_cast<size_t>(p.nz) * T * E * sizeof(float));
  p.off_ids = off; off += round_up(R * sizeof(int32_t));
  p.off_w = off; off += round_up(R * sizeof(float));
  p.off_sorted = off; off += round_up(static_cast<size_t>(p.cap) * sizeof(int32_t));
  p.off_eids = off; off += round_up(static_cast<size_t>(p.cap / p.bm) * sizeof(int32_t));
  p.off_ntpp = off; off += round_up(sizeof(int32_t));
  p.off_counts = off; off += round_up(static_cast<size_t>(ES) * sizeof(int32_t));
  p.off_runs = off; off += round_up(static_cast<size_t>(p.cap / p.bm + 1) * sizeof(int2));
  p.off_align = off; off += round_up(moe::align_ws_bytes(static_cast<int>(R), ES));
  p.off_fwd = off; off += forward_ws_full(T, H, I, ES, KS, dt);
  p.total = off;
  return p;
}
}  // namespace

size_t moe_layer_workspace_size(int T, int H, int I, int E, int k, moe_dtype dt) {
  if (T <= 0 || H <= 0 || I <= 0 || E <= 0 || k < 1 || !valid_expert_dt(dt)) return 0;
  return plan_layer(T, H, I, E, k, dt).total;
}

}  // extern "C"

namespace {

moe_status layer_impl(const void* x, const void* wg, const void* w13, const float* w13_scale,
                      const void* w2, const float* w2_scale, const int32_t* expert_map,
                      const moe_route_cfg* cfg, int T,
                      int H, int I, int E, int k, moe_dtype dt, void* out, int32_t* topk_ids_out,
                      float* topk_w_out, void* ws, size_t ws_bytes, void* stream,
                      int shared = 0) {
  moe_status st = check_tke(T, k, E);
  if (st != MOE_OK) return st;
  const int ES = E + shared, KS = k + shared;
  if (shared && (st = check_tke(T, KS, ES)) != MOE_OK) return st;
  if (shared && expert_map)
    return fail(MOE_ERR_UNSUPPORTED, "a shared expert with an expert map is not supported");
  if (!valid_expert_dt(dt)) return fail(MOE_ERR_INVALID_ARG, "dtype=%d", dt);
  // the sizes must suit the block_m this layer aligns with
  st = check_gemm_common(T, H, I, ES, KS, preferred_bm(T, H, I, ES, KS, dt), dt,
                         MOE_VARIANT_AUTO);
  if (st != MOE_OK) return st;
  if ((st = check_route_cfg(cfg, E, k)) != MOE_OK) return st;
  if ((st = check_scales(dt, w13_scale, w2_scale)) != MOE_OK) return st;
  if (T == 0) return ok();
  if (!x || !wg || !w13 || !w2 || !out) return fail(MOE_ERR_INVALID_ARG, "NULL tensor pointer");
  if (bf16_acts(dt) && (!aligned16(x) || !aligned16(wg) || !aligned16(w13) || !aligned16(w2) ||
                        !aligned16(out)))
    return fail(MOE_ERR_INVALID_ARG, "tensor not 16-byte aligned");
  const LayerPlan p = plan_layer(T, H, I, E, k, dt, shared);
  if (!ws || ws_bytes < p.total) return fail(MOE_ERR_WORKSPACE, "layer workspace needs %zu bytes", p.total);
  if (!aligned16(ws)) return fail(MOE_ERR_INVALID_ARG, "workspace not 16-byte aligned");
  uint8_t* b = static_cast<uint8_t*>(ws);
  float* logits = reinterpret_cast<float*>(b + p.off_logits);
  int32_t* ids = topk_ids_out ? topk_ids_out : reinterpret_cast<int32_t*>(b + p.off_ids);
  float* tw = topk_w_out ? topk_w_out : reinterpret_cast<float*>(b + p.off_w);
  int32_t* sorted = reinterpret_cast<int32_t*>(b + p.off_sorted);
  int32_t* eids = reinterpret_cast<int32_t*>(b + p.off_eids);
  int32_t* ntpp = reinterpret_cast<int32_t*>(b + p.off_ntpp);
  int32_t* counts = reinterpret_cast<int32_t*>(b + p.off_counts);
  int2* runs = reinterpret_cast<int2*>(b + p.off_runs);
  hipStream_t s = static_cast<hipStream_t>(stream);
  moe::RouteArgs ra = route_args(cfg);
  ra.shared = shared;
  hipError_t e = hipSuccess;
  if (p.route_in_gemm1 && !expert_map) {
    // one token: the router logits (whole), then GEMM1 routes the token itself (every wave
    // selects and ranks the experts; work-group 0 writes the routing and the table),
    // GEMM2, the combine
    e = moe::launch_router_logits_gemv(x, wg, H, E, logits, s);
    if (e != hipSuccess) return hip_status(e, "router logits");
    uint8_t* fw = b + p.off_fwd;
    void* a = fw;
    float* y = reinterpret_cast<float*>(fw + round_up(static_cast<size_t>(KS) * I * esize(dt)));
    moe::GemmArgs g1 = gemm_args(x, w13, w13_scale, a, nullptr, sorted, eids, ntpp, T, H, I, ES,
                                 KS, p.bm);
    e = moe::launch_decode_gemm1_routed(g1, logits, 1, ra, E, k, ids, tw, counts, s);
    if (e != hipSuccess) return hip_status(e, "gemm1 (routed)");
    moe::GemmArgs g2 = gemm_args(a, w2, w2_scale, y, tw, sorted, eids, ntpp, T, H, I, ES, KS,
                                 p.bm);
    g2.max_rows = 1;
    e = moe::launch_gemm2(g2, true, MOE_VARIANT_DECODE, s);
    if (e != hipSuccess) return hip_status(e, "gemm2");
    return hip_status(moe::launch_combine(y, T, H, KS, true, out, s), "combine");
  }
  if (!p.fused_route_align && moe::route_fused_ok(T, H, E, bf16_acts(dt))) {
    // prefill: logits and top-k in one launch, then the align table
    e = moe::launch_route_fused(x, wg, T, H, E, k, ra, ids, tw, nullptr, s);
    if (e != hipSuccess) return hip_status(e, "router");
    e = moe::launch_align(ids, T * KS, ES, p.bm, p.cap, sorted, eids, ntpp, counts,
                          reinterpret_cast<int32_t*>(b + p.off_align), expert_map, s, runs);
    if (e != hipSuccess) return hip_status(e, "align");
    return forward_impl(x, w13, w13_scale, w2, w2_scale, tw, sorted, eids, ntpp, T, H, I, ES, KS,
                        p.bm, dt, MOE_VARIANT_AUTO, out, b + p.off_fwd,
                        forward_ws_full(T, H, I, ES, KS, dt), stream, T, runs);
  }
  e = moe::launch_router_logits(x, wg, T, H, E, bf16_acts(dt), logits, s);
  if (e != hipSuccess) return hip_status(e, "router logits");
  if (p.fused_route_align) {
    e = moe::launch_route_align_small(logits, p.nz, nullptr, T, E, k, ra, ids, tw, p.bm, p.cap,
                                      sorted, eids, ntpp, counts, expert_map, s);
    if (e != hipSuccess) return hip_status(e, "route+align");
  } else {
    e = moe::launch_topk(logits, p.nz, nullptr, T, E, k, ra, ids, tw, s);
    if (e != hipSuccess) return hip_status(e, "top-k");
    e = moe::launch_align(ids, T * KS, ES, p.bm, p.cap, sorted, eids, ntpp, counts,
                          reinterpret_cast<int32_t*>(b + p.off_align), expert_map, s, runs);
    if (e != hipSuccess) return hip_status(e, "align");
  }
  return forward_impl(x, w13, w13_scale, w2, w2_scale, tw, sorted, eids, ntpp, T, H, I, ES, KS,
                      p.bm, dt, MOE_VARIANT_AUTO, out, b + p.off_fwd,
                      forward_ws_full(T, H, I, ES, KS, dt), stream,
                      T,    // the router's k experts of a token are distinct
                      p.fused_route_align ? nullptr : runs);
}

}  // namespace

extern "C" {

moe_status moe_layer(const void* x, const void* wg, const void* w13, const void* w2,
                     const moe_route_cfg* cfg, int T, int H, int I, int E, int k, moe_dtype dt,
                     void* out, int32_t* topk_ids_out, float* topk_w_out, void* ws,
                     size_t ws_bytes, void* stream) {
  return layer_impl(x, wg, w13, nullptr, w2, nullptr, nullptr, cfg, T, H, I, E, k, dt, out,
                    topk_ids_out, topk_w_out, ws, ws_bytes, stream);
}

moe_status moe_layer_fp8(const void* x, const void* wg, const uint8_t* w13,
                         const float* w13_scale, const uint8_t* w2, const float* w2_scale,
                         const moe_route_cfg* cfg, int T, int H, int I, int E, int k, void* out,
                         int32_t* topk_ids_out, float* topk_w_out, void* ws, size_t ws_bytes,
                         void* stream) {
  if (!w13_scale || !w2_scale) return fail(MOE_ERR_INVALID_ARG, "NULL scale pointer");
  return layer_impl(x, wg, w13, w13_scale, w2, w2_scale, nullptr, cfg, T, H, I, E, k,
                    MOE_BF16_FP8W, out, topk_ids_out, topk_w_out, ws, ws_bytes, stream);
}

size_t moe_layer_shared_workspace_size(int T, int H, int I, int E, int k, moe_dtype dt) {
  if (T <= 0 || H <= 0 || I <= 0 || E <= 0 || k < 1 || !valid_expert_dt(dt)) return 0;
  return plan_layer(T, H, I, E, k, dt, 1).total;
}

moe_status moe_layer_shared(const void* x, const void* wg, const void* w13,
                            const float* w13_scale, const void* w2, const float* w2_scale,
                            const moe_route_cfg* cfg, int T, int H, int I, int E, int k,
                            moe_dtype dt, void* out, int32_t* topk_ids_out, float* topk_w_out,
                            void* ws, size_t ws_bytes, void* stream) {
  return layer_impl(x, wg, w13, w13_scale, w2, w2_scale, nullptr, cfg, T, H, I, E, k, dt, out,
                    topk_ids_out, topk_w_out, ws, ws_bytes, stream, 1);
}

moe_status moe_layer_ep(const void* x, const void* wg, const void* w13, const float* w13_scale,
                        const void* w2, const float* w2_scale, const int32_t* expert_map,
                        const moe_route_cfg* cfg, int T, int H, int I, int E, int k,
                        moe_dtype dt, void* out, int32_t* topk_ids_out, float* topk_w_out,
                        void* ws, size_t ws_bytes, void* stream) {
  if (!expert_map) return fail(MOE_ERR_INVALID_ARG, "expert_map is NULL");
  return layer_impl(x, wg, w13, w13_scale, w2, w2_scale, expert_map, cfg, T, H, I, E, k, dt, out,
                    topk_ids_out, topk_w_out, ws, ws_bytes, stream);
}

}  // extern "C"

// ------------------------------------------------------------------ allocation-free layer
// The workspace of moe_layer_noalloc: a device array of the library, one per GPU (each
// device that runs the entry point holds its copy until the process ends).  Its name is
// a host-side stand-in; the device address of the current device's copy comes from
// hipGetSymbolAddress, taken once per device on that device's first call.
constexpr size_t kNoallocScratchBytes = static_cast<size_t>(96) << 20;
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

moe_status scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_layer_noalloc(const void* x, const void* wg, const void* w13, const void* w2,
                             const moe_route_cfg* cfg, int T, int H, int I, int E, int k,
                             moe_dtype dt, void* out, int32_t* topk_ids_out, float* topk_w_out,
                             void* stream) {
  if (dt == MOE_BF16_FP8W)
    return fail(MOE_ERR_UNSUPPORTED, "moe_layer_noalloc takes bf16 or fp32 expert weights");
  const size_t need = moe_layer_workspace_size(T, H, I, E, k, dt);
  if (T > 0 && need == 0) return fail(MOE_ERR_INVALID_ARG, "invalid sizes or dtype");
  if (need > kNoallocScratchBytes)
    return fail(MOE_ERR_WORKSPACE,
                "moe_layer_noalloc: this layer needs %zu bytes of workspace, above the %zu-byte "
                "static scratch (use moe_layer with a caller workspace)",
                need, kNoallocScratchBytes);
  void* ws = nullptr;
  if (T > 0) {
    const moe_status st = scratch_of_current_device(&ws);
    if (st != MOE_OK) return st;
  }
  return layer_impl(x, wg, w13, nullptr, w2, nullptr, nullptr, cfg, T, H, I, E, k, dt, out,
                    topk_ids_out, topk_w_out, ws, kNoallocScratchBytes, stream);
}

}  // extern "C"
