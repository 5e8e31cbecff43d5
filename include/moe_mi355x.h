/*
 * moe_mi355x.h -- C ABI of a fused top-k Mixture-of-Experts SwiGLU FFN layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (definition: "Mixture-of-Experts Kernels: Routing, Permutation, and
 * Grouped GEMM", section 1; data flow: section 2):
 *
 *   logits = x . Wg^T                      router GEMM, fp32            (moe_route)
 *   (topk_ids, topk_w) = rule(logits)      softmax/sigmoid + top-k      (moe_route)
 *   sorted_ids, expert_ids, padded total   histogram/pad/scan/scatter   (moe_align)
 *   a[r] = silu(x[r/k] W1[e]^T) * (x[r/k] W3[e]^T)   gathered GEMM1     (moe_gemm1_swiglu)
 *   y[r] = topk_w[r] * a[r] W2[e]^T                  GEMM2 x weight     (moe_gemm2_weighted)
 *   out[t] = sum_j y[t*k + j]                        combine            (moe_combine)
 *
 * where r = t*k + j is the flat routed row of token t, slot j, and e = topk_ids[t][j].
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers owned by the caller; the library
 *   allocates nothing, frees nothing and keeps no device state between calls.
 * - `stream` is a hipStream_t (NULL = the legacy default stream).  Every call only
 *   enqueues kernels on it: no host<->device copy, no synchronisation, no
 *   decision that depends on device data, so every call can be captured in a
 *   HIP graph.  The library is thread-safe and reentrant.
 * - Arguments are validated on the host before anything is enqueued.  On any
 *   error nothing is enqueued, outputs are untouched, and moe_last_error()
 *   returns a thread-local message.  A failed kernel launch returns MOE_ERR_HIP.
 * - Not checked on the device (preconditions): topk_ids values lie in [0, E)
 *   (moe_align skips, and counts nowhere, any that do not; see there) and each
 *   token's k ids are distinct (both hold for ids from moe_route);
 *   sorted_ids / expert_ids / num_tokens_post_padded come from moe_align with the
 *   same T, k, E, block_m.
 * - Layouts (row-major, "nn.Linear" [out, in] weights, section 11 of the
 *   routing/grouped GEMM page):  x [T,H];  Wg [E,H];  W13 [E,2I,H] whose rows
 *   0..I-1 are the gate projection W1[e] and rows I..2I-1 the up projection W3[e];
 *   W2 [E,H,I];  topk_ids [T,k] int32;  topk_w [T,k] fp32;  out [T,H].
 * - Element types: MOE_BF16 means x, Wg, W13, W2 and out are bf16 and the SwiGLU
 *   activation a is stored as bf16 (it is GEMM2's input); MOE_F32 means all of
 *   them are fp32.  Accumulation is fp32 in both; logits, topk_w and y are fp32.
 *   MOE_BF16_FP8W is MOE_BF16 with FP8 expert weights (the *_fp8 entry points):
 *   W13 and W2 hold one OCP E4M3 byte per weight (sign, 4 exponent bits with bias
 *   7, 3 mantissa bits; no infinities; 0x7F/0xFF are NaN) and come with fp32
 *   per-row scales W13_scale [E,2I] and W2_scale [E,H]; the weight used is
 *   decode(code[e,n,:]) * scale[e,n] (section 8 of the routing/grouped GEMM page
 *   prices an expert's weights at one byte each; section 9 lists FP8 weight
 *   variants).  The decoded values are exact in bf16, the products are accumulated
 *   in fp32 and the row scale multiplies the accumulator.
 * - Limits: 1 <= k <= 16, k <= E <= 512, T >= 0, T*k < 2^31; for MOE_BF16, H and I
 *   are multiples of 64 (128 for MOE_BF16_FP8W); x, W13, W2, out, a and y 16-byte
 *   aligned.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,   /* null/misaligned pointer, size out of range, bad mode */
  MOE_ERR_UNSUPPORTED = -2,   /* valid request outside this build's limits            */
  MOE_ERR_WORKSPACE = -3,     /* workspace pointer NULL or smaller than required      */
  MOE_ERR_HIP = -4            /* a HIP call failed (launch error)                     */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_BF16_FP8W = 2 } moe_dtype;

/* Routing rules ("Mixture-of-Experts Kernels: Routing, Permutation, and Grouped GEMM",
 * section 1 model table, section 3 `route`, section 4 grouped router). */
typedef enum {
  /* softmax over all E logits, top-k, weights renormalised to sum to 1 (Mixtral, Qwen3) */
  MOE_ROUTE_SOFTMAX_TOPK_RENORM = 0,
  /* top-k logits first, then softmax over those k (gpt-oss)                             */
  MOE_ROUTE_TOPK_THEN_SOFTMAX = 1,
  /* s = sigmoid(logit); c = s + select_bias chooses; groups of E/n_group contiguous
   * experts are scored by the sum of their two largest c, the best topk_group groups
   * stay eligible, top-k by c inside them; weights = routed_scaling * s / sum(s) over
   * the chosen experts, from the UNBIASED s (DeepSeek-V3)                              */
  MOE_ROUTE_SIGMOID_BIAS_GROUPED = 2
} moe_route_mode;

typedef struct {
  int32_t mode;               /* moe_route_mode                                          */
  const float* logit_offset;  /* device [E] or NULL: added (fp32) to every logit before   *
                               * selection and weighting                                  */
  const float* select_bias;   /* device [E] or NULL: mode 2 only, selection-only bias     */
  int32_t n_group;            /* mode 2: number of groups (divides E); 0 = no grouping    */
  int32_t topk_group;         /* mode 2: groups kept; 0 = no grouping                     */
  float routed_scaling;       /* mode 2: weight scale (2.5 for DeepSeek-V3); else ignored */
} moe_route_cfg;

/* ---------------------------------------------------------------------------------- */
/* Router.  Computes logits = x . Wg^T in fp32 and applies cfg's rule.
 *   topk_ids [T,k] int32: chosen experts, slot j in selection order (descending
 *            selection score, ties to the lower expert index; groups likewise).
 *   topk_w   [T,k] fp32: router weights of those slots.
 *   logits_out [T,E] fp32 or NULL: the raw x . Wg^T (before logit_offset).
 *   ws: scratch of at least moe_route_workspace_size(T,H,E,dt) bytes, always
 *       required: it holds the logits (for bf16 at T <= 64, the partial logits of
 *       the K-split router GEMM, added in a fixed order, so results stay
 *       deterministic).  logits_out, when given, receives a copy of the summed logits.
 * Selection decisions are taken on fp32 values: (logit + offset) for modes 0/1;
 * for mode 2 on c = s + bias with s = sigmoid(logit+offset) rounded to nearest fp32
 * and group scores c_a + c_b in fp32. */
moe_status moe_route(const void* x, const void* wg, int T, int H, int E, int k, moe_dtype dt,
                     const moe_route_cfg* cfg, int32_t* topk_ids, float* topk_w,
                     float* logits_out, void* ws, size_t ws_bytes, void* stream);
size_t moe_route_workspace_size(int T, int H, int E, moe_dtype dt);

/* The selection/weighting half of moe_route on caller-supplied fp32 logits [T,E]
 * (the same device code as moe_route's epilogue). */
moe_status moe_route_from_logits(const float* logits, int T, int E, int k,
                                 const moe_route_cfg* cfg, int32_t* topk_ids, float* topk_w,
                                 void* stream);

/* ---------------------------------------------------------------------------------- */
/* Align ("Mixture-of-Experts Kernels: ...", section 5; "fused-moe-kernel", Core
 * Technique).  From topk_ids [T,k] builds the block-aligned indirection table:
 *   expert_counts[e]  = n_e, rows routed to e (optional output, may be NULL);
 *   padded_e          = ceil(n_e / block_m) * block_m;  start_e = exclusive scan;
 *   *num_tokens_post_padded = total = sum_e padded_e;
 *   sorted_ids[start_e + i] = the i-th flat row r (ascending r) with topk_ids = e, and
 *                           the sentinel T*k on the padding positions and on the tail
 *                           [total, cap);
 *   expert_ids[p]      = expert owning rows [p*block_m, (p+1)*block_m) for p < total/
 *                           block_m (empty experts own no tile), -1 on [total/block_m,
 *                           cap/block_m).
 * Buffers are sized for the worst case cap = moe_align_capacity(T,k,E,block_m), so the
 * call is graph-capturable; the result is bit-exact and deterministic.
 * block_m: a power of two in [1, 256].  ws: moe_align_workspace_size(...) bytes.
 * Ids outside [0, E) (possible only for caller-supplied ids) are skipped on the device:
 * such a row is counted for no expert and appears in no tile, the rest of the table is
 * built as if it were absent, and no memory outside the buffers is touched; the host
 * detects it afterwards as sum(expert_counts) < T*k (the expert GEMMs then leave that
 * row of a/y unwritten, so its token's output is not defined). */
int64_t moe_align_capacity(int T, int k, int E, int block_m);
size_t moe_align_workspace_size(int T, int k, int E, int block_m);
moe_status moe_align(const int32_t* topk_ids, int T, int k, int E, int block_m,
                     int32_t* sorted_ids, int32_t* expert_ids,
                     int32_t* num_tokens_post_padded, int32_t* expert_counts,
                     void* ws, size_t ws_bytes, void* stream);

/* Align for one GPU of an expert-parallel layer (section 11 exercise of the routing/
 * grouped GEMM page: experts not on this GPU get expert_ids = -1 and the GEMMs skip
 * their tiles).  expert_map [E] int32 (device, not NULL): expert_map[e] is e's index
 * among this GPU's experts, or -1 when another GPU holds it.  The table is moe_align's
 * (same sorted_ids, total and counts) with each tile's owner e replaced by
 * expert_map[e].  Precondition (not checked on the device): the values are -1 or in
 * [0, E_local), E_local being the number of experts in the weights the GEMMs get. */
moe_status moe_align_ep(const int32_t* topk_ids, int T, int k, int E, int block_m,
                        const int32_t* expert_map, int32_t* sorted_ids, int32_t* expert_ids,
                        int32_t* num_tokens_post_padded, int32_t* expert_counts, void* ws,
                        size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------- */
/* Expert computation ("Mixture-of-Experts Kernels: ...", section 6).
 * Tiles past the device-side padded total exit at once; sentinel rows are never
 * stored; tiles of an expert with no rows do not exist, so its weights are never
 * read.  E is the expert count the table was built for (it sizes the grids through
 * the table's capacity).  Weights are indexed by the table's expert ids: with a
 * moe_align_ep table E is the global count while the weights hold this GPU's experts
 * only ([E_local, ...]); tiles marked -1 are skipped by GEMM1
 * and GEMM2 writes zeros into their rows of y, so the combine yields this GPU's share
 * (the shares of GPUs whose maps partition the experts add up to the layer). */

/* Variant of the expert GEMMs: 0 = automatic (from T, k, E, H, I on the host),
 * 1 = prefill (MFMA tiles staged through LDS), 2 = decode (weight streaming, small M).
 * bf16 block_m limits: prefill >= 32, decode >= 16 (MOE_ERR_UNSUPPORTED otherwise);
 * fp32 takes any block_m (16 x 64 MFMA tiles when block_m is a multiple of 16, one
 * thread per output below that).  FP8 weights: prefill block_m >= 128, decode >= 16.  The
 * decode variant takes tables of at most 65536 rows (moe_align_capacity), larger
 * requests are MOE_ERR_UNSUPPORTED. */
enum { MOE_VARIANT_AUTO = 0, MOE_VARIANT_PREFILL = 1, MOE_VARIANT_DECODE = 2 };

/* block_m that moe_forward's automatic variant wants moe_align to use (0 when T < 0,
 * E < 1, k < 1 or dt is not a moe_dtype). */
int moe_preferred_block_m(int T, int H, int I, int E, int k, moe_dtype dt);
/* The variant moe_forward will run for these sizes (1 or 2; 0 for invalid sizes as
 * above). */
int moe_auto_variant(int T, int H, int I, int E, int k, moe_dtype dt);

/* GEMM1 + SwiGLU: a[r, :] (dtype dt, [T*k, I]) for every non-sentinel row r of the
 * table; rows never routed are left untouched. */
moe_status moe_gemm1_swiglu(const void* x, const void* w13, const int32_t* sorted_ids,
                            const int32_t* expert_ids, const int32_t* num_tokens_post_padded,
                            int T, int H, int I, int E, int k, int block_m, moe_dtype dt,
                            int variant, void* a, void* stream);

/* GEMM2 x router weight: y[r, :] = topk_w[r] * a[r] . W2[e]^T (fp32, [T*k, H]). */
moe_status moe_gemm2_weighted(const void* a, const void* w2, const float* topk_w,
                              const int32_t* sorted_ids, const int32_t* expert_ids,
                              const int32_t* num_tokens_post_padded, int T, int H, int I,
                              int E, int k, int block_m, moe_dtype dt, int variant, float* y,
                              void* stream);

/* The same two GEMMs with FP8 expert weights (dtype MOE_BF16_FP8W: x and a bf16).
 * w13 / w2: E4M3 bytes [E,2I,H] / [E,H,I]; w13_scale [E,2I], w2_scale [E,H] fp32
 * (device, 4-byte aligned; a NULL scale is MOE_ERR_INVALID_ARG).  block_m limits as
 * above (prefill >= 128, decode >= 16). */
moe_status moe_gemm1_swiglu_fp8(const void* x, const uint8_t* w13, const float* w13_scale,
                                const int32_t* sorted_ids, const int32_t* expert_ids,
                                const int32_t* num_tokens_post_padded, int T, int H, int I,
                                int E, int k, int block_m, int variant, void* a, void* stream);
moe_status moe_gemm2_weighted_fp8(const void* a, const uint8_t* w2, const float* w2_scale,
                                  const float* topk_w, const int32_t* sorted_ids,
                                  const int32_t* expert_ids,
                                  const int32_t* num_tokens_post_padded, int T, int H, int I,
                                  int E, int k, int block_m, int variant, float* y,
                                  void* stream);

/* Combine: out[t, :] = sum_{j<k} y[t*k + j, :] in slot order (fp32), rounded once to
 * dt.  Every routed row of y must have been written. */
moe_status moe_combine(const float* y, int T, int H, int k, moe_dtype dt, void* out,
                       void* stream);

/* GEMM1+SwiGLU, GEMM2 x weight and combine.  ws: moe_forward_workspace_size bytes
 * (holds a and y; when the automatic variant is prefill, also 64 MiB of
 * partial sums for GEMM2's split last round of tiles).  A workspace that holds a and y
 * but not the partial sums is accepted: GEMM2 then runs its tiles unsplit. */
size_t moe_forward_workspace_size(int T, int H, int I, int E, int k, moe_dtype dt);
moe_status moe_forward(const void* x, const void* w13, const void* w2, const float* topk_w,
                       const int32_t* sorted_ids, const int32_t* expert_ids,
                       const int32_t* num_tokens_post_padded, int T, int H, int I, int E,
                       int k, int block_m, moe_dtype dt, int variant, void* out, void* ws,
                       size_t ws_bytes, void* stream);

/* moe_forward with FP8 expert weights (workspace: moe_forward_workspace_size with
 * MOE_BF16_FP8W). */
moe_status moe_forward_fp8(const void* x, const uint8_t* w13, const float* w13_scale,
                           const uint8_t* w2, const float* w2_scale, const float* topk_w,
                           const int32_t* sorted_ids, const int32_t* expert_ids,
                           const int32_t* num_tokens_post_padded, int T, int H, int I, int E,
                           int k, int block_m, int variant, void* out, void* ws,
                           size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------- */
/* The whole layer: route -> align (block_m = moe_preferred_block_m) -> forward.
 * topk_ids_out / topk_w_out ([T,k]) optionally receive the routing; when NULL the
 * routing lives in the workspace.  ws: moe_layer_workspace_size bytes. */
size_t moe_layer_workspace_size(int T, int H, int I, int E, int k, moe_dtype dt);
moe_status moe_layer(const void* x, const void* wg, const void* w13, const void* w2,
                     const moe_route_cfg* cfg, int T, int H, int I, int E, int k, moe_dtype dt,
                     void* out, int32_t* topk_ids_out, float* topk_w_out, void* ws,
                     size_t ws_bytes, void* stream);
/* moe_layer for callers that cannot allocate memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid it): the same launches, with the workspace taken
 * from a static device array of the library (96 MiB per GPU, held until the process ends;
 * enough for the DeepSeek-V3-shaped decode layer up to T = 256).  x, wg, w13, w2, out and
 * the optional routing outputs are as for moe_layer (bf16 or fp32; no FP8 weights).
 * Returns MOE_ERR_WORKSPACE, enqueuing nothing, when moe_layer_workspace_size(...) exceeds
 * 96 MiB.  Calls no allocating routine.  Every call on one GPU uses that GPU's one array,
 * so calls that overlap on a GPU (other streams, other threads) race; no kernel of the
 * layer reads workspace it has not written in the same call, so nothing is cleared. */
moe_status moe_layer_noalloc(const void* x, const void* wg, const void* w13, const void* w2,
                             const moe_route_cfg* cfg, int T, int H, int I, int E, int k,
                             moe_dtype dt, void* out, int32_t* topk_ids_out, float* topk_w_out,
                             void* stream);
/* moe_layer with FP8 expert weights: x, Wg and out bf16; w13/w2 E4M3 bytes with their
 * per-row scales (as for moe_forward_fp8).  ws: moe_layer_workspace_size(...,
 * MOE_BF16_FP8W) bytes. */
moe_status moe_layer_fp8(const void* x, const void* wg, const uint8_t* w13,
                         const float* w13_scale, const uint8_t* w2, const float* w2_scale,
                         const moe_route_cfg* cfg, int T, int H, int I, int E, int k, void* out,
                         int32_t* topk_ids_out, float* topk_w_out, void* ws, size_t ws_bytes,
                         void* stream);

/* The layer with one shared expert (DeepSeek-V3, Kimi K2: routed experts "+1 shared",
 * section 1 table of the routing/grouped GEMM page): an always-on SwiGLU expert of the
 * routed experts' shape whose output every token adds with weight 1.  Wg [E,H] routes
 * over the E routed experts; w13 [E+1,2I,H] and w2 [E+1,H,I] hold the routed experts
 * followed by the shared one (index E; FP8 weights and scales [E+1,...] likewise).  The
 * shared expert is one more routing slot, so topk_ids_out / topk_w_out are [T, k+1]
 * with column k = (E, 1.0), the flat row is r = t*(k+1) + j, and align, the GEMMs and
 * the combine run on k+1 slots over E+1 experts.  k <= 15, E+1 <= 512.
 * ws: moe_layer_shared_workspace_size(T,H,I,E,k,dt) bytes. */
size_t moe_layer_shared_workspace_size(int T, int H, int I, int E, int k, moe_dtype dt);
moe_status moe_layer_shared(const void* x, const void* wg, const void* w13,
                            const float* w13_scale, const void* w2, const float* w2_scale,
                            const moe_route_cfg* cfg, int T, int H, int I, int E, int k,
                            moe_dtype dt, void* out, int32_t* topk_ids_out, float* topk_w_out,
                            void* ws, size_t ws_bytes, void* stream);

/* One GPU's share of an expert-parallel layer: route over all E experts (Wg [E,H] is
 * global), moe_align_ep with expert_map, then the expert GEMMs on this GPU's experts
 * (w13 [E_local,2I,H], w2 [E_local,H,I]) and the combine; out = the sum over the slots
 * whose experts are local.  dt: MOE_F32, MOE_BF16 (scales NULL) or MOE_BF16_FP8W (E4M3
 * weights with their row scales [E_local,2I] / [E_local,H]).  ws: moe_layer_workspace_size
 * (T,H,I,E,k,dt) bytes. */
moe_status moe_layer_ep(const void* x, const void* wg, const void* w13, const float* w13_scale,
                        const void* w2, const float* w2_scale, const int32_t* expert_map,
                        const moe_route_cfg* cfg, int T, int H, int I, int E, int k,
                        moe_dtype dt, void* out, int32_t* topk_ids_out, float* topk_w_out,
                        void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------- */
const char* moe_status_string(int status);
/* Detail of the last error on the calling thread ("" if none). */
const char* moe_last_error(void);
/* Library version string. */
const char* moe_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
