"""Helpers shared by the GPU tests: host copies, oracle calls and the comparisons."""
from __future__ import annotations

import numpy as np
import torch

from oracle import moe_oracle as O


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def route_kwargs(wl, lay):
    kw = dict(n_group=wl.n_group, topk_group=wl.topk_group, scaling=wl.scaling)
    kw["offset"] = None if lay.offset is None else lay.offset.cpu().numpy()
    kw["bias"] = None if lay.bias is None else lay.bias.cpu().numpy()
    return kw


def lib_cfg(lib, wl, lay):
    return lib.route_cfg(wl.mode, logit_offset=lay.offset, select_bias=lay.bias,
                         n_group=wl.n_group, topk_group=wl.topk_group,
                         routed_scaling=wl.scaling)


def bf16_tol_check(got: np.ndarray, ref: np.ndarray, tol=2e-2, kernel_ref=None, kernel_c=1e-4):
    """bf16 output checks over every element.

    * The stated tolerance against the float64 oracle, on what the result adds beyond a
      correctly rounded bf16 output: |got - ref| <= |bf16(ref) - ref| + tol * RMS(ref).
      Half a bf16 ulp is 2^-6 RMS for outputs between 4 and 8 RMS and 2^-5 RMS above, so
      a raw max|got - ref| <= tol * RMS cannot hold at such outliers even for an exact
      result; the raw ratio is returned and reported beside it.
    * With ``kernel_ref`` (the oracle's GEMM2 x weight + combine run on the GPU's own SwiGLU
      activations a, so the two sides start from the same bf16 values): the error the
      expert GEMM2, any split of its K range and the combine add beyond the output's one
      rounding, |got - kernel_ref| <= |bf16(kernel_ref) - kernel_ref| + kernel_c * RMS(ref).
      The GPU rounds its fp32 result g once, so |bf16(g) - r| <= |bf16(r) - r| + 2|g - r|:
      the slack is twice GEMM2's fp32 accumulation error, a few 1e-6 of RMS.
    Returns (raw max|got - ref| / RMS, |ref| at that element / RMS)."""
    rms = float(np.sqrt(np.mean(ref * ref)))
    d = np.abs(got - ref)
    i = int(np.argmax(d))
    ratio = float(d.flat[i] / rms)
    beyond = (d - np.abs(O.bf16_round(ref) - ref)) / rms
    j = int(np.argmax(beyond))
    assert beyond.flat[j] <= tol, (
        f"error beyond the output rounding {beyond.flat[j]:.3e} RMS > {tol} (|ref|/RMS "
        f"{abs(ref.flat[j]) / rms:.2f}; raw max|d|/RMS {ratio:.3e})")
    if kernel_ref is not None:
        excess = (np.abs(got - kernel_ref) - np.abs(O.bf16_round(kernel_ref) - kernel_ref)) / rms
        k = int(np.argmax(excess))
        assert excess.flat[k] <= kernel_c, (
            f"GEMM2 + combine error beyond the output rounding {excess.flat[k]:.3e} RMS > "
            f"{kernel_c} (|ref|/RMS {abs(ref.flat[k]) / rms:.2f})")
    return ratio, abs(ref.flat[i]) / rms


def swiglu_flip_check(a_gpu: np.ndarray, a64: np.ndarray, rows: np.ndarray, max_frac=1e-2):
    """GEMM1's bf16 activations against the exact SwiGLU values: the GPU rounds an fp32 value
    whose accumulation error is ~1e-6 relative, so a small fraction of elements lying that
    close to a rounding tie come out as the other bf16 neighbour of the exact value.  A
    wrong rounding mode or a wrong operand would move most of them.  Returns the fraction."""
    g = a_gpu[rows]
    r = O.bf16_round(a64[rows])
    frac = float(np.mean(g != r)) if g.size else 0.0
    assert frac <= max_frac, f"{frac:.4f} of the SwiGLU activations differ from the rounded exact values"
    return frac


def f32_tol_check(got: np.ndarray, ref: np.ndarray, tol=1e-5):
    """Normwise relative error ||got - ref||_inf / ||ref||_inf <= tol."""
    r = float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-300))
    assert r <= tol, f"normwise relative error {r:.3e} > {tol}"
    return r


def logit_error_bound(x64: np.ndarray, wg64: np.ndarray) -> np.ndarray:
    """Per-token bound on |fp32-accumulated logit - exact logit| for a K-term dot product of
    exactly representable products: K * 2^-24 * sum_h |x_h w_h| (max over experts)."""
    K = x64.shape[1]
    s = np.abs(x64) @ np.abs(wg64).T
    return K * 2.0 ** -24 * s.max(axis=1) + 1e-30


def compact_experts(ids: np.ndarray, w13, w2):
    """Host float64 copies of only the experts used by ``ids``, with ids relabelled."""
    used = sorted(set(int(v) for v in ids.reshape(-1)))
    remap = {e: i for i, e in enumerate(used)}
    ids_c = np.vectorize(remap.get)(ids).astype(np.int32)
    w13c = np.stack([np64(w13[e]) for e in used])
    w2c = np.stack([np64(w2[e]) for e in used])
    return ids_c, w13c, w2c


DTYPE_CODE = {"f32": 0, "bf16": 1, "bf16_fp8w": 2}


def bf16_layer(wl) -> bool:
    """bf16 activations (bf16 weights, or FP8 weights with bf16 activations)."""
    return wl.dtype in ("bf16", "bf16_fp8w")


def run_layer(lib, lay, k, cfg, **kw):
    """moe_layer, or moe_layer_fp8 when the layer's expert weights are E4M3 codes."""
    if lay.w13_scale is not None:
        return lib.moe_layer_fp8(lay.x, lay.wg, lay.w13, lay.w13_scale, lay.w2, lay.w2_scale, k,
                                 cfg, **kw)
    return lib.moe_layer(lay.x, lay.wg, lay.w13, lay.w2, k, cfg, **kw)


def expert_weights64(lay, experts=None):
    """Host float64 expert weights (decoded and scaled for FP8 layers), optionally only
    the listed experts, in that order."""
    if lay.w13_scale is None:
        if experts is None:
            return np64(lay.w13), np64(lay.w2)
        return (np.stack([np64(lay.w13[e]) for e in experts]),
                np.stack([np64(lay.w2[e]) for e in experts]))
    idx = torch.tensor(list(range(lay.w13.shape[0])) if experts is None else list(experts),
                       device=lay.w13.device)
    w13 = O.dequant_rows(lay.w13.index_select(0, idx).cpu().numpy(),
                         lay.w13_scale.index_select(0, idx).cpu().numpy())
    w2 = O.dequant_rows(lay.w2.index_select(0, idx).cpu().numpy(),
                        lay.w2_scale.index_select(0, idx).cpu().numpy())
    return w13, w2


def score_error_bound(logit_bound: np.ndarray, mode: int, logits32, offset=None, bias=None):
    """Per-token bound on how far the GPU's selection scores can sit from the oracle's when
    their logits differ by at most ``logit_bound``: the softmax rules compare the logits
    (+ offset, one float32 rounding each side); the sigmoid rule compares
    fl32(fl32(sigmoid(l)) + bias), and sigmoid's slope is at most 1/4 (two float32
    roundings each side)."""
    sc = O.selection_scores(logits32, mode, offset, bias)
    ulp = 2.0 ** -23 * np.abs(sc).max(axis=1)
    if mode == O.SIGMOID_BIAS_GROUPED:
        return logit_bound / 4 + 2 * ulp + 2.0 ** -24
    return logit_bound + 2 * ulp


def same_set(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Per token: the same experts selected (slot order aside)."""
    return np.all(np.sort(a, axis=1) == np.sort(b, axis=1), axis=1)


def routing_vs_oracle(wl, lay, gids, k=None):
    """Oracle routing from float64 logits rounded to float32, and which tokens the GPU
    may route differently.  Asserts that every token the GPU routed to another set of
    experts lies within its selection margin of a tie.  Returns (rid, rw, same)."""
    k = wl.k if k is None else k
    x64, wg64 = np64(lay.x), np64(lay.wg)
    logits32 = O.router_logits(x64, wg64).astype(np.float32)
    kw = route_kwargs(wl, lay)
    rid, rw = O.route(logits32, k, wl.mode, **kw)
    margin = O.selection_margin(logits32, k, wl.mode, kw["offset"], kw["bias"], wl.n_group,
                                wl.topk_group)
    sb = score_error_bound(logit_error_bound(x64, wg64), wl.mode, logits32, kw["offset"],
                           kw["bias"])
    same = same_set(gids[:, :k], rid)
    bad = ~same & (margin > sb)
    assert not bad.any(), f"{int(bad.sum())} tokens routed differently with a clear margin"
    return rid, rw, same


def layer_check(lib, wl, lay, out, gids, gw):
    """A layer's output (moe_layer / _fp8 / _shared, whose routing the GPU returned as gids,
    gw) against the oracle on every element:
    * the GPU's routing differs from the oracle's only within the selection margin;
    * spec: the oracle's per-expert math (float64, a rounded to bf16 for bf16 layers) with
      the oracle's weights, on the GPU's routing where the two differ (near ties);
    * GEMM1: the SwiGLU activations the same kernels compute (recomputed through the stage
      entry points with the layer's block_m and variant) round to the exact values but
      for a small fraction near ties;
    * GEMM2 + combine: the output against the oracle's GEMM2 x weight + combine on those
      activations and the GPU's weights (bf16_tol_check's kernel check).
    Expert weights are converted to float64 a few experts at a time."""
    bf16 = bf16_layer(wl)
    T, H = lay.x.shape
    k = wl.k
    KS = gids.shape[1]                     # k, or k + 1 with the shared slot
    E_all = lay.w13.shape[0]
    I = lay.w13.shape[1] // 2
    rid, rw, same = routing_vs_oracle(wl, lay, gids, k=k)
    if KS > k:                             # the shared slot: expert E, weight 1
        rid, rw = O.add_shared_slot(rid, rw, wl.E)
    # oracle weights in the GPU's slot order where the sets agree, the GPU's elsewhere
    ref_w = gw.copy()
    for t in np.nonzero(same)[0]:
        pos = {int(e): j for j, e in enumerate(rid[t])}
        ref_w[t] = [rw[t, pos[int(e)]] for e in gids[t]]
    assert same.mean() > 0.5
    # the layer's activations, recomputed by the stage entry points
    dt = DTYPE_CODE[wl.dtype]
    bm = lib.moe_preferred_block_m(T, wl.H, I, E_all, KS, dt)
    sorted_ids, expert_ids, ntpp, _ = lib.moe_align(torch.from_numpy(gids).to(lay.x.device), E_all, bm)
    if lay.w13_scale is not None:
        a = lib.moe_gemm1_swiglu_fp8(lay.x, lay.w13, lay.w13_scale, sorted_ids, expert_ids, ntpp,
                                     KS, bm, 0)
    else:
        a = lib.moe_gemm1_swiglu(lay.x, lay.w13, sorted_ids, expert_ids, ntpp, KS, bm, 0)
    torch.cuda.synchronize()
    a_gpu = np64(a)
    del a
    x64 = np64(lay.x)
    used = sorted(set(int(v) for v in gids.reshape(-1)))
    per = (lay.w13[0].numel() + lay.w2[0].numel()) * 8
    step = max(1, int((6 << 30) // per))
    ref = np.zeros((T, H))
    kref = np.zeros((T, H))
    flips, nel = 0.0, 0
    for c0 in range(0, len(used), step):
        chunk = used[c0:c0 + step]
        emap = np.full(E_all, -1, np.int64)
        emap[chunk] = np.arange(len(chunk))
        loc = emap[gids]
        w13c, w2c = expert_weights64(lay, chunk)
        a64 = O.swiglu_rows(x64, w13c, loc)
        rows = np.nonzero(loc.reshape(-1) >= 0)[0]
        if bf16:
            f = swiglu_flip_check(a_gpu, a64, rows)
            flips += f * rows.size
            nel += rows.size
        ref += O.down_and_combine(O.bf16_round(a64) if bf16 else a64, w2c, loc, ref_w)
        kref += O.down_and_combine(a_gpu, w2c, loc, gw)
        del w13c, w2c, a64
    got = np64(out)
    if bf16:
        r, _ = bf16_tol_check(got, ref, kernel_ref=kref)
    else:
        r = f32_tol_check(got, ref)
    return r, float(same.mean()), (flips / nel if nel else 0.0)


def layer_reference(lay, ids, w, round_a, max_bytes=6 << 30):
    """The oracle's per-expert loop over the whole layer, for every token, with the given
    routing.  Expert weights are converted to float64 a few experts at a time: each chunk
    is one expert-parallel share (moe_loop_ep, pinned to sum to moe_loop), summed."""
    x64 = np64(lay.x)
    T, H = x64.shape
    E_all = lay.w13.shape[0]
    used = sorted(set(int(v) for v in np.asarray(ids).reshape(-1)))
    per = (lay.w13[0].numel() + lay.w2[0].numel()) * 8
    step = max(1, int(max_bytes // per))
    out = np.zeros((T, H))
    for c0 in range(0, len(used), step):
        chunk = used[c0:c0 + step]
        emap = np.full(E_all, -1, np.int32)
        emap[chunk] = np.arange(len(chunk), dtype=np.int32)
        w13c, w2c = expert_weights64(lay, chunk)
        out += O.moe_loop_ep(x64, w13c, w2c, ids, w, emap, round_a=round_a)
        del w13c, w2c
    return out
