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


def bf16_tol_check(got: np.ndarray, ref: np.ndarray, tol=2e-2):
    """max|got - ref| / RMS(ref) <= tol.  Returns (ratio, |ref| at the worst element / RMS)."""
    rms = float(np.sqrt(np.mean(ref * ref)))
    d = np.abs(got - ref)
    i = int(np.argmax(d))
    ratio = float(d.flat[i] / rms)
    assert ratio <= tol, f"max|d|/RMS = {ratio:.3e} > {tol} (|ref|/RMS at worst = {abs(ref.flat[i]) / rms:.2f})"
    return ratio, abs(ref.flat[i]) / rms


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
