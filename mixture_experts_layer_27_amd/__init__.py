"""Python binding of libmoe_mi355x.so (fused top-k MoE SwiGLU layer for MI355X).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  torch supplies device memory (outputs and workspaces are allocated
here as torch tensors) and the current HIP stream.  The C entry points and their
contracts are declared in include/moe_mi355x.h; each function below has the same
name and forwards to it.
"""
from __future__ import annotations

import ctypes
import os

import torch

from ._lib import lib, LIB_PATH, MoeError, RouteCfg, check  # noqa: F401

F32, BF16, BF16_FP8W = 0, 1, 2
ROUTE_SOFTMAX_TOPK_RENORM, ROUTE_TOPK_THEN_SOFTMAX, ROUTE_SIGMOID_BIAS_GROUPED = 0, 1, 2
VARIANT_AUTO, VARIANT_PREFILL, VARIANT_DECODE = 0, 1, 2

__all__ = [
    "moe_route", "moe_route_from_logits", "moe_align", "moe_align_capacity",
    "moe_gemm1_swiglu", "moe_gemm2_weighted", "moe_combine", "moe_forward", "moe_layer",
    "moe_gemm1_swiglu_fp8", "moe_gemm2_weighted_fp8", "moe_forward_fp8", "moe_layer_fp8",
    "moe_align_ep", "moe_layer_ep", "moe_layer_shared", "moe_layer_noalloc",
    "moe_preferred_block_m", "moe_auto_variant", "moe_layer_workspace_size",
    "moe_forward_workspace_size", "moe_align_workspace_size", "moe_route_workspace_size",
    "route_cfg", "MoeError", "LIB_PATH",
]


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _p(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _fp8(w, scale, rows):
    """Check an FP8 expert weight (uint8 E4M3 codes [E, N, K]) and its fp32 row scales
    [E, N]."""
    if w.dtype != torch.uint8:
        raise TypeError("FP8 weights are uint8 tensors of E4M3 codes")
    if scale is None or scale.dtype != torch.float32 or tuple(scale.shape) != (w.shape[0], rows):
        raise ValueError(f"scale must be fp32 [{w.shape[0]}, {rows}]")
    return _p(w), _p(scale)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def route_cfg(mode: int, logit_offset=None, select_bias=None, n_group: int = 0,
              topk_group: int = 0, routed_scaling: float = 1.0) -> RouteCfg:
    """Build the moe_route_cfg struct (keeps references to the device tensors)."""
    c = RouteCfg()
    c.mode = int(mode)
    c.logit_offset = None if logit_offset is None else logit_offset.data_ptr()
    c.select_bias = None if select_bias is None else select_bias.data_ptr()
    c.n_group = int(n_group)
    c.topk_group = int(topk_group)
    c.routed_scaling = float(routed_scaling)
    c._keep = (logit_offset, select_bias)
    for t in (logit_offset, select_bias):
        if t is not None and (t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous()):
            raise ValueError("offset/bias must be contiguous fp32 GPU tensors")
    return c


def moe_route_workspace_size(T: int, H: int, E: int, dtype: int) -> int:
    return lib.moe_route_workspace_size(T, H, E, dtype)


def moe_route(x, wg, k, cfg: RouteCfg, logits_out=None):
    """-> (topk_ids int32 [T,k], topk_w fp32 [T,k]); fills logits_out [T,E] if given."""
    T, H = x.shape
    E = wg.shape[0]
    ids = torch.empty(T, k, dtype=torch.int32, device=x.device)
    w = torch.empty(T, k, dtype=torch.float32, device=x.device)
    ws = _ws(lib.moe_route_workspace_size(T, H, E, _dt(x)), x.device)
    check(lib.moe_route(_p(x), _p(wg), T, H, E, k, _dt(x), ctypes.byref(cfg), _p(ids), _p(w),
                        _p(logits_out), _p(ws), ws.numel(), _stream()), "moe_route")
    return ids, w


def moe_route_from_logits(logits, k, cfg: RouteCfg):
    T, E = logits.shape
    ids = torch.empty(T, k, dtype=torch.int32, device=logits.device)
    w = torch.empty(T, k, dtype=torch.float32, device=logits.device)
    check(lib.moe_route_from_logits(_p(logits), T, E, k, ctypes.byref(cfg), _p(ids), _p(w),
                                    _stream()), "moe_route_from_logits")
    return ids, w


def moe_align_capacity(T: int, k: int, E: int, block_m: int) -> int:
    return lib.moe_align_capacity(T, k, E, block_m)


def moe_align_workspace_size(T: int, k: int, E: int, block_m: int) -> int:
    return lib.moe_align_workspace_size(T, k, E, block_m)


def _reject_bad_ids(counts, T: int, k: int, strict: bool):
    """The library skips ids outside [0, E) and counts them for no expert: with ``strict``
    (outside HIP-graph capture) read the counts back and raise when rows are missing."""
    if not strict or torch.cuda.is_current_stream_capturing():
        return
    got = int(counts.cpu().sum())
    if got != T * k:
        raise ValueError(f"moe_align: {T * k - got} topk_ids outside [0, E) were skipped")


def moe_align(topk_ids, E: int, block_m: int, out=None, strict: bool = True):
    """-> (sorted_ids [cap], expert_ids [cap/block_m], num_tokens_post_padded [1],
    expert_counts [E]), all int32 on the GPU.  ``out`` may supply those four buffers.
    ``strict`` raises ValueError when some ids were outside [0, E) (it waits for the call)."""
    T, k = topk_ids.shape
    cap = lib.moe_align_capacity(T, k, E, block_m)
    dev = topk_ids.device
    if out is None:
        sorted_ids = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)[:cap]
        expert_ids = torch.empty(max(cap // block_m, 1), dtype=torch.int32, device=dev)[:cap // block_m]
        ntpp = torch.empty(1, dtype=torch.int32, device=dev)
        counts = torch.empty(E, dtype=torch.int32, device=dev)
    else:
        sorted_ids, expert_ids, ntpp, counts = out
    ws = _ws(lib.moe_align_workspace_size(T, k, E, block_m), dev)
    check(lib.moe_align(_p(topk_ids), T, k, E, block_m, _p(sorted_ids), _p(expert_ids), _p(ntpp),
                        _p(counts), _p(ws), ws.numel(), _stream()), "moe_align")
    _reject_bad_ids(counts, T, k, strict)
    return sorted_ids, expert_ids, ntpp, counts


def moe_align_ep(topk_ids, E: int, block_m: int, expert_map, out=None, strict: bool = True):
    """moe_align for one GPU of an expert-parallel layer: tiles carry expert_map[e] (the
    expert's local index, -1 when another GPU holds it).  Returns the same four tensors."""
    T, k = topk_ids.shape
    cap = lib.moe_align_capacity(T, k, E, block_m)
    dev = topk_ids.device
    if expert_map.dtype != torch.int32 or expert_map.numel() != E:
        raise ValueError("expert_map must be int32 [E]")
    if out is None:
        sorted_ids = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)[:cap]
        expert_ids = torch.empty(max(cap // block_m, 1), dtype=torch.int32, device=dev)[:cap // block_m]
        ntpp = torch.empty(1, dtype=torch.int32, device=dev)
        counts = torch.empty(E, dtype=torch.int32, device=dev)
    else:
        sorted_ids, expert_ids, ntpp, counts = out
    ws = _ws(lib.moe_align_workspace_size(T, k, E, block_m), dev)
    check(lib.moe_align_ep(_p(topk_ids), T, k, E, block_m, _p(expert_map), _p(sorted_ids),
                           _p(expert_ids), _p(ntpp), _p(counts), _p(ws), ws.numel(), _stream()),
          "moe_align_ep")
    _reject_bad_ids(counts, T, k, strict)
    return sorted_ids, expert_ids, ntpp, counts


def moe_preferred_block_m(T, H, I, E, k, dtype) -> int:
    return lib.moe_preferred_block_m(T, H, I, E, k, dtype)


def moe_auto_variant(T, H, I, E, k, dtype) -> int:
    return lib.moe_auto_variant(T, H, I, E, k, dtype)


def moe_gemm1_swiglu(x, w13, sorted_ids, expert_ids, ntpp, k, block_m, variant=0, a=None, E=None):
    """E: experts the align table was built for (default: w13's; under expert parallelism
    the global count, while w13 holds this GPU's experts)."""
    T, H = x.shape
    El, I2, _ = w13.shape
    E = El if E is None else E
    I = I2 // 2
    if a is None:
        a = torch.zeros(T * k, I, dtype=x.dtype, device=x.device)
    check(lib.moe_gemm1_swiglu(_p(x), _p(w13), _p(sorted_ids), _p(expert_ids), _p(ntpp), T, H, I,
                               E, k, block_m, _dt(x), variant, _p(a), _stream()),
          "moe_gemm1_swiglu")
    return a


def moe_gemm2_weighted(a, w2, topk_w, sorted_ids, expert_ids, ntpp, T, k, block_m, variant=0,
                       y=None, E=None):
    El, H, I = w2.shape
    E = El if E is None else E
    if y is None:
        y = torch.zeros(T * k, H, dtype=torch.float32, device=a.device)
    check(lib.moe_gemm2_weighted(_p(a), _p(w2), _p(topk_w), _p(sorted_ids), _p(expert_ids),
                                 _p(ntpp), T, H, I, E, k, block_m, _dt(a), variant, _p(y),
                                 _stream()), "moe_gemm2_weighted")
    return y


def moe_combine(y, T, k, dtype, out=None):
    H = y.shape[1]
    if out is None:
        out = torch.empty(T, H, dtype=dtype, device=y.device)
    check(lib.moe_combine(_p(y), T, H, k, _dt(out), _p(out), _stream()), "moe_combine")
    return out


def moe_forward_workspace_size(T, H, I, E, k, dtype) -> int:
    return lib.moe_forward_workspace_size(T, H, I, E, k, dtype)


def moe_forward(x, w13, w2, topk_w, sorted_ids, expert_ids, ntpp, k, block_m, variant=0,
                out=None, ws=None, E=None):
    """E: experts the align table was built for (default: w13's; the global count under
    expert parallelism)."""
    T, H = x.shape
    El, I2, _ = w13.shape
    E = El if E is None else E
    I = I2 // 2
    if out is None:
        out = torch.empty(T, H, dtype=x.dtype, device=x.device)
    if ws is None:
        ws = _ws(lib.moe_forward_workspace_size(T, H, I, E, k, _dt(x)), x.device)
    check(lib.moe_forward(_p(x), _p(w13), _p(w2), _p(topk_w), _p(sorted_ids), _p(expert_ids),
                          _p(ntpp), T, H, I, E, k, block_m, _dt(x), variant, _p(out), _p(ws),
                          ws.numel(), _stream()), "moe_forward")
    return out


def moe_layer_workspace_size(T, H, I, E, k, dtype) -> int:
    return lib.moe_layer_workspace_size(T, H, I, E, k, dtype)


def moe_layer(x, wg, w13, w2, k, cfg: RouteCfg, out=None, ws=None, topk_ids_out=None,
              topk_w_out=None):
    """route -> align -> GEMM1+SwiGLU -> GEMM2 x weight -> combine; returns out [T,H]."""
    T, H = x.shape
    E, I2, _ = w13.shape
    I = I2 // 2
    if out is None:
        out = torch.empty(T, H, dtype=x.dtype, device=x.device)
    if ws is None:
        ws = _ws(lib.moe_layer_workspace_size(T, H, I, E, k, _dt(x)), x.device)
    check(lib.moe_layer(_p(x), _p(wg), _p(w13), _p(w2), ctypes.byref(cfg), T, H, I, E, k, _dt(x),
                        _p(out), _p(topk_ids_out), _p(topk_w_out), _p(ws), ws.numel(),
                        _stream()), "moe_layer")
    return out


def moe_layer_noalloc(x, wg, w13, w2, k, cfg: RouteCfg, out=None, topk_ids_out=None,
                      topk_w_out=None):
    """moe_layer with the workspace in the library's static device scratch (no workspace
    argument; see the C declaration for the size limit)."""
    T, H = x.shape
    E, I2, _ = w13.shape
    I = I2 // 2
    if out is None:
        out = torch.empty(T, H, dtype=x.dtype, device=x.device)
    check(lib.moe_layer_noalloc(_p(x), _p(wg), _p(w13), _p(w2), ctypes.byref(cfg), T, H, I, E, k,
                                _dt(x), _p(out), _p(topk_ids_out), _p(topk_w_out), _stream()),
          "moe_layer_noalloc")
    return out


# ----------------------------------------------------------------- FP8 expert weights

def moe_gemm1_swiglu_fp8(x, w13, w13_scale, sorted_ids, expert_ids, ntpp, k, block_m,
                         variant=0, a=None, E=None):
    T, H = x.shape
    El, I2, _ = w13.shape
    E = El if E is None else E
    I = I2 // 2
    pw, ps = _fp8(w13, w13_scale, I2)
    if a is None:
        a = torch.zeros(T * k, I, dtype=x.dtype, device=x.device)
    check(lib.moe_gemm1_swiglu_fp8(_p(x), pw, ps, _p(sorted_ids), _p(expert_ids), _p(ntpp), T, H,
                                   I, E, k, block_m, variant, _p(a), _stream()),
          "moe_gemm1_swiglu_fp8")
    return a


def moe_gemm2_weighted_fp8(a, w2, w2_scale, topk_w, sorted_ids, expert_ids, ntpp, T, k, block_m,
                           variant=0, y=None, E=None):
    El, H, I = w2.shape
    E = El if E is None else E
    pw, ps = _fp8(w2, w2_scale, H)
    if y is None:
        y = torch.zeros(T * k, H, dtype=torch.float32, device=a.device)
    check(lib.moe_gemm2_weighted_fp8(_p(a), pw, ps, _p(topk_w), _p(sorted_ids), _p(expert_ids),
                                     _p(ntpp), T, H, I, E, k, block_m, variant, _p(y), _stream()),
          "moe_gemm2_weighted_fp8")
    return y


def moe_forward_fp8(x, w13, w13_scale, w2, w2_scale, topk_w, sorted_ids, expert_ids, ntpp, k,
                    block_m, variant=0, out=None, ws=None, E=None):
    T, H = x.shape
    El, I2, _ = w13.shape
    E = El if E is None else E
    I = I2 // 2
    p13, s13 = _fp8(w13, w13_scale, I2)
    p2, s2 = _fp8(w2, w2_scale, H)
    if out is None:
        out = torch.empty(T, H, dtype=x.dtype, device=x.device)
    if ws is None:
        ws = _ws(lib.moe_forward_workspace_size(T, H, I, E, k, BF16_FP8W), x.device)
    check(lib.moe_forward_fp8(_p(x), p13, s13, p2, s2, _p(topk_w), _p(sorted_ids),
                              _p(expert_ids), _p(ntpp), T, H, I, E, k, block_m, variant, _p(out),
                              _p(ws), ws.numel(), _stream()), "moe_forward_fp8")
    return out


def moe_layer_fp8(x, wg, w13, w13_scale, w2, w2_scale, k, cfg: RouteCfg, out=None, ws=None,
                  topk_ids_out=None, topk_w_out=None):
    """moe_layer with FP8 expert weights (uint8 E4M3 codes + fp32 row scales)."""
    T, H = x.shape
    E, I2, _ = w13.shape
    I = I2 // 2
    p13, s13 = _fp8(w13, w13_scale, I2)
    p2, s2 = _fp8(w2, w2_scale, H)
    if out is None:
        out = torch.empty(T, H, dtype=x.dtype, device=x.device)
    if ws is None:
        ws = _ws(lib.moe_layer_workspace_size(T, H, I, E, k, BF16_FP8W), x.device)
    check(lib.moe_layer_fp8(_p(x), _p(wg), p13, s13, p2, s2, ctypes.byref(cfg), T, H, I, E, k,
                            _p(out), _p(topk_ids_out), _p(topk_w_out), _p(ws), ws.numel(),
                            _stream()), "moe_layer_fp8")
    return out


def moe_layer_ep(x, wg, w13, w2, k, cfg: RouteCfg, expert_map, w13_scale=None, w2_scale=None,
                 out=None, ws=None, topk_ids_out=None, topk_w_out=None):
    """One GPU's share of an expert-parallel layer: Wg covers all E experts, w13/w2 (and
    the row scales, for FP8 weights) hold this GPU's experts in local index order."""
    T, H = x.shape
    E = wg.shape[0]
    El, I2, _ = w13.shape
    I = I2 // 2
    if expert_map.dtype != torch.int32 or expert_map.numel() != E:
        raise ValueError("expert_map must be int32 [E]")
    if w13.dtype == torch.uint8:
        dt = BF16_FP8W
        p13, s13 = _fp8(w13, w13_scale, I2)
        p2, s2 = _fp8(w2, w2_scale, H)
    else:
        dt = _dt(x)
        p13, s13, p2, s2 = _p(w13), None, _p(w2), None
    if out is None:
        out = torch.empty(T, H, dtype=x.dtype, device=x.device)
    if ws is None:
        ws = _ws(lib.moe_layer_workspace_size(T, H, I, E, k, dt), x.device)
    check(lib.moe_layer_ep(_p(x), _p(wg), p13, s13, p2, s2, _p(expert_map), ctypes.byref(cfg), T,
                           H, I, E, k, dt, _p(out), _p(topk_ids_out), _p(topk_w_out), _p(ws),
                           ws.numel(), _stream()), "moe_layer_ep")
    return out


def moe_layer_shared(x, wg, w13, w2, k, cfg: RouteCfg, w13_scale=None, w2_scale=None, out=None,
                     ws=None, topk_ids_out=None, topk_w_out=None):
    """The layer with one shared expert: w13 / w2 hold the E routed experts followed by the
    shared one (index E); the routing outputs, if given, are [T, k+1]."""
    T, H = x.shape
    E = wg.shape[0]
    EW, I2, _ = w13.shape
    if EW != E + 1:
        raise ValueError("w13 must hold E routed experts + 1 shared")
    I = I2 // 2
    if w13.dtype == torch.uint8:
        dt = BF16_FP8W
        p13, s13 = _fp8(w13, w13_scale, I2)
        p2, s2 = _fp8(w2, w2_scale, H)
    else:
        dt = _dt(x)
        p13, s13, p2, s2 = _p(w13), None, _p(w2), None
    if out is None:
        out = torch.empty(T, H, dtype=x.dtype, device=x.device)
    if ws is None:
        ws = _ws(lib.moe_layer_shared_workspace_size(T, H, I, E, k, dt), x.device)
    check(lib.moe_layer_shared(_p(x), _p(wg), p13, s13, p2, s2, ctypes.byref(cfg), T, H, I, E, k,
                               dt, _p(out), _p(topk_ids_out), _p(topk_w_out), _p(ws), ws.numel(),
                               _stream()), "moe_layer_shared")
    return out
