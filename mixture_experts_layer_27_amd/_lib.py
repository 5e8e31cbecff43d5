"""ctypes loader of libmoe_mi355x.so with the C signatures of include/moe_mi355x.h.

There is no fallback: if the library is not built the import fails.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python mixture_experts_layer_27_amd/build.py`"
                      " (or __graft_entry__.build()) first")

lib = ctypes.CDLL(LIB_PATH)

_i, _sz, _p, _f = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float


class RouteCfg(ctypes.Structure):
    """moe_route_cfg"""
    _fields_ = [("mode", ctypes.c_int32), ("logit_offset", _p), ("select_bias", _p),
                ("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32),
                ("routed_scaling", ctypes.c_float)]


_SIGS = {
    "moe_route": (_i, [_p, _p, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _sz, _p]),
    "moe_route_workspace_size": (_sz, [_i, _i, _i, _i]),
    "moe_route_from_logits": (_i, [_p, _i, _i, _i, _p, _p, _p, _p]),
    "moe_align_capacity": (ctypes.c_int64, [_i, _i, _i, _i]),
    "moe_align_workspace_size": (_sz, [_i, _i, _i, _i]),
    "moe_align": (_i, [_p, _i, _i, _i, _i, _p, _p, _p, _p, _p, _sz, _p]),
    "moe_align_ep": (_i, [_p, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "moe_preferred_block_m": (_i, [_i, _i, _i, _i, _i, _i]),
    "moe_auto_variant": (_i, [_i, _i, _i, _i, _i, _i]),
    "moe_gemm1_swiglu": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i, _p, _p]),
    "moe_gemm2_weighted": (_i, [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i, _p, _p]),
    "moe_gemm1_swiglu_fp8": (_i, [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _p, _p]),
    "moe_gemm2_weighted_fp8": (_i, [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _p,
                                    _p]),
    "moe_combine": (_i, [_p, _i, _i, _i, _i, _p, _p]),
    "moe_forward_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i]),
    "moe_forward": (_i, [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i, _p, _p, _sz,
                         _p]),
    "moe_forward_fp8": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _p,
                             _p, _sz, _p]),
    "moe_layer_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i]),
    "moe_layer_fp8": (_i, [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _p, _p, _p, _p, _sz,
                           _p]),
    "moe_layer": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _sz, _p]),
    "moe_layer_noalloc": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p]),
    "moe_layer_shared_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i]),
    "moe_layer_shared": (_i, [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p,
                              _sz, _p]),
    "moe_layer_ep": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p,
                          _sz, _p]),
    "moe_status_string": (ctypes.c_char_p, [_i]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_version": (ctypes.c_char_p, []),
}

for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.moe_last_error().decode()
        super().__init__(f"{where}: {lib.moe_status_string(status).decode()} ({msg})")


def check(status: int, where: str) -> None:
    if status != 0:
        raise MoeError(status, where)
