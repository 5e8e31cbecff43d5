"""moe_layer_noalloc (workspace in the library's static device scratch) against moe_layer
(caller workspace) through the C ABI: two calls in a row on one GPU, the second with a
smaller input, at a decode-variant and a prefill-variant size; identical outputs and
routing (the same launches on the same inputs)."""
import numpy as np
import pytest
import torch

from synth import inputs as S
from tests.gpu_util import layer_check, lib_cfg

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _pair(lib, wl, lay):
    cfg = lib_cfg(lib, wl, lay)
    T, k = wl.T, wl.k
    outs = []
    for fn in (lib.moe_layer, lib.moe_layer_noalloc):
        ids = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
        w = torch.full((T, k), float("nan"), dtype=torch.float32, device=DEV)
        out = fn(lay.x, lay.wg, lay.w13, lay.w2, k, cfg, topk_ids_out=ids, topk_w_out=w)
        torch.cuda.synchronize()
        outs.append((out, ids, w))
    (o0, i0, w0), (o1, i1, w1) = outs
    assert torch.equal(i0, i1) and torch.equal(w0, w1)
    assert torch.equal(o0, o1)
    return o1, i1, w1


@pytest.mark.parametrize("name,Ts,scale", [("deepseek_decode", (16, 4), 4),
                                           ("mixtral", (96, 40), 16)])
def test_noalloc_matches_layer_twice(lib, name, Ts, scale):
    base = S.WORKLOADS[name]
    for T in Ts:           # the second call has the smaller input
        wl = base.scaled(T=T, H=base.H // scale // 64 * 64, I=base.I // scale // 64 * 64)
        lay = S.make_layer(wl, device=DEV, seed=T)
        print(f"[noalloc] {name} T={T} H={wl.H} I={wl.I} E={wl.E} k={wl.k}", flush=True)
        out, ids, w = _pair(lib, wl, lay)
        # and the oracle's bar on the no-alloc result
        layer_check(lib, wl, lay, out, ids.cpu().numpy(), w.cpu().numpy().astype(np.float64))


def test_noalloc_rejects_layers_beyond_the_scratch(lib):
    """The Mixtral-shaped layer at T=4096 needs far more than the static scratch: the call
    fails on the host and enqueues nothing (no tensor is touched)."""
    import ctypes
    wl = S.WORKLOADS["mixtral"]
    st = lib.lib.moe_layer_noalloc(None, None, None, None, None, wl.T, wl.H, wl.I, wl.E, wl.k, 1,
                                   None, None, None, None)
    assert st == -3           # MOE_ERR_WORKSPACE
    assert b"static scratch" in lib.lib.moe_last_error()
