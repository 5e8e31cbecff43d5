"""Benchmark of the fused top-k MoE SwiGLU layer on one MI355X.

One step = one moe_layer call through the C ABI (route -> align -> GEMM1+SwiGLU -> GEMM2 x
weight -> combine) over one batch of seeded synthetic input already resident in HBM, on
the current HIP stream.  Prints ONE JSON line.  `config` also carries the spread of single
steps (p10/p50/p90) and per-stage durations: K calls of one stage captured in one HIP graph
whose replay is timed between HIP events; the GEMM1 duration for the roofline comes from
there.

  python bench.py [--steps K] [--warmup W] [--workload mixtral|deepseek_decode|...] [--T n]

Default workload: the Mixtral-8x7B-shaped prefill layer (T=4096, H=4096, I=14336, E=8,
k=2, bf16), metric = useful TFLOPS = 2*T*k*3*H*I / step time.  The default run also
carries, measured in the same process: `decode` (the DeepSeek-V3-shaped layer at T = 1,
16 and 64: weight GB/s and fraction of HBM, stage times), `calibration` (a dense bf16 GEMM
of the same total size through torch, the comparison point the pages name for prefill),
and `cpu_baseline` (the oracle on the host cores, plus its timings on the tiny layer).  Decode workloads report
weight GB/s = active experts * 3*H*I*2 B / step time (FP8 weights: 1 B per weight plus the
active experts' fp32 row scales, (2I + H)*4 B each).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer TFLOPS (2·T·k·3HI/t) prefill; weight GB/s at decode; % of roofline"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=48)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral")
    ap.add_argument("--T", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true",
                    help="default Mixtral run: skip the DeepSeek decode sub-record and the "
                         "dense-GEMM calibration")
    ap.add_argument("--no-stages", action="store_true",
                    help="profiling runs: skip the per-stage timing (the standalone stage entry "
                         "points), so that every GEMM dispatch of the run is the layer's own; "
                         "the line then carries no roofline fraction")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches instead of HIP-graph replays of the step")
    ap.add_argument("--cpu-sample-tokens", type=int, default=None)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (a known-size "
                         "kernel that calibrates HBM byte counters)")
    ap.add_argument("--ep", type=int, default=1,
                    help="expert-parallel degree: this GPU holds every ep-th expert (e %% ep "
                         "== 0) and computes the share of the layer those experts give "
                         "(moe_layer_ep); value counts the local experts only")
    ap.add_argument("--block-m", type=int, default=None,
                    help="align block_m (the expert GEMM tile height follows it); times the "
                         "stage-by-stage calls instead of moe_layer")
    return ap.parse_args()


KERNEL_SOURCES = ("gemm_pipe.hip", "decode.hip", "gemm.hip", "common.hpp", "dma.hpp", "route_dev.hpp",
                  "align_dev.hpp")


def kernel_digest() -> str:
    """sha256 over the sources of the expert-GEMM kernels (ties counter data to them)."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "mixture_experts_layer_27_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(key: str):
    """HBM bytes per GEMM1 launch from the committed FETCH_SIZE/WRITE_SIZE passes
    (profiles/traffic.json), or None when they were taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as fh:
            rec = json.load(fh).get(key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_sha256") != kernel_digest():
        return None
    return rec["traffic_bytes_per_launch"]


def expert_bytes(wl) -> int:
    """Weight bytes of one expert: 3*H*I weights (2 B in bf16; 1 B in FP8 plus the fp32
    scales of its 2I + H rows)."""
    if wl.dtype == "bf16_fp8w":
        return 3 * wl.H * wl.I + (2 * wl.I + wl.H) * 4
    return 3 * wl.H * wl.I * (4 if wl.dtype == "f32" else 2)


def cpu_baseline(wl, lay, sample_T):
    """Time the CPU oracle (routing + per-expert loop) on the first sample_T tokens."""
    import numpy as np
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    x = lay.x[:sample_T].float().cpu().numpy()
    wg = lay.wg.float().cpu().numpy()
    kw = dict(offset=None if lay.offset is None else lay.offset.cpu().numpy(),
              bias=None if lay.bias is None else lay.bias.cpu().numpy(),
              n_group=wl.n_group, topk_group=wl.topk_group, scaling=wl.scaling)
    if lay.w13_scale is not None:
        c13, s13 = lay.w13.cpu().numpy(), lay.w13_scale.cpu().numpy()
        c2, s2 = lay.w2.cpu().numpy(), lay.w2_scale.cpu().numpy()
        t0 = time.perf_counter()
        out, ids, _, _ = O.moe_layer_fp8(x, wg, c13, s13, c2, s2, wl.k, wl.mode, **kw)
    else:
        w13 = lay.w13.float().cpu().numpy()
        w2 = lay.w2.float().cpu().numpy()
        layer = O.moe_layer_shared if wl.shared else O.moe_layer
        t0 = time.perf_counter()
        out, ids, _, _ = layer(x, wg, w13, w2, wl.k, wl.mode, round_a=wl.dtype == "bf16", **kw)
    dt = time.perf_counter() - t0
    flops = 2 * sample_T * (wl.k + wl.shared) * 3 * wl.H * wl.I
    if wl.T <= 256:  # decode: weight bytes of the experts the sample activates
        active = len(set(ids.reshape(-1).tolist()))
        value, unit = active * expert_bytes(wl) / dt / 1e9, "GB/s"
    else:
        value, unit = flops / dt / 1e12, "TFLOPS"
    return {"value": value, "unit": unit, "cores": int(cores), "kind": "oracle",
            "sample": f"{sample_T} of {wl.T} tokens of the same layer (numpy float64 oracle, "
                      f"route + per-expert loop), {dt:.2f} s",
            "cpu_model": cpu_model(), "os_cpu_count": os.cpu_count(),
            "threads_note": "cores = the BLAS threads numpy's matrix products ran on"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def tiny_oracle_timings(reps=20):
    """The oracle on the tiny fp32 layer (T=64, H=64, I=96, E=8, k=2): routing + per-expert
    loop with all BLAS threads and with one, and the dense run-every-expert version."""
    import numpy as np
    from oracle import moe_oracle as O
    from synth import inputs as S
    wl = S.WORKLOADS["tiny"]
    lay = S.make_layer(wl)
    x = lay.x.double().numpy()
    wg, w13, w2 = lay.wg.double().numpy(), lay.w13.double().numpy(), lay.w2.double().numpy()
    logits32 = O.router_logits(x, wg).astype(np.float32)
    ids, w = O.route(logits32, wl.k, wl.mode)

    def best(fn):
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return min(ts) * 1e3

    out = {"loop_ms": best(lambda: O.moe_layer(x, wg, w13, w2, wl.k, wl.mode)),
           "dense_ms": best(lambda: O.moe_dense(x, w13, w2, ids, w))}
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            out["loop_1thread_ms"] = best(lambda: O.moe_layer(x, wg, w13, w2, wl.k, wl.mode))
    except Exception:
        out["loop_1thread_ms"] = None
    out["note"] = "best of %d runs; loop includes routing, dense is the expert math alone" % reps
    return out


def measure(args, workload: str, T_override=None, with_cpu=True):
    """Time one workload's layer step (and its stages); returns the JSON record."""
    import torch
    import mixture_experts_layer_27_amd as m
    from synth import inputs as S

    wl = S.WORKLOADS[workload]
    if T_override is not None:
        wl = wl.with_T(T_override)
    dev = "cuda"
    lay = S.make_layer(wl, device=dev, seed=0)
    T, H, I, E, k = wl.T, wl.H, wl.I, wl.E, wl.k
    # a shared expert is one more routing slot (expert E, weight 1): the table, the GEMMs
    # and the combine see K1 = k + 1 slots over ES = E + 1 experts
    shared = wl.shared
    K1, ES = k + shared, E + shared
    # expert weights this GPU holds (all of them unless --ep)
    ep = args.ep
    emap = None
    w13, w2, s13, s2 = lay.w13, lay.w2, lay.w13_scale, lay.w2_scale
    if ep > 1:
        if shared:
            raise SystemExit("--ep with a shared expert is not supported")
        local = torch.arange(0, E, ep, device=dev)
        emap = torch.full((E,), -1, dtype=torch.int32, device=dev)
        emap[local] = torch.arange(local.numel(), dtype=torch.int32, device=dev)
        w13, w2 = w13[local].contiguous(), w2[local].contiguous()
        if s13 is not None:
            s13, s2 = s13[local].contiguous(), s2[local].contiguous()
        torch.cuda.empty_cache()
    fp8 = wl.dtype == "bf16_fp8w"
    dt = {"bf16": m.BF16, "f32": m.F32, "bf16_fp8w": m.BF16_FP8W}[wl.dtype]
    dta = m.BF16 if fp8 else dt      # activation type (router, combine)
    cfg = m.route_cfg(wl.mode, lay.offset, lay.bias, wl.n_group, wl.topk_group, wl.scaling)
    bm = args.block_m or m.moe_preferred_block_m(T, H, I, ES, K1, dt)
    variant = m.moe_auto_variant(T, H, I, ES, K1, dt)
    cap = m.moe_align_capacity(T, K1, ES, bm)
    R = T * K1
    # rotate activation batches for decode so successive steps route differently
    nx = 8 if T <= 256 else 1
    xs = [lay.x] + [S.make_x(wl, device=dev, seed=1000 + i) for i in range(nx - 1)]
    i32 = dict(dtype=torch.int32, device=dev)
    ids = torch.empty(T, K1, **i32)
    w = torch.empty(T, K1, dtype=torch.float32, device=dev)
    # the route stage alone writes the k routed slots (the full step fills ids / w)
    ids_r = torch.empty(T, k, **i32) if shared else ids
    w_r = torch.empty(T, k, dtype=torch.float32, device=dev) if shared else w
    rws = torch.empty(max(16, m.moe_route_workspace_size(T, H, E, dta)), dtype=torch.uint8, device=dev)
    sorted_ids = torch.empty(cap, **i32)
    expert_ids = torch.empty(cap // bm, **i32)
    ntpp = torch.empty(1, **i32)
    counts = torch.empty(ES, **i32)
    aws = torch.empty(max(16, m.moe_align_workspace_size(T, K1, ES, bm)), dtype=torch.uint8, device=dev)
    lws_n = (m.lib.moe_layer_shared_workspace_size if shared else m.moe_layer_workspace_size)(
        T, H, I, E, k, dt)
    lws = torch.empty(lws_n, dtype=torch.uint8, device=dev)
    a = torch.empty(R, I, dtype=lay.x.dtype, device=dev)
    y = torch.empty(R, H, dtype=torch.float32, device=dev)
    out = torch.empty(T, H, dtype=lay.x.dtype, device=dev)
    lib = m.lib
    import ctypes
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = torch.cuda.current_stream()
    staged = args.block_m is not None

    def launch_staged(i, sp, marks=None, only=None):
        """route -> align -> GEMM1+SwiGLU -> GEMM2 x weight -> combine, one call each; with
        `marks` (6 events) the boundaries between the stages are recorded on the stream;
        `only` = j runs stage j alone."""
        x = xs[i % nx]
        mark = (lambda j: marks[j].record(torch.cuda.current_stream())) if marks else (lambda j: None)
        run = lambda j: only is None or only == j
        mark(0)
        if run(0):
            m.check(lib.moe_route(P(x), P(lay.wg), T, H, E, k, dta, ctypes.byref(cfg), P(ids_r),
                                  P(w_r), None, P(rws), rws.numel(), sp), "route")
        mark(1)
        if run(1) and emap is not None:
            m.check(lib.moe_align_ep(P(ids), T, k, E, bm, P(emap), P(sorted_ids), P(expert_ids),
                                     P(ntpp), P(counts), P(aws), aws.numel(), sp), "align")
        elif run(1):
            m.check(lib.moe_align(P(ids), T, K1, ES, bm, P(sorted_ids), P(expert_ids), P(ntpp),
                                  P(counts), P(aws), aws.numel(), sp), "align")
        mark(2)
        if run(2) and fp8:
            m.check(lib.moe_gemm1_swiglu_fp8(P(x), P(w13), P(s13), P(sorted_ids),
                                             P(expert_ids), P(ntpp), T, H, I, ES, K1, bm, variant,
                                             P(a), sp), "gemm1")
        elif run(2):
            m.check(lib.moe_gemm1_swiglu(P(x), P(w13), P(sorted_ids), P(expert_ids), P(ntpp), T,
                                         H, I, ES, K1, bm, dt, variant, P(a), sp), "gemm1")
        mark(3)
        if run(3) and fp8:
            m.check(lib.moe_gemm2_weighted_fp8(P(a), P(w2), P(s2), P(w),
                                               P(sorted_ids), P(expert_ids), P(ntpp), T, H, I, ES,
                                               K1, bm, variant, P(y), sp), "gemm2")
        elif run(3):
            m.check(lib.moe_gemm2_weighted(P(a), P(w2), P(w), P(sorted_ids), P(expert_ids),
                                           P(ntpp), T, H, I, ES, K1, bm, dt, variant, P(y), sp),
                    "gemm2")
        mark(4)
        if run(4):
            m.check(lib.moe_combine(P(y), T, H, K1, dta, P(out), sp), "combine")
        mark(5)

    def launch(i, sp):
        """One step: the whole layer in one library call."""
        if staged:
            return launch_staged(i, sp)
        x = xs[i % nx]
        if shared:
            m.check(lib.moe_layer_shared(P(x), P(lay.wg), P(w13), P(s13) if fp8 else None, P(w2),
                                         P(s2) if fp8 else None, ctypes.byref(cfg), T, H, I, E, k,
                                         dt, P(out), P(ids), P(w), P(lws), lws.numel(), sp),
                    "layer")
            return
        if emap is not None:
            m.check(lib.moe_layer_ep(P(x), P(lay.wg), P(w13), P(s13) if fp8 else None, P(w2),
                                     P(s2) if fp8 else None, P(emap), ctypes.byref(cfg), T, H, I,
                                     E, k, dt, P(out), P(ids), P(w), P(lws), lws.numel(), sp),
                    "layer")
            return
        if fp8:
            m.check(lib.moe_layer_fp8(P(x), P(lay.wg), P(lay.w13), P(lay.w13_scale), P(lay.w2),
                                      P(lay.w2_scale), ctypes.byref(cfg), T, H, I, E, k, P(out),
                                      P(ids), P(w), P(lws), lws.numel(), sp), "layer")
            return
        m.check(lib.moe_layer(P(x), P(lay.wg), P(lay.w13), P(lay.w2), ctypes.byref(cfg), T, H, I, E,
                              k, dt, P(out), P(ids), P(w), P(lws), lws.numel(), sp), "layer")

    cur_sp = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if args.copy_probe_mib:
        src = torch.empty(args.copy_probe_mib << 19, dtype=torch.int16, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for i in range(args.warmup):
        launch(i, cur_sp())
    torch.cuda.synchronize()

    # the step as HIP graphs (one per activation batch): the library only enqueues work,
    # so a whole layer is capturable and replays without host launch gaps.  A model step
    # replays its layers from one graph, so the timed loop replays `chunk`, the nx steps
    # (activation batches in turn) captured in one graph, and single-step graphs only for
    # the remainder: no graph launch sits between the steps of a chunk.
    graphs = []
    chunk = None
    if not args.eager:
        cs = torch.cuda.Stream()
        cs.wait_stream(stream)
        for i in range(nx):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cs):
                launch(i, cur_sp())
            graphs.append(g)
        if nx > 1:
            chunk = torch.cuda.CUDAGraph()
            with torch.cuda.graph(chunk, stream=cs):
                for i in range(nx):
                    launch(i, cur_sp())
        torch.cuda.synchronize()
        for i in range(args.warmup):
            graphs[i % nx].replay()
        if chunk is not None:
            chunk.replay()
        torch.cuda.synchronize()

    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    i = 0
    while chunk is not None and i + nx <= args.steps:
        chunk.replay()
        i += nx
    for i in range(i, args.steps):
        if graphs:
            graphs[i % nx].replay()
        else:
            launch(i, cur_sp())
    t_end.record(stream)
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_end) / args.steps

    # spread of single steps (one event pair per replay, same work as above)
    per = []
    for i in range(args.steps):
        a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_ev.record(stream)
        if graphs:
            graphs[i % nx].replay()
        else:
            launch(i, cur_sp())
        b_ev.record(stream)
        per.append((a_ev, b_ev))
    torch.cuda.synchronize()
    per_ms = sorted(a_.elapsed_time(b_) for a_, b_ in per)
    pct = lambda q: per_ms[min(len(per_ms) - 1, int(round(q * (len(per_ms) - 1))))]

    # per-stage durations (GEMM1 among them): K calls of one stage captured back to back in
    # one HIP graph, one replay timed between two HIP events on the replay stream, so that
    # neither host nor graph launch latency enters (the stages read what the previous full
    # step left in the buffers)
    stage_names = ("route", "align", "gemm1", "gemm2", "combine")
    stages_ms = {}
    if args.no_stages:
        pass
    elif args.eager:
        marks = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
        for i in range(args.steps):
            launch_staged(i, cur_sp(), marks[i])
        torch.cuda.synchronize()
        for j, nm in enumerate(stage_names):
            stages_ms[nm] = sum(mk[j].elapsed_time(mk[j + 1]) for mk in marks) / args.steps
    else:
        launch_staged(0, cur_sp())
        torch.cuda.synchronize()
        for j, nm in enumerate(stage_names):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cs):
                for _ in range(args.steps):
                    launch_staged(0, cur_sp(), only=j)
            g.replay()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            stages_ms[nm] = e0.elapsed_time(e1) / args.steps
            del g
    g1_ms = stages_ms.get("gemm1")
    flops = 2 * T * K1 * 3 * H * I        # useful expert FLOPs (the shared slot included)
    g1_flops = 2 * R * 2 * I * H
    decode = T <= 256
    traffic_key = f"{wl.name}_T{T}" + (f"_ep{ep}" if ep > 1 else "")
    if decode:
        # active experts of each timed step, recomputed outside the timed region
        act = []
        for i in range(args.steps):
            launch(i, cur_sp())
            u = torch.unique(ids)
            act.append(int(u.numel() if emap is None else (emap[u.long()] >= 0).sum()))
        n_act = sum(act) / len(act)
        wbytes = n_act * expert_bytes(wl)
        value, unit = wbytes / (ms * 1e-3) / 1e9, "GB/s"
        # GEMM1 streams W13: 2I*H weights (+ 2I row scales with FP8 weights)
        g1_bytes = n_act * (2 * I * H + 2 * I * 4 if fp8 else 2 * I * H * 2)
        roof = {"bound": "hbm", "achieved": g1_bytes / (g1_ms * 1e-3) / 1e9 if g1_ms else None,
                "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "traffic": measured_traffic(traffic_key)}
    else:
        if emap is not None:
            # expert parallelism: only the routed rows of this GPU's experts are computed;
            # count them for each timed step, outside the timed region
            loc = []
            for i in range(args.steps):
                launch(i, cur_sp())
                loc.append(int((emap[ids.reshape(-1).long()] >= 0).sum()))
            r_local = sum(loc) / len(loc)
            flops = 2 * r_local * 3 * H * I
            g1_flops = 2 * r_local * 2 * I * H
        value, unit = flops / (ms * 1e-3) / 1e12, "TFLOPS"
        roof = {"bound": "mfma", "achieved": g1_flops / (g1_ms * 1e-3) / 1e12 if g1_ms else None,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "traffic": measured_traffic(traffic_key)}
    roof["frac"] = roof["achieved"] / roof["peak"] if roof["achieved"] else None
    roof["kernel"] = ("moe_decode_kernel<GEMM1+SwiGLU>" if variant == m.VARIANT_DECODE
                      else "moe_gemm_pipe_kernel<GEMM1+SwiGLU>")
    roof["kernel_ms"] = g1_ms
    if shared:
        roof["kernel"] += " (k+1 slots: the shared expert is slot k)"
    rec = {"metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
           "config": {"workload": f"{wl.name}", "T": T, "H": H, "I": I, "E": E, "k": k,
                      "route_mode": wl.mode, "shared_experts": shared, "block_m": bm,
                      "variant": variant,
                      "timing": "eager" if args.eager else "hip-graph replay",
                      "step": "stage-by-stage calls" if staged else "moe_layer",
                      "step_ms_p10_p50_p90": [pct(0.1), pct(0.5), pct(0.9)],
                      "stages_ms": {nm: round(v, 4) for nm, v in stages_ms.items()},
                      "route_align_combine_share": ((stages_ms["route"] + stages_ms["align"] +
                                                     stages_ms["combine"]) / sum(stages_ms.values())
                                                    if stages_ms else None),
                      "parallelism": "single-gpu"},
           "roofline": roof}
    if decode:
        rec["config"]["active_experts"] = n_act
    if not decode and not staged:
        # the per-stage GEMM2 call has no workspace and runs every tile whole; inside the
        # layer step GEMM2 may split a short last round of tiles (partial sums + fix-up)
        rec["config"]["stage_note"] = ("stages_ms.gemm2 is the standalone GEMM2 call (tiles "
                                       "whole); the layer step's GEMM2 may split its last "
                                       "round of tiles in K")
    if ep > 1:
        rec["config"]["expert_parallel"] = {"degree": ep, "local_experts": int(w13.shape[0]),
                                            "held": "experts e with e % degree == 0",
                                            "value_counts": "local experts only"}
    if wl.offset == "hot8":
        # share of the routed rows that the +3.0 logit offset sends to experts 0..7
        rec["config"]["hot_block_share"] = float((ids[:, :k] < 8).float().mean())
    if with_cpu and not args.no_cpu_baseline and ep == 1:
        st = args.cpu_sample_tokens or T
        rec["cpu_baseline"] = cpu_baseline(wl, lay, st)
    del lay, xs, graphs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def dense_calibration(T, H, I, k, steps):
    """The pages' comparison point for prefill: a dense bf16 GEMM of the same total size
    (the T*k routed rows against one expert's weights), timed through torch (hipBLASLt)."""
    import torch
    R = T * k
    g = torch.Generator(device="cuda").manual_seed(0)
    out = {}
    for name, (M, K, N) in (("gemm1", (R, H, 2 * I)), ("gemm2", (R, I, H))):
        a = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16)
        w = (torch.randn(N, K, device="cuda", generator=g) / K ** 0.5).to(torch.bfloat16)
        for _ in range(3):
            torch.nn.functional.linear(a, w)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            torch.nn.functional.linear(a, w)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        out[name + "_ms"] = ms
        out[name + "_tflops"] = 2 * M * K * N / (ms * 1e-3) / 1e12
        del a, w
    out["layer_gemms_ms"] = out["gemm1_ms"] + out["gemm2_ms"]
    out["note"] = ("torch.nn.functional.linear (hipBLASLt) on dense bf16 [T*k, H] x [H, 2I] "
                   "and [T*k, I] x [I, H]: the same total GEMM size as the layer's expert "
                   "GEMMs, with no gather, padding or expert boundaries")
    torch.cuda.empty_cache()
    return out


def decode_summary(rec):
    """The figures of a decode record kept in the headline line's decode sub-record."""
    c = rec["config"]
    return {"T": c["T"], "weight_GBps": rec["value"], "frac_of_hbm": rec["value"] / PEAK_HBM_GBS,
            "ms_per_step": rec["ms_per_step"], "active_experts": c.get("active_experts"),
            "stages_ms": c["stages_ms"], "step_ms_p10_p50_p90": c["step_ms_p10_p50_p90"],
            "gemm1_weight_GBps": rec["roofline"]["achieved"],
            "gemm1_frac_of_hbm": rec["roofline"]["frac"]}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this layer's benchmark runs on a single MI355X "
              "(no sharding); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)
    headline = (args.workload == "mixtral" and args.T is None and args.block_m is None
                and args.ep == 1 and not args.no_decode)
    decode = {}
    if headline:
        # the second headline target, measured in the same run (first, so that the one-token
        # step does not follow the dense calibration GEMMs): DeepSeek-V3-shaped decode
        for T in (1, 16, 64):
            decode[f"T{T}"] = decode_summary(measure(args, "deepseek_decode", T, with_cpu=False))
    rec = measure(args, args.workload, args.T)
    if headline:
        c = rec["config"]
        rec["calibration"] = dense_calibration(c["T"], c["H"], c["I"], c["k"], args.steps)
        rec["decode"] = {"workload": "deepseek_decode (E=256, k=8, H=7168, I=2048, bf16, "
                                     "sigmoid + bias grouped routing)", **decode}
        if "cpu_baseline" in rec:
            rec["cpu_baseline"]["tiny_layer"] = tiny_oracle_timings()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
