"""Seeded synthetic inputs for the top-k MoE SwiGLU layer.

This module only draws numbers.  It holds none of the layer's arithmetic
(no routing, no alignment, no expert math): it produces the tensors the
layer consumes, with the shapes, distributions and load structure of the
workloads the pages discuss, and it is shared by the CPU oracle tests and
the GPU path tests/bench so that both sides see identical input bits.

Workloads (shapes from the model table of "Mixture-of-Experts Kernels:
Routing, Permutation, and Grouped GEMM", section 1):

* ``tiny``            T=64,  H=64,   I=96,    E=8,   k=2, fp32, softmax top-2 renormalised.
                       Uses the page's own generator recipe (section 3, ground
                       truth script): global seed 0 draws x, a Generator with seed
                       0 draws Wg, W1, W3, W2 in that order, scaled 1/sqrt(fan_in).
* ``mixtral``         T=4096, H=4096, I=14336, E=8,  k=2, bf16, softmax top-2 renormalised.
* ``qwen3_balanced``  T=8192, H=4096, I=1536,  E=128, k=8, bf16, softmax top-8 renormalised.
* ``qwen3_skewed``    as above, plus +3.0 on the router logits of experts 0..7.
* ``deepseek_decode`` T in {1,16,64,256}, H=7168, I=2048, E=256, k=8, bf16,
                       sigmoid + selection bias ~ N(0, variance 0.1), 8 groups,
                       keep 4 groups, weights x2.5.
* ``deepseek_decode_bias01``  the same with the selection bias drawn with standard
                       deviation 0.1 (the other reading of "N(0, 0.1)").
* ``gptoss``          T=16384, H=2880, I=2880, E=128, k=4, bf16, top-4 then softmax,
                       per-expert logit offset 0.5*ln(Zipf(s=1.2) rank weight).

* ``kimi_k2_decode``  T in {1,16,64}, H=7168, I=2048, E=384 routed + 1 shared, k=8, bf16,
                       sigmoid + selection bias ~ N(0, variance 0.1), no groups, no
                       weight scale (the page gives none for this model); the shared
                       expert's W13/W2 follow the routed ones (index E), Wg has E rows.
* ``deepseek_decode_fp8`` / ``mixtral_fp8``: the same layers with FP8 expert
                       weights (dtype "bf16_fp8w"): each expert weight row drawn in
                       fp32 as for bf16, divided by its scale amax(|row|)/448 and
                       converted to OCP E4M3 by torch (round to nearest even); the
                       codes and the fp32 scales are the inputs.  x, Wg and out stay
                       bf16.

Every floating-point input is an fp32 normal draw; bf16 workloads round it
to bf16 (round-to-nearest-even, torch's conversion).  Weights follow
N(0, 1/fan_in): std 1/sqrt(H) for Wg, W1, W3 and 1/sqrt(I) for W2.
W13[e] is the row concatenation [W1[e]; W3[e]] (gate rows first).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch

# routing modes (same integer values as the C-ABI enum)
ROUTE_SOFTMAX_TOPK_RENORM = 0
ROUTE_TOPK_THEN_SOFTMAX = 1
ROUTE_SIGMOID_BIAS_GROUPED = 2


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    dtype: str                      # "f32", "bf16" or "bf16_fp8w" (bf16, FP8 expert weights)
    mode: int
    n_group: int = 0
    topk_group: int = 0
    scaling: float = 1.0
    offset: str | None = None       # None, "hot8", "zipf"
    bias_std: float | None = None   # selection bias std (sigmoid router)
    recipe: str = "device"          # "page_tiny" or "device"
    shared: int = 0                 # shared experts (0 or 1): expert E of W13/W2

    @property
    def R(self) -> int:
        return self.T * self.k

    @property
    def flops(self) -> int:
        """Useful expert FLOPs of one layer pass: 2*T*k*3*H*I."""
        return 2 * self.T * self.k * 3 * self.H * self.I

    def with_T(self, T: int) -> "Workload":
        return replace(self, T=T)

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 64, 64, 96, 8, 2, "f32", ROUTE_SOFTMAX_TOPK_RENORM,
                     recipe="page_tiny"),
    "mixtral": Workload("mixtral", 4096, 4096, 14336, 8, 2, "bf16", ROUTE_SOFTMAX_TOPK_RENORM),
    "qwen3_balanced": Workload("qwen3_balanced", 8192, 4096, 1536, 128, 8, "bf16",
                               ROUTE_SOFTMAX_TOPK_RENORM),
    "qwen3_skewed": Workload("qwen3_skewed", 8192, 4096, 1536, 128, 8, "bf16",
                             ROUTE_SOFTMAX_TOPK_RENORM, offset="hot8"),
    "deepseek_decode": Workload("deepseek_decode", 1, 7168, 2048, 256, 8, "bf16",
                                ROUTE_SIGMOID_BIAS_GROUPED, n_group=8, topk_group=4,
                                scaling=2.5, bias_std=math.sqrt(0.1)),
    # the bias read as standard deviation 0.1 instead of variance 0.1 (secondary sweep)
    "deepseek_decode_bias01": Workload("deepseek_decode_bias01", 1, 7168, 2048, 256, 8, "bf16",
                                       ROUTE_SIGMOID_BIAS_GROUPED, n_group=8, topk_group=4,
                                       scaling=2.5, bias_std=0.1),
    "gptoss": Workload("gptoss", 16384, 2880, 2880, 128, 4, "bf16",
                       ROUTE_TOPK_THEN_SOFTMAX, offset="zipf"),
    "deepseek_decode_fp8": Workload("deepseek_decode_fp8", 1, 7168, 2048, 256, 8, "bf16_fp8w",
                                    ROUTE_SIGMOID_BIAS_GROUPED, n_group=8, topk_group=4,
                                    scaling=2.5, bias_std=math.sqrt(0.1)),
    "mixtral_fp8": Workload("mixtral_fp8", 4096, 4096, 14336, 8, 2, "bf16_fp8w",
                            ROUTE_SOFTMAX_TOPK_RENORM),
    "kimi_k2_decode": Workload("kimi_k2_decode", 1, 7168, 2048, 384, 8, "bf16",
                               ROUTE_SIGMOID_BIAS_GROUPED, bias_std=math.sqrt(0.1), shared=1),
}

FP8_MAX = 448.0     # largest finite OCP E4M3 value


def quantize_fp8_rows(w: torch.Tensor):
    """Input recipe for FP8 expert weights: per row (last dim) scale = amax/448 in fp32,
    codes = torch's E4M3 conversion of w / scale, returned as uint8.  Returns
    (codes uint8 [..., N, K], scale fp32 [..., N])."""
    w = w.to(torch.float32)
    scale = (w.abs().amax(dim=-1) / FP8_MAX).clamp_min(2.0 ** -120)
    codes = (w / scale[..., None]).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale


def _torch_dtype(dt: str) -> torch.dtype:
    """Type of x, Wg and out (FP8-weight layers keep them bf16)."""
    return torch.float32 if dt == "f32" else torch.bfloat16


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def logit_offset(wl: Workload, seed: int = 0) -> torch.Tensor | None:
    """Per-expert fp32 offset added to the router logits (selection and weights)."""
    if wl.offset is None:
        return None
    if wl.offset == "hot8":
        off = torch.zeros(wl.E, dtype=torch.float32)
        off[: min(8, wl.E)] = 3.0
        return off
    if wl.offset == "zipf":
        # Zipf(s=1.2) rank weights, ranks assigned to experts by a seeded permutation.
        g = _gen("cpu", seed + 7)
        ranks = torch.randperm(wl.E, generator=g).to(torch.float64) + 1.0
        q = torch.arange(1, wl.E + 1, dtype=torch.float64)
        norm = (q ** -1.2).sum()
        return (0.5 * torch.log(ranks ** -1.2 / norm)).to(torch.float32)
    raise ValueError(wl.offset)


def selection_bias(wl: Workload, seed: int = 0) -> torch.Tensor | None:
    if wl.bias_std is None:
        return None
    g = _gen("cpu", seed + 11)
    return (torch.randn(wl.E, generator=g, dtype=torch.float32) * wl.bias_std)


@dataclass
class Layer:
    wl: Workload
    x: torch.Tensor          # [T, H]
    wg: torch.Tensor         # [E, H]
    w13: torch.Tensor        # [E (+1 shared), 2I, H]
    w2: torch.Tensor         # [E (+1 shared), H, I]
    offset: torch.Tensor | None = None   # [E] f32
    bias: torch.Tensor | None = None     # [E] f32
    w13_scale: torch.Tensor | None = None  # [E, 2I] f32 (FP8 weights: w13 holds uint8 codes)
    w2_scale: torch.Tensor | None = None   # [E, H] f32 (FP8 weights: w2 holds uint8 codes)
    extra: dict = field(default_factory=dict)


def make_layer(wl: Workload, device="cpu", seed: int = 0, x_seed: int | None = None) -> Layer:
    """Draw one layer's inputs.  ``x_seed`` re-draws only the activations."""
    dt = _torch_dtype(wl.dtype)
    E, H, I, T = wl.E, wl.H, wl.I, wl.T
    if wl.recipe == "page_tiny":
        # the page's ground-truth recipe: global seed 0 -> x, Generator(0) -> Wg, W1, W3, W2
        torch.manual_seed(seed)
        x = torch.randn(T, H)
        g = _gen("cpu", seed)
        s = 1.0 / H ** 0.5
        wg = torch.randn(E, H, generator=g) * s
        w1 = torch.randn(E, I, H, generator=g) * s
        w3 = torch.randn(E, I, H, generator=g) * s
        w2 = torch.randn(E, H, I, generator=g) / I ** 0.5
        w13 = torch.cat([w1, w3], dim=1)
        lay = Layer(wl, x.to(dt).to(device), wg.to(dt).to(device), w13.to(dt).to(device),
                    w2.to(dt).to(device))
    else:
        g = _gen(device, seed)
        x = torch.randn(T, H, generator=g, device=device).to(dt)
        wg = (torch.randn(E, H, generator=g, device=device) / math.sqrt(H)).to(dt)
        fp8 = wl.dtype == "bf16_fp8w"
        wdt = torch.uint8 if fp8 else dt
        EW = E + wl.shared                 # expert weights drawn: routed, then shared
        w13 = torch.empty(EW, 2 * I, H, dtype=wdt, device=device)
        w2 = torch.empty(EW, H, I, dtype=wdt, device=device)
        s13 = torch.empty(EW, 2 * I, dtype=torch.float32, device=device) if fp8 else None
        s2 = torch.empty(EW, H, dtype=torch.float32, device=device) if fp8 else None

        def put(dst, sdst, e, rows, w):
            if fp8:
                dst[e, rows], sdst[e, rows] = quantize_fp8_rows(w)
            else:
                dst[e, rows] = w.to(dt)

        # per expert, to bound the fp32 staging memory at the large shapes
        for e in range(EW):
            put(w13, s13, e, slice(0, I), torch.randn(I, H, generator=g, device=device) / math.sqrt(H))
            put(w13, s13, e, slice(I, 2 * I),
                torch.randn(I, H, generator=g, device=device) / math.sqrt(H))
            put(w2, s2, e, slice(0, H), torch.randn(H, I, generator=g, device=device) / math.sqrt(I))
        if x_seed is not None:
            gx = _gen(device, x_seed)
            x = torch.randn(T, H, generator=gx, device=device).to(dt)
        lay = Layer(wl, x, wg, w13, w2, w13_scale=s13, w2_scale=s2)
    off = logit_offset(wl, seed)
    bias = selection_bias(wl, seed)
    lay.offset = None if off is None else off.to(device)
    lay.bias = None if bias is None else bias.to(device)
    return lay


def make_x(wl: Workload, device="cpu", seed: int = 0) -> torch.Tensor:
    """A fresh activation batch for a workload (used to rotate decode inputs)."""
    g = _gen(device, seed)
    return torch.randn(wl.T, wl.H, generator=g, device=device).to(_torch_dtype(wl.dtype))


def page_test_case(name: str):
    """The four cases of the fused-kernel test matrix (section 6 of the routing/grouped
    GEMM page): H=64, I=96; global seed 1, layer Generator seed 2; expert 0 made popular
    by adding bias*u to its router row and 1.5*u to every token, u a random unit vector.
    Returns (x, wg, w1, w3, w2, k) as fp32 CPU tensors."""
    cases = {
        "uniform": (64, 8, 2, 0.0),
        "skewed": (50, 16, 4, 3.0),
        "decode": (1, 8, 2, 0.0),
        "top1": (37, 8, 1, 0.0),
    }
    T, E, k, bias = cases[name]
    H, I = 64, 96
    torch.manual_seed(1)
    g = _gen("cpu", 2)
    s = 1.0 / H ** 0.5
    wg = torch.randn(E, H, generator=g) * s
    w1 = torch.randn(E, I, H, generator=g) * s
    w3 = torch.randn(E, I, H, generator=g) * s
    w2 = torch.randn(E, H, I, generator=g) / I ** 0.5
    u = torch.randn(H)
    u = u / u.norm().clamp_min(1e-12)
    wg[0] += bias * u
    x = torch.randn(T, H) + 1.5 * u
    return x, wg, w1, w3, w2, k


def page_grouped_router_logits():
    """Logits and bias of the grouped sigmoid router example (section 4 of the routing/
    grouped GEMM page): global seed 0, logits ~ N(0,1) of shape [4, 16]; bias 0.5 on
    experts 0, 4, 8, 12."""
    torch.manual_seed(0)
    logits = torch.randn(4, 16)
    bias = torch.zeros(16)
    bias[torch.arange(16) % 4 == 0] = 0.5
    return logits, bias


def random_topk_ids(T: int, k: int, E: int, seed: int = 0, skew: float = 0.0,
                    hot: int | None = None) -> torch.Tensor:
    """Seeded [T, k] int32 expert ids, k distinct experts per token.  ``skew`` > 0 draws
    experts with Zipf-like probability 1/rank^skew; ``hot`` forces every token to pick
    expert ``hot`` in slot 0 (one expert receives every token)."""
    g = _gen("cpu", seed)
    if skew > 0:
        p = 1.0 / torch.arange(1, E + 1, dtype=torch.float64) ** skew
    else:
        p = torch.ones(E, dtype=torch.float64)
    p = p.expand(T, E).contiguous()
    if hot is not None:
        p[:, hot] = 0.0
        rest = torch.multinomial(p, k - 1, replacement=False, generator=g) if k > 1 else \
            torch.empty(T, 0, dtype=torch.int64)
        ids = torch.cat([torch.full((T, 1), hot, dtype=torch.int64), rest], dim=1)
    else:
        ids = torch.multinomial(p, k, replacement=False, generator=g)
    return ids.to(torch.int32)


def ids_with_counts(counts, k: int, seed: int = 0) -> torch.Tensor:
    """Seeded [T, k] ids (k distinct experts per token) whose per-expert loads equal
    ``counts`` exactly; requires sum(counts) = T*k and max(counts) <= T.  Rows are filled
    by dealing experts round-robin over tokens, then tokens are shuffled."""
    counts = [int(c) for c in counts]
    R = sum(counts)
    assert R % k == 0
    T = R // k
    assert max(counts) <= T
    # deal: expert list sorted by expert, sequence position p -> token p % T, slot p // T
    seq = [e for e, c in enumerate(counts) for _ in range(c)]
    ids = torch.empty(T, k, dtype=torch.int32)
    for p, e in enumerate(seq):
        ids[p % T, p // T] = e
    g = _gen("cpu", seed)
    perm = torch.randperm(T, generator=g)
    ids = ids[perm]
    # shuffle slots within each token too
    for t in range(T):
        ids[t] = ids[t][torch.randperm(k, generator=g)]
    return ids
