"""CPU oracle for the fused top-k Mixture-of-Experts SwiGLU layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import or call this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code with the HIP library.

It is deliberately plain and slow: numpy, float64 arithmetic for every
floating-point value it produces, no blocking or fusion.  Where a step takes
a discrete decision on floating-point values (which experts a token selects,
which groups stay eligible) the decision is taken on float32 values, the
precision of the kernel, as the rounding of the decision inputs is part of
what the layer computes.

Source pages (cited by title and section):

* [MKR] "Mixture-of-Experts Kernels: Routing, Permutation, and Grouped GEMM"
  (book chapter): section 1 (layer definition, model table), section 2 (route,
  align, grouped GEMM, combine; flat row r = t*k + j), section 3 (two ground-truth
  implementations: per-expert loop and dense run-all-then-mask), section 4
  (sigmoid + selection-bias + group-limited routing), section 5 (the
  sorted_ids / expert_ids / padded-total contract), section 6 (GEMM1 gathers
  x rows r//k against W13[e] = [W1;W3], GEMM2 multiplies by the router weight
  and stores at row r, combine sums the k slots), section 10 (test matrix),
  section 11 (exercises: counting align, expert_map for expert parallelism).
* [CKM] "Custom Kernels for Mixture-of-Experts": device-resident dispatch
  metadata (grouped GEMM section).
* [FMK] "fused-moe-kernel" skill page: padding ids must be >= the number of
  valid rows (Common Pitfalls).

Readings where the pages leave a step open (each also listed in the design doc):

1. ties: the lower expert index (and the lower group index) wins;
2. softmax-top-k-renormalise selects on the fp32 logits; because softmax is
   monotone and the full-softmax denominator cancels in the renormalisation,
   the weights equal a softmax over the k selected logits ([MKR] section 3);
3. slot order j is the selection order (descending score, ties by index);
4. the sigmoid score used for selection is sigma(l) evaluated in float64 and
   rounded to the nearest float32; the biased score and the group score are
   float32 additions;
5. sentinel = T*k; buffer tails past the padded total hold the sentinel in
   sorted_ids and -1 in expert_ids;
6. for bf16 layers the SwiGLU activation a (GEMM2's input) is rounded to bf16
   (round-to-nearest-even); all other intermediates stay in float64 here;
7. "FP8 weights" ([MKR] section 8 prices an expert's weights at one byte per
   element; section 9 lists FP8 weight variants of the fused kernel) are read as
   the OCP 8-bit E4M3 format with one float32 scale per weight row (output
   channel) of each expert: W = decode(code) * scale[e, row].  Activations, the
   router and the output keep the bf16 layer's types;
8. the shared expert of DeepSeek-V3 / Kimi K2 ([MKR] section 1 table, "+1
   shared") is an always-on SwiGLU expert of the routed experts' shape: every token
   adds its output with weight 1; here it is expert E, reached through one more
   routing slot j = k.
"""
from __future__ import annotations

import math

import numpy as np

SOFTMAX_TOPK_RENORM = 0
TOPK_THEN_SOFTMAX = 1
SIGMOID_BIAS_GROUPED = 2


# --------------------------------------------------------------------------- rounding

def bf16_round(a) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (8 significant bits,
    ties to even), returned as float64.  Normal range only (|a| >= 2^-126 or 0),
    which covers every value this layer produces."""
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)                 # a = m * 2**e with 0.5 <= |m| < 1
    q = np.rint(m * 256.0) / 256.0     # keep 8 significant bits, half to even
    return np.ldexp(q, e)


def f32(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float32)


# --------------------------------------------------------------------------- FP8 weights (reading 7)

def fp8_e4m3_value(code: int) -> float:
    """Value of one OCP E4M3 byte: sign bit, 4 exponent bits with bias 7, 3 mantissa
    bits.  Exponent field 0 holds the subnormals m/8 * 2^-6; the all-ones exponent
    with mantissa 7 is NaN (there is no infinity), so the largest value is 448."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def fp8_e4m3_decode(codes) -> np.ndarray:
    """Decode an array of E4M3 bytes (any integer dtype) to float64."""
    table = np.array([fp8_e4m3_value(c) for c in range(256)], np.float64)
    return table[np.asarray(codes).astype(np.int64) & 0xFF]


def dequant_rows(codes, scale) -> np.ndarray:
    """Expert weights from E4M3 codes [E, N, K] and per-row scales [E, N]:
    W[e, n, :] = decode(codes[e, n, :]) * scale[e, n]  (float64)."""
    return fp8_e4m3_decode(codes) * np.asarray(scale, np.float64)[..., None]


# --------------------------------------------------------------------------- routing ([MKR] s3, s4)

def router_logits(x, wg) -> np.ndarray:
    """logits[t, e] = sum_h x[t, h] * Wg[e, h]  (float64)."""
    return np.asarray(x, np.float64) @ np.asarray(wg, np.float64).T


def order_first(values_row, candidates=None) -> np.ndarray:
    """Indices sorted by the order rule: a before b iff v_a > v_b, or v_a == v_b and
    a < b.  Optionally restricted to ``candidates`` (an index array)."""
    v = np.asarray(values_row)
    idx = np.arange(v.shape[0]) if candidates is None else np.asarray(candidates)
    vv = v[idx]
    o = np.lexsort((idx, -vv.astype(np.float64)))   # primary: value desc, secondary: index asc
    return idx[o]


def sigmoid_f32(logits32) -> np.ndarray:
    """sigma(l) = 1/(1+exp(-l)) evaluated in float64, rounded to float32."""
    l = np.asarray(logits32, np.float64)
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-l))
    return s.astype(np.float32)


def route(logits32, k, mode, offset=None, bias=None, n_group=0, topk_group=0,
          scaling=1.0):
    """Route every token from its float32 router logits.

    Returns (ids int32 [T, k], w float64 [T, k]); slot j of token t is flat row t*k+j.

    * SOFTMAX_TOPK_RENORM ([MKR] s1 table: Mixtral, Qwen3; s3 ``route``): softmax over
      all E logits, top-k, renormalise the k weights to sum to 1.  Selection on the
      logits, weights = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the k selected.
    * TOPK_THEN_SOFTMAX ([MKR] s1 table: gpt-oss): top-k logits first, then softmax over
      those k.  Same arithmetic as the previous mode.
    * SIGMOID_BIAS_GROUPED ([MKR] s4): s = sigmoid(l); c = s + bias selects; each group of
      E/n_group contiguous experts scores the sum of its two largest c; the best
      ``topk_group`` groups stay eligible; top-k by c inside them; weights are the
      unbiased s of the chosen experts renormalised and multiplied by ``scaling``.
    ``offset`` (float32 [E]) is added to the logits before anything else (a float32 add).
    """
    l = f32(logits32)
    T, E = l.shape
    if offset is not None:
        l = (l + f32(offset)[None, :]).astype(np.float32)
    ids = np.zeros((T, k), np.int32)
    w = np.zeros((T, k), np.float64)
    if mode in (SOFTMAX_TOPK_RENORM, TOPK_THEN_SOFTMAX):
        for t in range(T):
            sel = order_first(l[t])[:k]
            ids[t] = sel
            ls = l[t, sel].astype(np.float64)
            ex = np.exp(ls - ls[0])
            w[t] = ex / ex.sum()
        return ids, w
    if mode != SIGMOID_BIAS_GROUPED:
        raise ValueError(mode)
    s = sigmoid_f32(l)
    b = np.zeros(E, np.float32) if bias is None else f32(bias)
    c = (s + b[None, :]).astype(np.float32)
    for t in range(T):
        if n_group and topk_group:
            gsz = E // n_group
            gscore = np.zeros(n_group, np.float32)
            for g in range(n_group):
                members = np.arange(g * gsz, (g + 1) * gsz)
                top2 = order_first(c[t], members)[:2]
                gscore[g] = np.float32(c[t, top2[0]]) + np.float32(c[t, top2[1]])
            kept = order_first(gscore)[:topk_group]
            cand = np.concatenate([np.arange(g * gsz, (g + 1) * gsz) for g in sorted(kept)])
        else:
            cand = None
        sel = order_first(c[t], cand)[:k]
        ids[t] = sel
        sw = s[t, sel].astype(np.float64)
        w[t] = scaling * sw / sw.sum()
    return ids, w


# --------------------------------------------------------------------------- align ([MKR] s5)

def align_capacity(T, k, E, block_m) -> int:
    """Worst-case padded length: the largest multiple of block_m not above
    T*k + min(E, T*k)*(block_m-1) (each non-empty expert pads by at most block_m-1)."""
    R = T * k
    bound = R + min(E, R) * (block_m - 1)
    return (bound // block_m) * block_m


def align_runs(topk_ids, E, block_m, cap=None):
    """The align table ([MKR] s5) built one expert run at a time.

    Walking the experts in ascending order, expert e owns a run of ceil(n_e / block_m)
    whole tiles that starts where the previous expert's run ended.  The run's first n_e
    slots hold the flat rows routed to e in ascending row order (the stable order the
    page calls a choice that makes the output deterministic); its remaining slots hold
    the sentinel R = T*k, and each of its tiles records e in expert_ids.  Slots past the
    last run (up to ``cap``) keep the sentinel and their tiles -1 (reading 5).

    Returns dict(sorted_ids, expert_ids, total, counts) with buffers of length ``cap``
    (default: the padded total) and cap // block_m.
    """
    flat = np.asarray(topk_ids, np.int64).reshape(-1)
    sentinel = flat.size
    runs, owners, counts = [], [], np.zeros(E, np.int32)
    for e in range(E):
        mine = np.flatnonzero(flat == e)             # ascending flat rows of expert e
        counts[e] = mine.size
        if mine.size == 0:
            continue                                 # an empty expert owns no tile
        ntiles = -(-mine.size // block_m)
        run = np.full(ntiles * block_m, sentinel, np.int64)
        run[: mine.size] = mine
        runs.append(run)
        owners.extend([e] * ntiles)
    table = np.concatenate(runs) if runs else np.zeros(0, np.int64)
    total = int(table.size)
    if cap is None:
        cap = total
    sorted_ids = np.full(cap, sentinel, np.int32)
    sorted_ids[:total] = table
    expert_ids = np.full(cap // block_m, -1, np.int32)
    expert_ids[: len(owners)] = owners
    return dict(sorted_ids=sorted_ids, expert_ids=expert_ids, total=total, counts=counts)


def align_counting(topk_ids, E, block_m, cap=None):
    """The same table without a sort: one counting pass, an exclusive scan over the
    padded counts, then a running cursor per expert while walking rows in order
    ([MKR] s11, first exercise).  Plain Python loops."""
    flat = [int(v) for v in np.asarray(topk_ids).reshape(-1)]
    R = len(flat)
    counts = [0] * E
    for e in flat:
        counts[e] += 1
    start = [0] * E
    run = 0
    for e in range(E):
        start[e] = run
        run += -(-counts[e] // block_m) * block_m
    total = run
    if cap is None:
        cap = total
    sorted_ids = [R] * cap
    cursor = [0] * E
    for r, e in enumerate(flat):
        sorted_ids[start[e] + cursor[e]] = r
        cursor[e] += 1
    expert_ids = [-1] * (cap // block_m)
    for e in range(E):
        for j in range(-(-counts[e] // block_m)):
            expert_ids[start[e] // block_m + j] = e
    return dict(sorted_ids=np.array(sorted_ids, np.int32),
                expert_ids=np.array(expert_ids, np.int32), total=total,
                counts=np.array(counts, np.int32))


# --------------------------------------------------------------------------- expert math ([MKR] s1, s3, s6)

def silu(z):
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z))  (float64)."""
    z = np.asarray(z, np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def _split_w13(w13):
    w13 = np.asarray(w13, np.float64)
    I = w13.shape[1] // 2
    return w13[:, :I, :], w13[:, I:, :]        # gate rows (W1) first, then up rows (W3)


def moe_loop(x, w13, w2, ids, w, round_a=False, return_rows=False):
    """Per-expert loop ([MKR] s3 ``moe_loop``): for each expert gather the token rows
    routed to it (flat rows r, token r // k), run the SwiGLU expert once on them, scale
    by the router weight of row r, then sum each token's k slots in slot order."""
    x = np.asarray(x, np.float64)
    w2 = np.asarray(w2, np.float64)
    W1, W3 = _split_w13(w13)
    T, H = x.shape
    E = W1.shape[0]
    ids = np.asarray(ids)
    k = ids.shape[1]
    flat_ids = ids.reshape(-1)
    flat_w = np.asarray(w, np.float64).reshape(-1)
    y = np.zeros((T * k, H))
    for e in range(E):
        rows = np.nonzero(flat_ids == e)[0]
        if rows.size == 0:
            continue                                   # an empty expert does nothing
        xe = x[rows // k]
        a = silu(xe @ W1[e].T) * (xe @ W3[e].T)
        if round_a:
            a = bf16_round(a)
        y[rows] = flat_w[rows, None] * (a @ w2[e].T)
    out = np.zeros((T, H))
    for j in range(k):                                 # combine: slot order
        out += y[j::k]
    return (out, y) if return_rows else out


def swiglu_rows(x, w13, ids):
    """GEMM1 + SwiGLU of every routed row ([MKR] s6: flat row r = t*k + j gathers token
    r // k and multiplies it by W13[e] = [W1[e]; W3[e]] of its expert e = ids[t, j]):
    a[r] = silu(x[t] W1[e]^T) * (x[t] W3[e]^T), float64, not rounded.  Slots whose id is
    outside [0, E) (an expert this call does not hold) are left zero."""
    x = np.asarray(x, np.float64)
    W1, W3 = _split_w13(w13)
    ids = np.asarray(ids)
    T, k = ids.shape
    a = np.zeros((T * k, W1.shape[1]))
    for e in range(W1.shape[0]):
        tt, jj = np.nonzero(ids == e)               # the slots routed to expert e
        if tt.size:
            xe = x[tt]
            a[tt * k + jj] = silu(xe @ W1[e].T) * (xe @ W3[e].T)
    return a


def down_and_combine(a, w2, ids, w):
    """GEMM2 x router weight and the combine ([MKR] s6) from given activations a [T*k, I]:
    out[t] = sum_j w[t, j] * (a[t*k + j] W2[e]^T), e = ids[t, j], float64.  Slots whose id
    is outside [0, E) add nothing."""
    a = np.asarray(a, np.float64)
    w2 = np.asarray(w2, np.float64)
    ids = np.asarray(ids)
    wv = np.asarray(w, np.float64)
    T, k = ids.shape
    out = np.zeros((T, w2.shape[1]))
    for e in range(w2.shape[0]):
        tt, jj = np.nonzero(ids == e)                # one slot per token: ids of a token differ
        if tt.size:
            out[tt] += wv[tt, jj, None] * (a[tt * k + jj] @ w2[e].T)
    return out


def moe_dense(x, w13, w2, ids, w, round_a=False):
    """Dense version ([MKR] s3 ``moe_dense``): run every expert on every token, then
    weight by a [T, E] gate matrix holding the k routed weights per token."""
    x = np.asarray(x, np.float64)
    w2 = np.asarray(w2, np.float64)
    W1, W3 = _split_w13(w13)
    T, H = x.shape
    E = W1.shape[0]
    gate = np.zeros((T, E))
    ids = np.asarray(ids)
    wv = np.asarray(w, np.float64)
    for t in range(T):
        for j in range(ids.shape[1]):
            gate[t, ids[t, j]] += wv[t, j]
    out = np.zeros((T, H))
    for e in range(E):
        a = silu(x @ W1[e].T) * (x @ W3[e].T)
        if round_a:
            a = bf16_round(a)
        out += gate[:, e:e + 1] * (a @ w2[e].T)
    return out


def moe_permute_grouped(x, w13, w2, ids, w, round_a=False):
    """Third implementation ([MKR] s2 'permute, then grouped GEMM'; s10 'three
    implementations'), written as matrix algebra.

    The routed (token, slot) pairs are listed expert by expert (ascending expert, and
    within an expert ascending token, then slot), so each expert's pairs form one
    contiguous segment of the list.  The permutation is a 0/1 gather matrix P [R, T]
    whose row i selects the token of pair i, so P @ x is the permuted activation copy;
    each segment goes through its expert's SwiGLU FFN as one dense GEMM chain; the
    un-permute and the weighted combine are a single matrix Q [T, R] with Q[t, i] =
    (router weight of pair i) when pair i belongs to token t, so out = Q @ Y.
    Shares no indexing code with ``moe_loop`` (no flat row numbers, no slot-order sum).
    """
    x = np.asarray(x, np.float64)
    w2 = np.asarray(w2, np.float64)
    W1, W3 = _split_w13(w13)
    T, H = x.shape
    E = W1.shape[0]
    ids = np.asarray(ids)
    wv = np.asarray(w, np.float64)
    pairs, seg_len = [], []
    for e in range(E):
        mine = [(t, j) for t in range(T) for j in range(ids.shape[1]) if ids[t, j] == e]
        pairs.extend(mine)
        seg_len.append(len(mine))
    R = len(pairs)
    P = np.zeros((R, T))
    Q = np.zeros((T, R))
    for i, (t, j) in enumerate(pairs):
        P[i, t] = 1.0
        Q[t, i] = wv[t, j]
    xp = P @ x                                        # permuted activations
    Y = np.zeros((R, H))
    lo = 0
    for e, n in enumerate(seg_len):                   # grouped GEMM: one segment per expert
        if n:
            seg = xp[lo:lo + n]
            a = silu(seg @ W1[e].T) * (seg @ W3[e].T)
            if round_a:
                a = bf16_round(a)
            Y[lo:lo + n] = a @ w2[e].T
        lo += n
    return Q @ Y                                      # un-permute and combine


def moe_bruteforce(x, w13, w2, ids, w, round_a=False):
    """Scalar Python loops per (token, slot, output element); tiny inputs only."""
    x = np.asarray(x, np.float64).tolist()
    w13 = np.asarray(w13, np.float64)
    w2 = np.asarray(w2, np.float64).tolist()
    I = w13.shape[1] // 2
    w13 = w13.tolist()
    T = len(x)
    H = len(x[0])
    out = [[0.0] * H for _ in range(T)]
    for t in range(T):
        for j, e in enumerate(np.asarray(ids)[t].tolist()):
            wt = float(np.asarray(w)[t, j])
            a = []
            for i in range(I):
                g = sum(x[t][h] * w13[e][i][h] for h in range(H))
                u = sum(x[t][h] * w13[e][I + i][h] for h in range(H))
                ai = (g / (1.0 + math.exp(-g)) if g > -700 else 0.0) * u
                if round_a:
                    ai = float(bf16_round(ai))
                a.append(ai)
            for h in range(H):
                out[t][h] += wt * sum(a[i] * w2[e][h][i] for i in range(I))
    return np.array(out)


def moe_layer(x, wg, w13, w2, k, mode, offset=None, bias=None, n_group=0, topk_group=0,
              scaling=1.0, round_a=False):
    """Whole layer: float64 router logits rounded to float32, routing, per-expert loop."""
    logits32 = router_logits(x, wg).astype(np.float32)
    ids, w = route(logits32, k, mode, offset, bias, n_group, topk_group, scaling)
    out = moe_loop(x, w13, w2, ids, w, round_a=round_a)
    return out, ids, w, logits32


def moe_layer_fp8(x, wg, w13_codes, w13_scale, w2_codes, w2_scale, k, mode, offset=None,
                  bias=None, n_group=0, topk_group=0, scaling=1.0):
    """The bf16 layer with FP8 expert weights (reading 7): the expert weights are the
    decoded codes times their row scales; everything else as ``moe_layer`` with the
    SwiGLU activation rounded to bf16."""
    w13 = dequant_rows(w13_codes, w13_scale)
    w2 = dequant_rows(w2_codes, w2_scale)
    return moe_layer(x, wg, w13, w2, k, mode, offset, bias, n_group, topk_group, scaling,
                     round_a=True)


# --------------------------------------------------------------------------- expert parallelism ([MKR] s11)

def align_ep(topk_ids, E, block_m, expert_map, cap=None):
    """The align table of one GPU under expert parallelism ([MKR] s11 exercise: experts
    not on this GPU get expert_ids = -1, and the GEMMs skip those tiles).  The table of
    all E experts (same sorted_ids, total and counts as ``align_runs``) with each
    tile's owner e replaced by expert_map[e]: its index among this GPU's experts, or -1."""
    r = align_runs(topk_ids, E, block_m, cap)
    emap = np.asarray(expert_map, np.int64)
    eids = r["expert_ids"].astype(np.int64)
    owned = eids >= 0
    eids[owned] = emap[eids[owned]]
    r["expert_ids"] = eids.astype(np.int32)
    return r


def moe_loop_ep(x, w13_local, w2_local, ids, w, expert_map, round_a=False):
    """One GPU's share of the layer under expert parallelism: the per-expert loop over
    the experts this GPU holds (local index l = expert_map[e], weights w13_local[l],
    w2_local[l]); slots routed to other GPUs' experts add nothing here.  Summing the
    shares of GPUs whose maps partition the experts gives the whole layer."""
    x = np.asarray(x, np.float64)
    w2_local = np.asarray(w2_local, np.float64)
    W1, W3 = _split_w13(w13_local)
    T, H = x.shape
    ids = np.asarray(ids)
    k = ids.shape[1]
    emap = np.asarray(expert_map, np.int64)
    flat_local = emap[ids.reshape(-1)]
    flat_w = np.asarray(w, np.float64).reshape(-1)
    y = np.zeros((T * k, H))
    for l in range(W1.shape[0]):
        rows = np.nonzero(flat_local == l)[0]
        if rows.size == 0:
            continue
        xe = x[rows // k]
        a = silu(xe @ W1[l].T) * (xe @ W3[l].T)
        if round_a:
            a = bf16_round(a)
        y[rows] = flat_w[rows, None] * (a @ w2_local[l].T)
    out = np.zeros((T, H))
    for j in range(k):
        out += y[j::k]
    return out


# --------------------------------------------------------------------------- shared expert ([MKR] s1 table)

def add_shared_slot(ids, w, E):
    """Routing with the shared expert (reading 17): every token gets one more slot, j = k,
    holding expert E (the shared one) with weight 1."""
    ids = np.asarray(ids)
    T = ids.shape[0]
    ids_s = np.concatenate([ids, np.full((T, 1), E, ids.dtype)], axis=1)
    w_s = np.concatenate([np.asarray(w, np.float64), np.ones((T, 1))], axis=1)
    return ids_s, w_s


def moe_layer_shared(x, wg, w13, w2, k, mode, offset=None, bias=None, n_group=0, topk_group=0,
                     scaling=1.0, round_a=False):
    """Layer with one shared expert ([MKR] s1 table: DeepSeek-V3 and Kimi K2 have routed
    experts '+1 shared'): routing over the E routed experts (Wg has E rows), then the
    per-expert loop over the k routed slots plus the shared slot (expert E of w13 / w2,
    weight 1)."""
    E = np.asarray(wg).shape[0]
    logits32 = router_logits(x, wg).astype(np.float32)
    ids, w = route(logits32, k, mode, offset, bias, n_group, topk_group, scaling)
    ids_s, w_s = add_shared_slot(ids, w, E)
    out = moe_loop(x, w13, w2, ids_s, w_s, round_a=round_a)
    return out, ids_s, w_s, logits32


def expert_flops(T, k, H, I) -> int:
    """Useful expert FLOPs: 2 * T * k * 3 * H * I (two GEMMs of 2I and I outputs)."""
    return 2 * T * k * 3 * H * I


# --------------------------------------------------------------------------- routing margins

def selection_scores(logits32, mode, offset=None, bias=None) -> np.ndarray:
    """The float32 scores the router compares (float64 copy): logits (+ offset) for the
    softmax rules, sigmoid(logit) + bias for the grouped sigmoid rule ([MKR] s4)."""
    l = f32(logits32)
    if offset is not None:
        l = (l + f32(offset)[None, :]).astype(np.float32)
    if mode == SIGMOID_BIAS_GROUPED:
        b = np.zeros(l.shape[1], np.float32) if bias is None else f32(bias)
        return (sigmoid_f32(l) + b[None, :]).astype(np.float32).astype(np.float64)
    return l.astype(np.float64)


def selection_margin(logits32, k, mode, offset=None, bias=None, n_group=0, topk_group=0):
    """Per token, a radius rho in selection-score units: every perturbation of the scores
    that moves no score by rho or more leaves the SET of selected experts unchanged (slot
    order may still swap between near-equal selected experts).  A token whose scores are
    known only to within rho may be routed either way by a correct implementation.

    Derivation (scores c; S = selected set, c_k = its smallest score):
    * plain top-k (the softmax rules, or the sigmoid rule without group limit): S changes
      only if a selected and an unselected score cross, each moving at most rho, so
      rho = (c_k - best unselected) / 2;
    * group-limited top-k ([MKR] s4): a group score is the sum of the group's two largest
      scores, so it moves by at most 2 rho.  Within the kept groups' candidates the
      k-th / (k+1)-th gap gives (gap) / 2 as above.  A kept group A can be displaced by a
      dropped group B only when G_A - G_B < 4 rho; that changes S if A holds a selected
      expert, and otherwise only if an expert of B then beats c_k, which needs
      (c_k - max c_B) < 2 rho.  So each (A, B) pair bounds rho by (G_A - G_B) / 4, or by
      the larger of that and (c_k - max c_B) / 2 when A holds no selected expert.
    rho is the minimum over these events: a sound lower bound of the true radius (exact
    when groups have two experts, where each event's perturbation is attained, up to the
    float32 rounding of the group sums, which the group events subtract)."""
    sc = selection_scores(logits32, mode, offset, bias)
    T, E = sc.shape
    rho = np.full(T, np.inf)
    grouped = mode == SIGMOID_BIAS_GROUPED and n_group and topk_group and topk_group < n_group
    for t in range(T):
        c = sc[t]
        if not grouped:
            o = order_first(c)
            if k < E:
                rho[t] = (c[o[k - 1]] - c[o[k]]) / 2
            continue
        gsz = E // n_group
        members = [np.arange(g * gsz, (g + 1) * gsz) for g in range(n_group)]
        # group scores as the router forms them (a float32 sum of the two largest)
        G = np.array([np.float32(np.sort(c[m])[-1]) + np.float32(np.sort(c[m])[-2])
                      for m in members], np.float32)
        kept = order_first(G)[:topk_group]
        dropped = [g for g in range(n_group) if g not in set(kept.tolist())]
        cand = np.concatenate([members[g] for g in kept])
        oc = order_first(c, cand)
        sel = set(oc[:k].tolist())
        ck = c[oc[k - 1]]
        r = (ck - c[oc[k]]) / 2 if oc.size > k else np.inf
        for A in kept:
            holds = any(e in sel for e in members[A].tolist())
            for B in dropped:
                # the float32 rounding of each perturbed group sum may add half an
                # ulp on either side of the pair
                ulp = float(np.spacing(np.float32(max(abs(G[A]), abs(G[B])))))
                eps = (float(G[A]) - float(G[B]) - 2 * ulp) / 4
                if not holds:
                    eps = max(eps, (ck - c[members[B]].max()) / 2)
                r = min(r, eps)
        rho[t] = max(r, 0.0)
    return rho
