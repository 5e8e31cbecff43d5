"""Pins of the CPU oracle to facts outside itself: values the pages print for worked
examples (tests/golden/*.json, each with its citation), closed forms, library routines,
brute force and invariants.  CPU only."""
import itertools
import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from synth import inputs as S

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------- align

def test_align_worked_example_both_implementations():
    g = gold("align_worked_example.json")
    ids = np.array(g["topk_ids"], np.int32)
    assert ids.reshape(-1).tolist() == g["flat"]
    for impl in (O.align_runs, O.align_counting):
        r = impl(ids, g["num_experts"], g["block_m"])
        assert r["sorted_ids"].tolist() == g["sorted_ids"]
        assert r["expert_ids"].tolist() == g["expert_ids"]
        assert r["total"] == g["total"]
        assert round(100 * (1 - g["useful"] / r["total"])) == g["waste_percent"]


def test_align_padded_totals_match_printed_test_matrix():
    g = gold("fused_test_matrix.json")
    bm = g["block_m"]
    for name, c in g["cases"].items():
        ids = S.ids_with_counts(c["loads"], c["k"], seed=3).numpy()
        assert ids.shape == (c["T"], c["k"])
        for impl in (O.align_runs, O.align_counting):
            r = impl(ids, c["E"], bm)
            assert r["total"] == c["padded"], name
            assert r["counts"].tolist() == c["loads"]


def _check_align_invariants(ids, E, bm, r, cap):
    flat = ids.reshape(-1)
    R = flat.size
    counts = r["counts"]
    assert counts.sum() == R
    total = r["total"]
    assert total % bm == 0 and total <= cap
    si, ei = r["sorted_ids"], r["expert_ids"]
    assert si.size == cap and ei.size == cap // bm
    real = si[:total][si[:total] < R]
    assert sorted(real.tolist()) == list(range(R))             # every row exactly once
    assert np.all(si[total:] == R) and np.all(ei[total // bm:] == -1)
    tiles = ei[: total // bm]
    assert np.all(np.diff(tiles) >= 0)                         # experts ascending
    for e in range(E):
        nt = int((tiles == e).sum())
        assert nt == -(-int(counts[e]) // bm)                  # ceil(n_e / BM) tiles, none if empty
    for p in range(total // bm):                               # each tile's rows belong to its expert,
        blk = si[p * bm:(p + 1) * bm]                          # in ascending order, sentinel after
        v = blk[blk < R]
        assert np.all(flat[v] == tiles[p])
        assert np.all(np.diff(v) > 0)
        nv = v.size
        assert np.all(blk[:nv] < R) and np.all(blk[nv:] == R)


@pytest.mark.parametrize("bm", [1, 4, 16, 64, 128, 256])
@pytest.mark.parametrize("T,k,E,skew", [(1, 8, 256, 0.0), (37, 1, 8, 0.0), (64, 2, 8, 0.0),
                                          (300, 8, 128, 1.2), (50, 4, 16, 0.0)])
def test_align_invariants_and_implementations_agree(bm, T, k, E, skew):
    ids = S.random_topk_ids(T, k, E, seed=T + E, skew=skew).numpy()
    cap = O.align_capacity(T, k, E, bm)
    a = O.align_runs(ids, E, bm, cap)
    b = O.align_counting(ids, E, bm, cap)
    for key in ("sorted_ids", "expert_ids", "counts"):
        assert np.array_equal(a[key], b[key]), key
    assert a["total"] == b["total"]
    _check_align_invariants(ids, E, bm, a, cap)


def test_align_edge_counts():
    """Experts at 0, 1, BM-1, BM, BM+1 rows, and one expert receiving every token."""
    bm = 16
    loads = [0, 1, bm - 1, bm, bm + 1, 0, 2 * bm, 3]
    k = 2
    pad = (-sum(loads)) % k
    loads[-1] += pad
    ids = S.ids_with_counts(loads, k, seed=5).numpy()
    cap = O.align_capacity(ids.shape[0], k, len(loads), bm)
    r = O.align_runs(ids, len(loads), bm, cap)
    _check_align_invariants(ids, len(loads), bm, r, cap)
    assert r["total"] == sum(-(-c // bm) * bm for c in loads)
    hot = S.random_topk_ids(100, 4, 16, seed=1, hot=3).numpy()
    r = O.align_counting(hot, 16, bm, O.align_capacity(100, 4, 16, bm))
    assert r["counts"][3] == 100
    _check_align_invariants(hot, 16, bm, r, O.align_capacity(100, 4, 16, bm))


def test_align_capacity_is_tight_bound():
    # every non-empty expert pads by at most BM-1 rows; the bound is reached when every
    # expert has exactly one row beyond a multiple of BM
    T, k, E, bm = 8, 2, 4, 4
    loads = [5, 5, 1, 5]
    ids = S.ids_with_counts(loads, k).numpy()
    r = O.align_runs(ids, E, bm)
    assert r["total"] == 8 + 8 + 4 + 8 == 28
    assert O.align_capacity(T, k, E, bm) >= r["total"]
    assert O.align_capacity(1, 8, 256, 64) == 8 * 64


# ----------------------------------------------------------------------------- routing

def test_tiny_layer_counts_and_flops():
    g = gold("tiny_layer.json")
    lay = S.make_layer(S.WORKLOADS["tiny"])
    x, wg = lay.x.numpy(), lay.wg.numpy()
    logits32 = O.router_logits(x, wg).astype(np.float32)
    ids, w = O.route(logits32, g["k"], O.SOFTMAX_TOPK_RENORM)
    counts = np.bincount(ids.reshape(-1), minlength=g["E"])
    assert counts.tolist() == g["tokens_per_expert"]
    assert counts.sum() == g["sum"]
    fl = O.expert_flops(g["T"], g["k"], g["H"], g["I"])
    assert fl == 4718592
    assert round(fl / 1e6, 1) == g["routed_mflop"]
    assert round(fl * g["E"] / g["k"] / 1e6, 1) == g["dense_mflop"]


def test_test_matrix_loads():
    g = gold("fused_test_matrix.json")
    for name, c in g["cases"].items():
        x, wg, w1, w3, w2, k = S.page_test_case(name)
        logits32 = O.router_logits(x.numpy(), wg.numpy()).astype(np.float32)
        ids, _ = O.route(logits32, k, O.SOFTMAX_TOPK_RENORM)
        assert np.bincount(ids.reshape(-1), minlength=c["E"]).tolist() == c["loads"], name
        assert O.align_runs(ids, c["E"], g["block_m"])["total"] == c["padded"]


def test_grouped_router_worked_example():
    g = gold("grouped_router_example.json")
    logits, bias = S.page_grouped_router_logits()
    l32 = logits.numpy().astype(np.float32)
    args = dict(n_group=g["n_group"], topk_group=g["topk_group"], scaling=g["scaling"])
    ids0, _ = O.route(l32, g["k"], O.SIGMOID_BIAS_GROUPED, bias=np.zeros(16, np.float32), **args)
    assert ids0.tolist() == g["ids_no_bias"]
    ids1, w1 = O.route(l32, g["k"], O.SIGMOID_BIAS_GROUPED, bias=bias.numpy(), **args)
    assert ids1.tolist() == g["ids_with_bias"]
    gsz = g["E"] // g["n_group"]
    assert [sorted(set((r // gsz).tolist())) for r in ids1] == g["groups_per_token"]
    assert np.allclose(w1, np.array(g["weights_right_3dp"]), atol=5e-4 + 1e-9)
    assert np.allclose(w1.sum(1), g["scaling"])
    # the bias leak: weights from the biased scores instead of the unbiased ones
    s = O.sigmoid_f32(l32).astype(np.float64)
    c = s + bias.numpy().astype(np.float64)[None, :]
    cb = np.take_along_axis(c, ids1.astype(np.int64), 1)
    w_bug = g["scaling"] * cb / cb.sum(1, keepdims=True)
    assert np.allclose(w_bug, np.array(g["weights_bias_leak_3dp"]), atol=5e-4 + 1e-9)
    assert round(float(np.abs(w1 - w_bug).max()), 3) == g["max_weight_error_bias_leak_3dp"]


def test_softmax_renorm_matches_library_softmax_topk():
    """Reduces to torch.softmax -> torch.topk -> renormalise (float64) when no two
    logits tie."""
    rng = np.random.default_rng(0)
    l32 = rng.standard_normal((200, 64)).astype(np.float32)
    for k in (1, 2, 4, 8):
        ids, w = O.route(l32, k, O.SOFTMAX_TOPK_RENORM)
        p = torch.softmax(torch.from_numpy(l32.astype(np.float64)), dim=-1)
        tw, tid = torch.topk(p, k, dim=-1)
        tw = tw / tw.sum(-1, keepdim=True)
        assert np.array_equal(ids, tid.numpy())
        assert np.allclose(w, tw.numpy(), rtol=1e-13, atol=0)
        ids2, w2 = O.route(l32, k, O.TOPK_THEN_SOFTMAX)   # identical arithmetic by the identity
        assert np.array_equal(ids, ids2) and np.array_equal(w, w2)
        if k == 1:
            assert np.all(w == 1.0)


def test_route_ties_lower_index_wins():
    l32 = np.array([[1.0, 3.0, 3.0, 2.0, 3.0]], np.float32)
    ids, _ = O.route(l32, 2, O.SOFTMAX_TOPK_RENORM)
    assert ids.tolist() == [[1, 2]]
    ids, _ = O.route(l32, 4, O.SOFTMAX_TOPK_RENORM)
    assert ids.tolist() == [[1, 2, 4, 3]]
    # groups: two groups with equal scores -> the lower group is kept
    l = np.zeros((1, 8), np.float32)
    ids, w = O.route(l, 2, O.SIGMOID_BIAS_GROUPED, n_group=2, topk_group=1, scaling=2.5)
    assert ids.tolist() == [[0, 1]] and np.allclose(w, 1.25)


def test_route_offset_applies_to_selection_and_weights():
    rng = np.random.default_rng(1)
    l32 = rng.standard_normal((64, 16)).astype(np.float32)
    off = np.zeros(16, np.float32)
    off[:2] = 3.0
    ids_o, w_o = O.route(l32, 4, O.TOPK_THEN_SOFTMAX, offset=off)
    ids_s, w_s = O.route((l32 + off).astype(np.float32), 4, O.TOPK_THEN_SOFTMAX)
    assert np.array_equal(ids_o, ids_s) and np.array_equal(w_o, w_s)
    assert (np.isin(ids_o, [0, 1]).sum(1) == 2).mean() > 0.8


def _brute_grouped(c_row, s_row, k, n_group, topk_group, scaling):
    """Enumerate every choice of groups, then every k-subset inside them."""
    E = c_row.size
    gsz = E // n_group
    gs = [sorted(c_row[g * gsz:(g + 1) * gsz].tolist())[-2:] for g in range(n_group)]
    gscore = [np.float32(a) + np.float32(b) for a, b in gs]
    best = max(itertools.combinations(range(n_group), topk_group),
               key=lambda G: (sorted([gscore[g] for g in G], reverse=True), [-g for g in G]))
    cand = [e for g in sorted(best) for e in range(g * gsz, (g + 1) * gsz)]
    sel = max(itertools.combinations(cand, k), key=lambda S_: (sorted([c_row[e] for e in S_], reverse=True),
                                                              [-e for e in sorted(S_)]))
    sel = sorted(sel, key=lambda e: (-c_row[e], e))
    sw = np.array([s_row[e] for e in sel], np.float64)
    return sel, scaling * sw / sw.sum()


def test_grouped_router_brute_force():
    rng = np.random.default_rng(2)
    E, k, G, TG = 12, 3, 4, 2
    l32 = rng.standard_normal((40, E)).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.3).astype(np.float32)
    ids, w = O.route(l32, k, O.SIGMOID_BIAS_GROUPED, bias=bias, n_group=G, topk_group=TG, scaling=2.5)
    s = O.sigmoid_f32(l32)
    c = (s + bias[None]).astype(np.float32)
    for t in range(40):
        sel, wb = _brute_grouped(c[t], s[t], k, G, TG, 2.5)
        assert ids[t].tolist() == sel
        assert np.allclose(w[t], wb, rtol=1e-14)


def test_sigmoid_f32_is_correctly_rounded():
    getcontext().prec = 60
    rng = np.random.default_rng(3)
    vals = np.concatenate([rng.standard_normal(400) * 4, rng.uniform(-30, 30, 400),
                           np.array([0.0, 1.0, -1.0, 20.0, -20.0])]).astype(np.float32)
    got = O.sigmoid_f32(vals)
    for v, s in zip(vals.tolist(), got.tolist()):
        ex = Decimal(1) / (Decimal(1) + (-Decimal(v)).exp())
        lo = np.float32(s)
        # the float32 neighbours of s must both be farther from the exact value
        up = np.nextafter(lo, np.float32(2))
        dn = np.nextafter(lo, np.float32(-1))
        d = abs(Decimal(float(lo)) - ex)
        assert d <= abs(Decimal(float(up)) - ex) and d <= abs(Decimal(float(dn)) - ex), v


# ----------------------------------------------------------------------------- rounding

def test_bf16_round_matches_torch_conversion():
    rng = np.random.default_rng(4)
    v = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-8, 8, 100000),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0])])
    v32 = v.astype(np.float32)                                 # exactly representable inputs
    ref = torch.from_numpy(v32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.bf16_round(v32.astype(np.float64)), ref)
    # ties go to even: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7
    assert O.bf16_round(1.0 + 2 ** -8) == 1.0
    assert O.bf16_round(1.0 + 3 * 2 ** -8) == 1.0 + 2 ** -6


# ----------------------------------------------------------------------------- expert math

def _rand_layer(T, H, I, E, k, seed, mode=O.SOFTMAX_TOPK_RENORM):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    wg = rng.standard_normal((E, H)) / math.sqrt(H)
    w13 = rng.standard_normal((E, 2 * I, H)) / math.sqrt(H)
    w2 = rng.standard_normal((E, H, I)) / math.sqrt(I)
    l32 = O.router_logits(x, wg).astype(np.float32)
    ids, w = O.route(l32, k, mode, n_group=2 if mode == 2 else 0, topk_group=1 if mode == 2 else 0,
                     scaling=2.5 if mode == 2 else 1.0)
    return x, wg, w13, w2, ids, w


def test_silu_known_value():
    # silu(1) = 1 / (1 + e^-1)
    assert O.silu(1.0) == pytest.approx(0.7310585786300049, rel=1e-15)
    # the layer reduces to it for H = I = E = k = 1 with unit weights
    out = O.moe_loop(np.ones((1, 1)), np.ones((1, 2, 1)), np.ones((1, 1, 1)),
                     np.zeros((1, 1), np.int32), np.ones((1, 1)))
    assert out[0, 0] == pytest.approx(0.7310585786300049, rel=1e-15)


def test_gate_and_up_roles():
    """W13 = [W1; W3]: the gate half goes through silu.  A very negative gate
    pre-activation switches the expert off whatever the up half is."""
    rng = np.random.default_rng(5)
    H, I = 8, 6
    x = np.abs(rng.standard_normal((3, H))) + 0.1
    w13 = rng.standard_normal((1, 2 * I, H))
    w13[0, :I] = -40.0                                   # gate rows
    w2 = rng.standard_normal((1, H, I))
    ids = np.zeros((3, 1), np.int32)
    out = O.moe_loop(x, w13, w2, ids, np.ones((3, 1)))
    assert np.abs(out).max() < 1e-30
    w13b = w13.copy()
    w13b[0, :I], w13b[0, I:] = w13[0, I:], w13[0, :I]     # swapped halves are not off
    assert np.abs(O.moe_loop(x, w13b, w2, ids, np.ones((3, 1)))).max() > 1e-3


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_loop_dense_bruteforce_agree(mode):
    x, wg, w13, w2, ids, w = _rand_layer(6, 8, 6, 4, 2, seed=10 + mode, mode=mode)
    a = O.moe_loop(x, w13, w2, ids, w)
    b = O.moe_dense(x, w13, w2, ids, w)
    c = O.moe_bruteforce(x, w13, w2, ids, w)
    assert np.abs(a - b).max() <= 1e-13 * np.abs(a).max()
    assert np.abs(a - c).max() <= 1e-13 * np.abs(a).max()
    ar = O.moe_loop(x, w13, w2, ids, w, round_a=True)
    cr = O.moe_bruteforce(x, w13, w2, ids, w, round_a=True)
    assert np.abs(ar - cr).max() <= 1e-12 * np.abs(ar).max()
    assert np.abs(ar - a).max() > 0                   # the bf16 rounding point is real


@pytest.mark.parametrize("mode", [0, 2])
def test_stage_functions_compose_to_the_layer(mode):
    """GEMM1+SwiGLU rows, the bf16 rounding of a, then GEMM2 x weight + combine give the
    per-expert loop and the scalar brute force; slots of experts outside [0, E) add
    nothing (the two halves of a split of the experts add up to the layer)."""
    rng = np.random.default_rng(mode + 40)
    T, H, I, E, k = 9, 12, 10, 6, 3
    x = rng.standard_normal((T, H))
    w13 = rng.standard_normal((E, 2 * I, H)) / np.sqrt(H)
    w2 = rng.standard_normal((E, H, I)) / np.sqrt(I)
    l32 = rng.standard_normal((T, E)).astype(np.float32)
    kw = dict(n_group=3, topk_group=2, scaling=2.5) if mode == 2 else {}
    ids, w = O.route(l32, k, mode, **kw)
    for rnd in (False, True):
        a = O.swiglu_rows(x, w13, ids)
        out = O.down_and_combine(O.bf16_round(a) if rnd else a, w2, ids, w)
        assert np.allclose(out, O.moe_loop(x, w13, w2, ids, w, round_a=rnd), rtol=1e-12, atol=1e-13)
        assert np.allclose(out, O.moe_bruteforce(x, w13, w2, ids, w, round_a=rnd), rtol=1e-11,
                           atol=1e-12)
    half = np.where(ids < 3, ids, -1)
    other = np.where(ids >= 3, ids - 3, -1)
    a0 = O.swiglu_rows(x, w13[:3], half)
    a1 = O.swiglu_rows(x, w13[3:], other)
    assert np.allclose(a0 + a1, O.swiglu_rows(x, w13, ids), rtol=0, atol=0)
    both = O.down_and_combine(a0, w2[:3], half, w) + O.down_and_combine(a1, w2[3:], other, w)
    assert np.allclose(both, O.moe_loop(x, w13, w2, ids, w), rtol=1e-12, atol=1e-13)


def test_loop_vs_dense_tiny_layer():
    g = gold("tiny_layer.json")
    lay = S.make_layer(S.WORKLOADS["tiny"])
    x, wg, w13, w2 = (t.numpy() for t in (lay.x, lay.wg, lay.w13, lay.w2))
    out, ids, w, _ = O.moe_layer(x, wg, w13, w2, 2, O.SOFTMAX_TOPK_RENORM)
    dense = O.moe_dense(x, w13, w2, ids, w)
    assert np.abs(out - dense).max() <= 1e-12 + g["max_abs_loop_minus_dense"]


def test_k_equals_E_is_dense_softmax_mixture():
    """k = E with renormalisation: every expert weighted by the full softmax."""
    x, wg, w13, w2, _, _ = _rand_layer(5, 8, 6, 4, 4, seed=20)
    l32 = O.router_logits(x, wg).astype(np.float32)
    ids, w = O.route(l32, 4, O.SOFTMAX_TOPK_RENORM)
    p = torch.softmax(torch.from_numpy(l32.astype(np.float64)), -1).numpy()
    assert np.allclose(np.take_along_axis(p, ids.astype(np.int64), 1), w, rtol=1e-13)
    out = O.moe_loop(x, w13, w2, ids, w)
    ref = O.moe_bruteforce(x, w13, w2, np.tile(np.arange(4, dtype=np.int32), (5, 1)), p)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-14)


def test_metamorphic_properties():
    x, wg, w13, w2, ids, w = _rand_layer(9, 8, 6, 5, 2, seed=30)
    out = O.moe_loop(x, w13, w2, ids, w)
    # scaling every W2 by 2 scales the output by exactly 2
    assert np.array_equal(O.moe_loop(x, w13, 2 * w2, ids, w), 2 * out)
    # permuting tokens permutes the output rows
    perm = np.random.default_rng(0).permutation(9)
    assert np.allclose(O.moe_loop(x[perm], w13, w2, ids[perm], w[perm]), out[perm], rtol=1e-14)
    # relabelling experts (router rows, weights, ids together) leaves the output unchanged
    rel = np.random.default_rng(1).permutation(5)
    inv = np.argsort(rel)
    out2 = O.moe_loop(x, w13[rel], w2[rel], inv[ids].astype(np.int32), w)
    assert np.allclose(out2, out, rtol=1e-14)
    # slot j's weight multiplies expert ids[t, j]: doubling expert e's W2 adds w_e * F_e
    e = int(ids[0, 0])
    w2b = w2.copy()
    w2b[e] *= 2
    only_e = np.where(ids == e, w, 0.0)
    f_e = O.moe_loop(x, w13, w2, ids, only_e)
    assert np.allclose(O.moe_loop(x, w13, w2b, ids, w), out + f_e, rtol=1e-13, atol=1e-15)
    # an expert that receives no rows never influences the output
    unused = [q for q in range(5) if q not in ids]
    if unused:
        w13c = w13.copy()
        w13c[unused[0]] = np.nan
        assert np.array_equal(O.moe_loop(x, w13c, w2, ids, w), out)


def test_identical_experts_sum_of_weights():
    """Two identical experts: the output is (sum of the token's weights) x one expert;
    the grouped router's weights sum to its scale."""
    rng = np.random.default_rng(7)
    T, H, I = 4, 8, 6
    x = rng.standard_normal((T, H))
    one13 = rng.standard_normal((1, 2 * I, H))
    one2 = rng.standard_normal((1, H, I))
    ref = O.moe_loop(x, one13, one2, np.zeros((T, 1), np.int32), np.ones((T, 1)))
    l32 = rng.standard_normal((T, 4)).astype(np.float32)
    ids, w = O.route(l32, 2, O.SIGMOID_BIAS_GROUPED, n_group=2, topk_group=1, scaling=2.5)
    out = O.moe_loop(x, np.repeat(one13, 4, 0), np.repeat(one2, 4, 0), ids, w)
    assert np.allclose(out, 2.5 * ref, rtol=1e-13)


def _bias_route_set(c_target, k, ng, tg):
    """Selected set of the grouped sigmoid router when every logit is 0 (sigmoid = 1/2
    exactly) and the bias carries the scores: c = fl32(1/2 + bias)."""
    b = (np.asarray(c_target, np.float64) - 0.5).astype(np.float32)
    ids, _ = O.route(np.zeros((1, b.size), np.float32), k, O.SIGMOID_BIAS_GROUPED, bias=b,
                     n_group=ng, topk_group=tg)
    return frozenset(ids[0].tolist())


def _bias_margin(c_target, k, ng, tg):
    b = (np.asarray(c_target, np.float64) - 0.5).astype(np.float32)
    return float(O.selection_margin(np.zeros((1, b.size), np.float32), k, O.SIGMOID_BIAS_GROUPED,
                                    bias=b, n_group=ng, topk_group=tg)[0])


def test_selection_margin_plain_topk_closed_form():
    """Plain top-k: half the gap between the k-th and (k+1)-th score (each side may move
    by the radius)."""
    l32 = np.array([[1.0, 0.5, 0.25, 0.0]], np.float32)
    assert O.selection_margin(l32, 2, 0)[0] == 0.125
    assert O.selection_margin(l32, 2, 1)[0] == 0.125
    # the offset is part of the selection score
    off = np.array([0.0, 0.0, 0.5, 0.0], np.float32)
    assert O.selection_margin(l32, 2, 0, offset=off)[0] == 0.125      # 0.75 vs 0.5
    assert O.selection_margin(l32, 4, 0)[0] == np.inf                 # k = E: nothing to swap


def test_selection_margin_grouped_closed_forms():
    """[MKR] s4 group-limited routing, scores set exactly through the bias (4 groups of 2,
    keep 2, top-2)."""
    # three groups tied at 1.5: the tie rule keeps groups 0 and 1, group 1 holds a selected
    # expert, so no perturbation is safe
    c = [0.9, 0.6, 0.8, 0.7, 0.75, 0.75, 0.5, 0.5]
    assert _bias_route_set(c, 2, 4, 2) == {0, 2}
    assert _bias_margin(c, 2, 4, 2) == 0.0
    # the kept/dropped group gap binds: G1 = 1.30 vs G2 = 1.28 -> about 0.02 / 4
    c = [0.95, 0.60, 0.90, 0.40, 0.66, 0.62, 0.1, 0.1]
    m = _bias_margin(c, 2, 4, 2)
    c32 = (np.float32(0.5) + (np.asarray(c) - 0.5).astype(np.float32)).astype(np.float64)
    g1 = float(np.float32(c32[2]) + np.float32(c32[3]))
    g2 = float(np.float32(c32[4]) + np.float32(c32[5]))
    assert m == pytest.approx((g1 - g2) / 4, abs=1e-6)
    # the last kept group holds no selected expert and the dropped group's best expert is
    # far below the k-th: the group swap cannot change the set, the expert gap binds
    c = [0.95, 0.90, 0.60, 0.59, 0.58, 0.57, 0.1, 0.1]
    assert _bias_route_set(c, 2, 4, 2) == {0, 1}
    c32 = (np.float32(0.5) + (np.asarray(c) - 0.5).astype(np.float32)).astype(np.float64)
    assert _bias_margin(c, 2, 4, 2) == pytest.approx((c32[1] - c32[2]) / 2, abs=1e-7)


def _grouped_instance(rng, E, ng, tg, k):
    """Scores for the bias-carried router: well separated values (no exact ties)."""
    return np.round(rng.uniform(0.0, 1.0, E), 4)


@pytest.mark.parametrize("E,ng,tg,k", [(8, 4, 2, 2), (8, 4, 1, 2), (8, 4, 3, 3), (8, 2, 1, 1),
                                       (6, 3, 1, 2)])
def test_selection_margin_grouped_brute_force(E, ng, tg, k):
    """Brute force over every perturbation with components in {-eps, 0, +eps} (3^E of
    them): below the reported radius the selected set never changes; just above it some
    perturbation changes it (groups of two experts, where the bound is exact).  Plus
    random perturbations inside the radius."""
    rng = np.random.default_rng(E * 100 + ng * 10 + tg + k)
    corners = np.array(list(itertools.product((-1.0, 0.0, 1.0), repeat=E)))
    exact = E // ng == 2
    checked = 0
    for trial in range(40):
        c = _grouped_instance(rng, E, ng, tg, k)
        m = _bias_margin(c, k, ng, tg)
        if not (1e-4 < m < 0.2):
            continue
        base = _bias_route_set(c, k, ng, tg)
        below = 0.999 * m
        for d in corners:
            assert _bias_route_set(c + below * d, k, ng, tg) == base
        for _ in range(200):
            d = rng.uniform(-below, below, E)
            assert _bias_route_set(c + d, k, ng, tg) == base
        if exact:
            above = 1.002 * m
            assert any(_bias_route_set(c + above * d, k, ng, tg) != base for d in corners), \
                f"radius {m} is not attained: the bound is loose on {c}"
        checked += 1
        if checked == 4:
            break
    assert checked >= 2


@pytest.mark.parametrize("mode", [0, 1])
def test_selection_margin_plain_brute_force(mode):
    """Softmax rules: perturbing the logits by just under the radius never changes the
    selected set; moving the k-th down and the (k+1)-th up by just over it does."""
    rng = np.random.default_rng(5 + mode)
    E, k = 7, 3
    for _ in range(30):
        l = rng.standard_normal((1, E)).astype(np.float32)
        m = float(O.selection_margin(l, k, mode)[0])
        base = set(O.route(l, k, mode)[0][0].tolist())
        for _ in range(300):
            d = rng.uniform(-0.999 * m, 0.999 * m, E).astype(np.float32)
            assert set(O.route((l + d).astype(np.float32), k, mode)[0][0].tolist()) == base
        o = np.argsort(-l[0].astype(np.float64), kind="stable")
        d = np.zeros(E, np.float32)
        d[o[k - 1]], d[o[k]] = -1.002 * m, 1.002 * m
        assert set(O.route((l + d[None]).astype(np.float32), k, mode)[0][0].tolist()) != base


# ----------------------------------------------------------------------------- FP8 weights

def _torch_e4m3(codes):
    """torch's own E4M3 decoding (the library routine, independent of the oracle's)."""
    c = torch.as_tensor(np.asarray(codes, np.uint8))
    return c.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_fp8_decode_all_codes_match_library():
    codes = np.arange(256)
    ours = O.fp8_e4m3_decode(codes)
    ref = _torch_e4m3(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))


def test_fp8_decode_closed_forms():
    # OCP 8-bit floating point, E4M3: bias 7, no infinities, one NaN mantissa pattern
    v = O.fp8_e4m3_value
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0              # largest finite
    assert v(0x01) == 2.0 ** -9 and v(0x07) == 7 * 2.0 ** -9   # subnormals m/8 * 2^-6
    assert v(0x08) == 2.0 ** -6                                # smallest normal
    assert v(0x38) == 1.0 and v(0xB8) == -1.0 and v(0x3C) == 1.5
    assert v(0x00) == 0.0 and math.copysign(1.0, v(0x80)) == -1.0
    nan = [c for c in range(256) if math.isnan(v(c))]
    assert nan == [0x7F, 0xFF]
    pos = [v(c) for c in range(0x7F)]
    assert all(b > a for a, b in zip(pos, pos[1:]))              # codes order the values
    assert all(v(c | 0x80) == -v(c) for c in range(0x7F))


def test_fp8_row_quantisation_error_bound():
    """Decoded codes times the row scale recover each weight to E4M3's rounding bound:
    half an ulp (2^-4 relative) in the normal range, half the subnormal step (2^-10 of
    the scale) below it.  A scale applied along the wrong axis breaks the bound."""
    g = torch.Generator().manual_seed(5)
    w = torch.randn(3, 40, 24, generator=g) * torch.rand(3, 40, 1, generator=g) * 4
    codes, scale = S.quantize_fp8_rows(w)
    deq = O.dequant_rows(codes.numpy(), scale.numpy())
    wn = w.double().numpy()
    sc = scale.double().numpy()[..., None]
    bound = np.maximum(2.0 ** -4 * np.abs(wn), 2.0 ** -10 * sc) * (1 + 1e-6) + 1e-30
    assert np.all(np.abs(deq - wn) <= bound)
    # the row maximum maps onto the largest code
    assert np.all(np.abs(deq).max(axis=-1) == pytest.approx(np.abs(wn).max(axis=-1), rel=1e-6))


def test_fp8_layer_matches_bruteforce():
    wl = S.WORKLOADS["deepseek_decode_fp8"].scaled(T=3, H=16, I=12, E=32, n_group=8,
                                                   topk_group=4)
    lay = S.make_layer(wl, seed=3)
    x = lay.x.double().numpy()
    out, ids, w, _ = O.moe_layer_fp8(x, lay.wg.double().numpy(), lay.w13.numpy(),
                                     lay.w13_scale.numpy(), lay.w2.numpy(), lay.w2_scale.numpy(),
                                     wl.k, wl.mode, None, lay.bias.numpy(), wl.n_group,
                                     wl.topk_group, wl.scaling)
    w13 = _torch_e4m3(lay.w13.numpy()) * lay.w13_scale.double().numpy()[..., None]
    w2 = _torch_e4m3(lay.w2.numpy()) * lay.w2_scale.double().numpy()[..., None]
    ref = O.moe_bruteforce(x, w13, w2, ids, w, round_a=True)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- expert parallelism

def _half_maps(E, seed):
    """Two expert maps that split the E experts between two GPUs at random."""
    perm = np.random.default_rng(seed).permutation(E)
    owner = np.zeros(E, np.int64)
    owner[perm[E // 2:]] = 1
    maps = []
    for g in range(2):
        m = np.full(E, -1, np.int32)
        mine = np.nonzero(owner == g)[0]
        m[mine] = np.arange(mine.size)
        maps.append(m)
    return maps


def test_ep_shares_sum_to_the_layer():
    """[MKR] s11 exercise, 'half the experts remote': the two GPUs' shares add up to the
    whole layer, and a map that keeps every expert local is the layer itself."""
    x, wg, w1, w3, w2, k = S.page_test_case("skewed")
    w13 = torch.cat([w1, w3], dim=1).double().numpy()
    w2 = w2.double().numpy()
    x = x.double().numpy()
    l32 = O.router_logits(x, wg.double().numpy()).astype(np.float32)
    ids, w = O.route(l32, k, O.SOFTMAX_TOPK_RENORM)
    full = O.moe_loop(x, w13, w2, ids, w)
    E = w13.shape[0]
    parts = []
    for m in _half_maps(E, 4):
        mine = np.nonzero(m >= 0)[0]
        order = np.argsort(m[mine])
        parts.append(O.moe_loop_ep(x, w13[mine[order]], w2[mine[order]], ids, w, m))
        # each share alone misses the other half's experts
        assert np.abs(parts[-1] - full).max() > 1e-3
    assert np.allclose(parts[0] + parts[1], full, rtol=1e-12, atol=1e-12)
    ident = np.arange(E, dtype=np.int32)
    assert np.allclose(O.moe_loop_ep(x, w13, w2, ids, w, ident), full, rtol=1e-13, atol=1e-13)
    none = np.full(E, -1, np.int32)
    assert np.all(O.moe_loop_ep(x, w13[:0], w2[:0], ids, w, none) == 0.0)


def test_ep_align_marks_remote_tiles():
    """The EP table keeps the global sorted_ids and total; tiles of remote experts carry -1,
    local ones the local index, the cap tail stays -1."""
    ids = S.random_topk_ids(300, 8, 64, seed=3, skew=0.8).numpy()
    for bm in (16, 64):
        cap = O.align_capacity(300, 8, 64, bm)
        ref = O.align_runs(ids, 64, bm, cap)
        for m in _half_maps(64, bm):
            r = O.align_ep(ids, 64, bm, m, cap)
            assert np.array_equal(r["sorted_ids"], ref["sorted_ids"])
            assert r["total"] == ref["total"]
            nt = ref["total"] // bm
            for p in range(cap // bm):
                e = ref["expert_ids"][p]
                assert r["expert_ids"][p] == (m[e] if p < nt else -1)
            # every routed row of a local expert sits in a tile marked with its local index
            for p in range(nt):
                rows = r["sorted_ids"][p * bm:(p + 1) * bm]
                rows = rows[rows < ids.size]
                owner = m[ids.reshape(-1)[rows]]
                assert np.all(owner == r["expert_ids"][p])


# ----------------------------------------------------------------------------- shared expert

def test_shared_expert_adds_a_dense_swiglu_ffn():
    """The shared slot adds exactly the dense SwiGLU FFN of expert E to every token (no
    router weight); zero shared weights give the routed layer; the routing itself is the
    routed experts' (Wg has E rows)."""
    rng = np.random.default_rng(7)
    T, H, I, E, k = 9, 12, 10, 6, 2
    x = rng.standard_normal((T, H))
    wg = rng.standard_normal((E, H)) / H ** 0.5
    w13 = rng.standard_normal((E + 1, 2 * I, H)) / H ** 0.5
    w2 = rng.standard_normal((E + 1, H, I)) / I ** 0.5
    out, ids_s, w_s, l32 = O.moe_layer_shared(x, wg, w13, w2, k, O.SOFTMAX_TOPK_RENORM)
    routed, ids, w, _ = O.moe_layer(x, wg, w13[:E], w2[:E], k, O.SOFTMAX_TOPK_RENORM)
    assert np.array_equal(ids_s[:, :k], ids) and np.all(ids_s[:, k] == E)
    assert np.all(w_s[:, k] == 1.0) and np.allclose(w_s[:, :k], w)
    g = x @ w13[E, :I].T
    u = x @ w13[E, I:].T
    dense = (g / (1 + np.exp(-g)) * u) @ w2[E].T
    assert np.allclose(out - routed, dense, rtol=1e-11, atol=1e-12)
    z13, z2 = w13.copy(), w2.copy()
    z13[E] = 0.0
    z2[E] = 0.0
    out0, _, _, _ = O.moe_layer_shared(x, wg, z13, z2, k, O.SOFTMAX_TOPK_RENORM)
    assert np.allclose(out0, routed, rtol=1e-13, atol=1e-13)
    # brute force with the extra slot
    bf = O.moe_bruteforce(x, w13, w2, ids_s, w_s)
    assert np.allclose(out, bf, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- third implementation

@pytest.mark.parametrize("case", ["uniform", "skewed", "decode", "top1"])
def test_permute_grouped_matches_loop_and_library_grouped_mm(case):
    """[MKR] s10: loop, fused kernel and F.grouped_mm with explicit permute / un-permute.
    The oracle's permute path agrees with the per-expert loop (float64), and torch's own
    grouped GEMM on the same permuted layout (fp32, library routine) agrees with both."""
    import torch.nn.functional as F
    x, wg, w1, w3, w2, k = S.page_test_case(case)
    w13 = torch.cat([w1, w3], dim=1)
    x64, w13_64, w2_64 = x.double().numpy(), w13.double().numpy(), w2.double().numpy()
    l32 = O.router_logits(x64, wg.double().numpy()).astype(np.float32)
    ids, w = O.route(l32, k, O.SOFTMAX_TOPK_RENORM)
    loop = O.moe_loop(x64, w13_64, w2_64, ids, w)
    perm = O.moe_permute_grouped(x64, w13_64, w2_64, ids, w)
    assert np.allclose(perm, loop, rtol=1e-12, atol=1e-12)
    assert np.allclose(O.moe_permute_grouped(x64, w13_64, w2_64, ids, w, round_a=True),
                       O.moe_loop(x64, w13_64, w2_64, ids, w, round_a=True), rtol=1e-12, atol=1e-12)
    # torch's grouped GEMM (F.grouped_mm, fp32 on the CPU) as the library leg.  Its
    # contract: rows [ends[g-1], ends[g]) of the left operand multiply the g-th matrix of
    # the right one.  Routed (token, slot) pairs are ranked by the key expert * T*k +
    # (pair index), so each expert's pairs are one contiguous run; the runs' ends come
    # from where each expert's keys stop.
    E, I, T = w13.shape[0], w13.shape[1] // 2, x.shape[0]
    R = T * k
    eid = torch.from_numpy(ids.astype(np.int64)).reshape(-1)
    key, rank = torch.sort(eid * R + torch.arange(R))
    tok = rank // k
    ends = torch.searchsorted(key, (torch.arange(E) + 1) * R).to(torch.int32)
    lhs = x.index_select(0, tok)
    gate = F.grouped_mm(lhs, w13[:, :I].permute(0, 2, 1).contiguous(), offs=ends)
    up = F.grouped_mm(lhs, w13[:, I:].permute(0, 2, 1).contiguous(), offs=ends)
    act = (gate * torch.sigmoid(gate) * up).contiguous()
    rows = F.grouped_mm(act, w2.permute(0, 2, 1).contiguous(), offs=ends)
    wt = torch.from_numpy(w.astype(np.float32)).reshape(-1).index_select(0, rank)
    lib = torch.zeros(T, x.shape[1]).scatter_add_(
        0, tok[:, None].expand(-1, x.shape[1]), rows * wt[:, None]).double().numpy()
    assert np.abs(lib - loop).max() / np.abs(loop).max() < 1e-5
