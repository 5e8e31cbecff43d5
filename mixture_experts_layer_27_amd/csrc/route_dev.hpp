// Per-token expert selection by one wave (the top-k rules of "Mixture-of-Experts Kernels:
// Routing, Permutation, and Grouped GEMM", section 3 `route` and section 4 grouped
// sigmoid router), shared by the routing kernels and the single-token decode GEMM.
//
// Lane l owns experts l, l+64, ...; each of the k selections is a wave arg-max on
// (value desc, index asc) over the heads of per-lane sorted candidate lists.
#pragma once
#include "common.hpp"

namespace moe {
namespace rdev {

// (m1, m2) <- the two largest of {m1, m2, o1, o2}, given m1 >= m2 and o1 >= o2
__device__ __forceinline__ void top2_merge(float& m1, float& m2, float o1, float o2) {
  const float n2 = fmaxf(fminf(m1, o1), fmaxf(m2, o2));
  m1 = fmaxf(m1, o1);
  m2 = n2;
}

template <int CTRL, int NSLOT>
__device__ __forceinline__ void top2_steps(float (&m1)[NSLOT], float (&m2)[NSLOT]) {
#pragma unroll
  for (int i = 0; i < NSLOT; ++i) {
    const float o1 = __int_as_float(dpp_move<CTRL>(__float_as_int(m1[i])));
    const float o2 = __int_as_float(dpp_move<CTRL>(__float_as_int(m2[i])));
    top2_merge(m1[i], m2[i], o1, o2);
  }
}

// Maximum of an unsigned value over the wave, returned to every lane: four in-row DPP
// steps leave each 16-lane row's maximum in all its lanes (the moves write every lane),
// then the four row maxima are combined on the scalar unit.
template <int CTRL>
__device__ __forceinline__ uint32_t umax_step(uint32_t v) {
  const uint32_t o = static_cast<uint32_t>(dpp_move<CTRL>(static_cast<int>(v)));
  return o > v ? o : v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = umax_step<dpp::kQuadXor1>(v);
  v = umax_step<dpp::kQuadXor2>(v);
  v = umax_step<dpp::kRowHalfMirror>(v);
  v = umax_step<dpp::kRowMirror>(v);
  const uint32_t r0 = static_cast<uint32_t>(read_lane(static_cast<int>(v), 0));
  const uint32_t r1 = static_cast<uint32_t>(read_lane(static_cast<int>(v), 16));
  const uint32_t r2 = static_cast<uint32_t>(read_lane(static_cast<int>(v), 32));
  const uint32_t r3 = static_cast<uint32_t>(read_lane(static_cast<int>(v), 48));
  const uint32_t a = r0 > r1 ? r0 : r1, b = r2 > r3 ? r2 : r3;
  return a > b ? a : b;
}

__device__ __forceinline__ float sigmoid_rn(float l) {
  // sigma(l) evaluated in double and rounded once to the nearest float
  return static_cast<float>(1.0 / (1.0 + exp(-static_cast<double>(l))));
}

struct TopkParams {
  const float* logits;     // nz slabs of [T][E] (nz == 1: the logits themselves); row t of
                           // a slab is token t0 + t
  int t0;
  int nz;
  float* logits_out;       // [T][E] or null: receives the summed logits (nz > 1)
  int T, E, k, mode;
  const float* offset;
  const float* bias;
  int n_group, topk_group;
  float scaling;
  int32_t* ids;            // [T][k + shared]
  float* w;
  int shared;              // 1: slot k is the shared expert (id E, weight 1)
};

// LDS of one wave's top-k (group segment pairs)
struct TopkLds {
  float cval[512];
};

// Routes token t with the calling wave: lane j < k + shared returns slot j's expert and
// weight in (out_id, out_w) (the shared slot: expert E, weight 1); writes the summed
// logits of t to logits_out when given.  NSLOT = experts per lane (E <= 64*NSLOT);
// ZC = logit slabs loaded per round trip (bounded by the registers the launch allows).
template <int NSLOT, int ZC>
__device__ void topk_select(const TopkParams& p, int t, TopkLds& sh, int& out_id, float& out_w) {
  const int lane = lane_id();
  const int E = p.E, k = p.k, mode = p.mode;
  const float kNegInf = -__builtin_inff();
  // every load first, at clamped indices, so that all of them are in flight together;
  // slabs are added in ascending order
  float lv[NSLOT], ov[NSLOT], bv[NSLOT];
  const float* lrow = p.logits + static_cast<int64_t>(t - p.t0) * E;
  const int64_t slab = static_cast<int64_t>(p.T) * E;
#pragma unroll
  for (int i = 0; i < NSLOT; ++i) {
    const int ec = min(lane + kWave * i, E - 1);
    lv[i] = lrow[ec];
    ov[i] = p.offset ? p.offset[ec] : 0.f;
    bv[i] = p.bias ? p.bias[ec] : 0.f;
  }
  if (p.nz > 1) {
    for (int z0 = 1; z0 < p.nz; z0 += ZC) {
      float part[ZC][NSLOT];
#pragma unroll
      for (int q = 0; q < ZC; ++q) {
        const int zc = min(z0 + q, p.nz - 1);
#pragma unroll
        for (int i = 0; i < NSLOT; ++i)
          part[q][i] = lrow[zc * slab + min(lane + kWave * i, E - 1)];
      }
#pragma unroll
      for (int q = 0; q < ZC; ++q) {
#pragma unroll
        for (int i = 0; i < NSLOT; ++i) lv[i] = z0 + q < p.nz ? lv[i] + part[q][i] : lv[i];
      }
    }
  }
  float sel[NSLOT];    // selection value (-inf = not eligible / taken)
  float wsrc[NSLOT];   // weight source: logit (modes 0,1) or unbiased sigmoid (2)
#pragma unroll
  for (int i = 0; i < NSLOT; ++i) {
    const int e = lane + kWave * i;
    if (p.logits_out && e < E) p.logits_out[static_cast<int64_t>(t) * E + e] = lv[i];
    float l = lv[i];
    if (p.offset) l = l + ov[i];
    float v, ws;
    if (mode == 2) {
      const float s = sigmoid_rn(l);
      v = p.bias ? s + bv[i] : s;
      ws = s;
    } else {
      v = l;
      ws = l;
    }
    sel[i] = e < E ? v : kNegInf;
    wsrc[i] = e < E ? ws : 0.f;
  }
  if (mode == 2 && p.n_group > 0 && p.topk_group > 0) {
    // group score = sum of the two largest biased scores of a contiguous group of
    // gsz = E / n_group experts.  Only values enter the score, so the merge order does not
    // change it.
    const int gsz = E / p.n_group;
    // group of expert e: a shift when gsz is a power of two (uniform branch)
    const int gsz_sh = (gsz & (gsz - 1)) == 0 ? __builtin_ctz(static_cast<unsigned>(gsz)) : -1;
    auto group_of = [&](int e) { return gsz_sh >= 0 ? e >> gsz_sh : e / gsz; };
    float gs = kNegInf;                            // lane g < n_group: score of group g
    float m1[NSLOT], m2[NSLOT];
#pragma unroll
    for (int i = 0; i < NSLOT; ++i) { m1[i] = sel[i]; m2[i] = kNegInf; }
    if ((gsz == 16 || gsz == 32 || gsz == 64) && E == gsz * p.n_group) {
      // a group is one, two or four whole 16-lane rows of a slot: top-2 pairs within each
      // row by DPP moves, then across rows by lane swaps, so that every lane of a group
      // holds its pair; lane g then reads group g's score from the lane that opens it
      top2_steps<dpp::kQuadXor1, NSLOT>(m1, m2);
      top2_steps<dpp::kQuadXor2, NSLOT>(m1, m2);
      top2_steps<dpp::kRowHalfMirror, NSLOT>(m1, m2);
      top2_steps<dpp::kRowMirror, NSLOT>(m1, m2);
      for (int x = 16; x < gsz; x <<= 1) {
#pragma unroll
        for (int i = 0; i < NSLOT; ++i)
          top2_merge(m1[i], m2[i], __shfl_xor(m1[i], x, kWave), __shfl_xor(m2[i], x, kWave));
      }
      const int e0 = min(lane, p.n_group - 1) * gsz;   // first expert of group `lane`
      float g[NSLOT];
#pragma unroll
      for (int i = 0; i < NSLOT; ++i) g[i] = __shfl(m1[i] + m2[i], e0 & (kWave - 1), kWave);
      const int slot = e0 >> 6;
#pragma unroll
      for (int i = 0; i < NSLOT; ++i) gs = slot == i ? g[i] : gs;
      if (lane >= p.n_group) gs = kNegInf;
    } else {
      // segments of `sub` lanes (the largest power of two <= 16 dividing gsz) merged
      // with DPP moves; lane g then merges the gsz/sub segment pairs of group g from LDS
      const int sub = min(16, gsz & -gsz);
      const int sub_sh = __builtin_ctz(static_cast<unsigned>(sub));
      if (sub >= 2) top2_steps<dpp::kQuadXor1, NSLOT>(m1, m2);
      if (sub >= 4) top2_steps<dpp::kQuadXor2, NSLOT>(m1, m2);
      if (sub >= 8) top2_steps<dpp::kRowHalfMirror, NSLOT>(m1, m2);
      if (sub >= 16) top2_steps<dpp::kRowMirror, NSLOT>(m1, m2);
      // segment pairs: first value at cval[s], second at cval[256 + s] (sub >= 2 leaves
      // at most 256 segments; with sub == 1 every second value is -inf and not stored)
#pragma unroll
      for (int i = 0; i < NSLOT; ++i) {
        const int e = lane + kWave * i;
        if (e < E && (lane & (sub - 1)) == 0) {
          const int sg = e >> sub_sh;
          sh.cval[sg] = m1[i];
          if (sub > 1) sh.cval[256 + sg] = m2[i];
        }
      }
      wave_sync();
      if (lane < p.n_group) {
        const int nps = gsz >> sub_sh;
        const int s0 = lane * nps;
        float g1 = sh.cval[s0];
        float g2 = sub > 1 ? sh.cval[256 + s0] : kNegInf;
        for (int q = 1; q < nps; ++q)
          top2_merge(g1, g2, sh.cval[s0 + q], sub > 1 ? sh.cval[256 + s0 + q] : kNegInf);
        gs = g1 + g2;
      }
      wave_sync();                                 // cval is reused by the next token
    }
    // keep the topk_group groups of highest score (ties to the lower group index):
    // group g is kept when fewer than topk_group groups beat it
    int beaten_by = 0;
    for (int h = 0; h < p.n_group; ++h) {
      const float o = read_lane(gs, h);
      beaten_by += ((o > gs) | ((o == gs) & (h < lane))) ? 1 : 0;
    }
    const uint64_t keep = __ballot(lane < p.n_group && beaten_by < p.topk_group);
#pragma unroll
    for (int i = 0; i < NSLOT; ++i) {
      const int e = min(lane + kWave * i, E - 1);
      sel[i] = (keep >> group_of(e)) & 1ull ? sel[i] : kNegInf;
    }
  }
  // k selections; lane j keeps the j-th chosen (id, weight source) pair.  Candidates are
  // 32-bit keys: the selection value's bits mapped to an unsigned order (-0 folded into
  // +0, so equal values give equal keys); masked, invalid, taken and NaN candidates hold
  // key 0, below every eligible key.  Each lane first sorts its NSLOT candidates (key
  // descending, index ascending), so its best one is always its head; a pick is then the
  // wave maximum of the heads, whose owner pops it.  Equal keys go to the lowest expert
  // index: a lone matching head needs nothing more, several take the minimum index.
  uint32_t hk[NSLOT];
  int hi[NSLOT];
  float hs[NSLOT];
#pragma unroll
  for (int i = 0; i < NSLOT; ++i) {
    const uint32_t b = __float_as_uint(sel[i] + 0.f);
    const uint32_t ord = b ^ (static_cast<uint32_t>(static_cast<int32_t>(b) >> 31) | 0x80000000u);
    hk[i] = (sel[i] > kNegInf) ? ord : 0u;        // false for -inf and NaN
    hi[i] = lane + kWave * i;
    hs[i] = wsrc[i];
  }
  auto cx = [&](int a, int b) {                    // order slots a < b: (key desc, index asc)
    const bool sw = hk[b] > hk[a] || (hk[b] == hk[a] && hi[b] < hi[a]);
    const uint32_t tk = hk[a]; const int ti = hi[a]; const float ts = hs[a];
    hk[a] = sw ? hk[b] : hk[a]; hi[a] = sw ? hi[b] : hi[a]; hs[a] = sw ? hs[b] : hs[a];
    hk[b] = sw ? tk : hk[b];    hi[b] = sw ? ti : hi[b];    hs[b] = sw ? ts : hs[b];
  };
  if constexpr (NSLOT == 4) {
    cx(0, 1); cx(2, 3); cx(0, 2); cx(1, 3); cx(1, 2);
  } else {                                         // insertion sort
#pragma unroll
    for (int a = 1; a < NSLOT; ++a)
#pragma unroll
      for (int b = a; b > 0; --b) cx(b - 1, b);
  }
  int my_id = 0;
  float my_src = 0.f;
  for (int j = 0; j < k; ++j) {
    const uint32_t best = wave_max_u32(hk[0]);
    int bi = -1, owner = 0;                         // bi stays -1 if nothing eligible is left
    if (best != 0u) {
      const uint64_t m = __ballot(hk[0] == best);
      owner = __builtin_ctzll(m);
      bi = read_lane(hi[0], owner);
      for (uint64_t r = m & (m - 1); r; r &= r - 1) {   // equal keys: lowest index
        const int l = __builtin_ctzll(r);
        const int c = read_lane(hi[0], l);
        if (c < bi) { bi = c; owner = l; }
      }
    }
    const float src = read_lane(hs[0], owner);      // the owner lane's weight source
    if (bi >= 0 && lane == owner) {                 // pop the head
#pragma unroll
      for (int i = 0; i + 1 < NSLOT; ++i) { hk[i] = hk[i + 1]; hi[i] = hi[i + 1]; hs[i] = hs[i + 1]; }
      hk[NSLOT - 1] = 0u;
    }
    my_id = lane == j ? bi : my_id;
    my_src = lane == j ? src : my_src;
  }
  // weights in double: modes 0/1 exp(l_j - l_0) / sum, mode 2 scale * s_j / sum; the
  // sum runs over j = 0..k-1 in order
  const double l0 = static_cast<double>(read_lane(my_src, 0));
  const double myv = mode == 2 ? static_cast<double>(my_src)
                               : exp(static_cast<double>(my_src) - l0);
  double sum = 0.0;
  for (int j = 0; j < k; ++j) sum += read_lane(myv, j);
  // k + shared slots; the shared expert takes slot k with weight 1
  const double wt = mode == 2 ? static_cast<double>(p.scaling) * myv / sum : myv / sum;
  out_id = lane < k ? my_id : p.E;
  out_w = lane < k ? static_cast<float>(wt) : 1.f;
}

// topk_select, then the ids and weights of token t into p.ids / p.w (rows of k + shared
// slots), and the ids into ids_lds when given.
template <int NSLOT, int ZC>
__device__ void topk_token(const TopkParams& p, int t, TopkLds& sh, int32_t* ids_lds) {
  int id;
  float w;
  topk_select<NSLOT, ZC>(p, t, sh, id, w);
  const int lane = lane_id(), ko = p.k + p.shared;
  if (lane < ko) {
    p.ids[static_cast<int64_t>(t) * ko + lane] = id;
    p.w[static_cast<int64_t>(t) * ko + lane] = w;
    if (ids_lds) ids_lds[t * ko + lane] = id;
  }
}


}  // namespace rdev
}  // namespace moe
