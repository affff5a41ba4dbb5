// Per-token top-k selection and gates, shared by the routing kernel
// (moe_route) and the router kernel that routes its own logits in the
// forward pass, so both make the same choice bit for bit from the same
// logits.
//
// Routing follows the pages' description of the layer: a sigmoid router with
// a per-expert bias that only steers selection (Apex-3 code page, "What's
// inside", row "Fine-grained MoE"), or a softmax top-k router (KempnerForge
// README, "Features / Architecture"), on fp32 logits (Ultimate MoE Training
// Handbook, section 2.5, fp32 router dtype).
#pragma once

#include "kernels.h"

namespace moe {
namespace rte {

// Map an fp32 key to an unsigned integer with the same order.  -0 is folded
// onto +0 and NaN onto the very bottom, so NaN keys are picked last.
MOE_DEV uint32_t ordered_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN
  if (u == 0x80000000u) u = 0u;                     // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Candidate code: key in the high word, (0xffffffff - expert) in the low word,
// so the maximum is the best key and, among equal keys, the lowest expert.
MOE_DEV uint64_t cand_code(float key, int e) {
  return ((uint64_t)ordered_bits(key) << 32) | (uint64_t)(0xffffffffu - (uint32_t)e);
}

// Cross-lane moves within rows of 16 lanes (DPP, VALU latency): quad_perm
// [1,0,3,2] and [2,3,0,1] exchange neighbours at distance 1 and 2, half-row
// mirror pairs each quad with the other quad of its 8 lanes, row mirror each
// half-row with the other half.  After the four steps every lane of a row
// holds the combination of all 16 of its values, and lanes paired at each
// step combine the same two partial results, so every lane holds the same
// bits (for a sum as well as a maximum).  Groups wider than a row continue
// with lane shuffles across rows.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
template <int CTRL>
MOE_DEV int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
MOE_DEV uint64_t dpp_u64(uint64_t v) {
  const int lo = dpp_i32<CTRL>((int)(uint32_t)v), hi = dpp_i32<CTRL>((int)(uint32_t)(v >> 32));
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
template <int CTRL>
MOE_DEV double dpp_f64(double v) {
  return __builtin_bit_cast(double, dpp_u64<CTRL>(__builtin_bit_cast(uint64_t, v)));
}
template <int CTRL>
MOE_DEV float dpp_f32(float v) {
  return __int_as_float(dpp_i32<CTRL>(__float_as_int(v)));
}

template <int L>
MOE_DEV uint64_t group_max_u64(uint64_t v) {
  static_assert(L >= 16, "groups of whole DPP rows");
  uint64_t o;
  o = dpp_u64<kDppXor1>(v); v = o > v ? o : v;
  o = dpp_u64<kDppXor2>(v); v = o > v ? o : v;
  o = dpp_u64<kDppHalfMirror>(v); v = o > v ? o : v;
  o = dpp_u64<kDppMirror>(v); v = o > v ? o : v;
#pragma unroll
  for (int m = 16; m < L; m <<= 1) {
    o = __shfl_xor(v, m, L);
    v = o > v ? o : v;
  }
  return v;
}
template <int L>
MOE_DEV double group_sum_f64(double v) {
  static_assert(L >= 16, "groups of whole DPP rows");
  v += dpp_f64<kDppXor1>(v);
  v += dpp_f64<kDppXor2>(v);
  v += dpp_f64<kDppHalfMirror>(v);
  v += dpp_f64<kDppMirror>(v);
#pragma unroll
  for (int m = 16; m < L; m <<= 1) v += __shfl_xor(v, m, L);
  return v;
}
template <int L>
MOE_DEV float group_max_f32(float v) {
  static_assert(L >= 16, "groups of whole DPP rows");
  v = fmaxf(v, dpp_f32<kDppXor1>(v));
  v = fmaxf(v, dpp_f32<kDppXor2>(v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppMirror>(v));
#pragma unroll
  for (int m = 16; m < L; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, L));
  return v;
}

// sigmoid evaluated in fp64 and rounded once to fp32
MOE_DEV float sigmoid_rounded(float l) { return (float)(1.0 / (1.0 + exp(-(double)l))); }

// One token routed by a group of L lanes (li = lane within the group); lane
// i holds experts i, i+L, ... (V = ceil(E / L) values).  lrow: the token's E
// logits (global memory or LDS).  Slot j (j < k) is written by lane j:
// idx[j], gate[j]; each picked expert is counted in s_hist (LDS).
template <int L, int V>
MOE_DEV void route_token(const float* lrow, const float* __restrict__ bias, int E, int k, int score,
                         int renorm, int li, int32_t* idx, float* gate, int* s_hist) {
  float lv[V];
  float sc[V];
  uint64_t cand[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int e = li + v * L;
    lv[v] = (e < E) ? lrow[e] : -INFINITY;
  }
  if (score == MOE_SIGMOID) {
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int e = li + v * L;
      sc[v] = sigmoid_rounded(lv[v]);
      const float key = bias ? (sc[v] + (e < E ? bias[e] : 0.0f)) : sc[v];
      cand[v] = (e < E) ? cand_code(key, e) : 0ull;
    }
  } else {
    float m = lv[0];
#pragma unroll
    for (int v = 1; v < V; ++v) m = fmaxf(m, lv[v]);
    m = group_max_f32<L>(m);
    double z[V], zs = 0.0;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int e = li + v * L;
      z[v] = (e < E) ? exp((double)lv[v] - (double)m) : 0.0;
      zs += z[v];
    }
    zs = group_sum_f64<L>(zs);
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int e = li + v * L;
      sc[v] = (float)(z[v] / zs);
      cand[v] = (e < E) ? cand_code(lv[v], e) : 0ull;
    }
  }
  // k rounds of group arg-max; slot j's expert lands in lane j
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t b = cand[0];
#pragma unroll
    for (int v = 1; v < V; ++v) b = cand[v] > b ? cand[v] : b;
    b = group_max_u64<L>(b);
    const int e = (int)(0xffffffffu - (uint32_t)(b & 0xffffffffu));
    const int owner = e % L, ov = e / L;
    if (li == owner) {
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (v == ov) cand[v] = 0ull;
    }
    if (li == j) my_e = e;
  }
  // each slot's score from the lane that holds its expert (V independent
  // reads of that lane, one of which is the expert's)
  float my_s = 0.0f;
  {
    const int owner = my_e % L, ov = my_e / L;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const float t = __shfl(sc[v], owner, L);
      if (v == ov) my_s = t;
    }
  }
  double gsum = (li < k) ? (double)my_s : 0.0;
  gsum = group_sum_f64<L>(gsum);
  if (li < k) {
    float g;
    if (score == MOE_SOFTMAX && !renorm)
      g = my_s;
    else
      g = (float)((double)my_s / gsum);
    idx[li] = my_e;
    gate[li] = g;
    atomicAdd(&s_hist[my_e], 1);
  }
}

}  // namespace rte
}  // namespace moe
