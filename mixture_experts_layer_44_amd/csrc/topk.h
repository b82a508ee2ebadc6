// Per-token softmax + top-k + renormalised gates for one wave (64 lanes), shared by the
// router's top-k kernel and the small-batch routing kernel.
//
// Pages: "MoE Architecture" §2 "Gating Function" (softmax over the expert scores, top-k,
// renormalise the kept weights); "MoE (Mixture of Experts) Deep Dive", "Weighted Sum Output"
// (kept probabilities divided by their sum); "Mixture of experts (MoE)" handbook, "Load
// balancing" (the balancing bias only chooses experts).
//
// Wave reductions use DPP row shifts and row broadcasts (VALU, no LDS round trips) in a
// fixed order: the result lands in lane 63 and is broadcast with readlane, so every lane
// gets the same bits and the reduction is run-to-run deterministic.
#pragma once

#include "moe_internal.h"

namespace moe {

template <int CTRL, int ROW_MASK, int BANK_MASK>
__device__ __forceinline__ int dpp(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, BANK_MASK, false);
}

// row_shr:1, row_shr:2, row_shr:4 (banks 1-3), row_shr:8 (banks 2-3), row_bcast:15 (rows
// 1,3), row_bcast:31 (rows 2,3): afterwards lane 63 holds the reduction of all 64 lanes.
template <typename Op>
__device__ __forceinline__ int wave_reduce_bits(int v, int identity, Op op) {
  v = op(v, dpp<0x111, 0xF, 0xF>(identity, v));
  v = op(v, dpp<0x112, 0xF, 0xF>(identity, v));
  v = op(v, dpp<0x114, 0xF, 0xE>(identity, v));
  v = op(v, dpp<0x118, 0xF, 0xC>(identity, v));
  v = op(v, dpp<0x142, 0xA, 0xF>(identity, v));
  v = op(v, dpp<0x143, 0xC, 0xF>(identity, v));
  return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ float wave_max_f(float x) {
  const int r = wave_reduce_bits(__float_as_int(x), __float_as_int(-INFINITY), [](int a, int b) {
    return __float_as_int(fmaxf(__int_as_float(a), __int_as_float(b)));
  });
  return __int_as_float(r);
}

__device__ __forceinline__ float wave_sum_f(float x) {
  const int r = wave_reduce_bits(__float_as_int(x), __float_as_int(0.f), [](int a, int b) {
    return __float_as_int(__int_as_float(a) + __int_as_float(b));
  });
  return __int_as_float(r);
}

// Router logit of (token t, expert e): the K-split partials added in slice order. The loads
// are issued together (up to 16 slices) before the fixed-order sum.
__device__ __forceinline__ float sum_partials(const float* __restrict__ part, int KS, int T,
                                              int E_pad, int t, int e) {
  float v[16];
#pragma unroll
  for (int z = 0; z < 16; ++z)
    v[z] = z < KS ? part[((size_t)z * T + t) * E_pad + e] : 0.f;
  float s = 0.f;
#pragma unroll
  for (int z = 0; z < 16; ++z)
    if (z < KS) s += v[z];
  return s;
}

// order-preserving map of an fp32 key to uint32 (larger key -> larger uint)
__device__ __forceinline__ uint32_t sortable(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Arg-max over the wave of (key, expert): larger key first, lower expert index on equal keys.
// Each lane offers one candidate (key_u = sortable key, or 0 for none; tag = 255 - expert).
// Returns the winning expert.
__device__ __forceinline__ int wave_argmax(uint32_t key_u, int expert) {
  int hi = (int)key_u, lo = 255 - expert;
  auto step = [&](int nh, int nl) {
    const bool take = ((uint32_t)nh > (uint32_t)hi) || (nh == hi && nl > lo);
    hi = take ? nh : hi;
    lo = take ? nl : lo;
  };
  step(dpp<0x111, 0xF, 0xF>(hi, hi), dpp<0x111, 0xF, 0xF>(lo, lo));
  step(dpp<0x112, 0xF, 0xF>(hi, hi), dpp<0x112, 0xF, 0xF>(lo, lo));
  step(dpp<0x114, 0xF, 0xE>(hi, hi), dpp<0x114, 0xF, 0xE>(lo, lo));
  step(dpp<0x118, 0xF, 0xC>(hi, hi), dpp<0x118, 0xF, 0xC>(lo, lo));
  step(dpp<0x142, 0xA, 0xF>(hi, hi), dpp<0x142, 0xA, 0xF>(lo, lo));
  step(dpp<0x143, 0xC, 0xF>(hi, hi), dpp<0x143, 0xC, 0xF>(lo, lo));
  return 255 - __builtin_amdgcn_readlane(lo, 63);
}

// Softmax + top-k of one token. logits[i] / live[i] for experts lane + 64 i (i < 4,
// E <= 256); sel_bias (may be null) shifts only the keys. On return lanes j < k hold the
// j-th selected expert (out_e) and its renormalised gate (out_g); pr[] holds each lane's
// probabilities (0 for dead experts).
__device__ __forceinline__ void token_topk(const float (&lg)[4], const bool (&live)[4],
                                           const float* __restrict__ sel_bias, int k, int lane,
                                           float (&pr)[4], int& out_e, float& out_g) {
  const float m = wave_max_f(fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3])));
  float ex[4], loc = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ex[i] = live[i] ? expf(lg[i] - m) : 0.f;
    loc += ex[i];
  }
  const float inv = 1.0f / wave_sum_f(loc);
  uint32_t key[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pr[i] = ex[i] * inv;
    const float kf = sel_bias && live[i] ? lg[i] + sel_bias[lane + 64 * i] : lg[i];
    key[i] = live[i] ? sortable(kf) : 0u;
  }
  bool taken[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) taken[i] = !live[i];
  int my_e = 0;
  float my_p = 0.f;
  for (int j = 0; j < k; ++j) {
    // this lane's best remaining candidate (experts lane, lane+64, ... ascending, so the
    // first strictly larger key wins and equal keys keep the lower expert)
    uint32_t bk = 0u;
    int be = 255, bi = -1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (!taken[i] && (bi < 0 || key[i] > bk)) { bk = key[i]; be = lane + 64 * i; bi = i; }
    }
    const int win = wave_argmax(bi < 0 ? 0u : bk, bi < 0 ? 255 : be);
    const int owner = win & 63, sl = win >> 6;
    const float cand = sl == 0 ? pr[0] : sl == 1 ? pr[1] : sl == 2 ? pr[2] : pr[3];
    const float pw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cand), owner));
    if (lane == owner) {
      if (sl == 0) taken[0] = true;
      else if (sl == 1) taken[1] = true;
      else if (sl == 2) taken[2] = true;
      else taken[3] = true;
    }
    if (lane == j) { my_e = win; my_p = pw; }
  }
  const float psel = wave_sum_f(lane < k ? my_p : 0.f);
  out_e = my_e;
  out_g = my_p / psel;
}

}  // namespace moe
