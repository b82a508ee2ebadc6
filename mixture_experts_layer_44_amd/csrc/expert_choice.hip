// Expert-choice routing: each expert picks its C tokens.
//
// Pages: "One Deep Concept #04 -- Mixture of Experts", "Expert Choice -- Reverse Who Selects
// Whom" (experts choose tokens; fixed bucket sizes; a token may get any number of experts).
// Scores are the router's softmax probabilities ("MoE Architecture" §2 "Gating Function").
// Expert e takes the C tokens with the largest p[t,e], equal scores going to the lower token;
// its bucket lists them in ascending token order, with weight p[t,e] (no renormalisation).
//
//   ec_probs:   one wave per token: logits (K-split partials + offset), max-shifted softmax;
//               written expert-major (probsT[e][t]) through LDS, plus per-workgroup sums.
//   ec_select:  one 1024-thread workgroup per expert: the C-th largest key by a 4-pass radix
//               select over the order-preserving uint32 image of p, then a compaction in token
//               order (ballot prefix counts) that takes every key above the threshold and the
//               first ties at it. Writes the bucket (tokens, weights), the expert's segment
//               offset and pos[t][e] (row of (t,e) in the buckets, or -1).
//   ec_combine: one workgroup per token: the shared row, then the rows of the experts that
//               chose the token, in expert order.
#include "topk.h"

namespace moe {

namespace {

constexpr int EC_TOK = 16;   // tokens per probability workgroup (4 waves x 4)

__global__ __launch_bounds__(256) void ec_probs_kernel(const float* __restrict__ part, int KS, int T,
                                                       int E, int E_pad,
                                                       const float* __restrict__ logit_bias,
                                                       float* __restrict__ probsT,
                                                       float* __restrict__ psum_part) {
  __shared__ float prob[EC_TOK][256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int tt = 0; tt < EC_TOK / 4; ++tt) {
    const int tr = wave * (EC_TOK / 4) + tt;
    const int t = blockIdx.x * EC_TOK + tr;
    if (t >= T) {                     // uniform across the wave
#pragma unroll
      for (int i = 0; i < 4; ++i) prob[tr][lane + 64 * i] = 0.f;
      continue;
    }
    float lg[4];
    bool live[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      live[i] = e < E;
      float v = -INFINITY;
      if (live[i]) v = sum_partials(part, KS, T, E_pad, t, e) + (logit_bias ? logit_bias[e] : 0.f);
      lg[i] = v;
    }
    const float m = wave_max_f(fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3])));
    float ex[4], loc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ex[i] = live[i] ? expf(lg[i] - m) : 0.f;
      loc += ex[i];
    }
    const float inv = 1.0f / wave_sum_f(loc);
#pragma unroll
    for (int i = 0; i < 4; ++i) prob[tr][lane + 64 * i] = ex[i] * inv;
  }
  __syncthreads();
  const int t0 = blockIdx.x * EC_TOK;
  for (int idx = tid; idx < E * EC_TOK; idx += 256) {   // EC_TOK consecutive tokens per expert
    const int e = idx / EC_TOK, tr = idx % EC_TOK;
    if (t0 + tr < T) probsT[(size_t)e * T + t0 + tr] = prob[tr][e];
  }
  if (psum_part) {
    for (int e = tid; e < E; e += 256) {
      float s = 0.f;
      for (int tr = 0; tr < EC_TOK; ++tr) s += prob[tr][e];
      psum_part[(size_t)blockIdx.x * E + e] = s;
    }
  }
}

// Exclusive prefix count of `flag` over the 1024 threads in thread order; *total = the count.
__device__ int count_scan1024(bool flag, int* wsum, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t b = __ballot(flag);
  const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  if (lane == 0) wsum[wave] = __popcll(b);
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < 16; ++w) {
    const int c = wsum[w];
    before += w < wave ? c : 0;
    all += c;
  }
  __syncthreads();                    // wsum is reused by the next call
  *total = all;
  return before + __popcll(b & lt);
}

__global__ __launch_bounds__(1024) void ec_select_kernel(const float* __restrict__ probsT, int T,
                                                         int E, int C, int32_t* __restrict__ tokens,
                                                         float* __restrict__ gates,
                                                         int32_t* __restrict__ pos_table,
                                                         int32_t* __restrict__ offsets) {
  __shared__ int hist[256];
  __shared__ int wsum[16];
  __shared__ int s_digit, s_above;
  const int e = blockIdx.x, tid = threadIdx.x;
  const float* col = probsT + (size_t)e * T;
  if (tid == 0) {
    offsets[e] = e * C;
    if (e == 0) offsets[E] = E * C;
  }
  // ---- radix select: key of the C-th largest score, 8 bits per pass from the top
  uint32_t prefix = 0, mask = 0;
  int remaining = C;                  // how many of the keys matching `prefix` still to take
  if (C > 0) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      for (int t = tid; t < T; t += 1024) {
        const uint32_t u = sortable(col[t]);
        if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255], 1);
      }
      __syncthreads();
      // counts of digits 255, 254, ... (descending); the digit where the running count first
      // reaches `remaining` holds the C-th largest key
      const int own = tid < 256 ? hist[255 - tid] : 0;
      __syncthreads();
      if (tid < 256) hist[tid] = own;
      __syncthreads();
      for (int o = 1; o < 256; o <<= 1) {
        const int v = (tid < 256 && tid >= o) ? hist[tid - o] : 0;
        __syncthreads();
        if (tid < 256) hist[tid] += v;
        __syncthreads();
      }
      if (tid < 256) {
        const int incl = hist[tid];
        if (incl >= remaining && incl - own < remaining) {
          s_digit = 255 - tid;
          s_above = incl - own;
        }
      }
      __syncthreads();
      remaining -= s_above;
      prefix |= (uint32_t)s_digit << shift;
      mask |= 0xFFu << shift;
      __syncthreads();
    }
  }
  // ---- compaction in token order: keys above the threshold, then the first `remaining` ties
  const uint32_t kstar = prefix;
  int eq_carry = 0, sel_carry = 0;
  for (int base = 0; base < T; base += 1024) {
    const int t = base + tid;
    const bool in = t < T;
    const float p = in ? col[t] : 0.f;
    const uint32_t u = sortable(p);
    const bool eq = in && C > 0 && u == kstar;
    int eq_tot, sel_tot;
    const int eq_pre = eq_carry + count_scan1024(eq, wsum, &eq_tot);
    const bool sel = in && C > 0 && (u > kstar || (eq && eq_pre < remaining));
    const int sel_pre = sel_carry + count_scan1024(sel, wsum, &sel_tot);
    if (in) {
      int pos = -1;
      if (sel && sel_pre < C) {        // exactly C are selected; the bound only guards the write
        pos = e * C + sel_pre;
        tokens[pos] = t;
        gates[pos] = p;
      }
      pos_table[(size_t)t * E + e] = pos;
    }
    eq_carry += eq_tot;
    sel_carry += sel_tot;
  }
}

__global__ __launch_bounds__(256) void ec_combine_kernel(const int32_t* __restrict__ pos_table,
                                                         const float* __restrict__ gates,
                                                         const float* __restrict__ out_rows,
                                                         const float* __restrict__ out_rows_b,
                                                         const float* __restrict__ shared_out,
                                                         int E, int d, float* __restrict__ y) {
  __shared__ int rows[256];
  __shared__ float wts[256];
  __shared__ int wcount[4];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // the experts that chose this token, compacted in expert order (thread e looks at expert e)
  const int r = tid < E ? pos_table[(size_t)t * E + tid] : -1;
  const uint64_t b = __ballot(r >= 0);
  const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  if (lane == 0) wcount[wave] = __popcll(b);
  __syncthreads();
  int before = 0, n = 0;
  for (int w = 0; w < 4; ++w) {
    before += w < wave ? wcount[w] : 0;
    n += wcount[w];
  }
  if (r >= 0) {
    const int slot = before + __popcll(b & lt);
    rows[slot] = r;
    wts[slot] = gates[r];
  }
  __syncthreads();
  const int d4 = d >> 2;
  for (int c = tid; c < d4; c += 256) {
    f32x4 acc = shared_out ? *(const f32x4*)(shared_out + (size_t)t * d + 4 * c)
                           : f32x4{0.f, 0.f, 0.f, 0.f};
    // four rows at a time: their loads are issued together, then they are added in order
    for (int j0 = 0; j0 < n; j0 += 4) {
      f32x4 v[4], vb[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        v[u] = vb[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (j0 + u >= n) continue;   // uniform
        const size_t off = (size_t)rows[j0 + u] * d + 4 * c;
        v[u] = *(const f32x4*)(out_rows + off);
        if (out_rows_b) vb[u] = *(const f32x4*)(out_rows_b + off);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (j0 + u >= n) continue;
        if (out_rows_b) {
          v[u][0] += vb[u][0];
          v[u][1] += vb[u][1];
          v[u][2] += vb[u][2];
          v[u][3] += vb[u][3];
        }
        const float g = wts[j0 + u];
        acc[0] = fmaf(g, v[u][0], acc[0]);
        acc[1] = fmaf(g, v[u][1], acc[1]);
        acc[2] = fmaf(g, v[u][2], acc[2]);
        acc[3] = fmaf(g, v[u][3], acc[3]);
      }
    }
    *(f32x4*)(y + (size_t)t * d + 4 * c) = acc;
  }
}

}  // namespace

int ec_probs_blocks(const moe_problem& p) { return ceil_div(p.T, EC_TOK); }

hipError_t launch_ec_probs(const moe_problem& p, const float* logits_part, const float* logit_bias,
                           float* probsT, float* psum_part, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  const int E_pad = ceil_div(p.E, 16) * 16;
  hipLaunchKernelGGL(ec_probs_kernel, dim3(ec_probs_blocks(p)), dim3(256), 0, s, logits_part,
                     route_ksplit(p), p.T, p.E, E_pad, logit_bias, probsT, psum_part);
  return hipGetLastError();
}

hipError_t launch_ec_select(const moe_problem& p, int C, const float* probsT, int32_t* tokens,
                            float* gates, int32_t* pos_table, int32_t* offsets, hipStream_t s) {
  hipLaunchKernelGGL(ec_select_kernel, dim3(p.E), dim3(1024), 0, s, probsT, p.T, p.E, C, tokens,
                     gates, pos_table, offsets);
  return hipGetLastError();
}

hipError_t launch_ec_combine(const moe_problem& p, const int32_t* pos_table, const float* gates,
                             const float* out_rows, const float* out_rows_b,
                             const float* shared_out, float* y, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  hipLaunchKernelGGL(ec_combine_kernel, dim3(p.T), dim3(256), 0, s, pos_table, gates, out_rows,
                     out_rows_b, shared_out, p.E, p.d, y);
  return hipGetLastError();
}

}  // namespace moe
