// Router: logits = x . w_gate^T (+ logit_bias), softmax, top-k on logits (+ sel_bias),
// renormalised gates, per-workgroup probability sums.
//
// Pages: "MoE Architecture" §2 "Gating Function" (softmax of x W_gate, top-k, weights
// renormalised over the k kept scores); "MoE (Mixture of Experts) Deep Dive", "Weighted
// Sum Output" (kept probabilities divided by their sum); "Mixture of experts (MoE)"
// handbook, "Load balancing" (the balancing bias only chooses experts).
//
// One workgroup = 16 tokens x all E experts (E <= 256), 4 waves of 64 lanes.
// bf16: v_mfma_f32_16x16x32_bf16 tiles of 16 tokens x 16 experts; the fp32 logits stay in
// LDS (never rounded to bf16). With >= 4 expert tiles each wave owns whole tiles over the
// full d; with fewer, the 4 waves split d and their partial logits are summed in a fixed
// order. Then each wave takes 4 tokens: softmax and k rounds of a 64-lane arg-max
// (larger key first, lower expert index on equal keys) with shuffles.
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kWaves = 4;
constexpr int kMaxNT = 16;  // 256 experts / 16

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  // xor butterfly: every lane adds the same pairs, so all lanes get identical bits
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <bool BF16>
__global__ __launch_bounds__(256) void route_kernel(
    const void* __restrict__ xv, const void* __restrict__ wv, const float* __restrict__ logit_bias,
    const float* __restrict__ sel_bias, int T, int d, int E, int k, int32_t* __restrict__ ids,
    float* __restrict__ gates, float* __restrict__ psum_part) {
  const int n_tiles = (E + 15) / 16;
  const int E_pad = n_tiles * 16;
  const bool ksplit = n_tiles < kWaves;            // small E: waves split d instead of experts
  // part[s][tok][e]: s < 4 partial logits (ksplit) or s = 0 only
  extern __shared__ float lds[];
  float* part = lds;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tok0 = blockIdx.x * kRouteTok;

  if constexpr (BF16) {
    const bf16_t* x = (const bf16_t*)xv;
    const bf16_t* w = (const bf16_t*)wv;
    // this wave's expert tiles and d range
    int nt_first = ksplit ? 0 : wave, nt_step = ksplit ? 1 : kWaves;
    int kb0 = ksplit ? wave * (d / kWaves) : 0;
    int kb1 = ksplit ? kb0 + d / kWaves : d;
    const int r = lane & 15, kq = (lane >> 4) * 8;
    const int trow = tok0 + r;
    const bool a_ok = trow < T;
    const bf16_t* a_ptr = x + (size_t)(a_ok ? trow : 0) * d + kq;
    f32x4 acc[4];
    const bf16_t* b_ptr[4];
    bool b_ok[4];
    int nt_list[4];
    int nn = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      int nt = nt_first + i * nt_step;
      nt_list[i] = nt;
      bool have = nt < n_tiles && (ksplit ? (i < n_tiles) : true);
      if (have) nn = i + 1;
      int e = nt * 16 + r;
      b_ok[i] = have && e < E;
      b_ptr[i] = w + (size_t)(b_ok[i] ? e : 0) * d + kq;
    }
    const bf16x8 zero8 = {};
    for (int kb = kb0; kb < kb1; kb += 32) {
      bf16x8 a = a_ok ? *(const bf16x8*)(a_ptr + kb) : zero8;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i < nn) {
          bf16x8 b = b_ok[i] ? *(const bf16x8*)(b_ptr[i] + kb) : zero8;
          acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[i], 0, 0, 0);
        }
      }
    }
    // C layout (16x16): lane holds column (expert) lane%16, rows (tokens) 4*(lane/16)+j
    const int slot = ksplit ? wave : 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < nn) {
        int e = nt_list[i] * 16 + (lane & 15);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          int tr = (lane >> 4) * 4 + j;
          part[(slot * kRouteTok + tr) * E_pad + e] = acc[i][j];
        }
      }
    }
  } else {
    const float* x = (const float*)xv;
    const float* w = (const float*)wv;
    for (int idx = tid; idx < kRouteTok * E_pad; idx += 256) {
      int tr = idx / E_pad, e = idx - tr * E_pad;
      int t = tok0 + tr;
      float s = 0.f;
      if (t < T && e < E) {
        const float* xr = x + (size_t)t * d;
        const float* wr = w + (size_t)e * d;
        for (int i = 0; i < d; ++i) s = fmaf(xr[i], wr[i], s);
      }
      part[tr * E_pad + e] = s;
    }
  }
  __syncthreads();

  const bool split_sum = BF16 && ksplit;
  // softmax + top-k: wave w handles tokens 4w..4w+3
  for (int tt = 0; tt < kRouteTok / kWaves; ++tt) {
    const int tr = wave * (kRouteTok / kWaves) + tt;
    const int t = tok0 + tr;
    float lg[4], key[4];
    bool live[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int e = lane + 64 * i;
      live[i] = e < E;
      float v = -INFINITY;
      if (live[i]) {
        v = part[tr * E_pad + e];
        if (split_sum) {
          v += part[(1 * kRouteTok + tr) * E_pad + e];
          v += part[(2 * kRouteTok + tr) * E_pad + e];
          v += part[(3 * kRouteTok + tr) * E_pad + e];
        }
        if (logit_bias) v += logit_bias[e];
      }
      lg[i] = v;
      key[i] = live[i] ? (sel_bias ? v + sel_bias[e] : v) : -INFINITY;
    }
    float m = wave_max(fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3])));
    float ex[4], loc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ex[i] = live[i] ? expf(lg[i] - m) : 0.f;
      loc += ex[i];
    }
    const float s = wave_sum(loc);
    const float inv = 1.0f / s;
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = ex[i] * inv;
    // keep probabilities for the per-workgroup sums (slot 0 entries of this token;
    // each lane overwrites only what it alone has read)
    if (t < T) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (live[i]) part[tr * E_pad + lane + 64 * i] = pr[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (live[i]) part[tr * E_pad + lane + 64 * i] = 0.f;
    }
    if (t >= T) continue;  // uniform across the wave
    bool taken[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) taken[i] = !live[i];
    int my_e = 0;
    float my_p = 0.f;
    for (int j = 0; j < k; ++j) {
      float bk = -INFINITY;
      int be = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int e = lane + 64 * i;
        if (!taken[i] && (key[i] > bk || (key[i] == bk && e < be))) { bk = key[i]; be = e; }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        float ok = __shfl_xor(bk, o);
        int oe = __shfl_xor(be, o);
        if (ok > bk || (ok == bk && oe < be)) { bk = ok; be = oe; }
      }
      const int owner = be & 63, sl = be >> 6;
      float cand = sl == 0 ? pr[0] : sl == 1 ? pr[1] : sl == 2 ? pr[2] : pr[3];
      float pw = __shfl(cand, owner);
      if (lane == owner) {
        if (sl == 0) taken[0] = true;
        else if (sl == 1) taken[1] = true;
        else if (sl == 2) taken[2] = true;
        else taken[3] = true;
      }
      if (lane == j) { my_e = be; my_p = pw; }
    }
    const float psel = wave_sum(lane < k ? my_p : 0.f);
    if (lane < k) {
      ids[(size_t)t * k + lane] = my_e;
      gates[(size_t)t * k + lane] = my_p / psel;
    }
  }
  if (psum_part) {
    __syncthreads();
    for (int e = tid; e < E; e += 256) {
      float s = 0.f;
      for (int tr = 0; tr < kRouteTok; ++tr) s += part[tr * E_pad + e];
      psum_part[(size_t)blockIdx.x * E + e] = s;
    }
  }
}

// prob_sum[e] = sum over router workgroups (in order) of their partial sums
__global__ __launch_bounds__(256) void psum_reduce_kernel(const float* __restrict__ part, int nblk,
                                                          int E, float* __restrict__ out) {
  for (int e = threadIdx.x; e < E; e += 256) {
    float s = 0.f;
    for (int b = 0; b < nblk; ++b) s += part[(size_t)b * E + e];
    out[e] = s;
  }
}

}  // namespace

hipError_t launch_route(const moe_problem& p, const void* x, const void* w_gate,
                        const float* logit_bias, const float* sel_bias, int32_t* ids,
                        float* gates, float* prob_sum, float* psum_part, hipStream_t s) {
  const int nblk = ceil_div(p.T, kRouteTok);
  const int n_tiles = ceil_div(p.E, 16);
  const int E_pad = n_tiles * 16;
  const bool ksplit = p.dtype == MOE_BF16 && n_tiles < kWaves;
  const size_t lds = (size_t)(ksplit ? 4 : 1) * kRouteTok * E_pad * sizeof(float);
  float* part = prob_sum ? psum_part : nullptr;
  if (nblk == 0) {
    if (!prob_sum) return hipSuccess;
  } else if (p.dtype == MOE_BF16)
    hipLaunchKernelGGL(route_kernel<true>, dim3(nblk), dim3(256), lds, s, x, w_gate, logit_bias,
                       sel_bias, p.T, p.d, p.E, p.k, ids, gates, part);
  else
    hipLaunchKernelGGL(route_kernel<false>, dim3(nblk), dim3(256), lds, s, x, w_gate, logit_bias,
                       sel_bias, p.T, p.d, p.E, p.k, ids, gates, part);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !prob_sum) return err;
  hipLaunchKernelGGL(psum_reduce_kernel, dim3(1), dim3(256), 0, s, psum_part, nblk, p.E, prob_sum);
  return hipGetLastError();
}

}  // namespace moe
