// Small-batch routing (T*k <= 1024, decode-sized batches).
//
// Two paths, both with the definitions of route.hip (top-k, renormalised gates: "MoE
// Architecture" §2 "Gating Function"; "MoE (Mixture of Experts) Deep Dive", "Router Network
// Computation" and "Weighted Sum Output") and align.hip (histogram, prefix sum, stable order by
// expert, first-come capacity dropping: "Mixture of experts (MoE)" handbook, "Implementation";
// "MoE Architecture" §2 "Expert capacity and token dropping"):
//   - topk_align_small_kernel (T <= 16): after the logits kernel, softmax / top-k with wave
//     reductions, then grouping and the GEMM schedule, in one launch.
//   - align_small_kernel: after the logits and the multi-workgroup top-k (larger small
//     batches), probability sums + grouping + schedule in one workgroup.
// The grouping is bit-identical to the multi-launch align kernels. At decode sizes each of
// those steps is a few microseconds of launch latency and almost no work, so a single
// 1024-thread workgroup does them back to back out of LDS.
#include "topk.h"

namespace moe {

namespace {

constexpr int NWAVE = 16;

// exclusive scan of v over the first 320 threads (5 waves; the values live in threads < 257,
// the others pass 0); all 1024 threads call it. Each wave scans its 64 values with DPP steps,
// then adds the totals of the waves before it.
__device__ int scan320(int v, int* wsum, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int x = wave_incl_scan(v);
  if (lane == 63 && wave < 5) wsum[wave] = x;
  __syncthreads();
  int base = 0;
#pragma unroll
  for (int w = 0; w < 5; ++w) base += w < wave ? wsum[w] : 0;
  *total = wsum[0] + wsum[1] + wsum[2] + wsum[3] + wsum[4];
  __syncthreads();   // wsum is reused by the next call
  return base + x - v;
}

// LDS of the grouping step
struct AlignLds {
  int s_ids[1024];        // the T*k expert ids, flat assignment order
  int wcnt[NWAVE][256];   // assignments of expert e in wave w
  int s_off[257];
  int wsum[5];
};

// Grouping by expert + grouped-GEMM schedule out of LDS, at most one assignment per thread: all
// 1024 threads call it after L.s_ids[0..n) is filled and L.wcnt zeroed (and a barrier). Ranks
// come from ballots inside a wave plus the per-wave counts of earlier waves, i.e. ascending flat
// index a inside each expert, as the multi-launch path's stable order.
__device__ void align_schedule_lds(AlignLds& L, int n, int T, int E, int cap,
                                   int32_t* __restrict__ counts_pre, int32_t* __restrict__ counts,
                                   int32_t* __restrict__ offsets,
                                   int32_t* __restrict__ sorted_assign,
                                   int32_t* __restrict__ assign_pos, int n_shared,
                                   const Schedule& sc) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Wave w takes assignments [w*per, (w+1)*per) in lane order. With at most 256 of them, 16 per
  // wave: the ballot loop below runs once per distinct expert among a wave's assignments, a
  // serial chain, so spreading a few assignments over all 16 waves shortens it.
  const int per = n <= 16 * NWAVE ? 16 : 64;
  const int a = lane < per ? wave * per + lane : n;   // n: no assignment
  const bool has_a = a < n;
  const int e = has_a ? L.s_ids[a] : -1;
  const bool valid = e >= 0 && e < E;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int my_rank = 0;
  uint64_t active = __ballot(valid);
  while (active) {
    const int leader = __ffsll((unsigned long long)active) - 1;
    const int le = __builtin_amdgcn_readlane(e, leader);   // leader is wave-uniform
    const uint64_t msk = __ballot(valid && e == le);
    if (valid && e == le) {
      my_rank = __popcll(msk & lt_mask);
      if (lane == leader) L.wcnt[wave][e] = __popcll(msk);
    }
    active &= ~msk;
  }
  __syncthreads();
  int c = 0, kept = 0;
  if (tid < E) {
    for (int w = 0; w < NWAVE; ++w) c += L.wcnt[w][tid];
    kept = (cap >= 0 && c > cap) ? cap : c;
  }
  int total;
  const int off = scan320(tid < E ? kept : 0, L.wsum, &total);
  if (tid < E) {
    counts_pre[tid] = c;
    counts[tid] = kept;
    offsets[tid] = off;
    L.s_off[tid] = off;
  }
  if (tid == 0) {
    offsets[E] = total;
    L.s_off[E] = total;
  }
  __syncthreads();
  if (has_a) {
    int pos = -1;
    if (valid) {
      int rank = my_rank;
      for (int w = 0; w < wave; ++w) rank += L.wcnt[w][e];
      if (cap < 0 || rank < cap) {
        pos = L.s_off[e] + rank;
        sorted_assign[pos] = a;
      }
    }
    assign_pos[a] = pos;
  }

  // ---- grouped-GEMM schedule (same as schedule_kernel)
  const int G = E + n_shared;
  int rows = 0;
  if (tid < E) rows = L.s_off[tid + 1] - L.s_off[tid];
  else if (tid < G) rows = T;
  const int mts = (rows + sc.BM - 1) / sc.BM;
  int mt_total;
  const int base = scan320(tid < G ? mts : 0, L.wsum, &mt_total);
  if (tid < G) {
    const int m0 = min(base, sc.max_mtiles);
    const int m1 = min(base + mts, sc.max_mtiles);
    sc.grp_rows[tid] = min(rows, (m1 - m0) * sc.BM);
    sc.grp_off[tid] = tid < E ? L.s_off[tid] : 0;
    sc.mt_start[tid] = m0;
    const int grows = min(rows, (m1 - m0) * sc.BM), goff = tid < E ? L.s_off[tid] : 0;
    for (int m = m0; m < m1; ++m) {
      sc.mt_group[m] = tid;
      if (sc.mt_info) {
        ((int4*)sc.mt_info)[2 * m] = int4{tid, m0, m1 - m0, grows};
        ((int4*)sc.mt_info)[2 * m + 1] = int4{goff, 0, 0, 0};
      }
    }
  }
  if (tid == 0) sc.mt_start[G] = min(mt_total, sc.max_mtiles);
}

__global__ __launch_bounds__(1024) void align_small_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ psum_part, int nblk, int T, int E,
    int k, int cap, float* __restrict__ prob_sum, int32_t* __restrict__ counts_pre,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_assign, int32_t* __restrict__ assign_pos, int n_shared,
    Schedule sc) {
  __shared__ AlignLds L;
  const int tid = threadIdx.x;
  const int n = T * k;
  // the ids are loaded first, so their latency overlaps the sums below
  const int my_id = tid < n ? ids[tid] : 0;

  // probability sums: the top-k workgroups' partials, added in workgroup order, with up to 32
  // loads in flight (a decode batch of 128 tokens has 32 partial rows; the kernel took the same
  // time, 9.6-9.8 us, with eight in flight)
  if (prob_sum && tid < E) {
    float s = 0.f;
    int b = 0;
    for (; b + 32 <= nblk; b += 32) {
      float v[32];
#pragma unroll
      for (int u = 0; u < 32; ++u) v[u] = psum_part[(size_t)(b + u) * E + tid];
#pragma unroll
      for (int u = 0; u < 32; ++u) s += v[u];
    }
    for (; b + 8 <= nblk; b += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = psum_part[(size_t)(b + u) * E + tid];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; b < nblk; ++b) s += psum_part[(size_t)b * E + tid];
    prob_sum[tid] = s;
  }
  if (tid < n) L.s_ids[tid] = my_id;
  for (int i = tid; i < NWAVE * 256; i += 1024) (&L.wcnt[0][0])[i] = 0;
  __syncthreads();
  align_schedule_lds(L, n, T, E, cap, counts_pre, counts, offsets, sorted_assign, assign_pos,
                     n_shared, sc);
}

// ------------------------------------------------------------------ fused top-k + grouping
// After the router's logits kernel (split-K fp32 partials, many workgroups), one workgroup of 16
// waves does the rest of the routing of a small batch (T <= 16, T*k <= 1024) in one launch:
//   1. one token per wave at a time: the K-split partials added in slice order, the offset,
//      softmax, top-k and renormalised gates with the DPP wave reductions of topk.h -- the same
//      per-token code as route_topk_kernel, so ids and gates are the same bits; each wave keeps
//      running probability sums, added in wave order at the end (prob_sum);
//   2. grouping by expert with the capacity limit, and the grouped-GEMM schedule, out of LDS.
// At decode sizes each launch costs a few microseconds of fixed latency for almost no work; this
// replaces the top-k launch and the grouping launch with one. (Computing the logits in this
// workgroup too was measured slower: one CU streams w_gate at a fraction of the rate that the
// logits kernel's workgroups reach together.)
constexpr int kSmallTopkTokens = 16;   // one token per wave

__global__ __launch_bounds__(1024) void topk_align_small_kernel(
    const float* __restrict__ part, int KS, int T, int E, int E_pad, int k,
    const float* __restrict__ logit_bias, const float* __restrict__ sel_bias,
    int32_t* __restrict__ ids, float* __restrict__ gates, float* __restrict__ prob_sum, int do_align,
    int cap, int32_t* __restrict__ counts_pre, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_assign,
    int32_t* __restrict__ assign_pos, int n_shared, Schedule sc) {
  __shared__ float pw[NWAVE][256];
  __shared__ AlignLds L;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- 1. softmax, top-k, gates; per-wave probability sums
  float pacc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int t = wave; t < T; t += NWAVE) {
    float lgv[4], pr[4];
    bool live[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      live[i] = e < E;
      lgv[i] = live[i] ? sum_partials(part, KS, T, E_pad, t, e) + (logit_bias ? logit_bias[e] : 0.f)
                       : -INFINITY;
    }
    int my_e;
    float my_g;
    token_topk(lgv, live, sel_bias, k, lane, pr, my_e, my_g);
#pragma unroll
    for (int i = 0; i < 4; ++i) pacc[i] += pr[i];
    if (lane < k) {
      ids[(size_t)t * k + lane] = my_e;
      gates[(size_t)t * k + lane] = my_g;
      L.s_ids[t * k + lane] = my_e;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) pw[wave][lane + 64 * i] = pacc[i];
  for (int i = tid; i < NWAVE * 256; i += 1024) (&L.wcnt[0][0])[i] = 0;
  __syncthreads();
  if (prob_sum && tid < E) {
    float s = 0.f;
    for (int wv = 0; wv < NWAVE; ++wv) s += pw[wv][tid];
    prob_sum[tid] = s;
  }
  if (!do_align) return;   // uniform

  // ---- 2. grouping + schedule
  align_schedule_lds(L, T * k, T, E, cap, counts_pre, counts, offsets, sorted_assign, assign_pos,
                     n_shared, sc);
}

}  // namespace

bool small_routing(const moe_problem& p) { return (long long)p.T * p.k <= 1024; }

// top-k and grouping in one workgroup after the logits: at most 4 tokens per wave
bool small_topk_fused(const moe_problem& p) {
  return p.T >= 1 && p.T <= kSmallTopkTokens && small_routing(p);
}

hipError_t launch_topk_align_small(const moe_problem& p, int cap, const float* logits_part,
                                   const float* logit_bias, const float* sel_bias, int32_t* ids,
                                   float* gates, float* prob_sum, bool do_align,
                                   int32_t* counts_pre, int32_t* counts, int32_t* offsets,
                                   int32_t* sorted_assign, int32_t* assign_pos, const Schedule& sc,
                                   hipStream_t s) {
  if (!small_topk_fused(p)) return hipErrorInvalidValue;
  const int E_pad = ceil_div(p.E, 16) * 16;
  hipLaunchKernelGGL(topk_align_small_kernel, dim3(1), dim3(1024), 0, s, logits_part,
                     route_ksplit(p), p.T, p.E, E_pad, p.k, logit_bias, sel_bias, ids, gates,
                     prob_sum, do_align ? 1 : 0, cap, counts_pre, counts, offsets, sorted_assign,
                     assign_pos, p.n_shared, sc);
  return hipGetLastError();
}

hipError_t launch_route_align_small(const moe_problem& p, int cap, const float* logits_part,
                                    const float* logit_bias, const float* sel_bias, int32_t* ids,
                                    float* gates, float* prob_sum, float* psum_part,
                                    int32_t* counts_pre, int32_t* counts, int32_t* offsets,
                                    int32_t* sorted_assign, int32_t* assign_pos, const Schedule& sc,
                                    hipStream_t s) {
  hipError_t err = launch_route_topk(p, logits_part, logit_bias, sel_bias, ids, gates,
                                     prob_sum ? psum_part : nullptr, s);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(align_small_kernel, dim3(1), dim3(1024), 0, s, ids, psum_part,
                     route_topk_blocks(p), p.T, p.E, p.k, cap, prob_sum, counts_pre, counts,
                     offsets, sorted_assign, assign_pos, p.n_shared, sc);
  return hipGetLastError();
}

}  // namespace moe
