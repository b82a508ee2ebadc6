// Small-batch grouping in one launch: probability sums + grouping by expert (with the capacity
// limit) + grouped-GEMM schedule, for T*k <= 1024 (decode-sized batches). The top-k before it
// runs one token per wave over many workgroups (route.hip).
//
// Same definitions as route.hip (top-k, renormalised gates: "MoE Architecture" §2 "Gating
// Function"; "MoE (Mixture of Experts) Deep Dive", "Weighted Sum Output") and align.hip
// (histogram, prefix sum, stable order by expert, first-come capacity dropping: "Mixture of
// experts (MoE)" handbook, "Implementation"; "MoE Architecture" §2 "Expert capacity and
// token dropping"); the outputs are bit-identical to those launches. At decode sizes each
// of those steps is a few microseconds of launch latency and almost no work, so a single
// 1024-thread workgroup does them back to back out of LDS.
#include "topk.h"

namespace moe {

namespace {

constexpr int NWAVE = 16;

// exclusive scan of v over the first 320 threads (5 waves; the values live in threads < 257,
// the others pass 0); all 1024 threads call it. Each wave scans its 64 values with shuffles,
// then adds the totals of the waves before it.
__device__ int scan320(int v, int* wsum, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63 && wave < 5) wsum[wave] = x;
  __syncthreads();
  int base = 0;
#pragma unroll
  for (int w = 0; w < 5; ++w) base += w < wave ? wsum[w] : 0;
  *total = wsum[0] + wsum[1] + wsum[2] + wsum[3] + wsum[4];
  __syncthreads();   // wsum is reused by the next call
  return base + x - v;
}

__global__ __launch_bounds__(1024) void align_small_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ psum_part, int nblk, int T, int E,
    int k, int cap, float* __restrict__ prob_sum, int32_t* __restrict__ counts_pre,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_assign, int32_t* __restrict__ assign_pos, int n_shared,
    Schedule sc) {
  __shared__ int s_ids[1024];
  __shared__ int wcnt[NWAVE][256];    // assignments of expert e in wave w
  __shared__ int s_off[257];
  __shared__ int wsum[5];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = T * k;

  // probability sums: the top-k workgroups' partials, added in workgroup order
  if (prob_sum && tid < E) {
    float s = 0.f;
    int b = 0;
    for (; b + 8 <= nblk; b += 8) {   // eight loads in flight, added in block order
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = psum_part[(size_t)(b + u) * E + tid];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; b < nblk; ++b) s += psum_part[(size_t)b * E + tid];
    prob_sum[tid] = s;
  }
  if (tid < n) s_ids[tid] = ids[tid];
  for (int i = tid; i < NWAVE * 256; i += 1024) (&wcnt[0][0])[i] = 0;
  __syncthreads();

  // ---- grouping: one assignment per thread, ranks from ballots + per-wave counts
  const int a = tid;
  const int e = a < n ? s_ids[a] : -1;
  const bool valid = e >= 0 && e < E;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int my_rank = 0;
  uint64_t active = __ballot(valid);
  while (active) {
    const int leader = __ffsll((unsigned long long)active) - 1;
    const int le = __shfl(e, leader);
    const uint64_t msk = __ballot(valid && e == le);
    if (valid && e == le) {
      my_rank = __popcll(msk & lt_mask);
      if (lane == leader) wcnt[wave][e] = __popcll(msk);
    }
    active &= ~msk;
  }
  __syncthreads();
  int c = 0, kept = 0;
  if (tid < E) {
    for (int w = 0; w < NWAVE; ++w) c += wcnt[w][tid];
    kept = (cap >= 0 && c > cap) ? cap : c;
  }
  int total;
  const int off = scan320(tid < E ? kept : 0, wsum, &total);
  if (tid < E) {
    counts_pre[tid] = c;
    counts[tid] = kept;
    offsets[tid] = off;
    s_off[tid] = off;
  }
  if (tid == 0) {
    offsets[E] = total;
    s_off[E] = total;
  }
  __syncthreads();
  if (a < n) {
    int pos = -1;
    if (valid) {
      int rank = my_rank;
      for (int w = 0; w < wave; ++w) rank += wcnt[w][e];
      if (cap < 0 || rank < cap) {
        pos = s_off[e] + rank;
        sorted_assign[pos] = a;
      }
    }
    assign_pos[a] = pos;
  }

  // ---- grouped-GEMM schedule (same as schedule_kernel)
  const int G = E + n_shared;
  int rows = 0;
  if (tid < E) rows = s_off[tid + 1] - s_off[tid];
  else if (tid < G) rows = T;
  const int mts = (rows + sc.BM - 1) / sc.BM;
  int mt_total;
  const int base = scan320(tid < G ? mts : 0, wsum, &mt_total);
  if (tid < G) {
    const int m0 = min(base, sc.max_mtiles);
    const int m1 = min(base + mts, sc.max_mtiles);
    sc.grp_rows[tid] = min(rows, (m1 - m0) * sc.BM);
    sc.grp_off[tid] = tid < E ? s_off[tid] : 0;
    sc.mt_start[tid] = m0;
    for (int m = m0; m < m1; ++m) sc.mt_group[m] = tid;
  }
  if (tid == 0) sc.mt_start[G] = min(mt_total, sc.max_mtiles);
}

}  // namespace

bool small_routing(const moe_problem& p) { return (long long)p.T * p.k <= 1024; }

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
