// Small-batch routing (T*k <= 1024, decode-sized batches).
//
// Two paths, both with the definitions of route.hip (top-k, renormalised gates: "MoE
// Architecture" §2 "Gating Function"; "MoE (Mixture of Experts) Deep Dive", "Router Network
// Computation" and "Weighted Sum Output") and align.hip (histogram, prefix sum, stable order by
// expert, first-come capacity dropping: "Mixture of experts (MoE)" handbook, "Implementation";
// "MoE Architecture" §2 "Expert capacity and token dropping"):
//   - route_small_kernel (bf16, T <= 128): the fused router, one launch: logits kept in LDS,
//     softmax / top-k with wave reductions, then grouping and the GEMM schedule.
//   - align_small_kernel: after the multi-launch logits and top-k (fp32 storage, or batches the
//     fused kernel does not take), probability sums + grouping + schedule in one workgroup.
// The grouping is bit-identical to the multi-launch align kernels. At decode sizes each of
// those steps is a few microseconds of launch latency and almost no work, so a single
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

// LDS of the grouping step
struct AlignLds {
  int s_ids[1024];        // the T*k expert ids, flat assignment order
  int wcnt[NWAVE][256];   // assignments of expert e in wave w
  int s_off[257];
  int wsum[5];
};

// Grouping by expert + grouped-GEMM schedule out of LDS, one assignment per thread: all 1024
// threads call it after L.s_ids[0..n) is filled and L.wcnt zeroed (and a barrier). Ranks come
// from ballots inside a wave plus the per-wave counts of earlier waves, i.e. ascending flat
// index a inside each expert, as the multi-launch path's stable order.
__device__ void align_schedule_lds(AlignLds& L, int n, int T, int E, int cap,
                                   int32_t* __restrict__ counts_pre, int32_t* __restrict__ counts,
                                   int32_t* __restrict__ offsets,
                                   int32_t* __restrict__ sorted_assign,
                                   int32_t* __restrict__ assign_pos, int n_shared,
                                   const Schedule& sc) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int a = tid;
  const int e = a < n ? L.s_ids[a] : -1;
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
  if (a < n) {
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
    for (int m = m0; m < m1; ++m) sc.mt_group[m] = tid;
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
  if (tid < n) L.s_ids[tid] = ids[tid];
  for (int i = tid; i < NWAVE * 256; i += 1024) (&L.wcnt[0][0])[i] = 0;
  __syncthreads();
  align_schedule_lds(L, n, T, E, cap, counts_pre, counts, offsets, sorted_assign, assign_pos,
                     n_shared, sc);
}

// ------------------------------------------------------------------ fused decode router
// The whole router of a small batch in one workgroup, the logits never leaving the CU:
//   1. logits [T][E_pad] = x . w_gate^T with v_mfma_f32_16x16x32_bf16 (fp32 accumulate). Wave w
//      takes expert tile w % tiles (16 experts) over K slice w / tiles (d / S columns); its
//      16-byte operand loads go straight to registers, U steps of 32 ahead. The S slices' partial
//      logits are added into LDS in slice order (deterministic).
//   2. one token per wave at a time: offset, softmax, top-k and renormalised gates with the DPP
//      wave reductions of topk.h; each wave keeps its own running probability sums, added in wave
//      order at the end (prob_sum).
//   3. grouping by expert with the capacity limit and the grouped-GEMM schedule, out of LDS.
// At decode sizes the multi-launch router spends most of its time in launch latency and global
// round trips between its three kernels; here one CU streams w_gate once (512 KB for E = 128,
// d = 2048) and everything after stays on chip.
constexpr int kSmallLogits = 16384;   // T * E_pad logits kept in LDS (64 KB)

template <int NF>
__global__ __launch_bounds__(1024) void route_small_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ w, int T, int d, int E, int E_pad,
    int k, int S, const float* __restrict__ logit_bias, const float* __restrict__ sel_bias,
    int32_t* __restrict__ ids, float* __restrict__ gates, float* __restrict__ prob_sum,
    int do_align, int cap, int32_t* __restrict__ counts_pre, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_assign,
    int32_t* __restrict__ assign_pos, int n_shared, Schedule sc) {
  __shared__ float lg[kSmallLogits];
  __shared__ float pw[NWAVE][256];
  __shared__ AlignLds L;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tiles = E_pad / 16;
  const bool gemm_wave = wave < tiles * S;
  const int tile = wave % tiles, slice = wave / tiles;
  const int r = lane & 15, kq = (lane >> 4) * 8;
  const int e_b = tile * 16 + r;

  // ---- 1. logits
  f32x4 acc[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (gemm_wave) {
    const int klen = d / S, kb0 = slice * klen;
    const bool b_ok = e_b < E;
    const bf16_t* bp = w + (size_t)(b_ok ? e_b : 0) * d + kb0 + kq;
    const bf16_t* ap[NF];
    bool a_ok[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int t = 16 * f + r;
      a_ok[f] = t < T;
      ap[f] = x + (size_t)(a_ok[f] ? t : 0) * d + kb0 + kq;   // rows past T read row 0, zeroed
    }
    const bf16x8 z8 = {};
    constexpr int U = NF == 1 ? 8 : (NF == 2 ? 4 : (NF == 4 ? 2 : 1));
    const int nsteps = klen / 32;
    int st = 0;
    for (; st + U <= nsteps; st += U) {
      bf16x8 a[U][NF], b[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        b[u] = *(const bf16x8*)(bp + (st + u) * 32);
#pragma unroll
        for (int f = 0; f < NF; ++f) a[u][f] = *(const bf16x8*)(ap[f] + (st + u) * 32);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int f = 0; f < NF; ++f)
          acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_ok[f] ? a[u][f] : z8,
                                                           b_ok ? b[u] : z8, acc[f], 0, 0, 0);
    }
    for (; st < nsteps; ++st) {
      const bf16x8 b = *(const bf16x8*)(bp + st * 32);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const bf16x8 a = *(const bf16x8*)(ap[f] + st * 32);
        acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_ok[f] ? a : z8, b_ok ? b : z8, acc[f],
                                                         0, 0, 0);
      }
    }
  }
  // C layout (16x16): lane holds column (expert) lane%16, rows (tokens) 4*(lane/16)+i. The
  // slices are added in slice order: slice 0 writes, then each later slice adds its part.
  for (int sl = 0; sl < S; ++sl) {
    if (gemm_wave && slice == sl) {
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * f + 4 * (lane >> 4) + i;
          if (t < T) {
            float* dst = &lg[t * E_pad + e_b];
            *dst = sl == 0 ? acc[f][i] : *dst + acc[f][i];
          }
        }
    }
    __syncthreads();
  }

  // ---- 2. softmax, top-k, gates; per-wave probability sums
  float pacc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int t = wave; t < T; t += NWAVE) {
    float lgv[4], pr[4];
    bool live[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      live[i] = e < E;
      lgv[i] = live[i] ? lg[t * E_pad + e] + (logit_bias ? logit_bias[e] : 0.f) : -INFINITY;
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

  // ---- 3. grouping + schedule
  align_schedule_lds(L, T * k, T, E, cap, counts_pre, counts, offsets, sorted_assign, assign_pos,
                     n_shared, sc);
}

}  // namespace

bool small_routing(const moe_problem& p) { return (long long)p.T * p.k <= 1024; }

// the fused one-workgroup router: bf16, T*k <= 1024, at most 128 tokens (8 row fragments) and
// their logits fit the LDS table
bool small_route_fused(const moe_problem& p) {
  const int E_pad = ceil_div(p.E, 16) * 16;
  return p.dtype == MOE_BF16 && p.T >= 1 && p.T <= 128 && small_routing(p) &&
         (long long)p.T * E_pad <= kSmallLogits;
}

hipError_t launch_route_small(const moe_problem& p, int cap, const void* x, const void* w_gate,
                              const float* logit_bias, const float* sel_bias, int32_t* ids,
                              float* gates, float* prob_sum, bool do_align, int32_t* counts_pre,
                              int32_t* counts, int32_t* offsets, int32_t* sorted_assign,
                              int32_t* assign_pos, const Schedule& sc, hipStream_t s) {
  if (!small_route_fused(p)) return hipErrorInvalidValue;
  const int E_pad = ceil_div(p.E, 16) * 16;
  const int tiles = E_pad / 16;
  // K slices: as many as the 16 waves allow, each a whole number of 32-column steps
  int S = NWAVE / tiles;
  while (S > 1 && p.d % (32 * S)) --S;
  auto kern = p.T <= 16 ? route_small_kernel<1>
            : p.T <= 32 ? route_small_kernel<2>
            : p.T <= 64 ? route_small_kernel<4> : route_small_kernel<8>;
  hipLaunchKernelGGL(kern, dim3(1), dim3(1024), 0, s, (const bf16_t*)x, (const bf16_t*)w_gate, p.T,
                     p.d, p.E, E_pad, p.k, S, logit_bias, sel_bias, ids, gates, prob_sum,
                     do_align ? 1 : 0, cap, counts_pre, counts, offsets, sorted_assign, assign_pos,
                     p.n_shared, sc);
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
