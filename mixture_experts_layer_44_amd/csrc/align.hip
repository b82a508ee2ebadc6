// Grouping of the T*k assignments by expert, with an optional capacity limit.
//
// Pages: "Mixture of experts (MoE)" handbook, "Implementation: token by token vs. grouped
// by expert" (count per expert = histogram, segment start = prefix sum, a stable sort by
// expert keeps each expert's assignments in their original order); "MoE Architecture" §2
// "Expert capacity and token dropping" (assignments beyond an expert's capacity add
// nothing). Overflow is dropped first-come in ascending flat index a = t*k + j.
//
// Three launches, all deterministic (positions never depend on atomic arrival order):
//   count:   one workgroup per 1024-assignment chunk; LDS histogram -> blk_counts[b][e].
//   scan:    one workgroup; per expert, exclusive prefix over chunks (blk_base), the
//            pre-drop count, the capacity clamp and the exclusive prefix over experts.
//   scatter: one workgroup of 16 waves per chunk, one assignment per thread. Inside a wave
//            the rank among equal experts comes from ballots (lanes below with the same
//            expert); across waves from per-wave LDS counts of the waves before.
//            rank = blk_base + in-chunk rank; kept iff rank < cap.
// A separate one-workgroup kernel turns the offsets into the grouped-GEMM m-tile list.
#include "moe_internal.h"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void align_count_kernel(const int32_t* __restrict__ ids, int n,
                                                          int E, int32_t* __restrict__ blk_counts) {
  __shared__ int hist[256];
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int a0 = blockIdx.x * kAlignChunk;
  for (int i = threadIdx.x; i < kAlignChunk; i += 256) {
    int a = a0 + i;
    if (a < n) {
      int e = ids[a];
      if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) blk_counts[(size_t)blockIdx.x * E + e] = hist[e];
}

// exclusive block scan of one int per thread (256 threads)
__device__ int block_exclusive_scan(int v, int* tmp, int* total) {
  const int tid = threadIdx.x;
  tmp[tid] = v;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    int add = tid >= o ? tmp[tid - o] : 0;
    __syncthreads();
    tmp[tid] += add;
    __syncthreads();
  }
  int incl = tmp[tid];
  *total = tmp[255];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(256) void align_scan_kernel(
    const int32_t* __restrict__ blk_counts, int nblk, int E, int cap,
    int32_t* __restrict__ blk_base, int32_t* __restrict__ counts_pre, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets) {
  __shared__ int tmp[256];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    // the chunk counts are loaded eight at a time before they are added (one dependent round
    // trip per chunk made this a dozen microseconds at 32 chunks)
    int b = 0;
    for (; b + 8 <= nblk; b += 8) {
      int c[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) c[u] = blk_counts[(size_t)(b + u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        blk_base[(size_t)(b + u) * E + e] = run;
        run += c[u];
      }
    }
    for (; b < nblk; ++b) {
      blk_base[(size_t)b * E + e] = run;
      run += blk_counts[(size_t)b * E + e];
    }
  }
  const int kept = e < E ? (cap >= 0 && run > cap ? cap : run) : 0;
  int total;
  const int off = block_exclusive_scan(kept, tmp, &total);
  if (e < E) {
    counts_pre[e] = run;
    counts[e] = kept;
    offsets[e] = off;
  }
  if (e == 0) offsets[E] = total;
}

__global__ __launch_bounds__(1024) void align_scatter_kernel(
    const int32_t* __restrict__ ids, int n, int E, int cap, const int32_t* __restrict__ blk_base,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_assign,
    int32_t* __restrict__ assign_pos) {
  static_assert(kAlignChunk == 1024, "one assignment per thread");
  constexpr int NW = 16;
  __shared__ int wcnt[NW][256];  // assignments of expert e in wave w of this chunk
  __shared__ int cbase[256];     // this chunk's base rank of expert e
  __shared__ int first[256];     // offsets[e] + cbase[e]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < NW * 256; i += 1024) (&wcnt[0][0])[i] = 0;
  if (tid < E) {
    cbase[tid] = blk_base[(size_t)blockIdx.x * E + tid];
    first[tid] = offsets[tid] + cbase[tid];
  }
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int a = blockIdx.x * kAlignChunk + tid;
  int e = -1;
  if (a < n) {
    e = ids[a];
    if ((unsigned)e >= (unsigned)E) e = -1;
  }
  const bool valid = e >= 0;
  __syncthreads();   // wcnt zeroed
  int my_rank = 0;
  uint64_t active = __ballot(valid);
  while (active) {
    const int leader = __ffsll((unsigned long long)active) - 1;
    const int le = __builtin_amdgcn_readlane(e, leader);   // leader is wave-uniform
    const uint64_t m = __ballot(valid && e == le);
    if (valid && e == le) {
      my_rank = __popcll(m & lt_mask);
      if (lane == leader) wcnt[wave][e] = __popcll(m);
    }
    active &= ~m;
  }
  __syncthreads();
  if (a < n) {
    int pos = -1;
    if (valid) {
      int rank = my_rank;   // rank inside this chunk: lanes below, then the waves before
      for (int w = 0; w < wave; ++w) rank += wcnt[w][e];
      if (cap < 0 || cbase[e] + rank < cap) {
        pos = first[e] + rank;
        sorted_assign[pos] = a;
      }
    }
    assign_pos[a] = pos;
  }
}

// m-tile list for the grouped GEMMs: group g has ceil(rows_g / BM) m-tiles.
// Offsets that did not come from align (decreasing, or past T*k) are clamped so that every
// group stays inside [0, T*k) and the m-tile count inside the list's capacity.
__global__ __launch_bounds__(256) void schedule_kernel(const int32_t* __restrict__ offsets, int E,
                                                       int n_shared, int T, int n, int BM,
                                                       Schedule sc) {
  __shared__ int tmp[256];
  const int G = E + n_shared;   // n: rows that the routed segments can span
  // each thread owns groups 2*tid, 2*tid+1 (G <= 257 < 512)
  int rows[2], offs[2], mts[2];
  for (int i = 0; i < 2; ++i) {
    int g = 2 * threadIdx.x + i;
    rows[i] = 0;
    offs[i] = 0;
    if (g < E) {
      const int o0 = min(max(offsets[g], 0), n);
      const int o1 = min(max(offsets[g + 1], o0), n);
      offs[i] = o0;
      rows[i] = o1 - o0;
    } else if (g < G) {
      rows[i] = T;
    }
    mts[i] = (rows[i] + BM - 1) / BM;
  }
  int total;
  int base = block_exclusive_scan(mts[0] + mts[1], tmp, &total);
  for (int i = 0; i < 2; ++i) {
    int g = 2 * threadIdx.x + i;
    if (g < G) {
      const int m0 = min(base, sc.max_mtiles);
      const int m1 = min(base + mts[i], sc.max_mtiles);
      sc.grp_rows[g] = min(rows[i], (m1 - m0) * BM);
      sc.grp_off[g] = offs[i];
      sc.mt_start[g] = m0;
      for (int m = m0; m < m1; ++m) {
        sc.mt_group[m] = g;
        if (sc.mt_info) {
          ((int4*)sc.mt_info)[2 * m] = int4{g, m0, m1 - m0, min(rows[i], (m1 - m0) * BM)};
          ((int4*)sc.mt_info)[2 * m + 1] = int4{offs[i], 0, 0, 0};
        }
      }
    }
    base += mts[i];
  }
  if (threadIdx.x == 0) sc.mt_start[G] = min(total, sc.max_mtiles);
}

}  // namespace

int max_mtiles(long long n_rows, int T, int E, int n_shared, int BM) {
  long long m = (n_rows + BM - 1) / BM + E + (n_shared ? (T + BM - 1) / BM + 1 : 0);
  return (int)m;
}

hipError_t launch_align(const moe_problem& p, int cap, const int32_t* ids, int32_t* counts_pre,
                        int32_t* counts, int32_t* offsets, int32_t* sorted_assign,
                        int32_t* assign_pos, int32_t* blk_counts, int32_t* blk_base, hipStream_t s) {
  const int n = p.T * p.k;
  const int nblk = ceil_div(n, kAlignChunk);
  if (nblk > 0) {
    hipLaunchKernelGGL(align_count_kernel, dim3(nblk), dim3(256), 0, s, ids, n, p.E, blk_counts);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(align_scan_kernel, dim3(1), dim3(256), 0, s, blk_counts, nblk, p.E, cap,
                     blk_base, counts_pre, counts, offsets);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || nblk == 0) return err;
  hipLaunchKernelGGL(align_scatter_kernel, dim3(nblk), dim3(1024), 0, s, ids, n, p.E, cap, blk_base,
                     offsets, sorted_assign, assign_pos);
  return hipGetLastError();
}

hipError_t launch_schedule(const moe_problem& p, const int32_t* offsets, const Schedule& sc,
                           hipStream_t s, long long n_rows) {
  const int n = (int)(n_rows < 0 ? (long long)p.T * p.k : n_rows);
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(256), 0, s, offsets, p.E, p.n_shared, p.T, n,
                     sc.BM, sc);
  return hipGetLastError();
}

}  // namespace moe
