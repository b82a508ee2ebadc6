// Gate-weighted combine back to token order, and the balance statistics.
//
// Pages: "MoE Architecture" §1 (y is the sum over the chosen experts of gate times expert
// output) and §3 "Shared Experts (DeepSeek)" (shared experts are added to the routed sum);
// "Mixture of experts (MoE)" handbook, "Implementation" (results are scattered back to
// their original positions with their weights); "MoE Architecture" §2 "Load Balancing"
// (L = alpha * E * sum_i f_i p_i).
//
// combine: one workgroup per token row, 16-byte loads/stores along d; the loads of up to 8
// slots are issued together, and the slots are added in slot order after the shared row, so y
// is bit-reproducible from run to run. The expert rows are read once and y is written once:
// both go with the non-temporal hint (DeepSeek-V3-shaped combine 262 -> 215 us).
#include "moe_internal.h"

namespace moe {

namespace {

template <int NS>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ out_rows,
                                                      const float* __restrict__ out_rows_b,
                                                      const int32_t* __restrict__ assign_pos,
                                                      const float* __restrict__ topk_w,
                                                      const float* __restrict__ shared_out, int d,
                                                      int k, float* __restrict__ y) {
  const int t = blockIdx.x;
  const int n = gridDim.x * k;   // rows of out_rows that can exist: T*k
  __shared__ int pos[32];
  __shared__ float wt[32];
  if (threadIdx.x < k) {
    pos[threadIdx.x] = assign_pos[(size_t)t * k + threadIdx.x];
    wt[threadIdx.x] = topk_w[(size_t)t * k + threadIdx.x];
  }
  __syncthreads();
  // the first NS slots of this token in registers (the same in every lane)
  int r8[NS];
  float g8[NS];
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    const int r = u < k ? pos[u] : -1;
    r8[u] = r >= 0 && r < n ? r : -1;
    g8[u] = u < k ? wt[u] : 0.f;
  }
  const int d4 = d >> 2;
  // Two 16-byte column chunks per thread and pass (c and c + 256): the loads of both are issued
  // before either is added, so a short row (decode) takes one round trip instead of two.
  for (int c0 = threadIdx.x; c0 < d4; c0 += 512) {
    const bool two = c0 + 256 < d4;   // uniform except in the last pass of a ragged row
    f32x4 acc[2];
    f32x4 v[2][NS], vb[2][NS];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = c0 + 256 * h;
      const bool live = h == 0 || two;
      acc[h] = shared_out && live
                   ? __builtin_nontemporal_load((const f32x4*)(shared_out + (size_t)t * d + 4 * c))
                   : f32x4{0.f, 0.f, 0.f, 0.f};
      // the loads of the kept slots among the first NS (a dropped slot loads nothing: out_rows
      // may hold only kept rows)
#pragma unroll
      for (int u = 0; u < NS; ++u) {
        v[h][u] = vb[h][u] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (r8[u] < 0 || !live) continue;
        const size_t o = (size_t)r8[u] * d + 4 * c;
        v[h][u] = __builtin_nontemporal_load((const f32x4*)(out_rows + o));
        if (out_rows_b) vb[h][u] = __builtin_nontemporal_load((const f32x4*)(out_rows_b + o));
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = c0 + 256 * h;
      if (h == 1 && !two) break;
      // slots added in slot order after the shared row
#pragma unroll
      for (int u = 0; u < NS; ++u) {
        if (r8[u] < 0) continue;
        f32x4 w = v[h][u];
        if (out_rows_b) {
          w[0] += vb[h][u][0];
          w[1] += vb[h][u][1];
          w[2] += vb[h][u][2];
          w[3] += vb[h][u][3];
        }
        acc[h][0] = fmaf(g8[u], w[0], acc[h][0]);
        acc[h][1] = fmaf(g8[u], w[1], acc[h][1]);
        acc[h][2] = fmaf(g8[u], w[2], acc[h][2]);
        acc[h][3] = fmaf(g8[u], w[3], acc[h][3]);
      }
      for (int j = NS; j < k; ++j) {   // slots past the first NS, one at a time
        const int r = pos[j];
        if (r < 0 || r >= n) continue;
        f32x4 w = *(const f32x4*)(out_rows + (size_t)r * d + 4 * c);
        if (out_rows_b) {
          const f32x4 wb = *(const f32x4*)(out_rows_b + (size_t)r * d + 4 * c);
          w[0] += wb[0];
          w[1] += wb[1];
          w[2] += wb[2];
          w[3] += wb[3];
        }
        const float g = wt[j];
        acc[h][0] = fmaf(g, w[0], acc[h][0]);
        acc[h][1] = fmaf(g, w[1], acc[h][1]);
        acc[h][2] = fmaf(g, w[2], acc[h][2]);
        acc[h][3] = fmaf(g, w[3], acc[h][3]);
      }
      __builtin_nontemporal_store(acc[h], (f32x4*)(y + (size_t)t * d + 4 * c));
    }
  }
}

// out_rows[r] += out_rows_b[r] over the kept rows (offsets[E] of them), 16 bytes per lane
__global__ __launch_bounds__(256) void add_rows_kernel(float* __restrict__ out_rows,
                                                       const float* __restrict__ out_rows_b,
                                                       const int32_t* __restrict__ offsets, int E,
                                                       int d) {
  const long long n4 = (long long)offsets[E] * (d >> 2);
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n4;
       i += (long long)gridDim.x * 256) {
    f32x4 a = ((f32x4*)out_rows)[i];
    const f32x4 b = ((const f32x4*)out_rows_b)[i];
    a[0] += b[0];
    a[1] += b[1];
    a[2] += b[2];
    a[3] += b[3];
    ((f32x4*)out_rows)[i] = a;
  }
}

__global__ __launch_bounds__(256) void balance_kernel(const int32_t* __restrict__ counts_pre,
                                                      const float* __restrict__ prob_sum, int T,
                                                      int k, int E, float alpha,
                                                      float* __restrict__ f, float* __restrict__ P,
                                                      float* __restrict__ L) {
  __shared__ double part[256];
  const int e = threadIdx.x;
  double fp = 0.0;
  if (e < E) {
    const double fe = T > 0 ? (double)counts_pre[e] / ((double)T * k) : 0.0;
    const double pe = T > 0 ? (double)prob_sum[e] / (double)T : 0.0;
    f[e] = (float)fe;
    P[e] = (float)pe;
    fp = fe * pe;
  }
  part[e] = fp;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (e < o) part[e] += part[e + o];
    __syncthreads();
  }
  if (e == 0) L[0] = (float)((double)alpha * E * part[0]);
}

// sel_bias[e] += gamma * sign(T*k - E*counts_pre[e]) (64-bit integer comparison, fp32 step)
__global__ __launch_bounds__(256) void bias_update_kernel(const int32_t* __restrict__ counts_pre,
                                                          int T, int k, int E, float gamma,
                                                          float* __restrict__ sel_bias) {
  const int e = threadIdx.x;
  if (e >= E) return;
  const long long load = (long long)E * counts_pre[e], mean = (long long)T * k;
  const float dir = load < mean ? 1.0f : (load > mean ? -1.0f : 0.0f);
  sel_bias[e] = sel_bias[e] + gamma * dir;
}

}  // namespace

hipError_t launch_bias_update(const moe_problem& p, const int32_t* counts_pre, float gamma,
                              float* sel_bias, hipStream_t s) {
  hipLaunchKernelGGL(bias_update_kernel, dim3(1), dim3(256), 0, s, counts_pre, p.T, p.k, p.E,
                     gamma, sel_bias);
  return hipGetLastError();
}

hipError_t launch_combine(const moe_problem& p, const float* out_rows, const float* out_rows_b,
                          const int32_t* assign_pos, const float* topk_w, const float* shared_out,
                          float* y, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  // slots whose loads are issued together: enough for k up to 8, few registers for small k
  auto kern = p.k <= 2 ? combine_kernel<2> : (p.k <= 4 ? combine_kernel<4> : combine_kernel<8>);
  hipLaunchKernelGGL(kern, dim3(p.T), dim3(256), 0, s, out_rows, out_rows_b, assign_pos, topk_w,
                     shared_out, p.d, p.k, y);
  return hipGetLastError();
}

hipError_t launch_add_rows(const moe_problem& p, float* out_rows, const float* out_rows_b,
                           const int32_t* offsets, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  hipLaunchKernelGGL(add_rows_kernel, dim3(1024), dim3(256), 0, s, out_rows, out_rows_b, offsets,
                     p.E, p.d);
  return hipGetLastError();
}

hipError_t launch_balance(const moe_problem& p, const int32_t* counts_pre, const float* prob_sum,
                          float alpha, float* f, float* P, float* L, hipStream_t s) {
  hipLaunchKernelGGL(balance_kernel, dim3(1), dim3(256), 0, s, counts_pre, prob_sum, p.T, p.k, p.E,
                     alpha, f, P, L);
  return hipGetLastError();
}

}  // namespace moe
