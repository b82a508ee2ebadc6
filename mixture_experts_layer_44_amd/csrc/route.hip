// Router: logits = x . w_gate^T (+ logit_bias), softmax, top-k on logits (+ sel_bias),
// renormalised gates, per-workgroup probability sums.
//
// Pages: "MoE Architecture" §2 "Gating Function" (softmax of x W_gate, top-k, weights
// renormalised over the k kept scores); "MoE (Mixture of Experts) Deep Dive", "Weighted
// Sum Output" (kept probabilities divided by their sum); "Mixture of experts (MoE)"
// handbook, "Load balancing" (the balancing bias only chooses experts).
//
// Two launches:
//  logits: grid (token tiles of 64) x (expert groups of 64) x (KS slices of d). A workgroup
//          of 4 waves computes a 64 x 64 block of partial logits over its d slice with
//          v_mfma_f32_16x16x32_bf16 (fp32 accumulate): each wave takes the whole block over a
//          quarter of the slice (4 token rows and up to 4 expert rows loaded per 16 MFMAs, so
//          every x and W_gate byte a workgroup needs is loaded once), and the four partials
//          are added in wave order through LDS. Loads are issued four k-steps ahead of the
//          MFMAs. KS is chosen on the host so that the grid has >= ~512 workgroups; the fp32
//          partials [KS][T][E_pad] never round to bf16. (fp32 storage: one partial logit per
//          wave, route_logits_f32_kernel.)
//  topk:   one wave per token. Sums the KS partials in slice order (run-to-run identical),
//          adds logit_bias, softmax, keys = logits (+ sel_bias), k rounds of a 64-lane
//          arg-max (larger key first, lower expert index on equal keys), gates = kept p /
//          their sum; per-workgroup sums of p for prob_sum.
#include <type_traits>

#include "topk.h"

namespace moe {

namespace {

constexpr int TM = 64;        // tokens per logits workgroup
constexpr int EN = 64;        // experts per logits workgroup
constexpr int UNROLL = 4;     // k-steps of loads in flight per wave
constexpr int TOPK_TOK = 4;   // tokens per top-k workgroup (one per wave)

// partial logits of a 64-token x 64-expert block over the d slice blockIdx.z
__global__ __launch_bounds__(256) void route_logits_kernel(const void* __restrict__ xv,
                                                           const void* __restrict__ wv, int T,
                                                           int d, int E, int E_pad, int KS,
                                                           float* __restrict__ part) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tok0 = blockIdx.x * TM;
  const int e0 = blockIdx.y * EN;
  const int ntiles = min(EN, E_pad - e0) / 16;      // 1..4 expert tiles in this group
  const int slice = d / KS, k_begin = blockIdx.z * slice;
  float* out = part + (size_t)blockIdx.z * T * E_pad;

  {
    constexpr int RS = EN + 4;                        // padded row of a wave's partials
    __shared__ float red[4][TM * RS];
    const bf16_t* x = (const bf16_t*)xv;
    const bf16_t* w = (const bf16_t*)wv;
    const int sub_len = slice / 4;                    // this wave's quarter of the slice
    const int kb0 = k_begin + wave * sub_len;
    const int r = lane & 15, kq = (lane >> 4) * 8;
    const bf16x8 z8 = {};
    // The block for NT expert tiles. Operand rows past T or E read row 0 and are zeroed.
    auto run = [&](auto nt_tag) {
      constexpr int NT = decltype(nt_tag)::value;
      const bf16_t* ap[4];
      bool a_ok[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = tok0 + 16 * i + r;
        a_ok[i] = t < T;
        ap[i] = x + (size_t)(a_ok[i] ? t : 0) * d + kq;
      }
      const bf16_t* bp[NT];
      bool b_ok[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int e = e0 + 16 * j + r;
        b_ok[j] = e < E;
        bp[j] = w + (size_t)(b_ok[j] ? e : 0) * d + kq;
      }
      f32x4 acc[4][NT];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      // walk the sub-slice starting at a per-workgroup offset (wrapping): rows are d*2 bytes
      // apart, and workgroups reading the same k offset at once collide on memory channels
      const int nsteps = sub_len / 32;
      const int rot = (blockIdx.x + blockIdx.y * 7) % nsteps;
      auto kpos = [&](int step) { return kb0 + ((step + rot) % nsteps) * 32; };
      auto mma = [&](const bf16x8 (&a)[4], const bf16x8 (&b)[NT]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x8 av = a_ok[i] ? a[i] : z8;
#pragma unroll
          for (int j = 0; j < NT; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b_ok[j] ? b[j] : z8, acc[i][j],
                                                                0, 0, 0);
        }
      };
      int st = 0;
      for (; st + UNROLL <= nsteps; st += UNROLL) {
        bf16x8 a[UNROLL][4], b[UNROLL][NT];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
          const int kb = kpos(st + u);
#pragma unroll
          for (int i = 0; i < 4; ++i) a[u][i] = *(const bf16x8*)(ap[i] + kb);
#pragma unroll
          for (int j = 0; j < NT; ++j) b[u][j] = *(const bf16x8*)(bp[j] + kb);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) mma(a[u], b[u]);
      }
      for (; st < nsteps; ++st) {
        const int kb = kpos(st);
        bf16x8 a[4], b[NT];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = *(const bf16x8*)(ap[i] + kb);
#pragma unroll
        for (int j = 0; j < NT; ++j) b[j] = *(const bf16x8*)(bp[j] + kb);
        mma(a, b);
      }
      // C layout (16x16): lane holds column (expert) lane%16, rows (tokens) 4*(lane/16)+q
      float* my = red[wave];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            my[(16 * i + 4 * (lane >> 4) + q) * RS + 16 * j + (lane & 15)] = acc[i][j][q];
    };
    if (ntiles >= 4) run(std::integral_constant<int, 4>{});
    else if (ntiles == 3) run(std::integral_constant<int, 3>{});
    else if (ntiles == 2) run(std::integral_constant<int, 2>{});
    else run(std::integral_constant<int, 1>{});
    __syncthreads();
    // thread -> (token, expert) of this block; the four quarters added in wave order
    const int ecount = ntiles * 16;
    for (int idx = tid; idx < TM * ecount; idx += 256) {
      const int tr = idx / ecount, ec = idx % ecount;
      const float s = ((red[0][tr * RS + ec] + red[1][tr * RS + ec]) + red[2][tr * RS + ec]) +
                      red[3][tr * RS + ec];
      if (tok0 + tr < T) out[(size_t)(tok0 + tr) * E_pad + e0 + ec] = s;
    }
  }
}

// fp32 storage: one partial logit (slice z, token t, expert e) per wave, the 64 lanes striding
// the slice (coalesced rows) and a DPP wave sum at the end (a fixed order). Enough waves for a
// small problem to spread over the CUs.
__global__ __launch_bounds__(256) void route_logits_f32_kernel(const float* __restrict__ x,
                                                               const float* __restrict__ w, int T,
                                                               int d, int E, int E_pad, int KS,
                                                               float* __restrict__ part) {
  const int lane = threadIdx.x & 63;
  const long long ntask = (long long)KS * T * E_pad;
  const int slice = d / KS;
  // wave-uniform loop over the tasks (the grid is capped by the launcher)
  for (long long task = (long long)blockIdx.x * 4 + (threadIdx.x >> 6); task < ntask;
       task += (long long)gridDim.x * 4) {
    const int e = (int)(task % E_pad);
    const long long rest = task / E_pad;
    const int t = (int)(rest % T), z = (int)(rest / T);
    const int k0 = z * slice;
    float s = 0.f;
    if (e < E) {
      const float* xr = x + (size_t)t * d + k0;
      const float* wr = w + (size_t)e * d + k0;
      for (int i = lane; i < slice; i += 64) s = fmaf(xr[i], wr[i], s);
      s = wave_sum_f(s);
    }
    if (lane == 0) part[((size_t)z * T + t) * E_pad + e] = s;
  }
}

// The smallest batches (bf16, T <= 4, d a multiple of 512 up to 4096): one expert per wave, its
// w_gate row held in registers (lane l takes the 16-byte pieces l, l + 64, ...), the tokens' x
// rows read the same way; per token a lane-order dot product and a DPP wave sum. One partial
// slice (KS = 1): the top-k reads one value per logit. Decode T = 1: routing 7.9 -> 6.5 us,
// step 35.0 -> 32.3 us; at T = 8 (two batches of four tokens) the split-K MFMA tiles were faster.
__global__ __launch_bounds__(256) void route_logits_gemv_kernel(const bf16_t* __restrict__ x,
                                                                const bf16_t* __restrict__ w,
                                                                int T, int d, int E, int E_pad,
                                                                float* __restrict__ part) {
  constexpr int MAXC = 8;   // 16-byte pieces per lane: d <= 4096
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E_pad) return;   // wave-uniform
  const int nc = d / 512;
  u32x4 wr[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c)
    wr[c] = (c < nc && e < E) ? *(const u32x4*)(w + (size_t)e * d + (size_t)(lane + 64 * c) * 8)
                              : u32x4{0u, 0u, 0u, 0u};
  auto lo = [](uint32_t v) { return __uint_as_float(v << 16); };
  auto hi = [](uint32_t v) { return __uint_as_float(v & 0xffff0000u); };
  for (int t0 = 0; t0 < T; t0 += 4) {
    u32x4 xr[4][MAXC];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int c = 0; c < MAXC; ++c)
        xr[u][c] = (t0 + u < T && c < nc)
                       ? *(const u32x4*)(x + (size_t)(t0 + u) * d + (size_t)(lane + 64 * c) * 8)
                       : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (t0 + u >= T) break;   // uniform
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < MAXC; ++c)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          s = fmaf(lo(xr[u][c][q]), lo(wr[c][q]), s);
          s = fmaf(hi(xr[u][c][q]), hi(wr[c][q]), s);
        }
      s = wave_sum_f(s);
      if (lane == 0) part[(size_t)(t0 + u) * E_pad + e] = s;
    }
  }
}

// TOK tokens per workgroup of 4 waves (TOK/4 per wave, one after the other)
template <int TOK>
__global__ __launch_bounds__(256) void route_topk_kernel(
    const float* __restrict__ part, int KS, int T, int E, int E_pad, int k,
    const float* __restrict__ logit_bias, const float* __restrict__ sel_bias,
    int32_t* __restrict__ ids, float* __restrict__ gates, float* __restrict__ psum_part) {
  __shared__ float prob[TOK][256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int tt = 0; tt < TOK / 4; ++tt) {
    const int tr = wave * (TOK / 4) + tt;
    const int t = blockIdx.x * TOK + tr;
    if (t >= T) {                     // uniform across the wave
#pragma unroll
      for (int i = 0; i < 4; ++i) prob[tr][lane + 64 * i] = 0.f;
      continue;
    }
    float lg[4], pr[4];
    bool live[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      live[i] = e < E;
      float v = -INFINITY;
      if (live[i]) v = sum_partials(part, KS, T, E_pad, t, e) + (logit_bias ? logit_bias[e] : 0.f);
      lg[i] = v;
    }
    int my_e;
    float my_g;
    token_topk(lg, live, sel_bias, k, lane, pr, my_e, my_g);
#pragma unroll
    for (int i = 0; i < 4; ++i) prob[tr][lane + 64 * i] = pr[i];
    if (lane < k) {
      ids[(size_t)t * k + lane] = my_e;
      gates[(size_t)t * k + lane] = my_g;
    }
  }
  if (psum_part) {
    __syncthreads();
    for (int e = tid; e < E; e += 256) {
      float s = 0.f;
      for (int tr = 0; tr < TOK; ++tr) s += prob[tr][e];
      psum_part[(size_t)blockIdx.x * E + e] = s;
    }
  }
}

// out[e] = sum over the nblk rows of a [nblk][E] table of per-workgroup partial sums (the top-k
// workgroups' probability sums, or the backward's logit-bias gradient). A fixed tree, so the
// result is identical from run to run: thread (c, e) adds the rows of chunk c of C = 1024/E
// in order, 64 loads in flight; then thread e adds the C chunk sums in order. With G workgroups,
// workgroup g does this over rows [nblk*g/G, nblk*(g+1)/G) and writes row g of out (G = 1: out
// is the sum); the launcher chains a G-workgroup pass and a one-workgroup pass over its G rows
// for many partials, still a fixed tree.
__global__ __launch_bounds__(1024) void psum_reduce_kernel(const float* __restrict__ part, int nblk,
                                                           int E, float* __restrict__ out) {
  __shared__ float csum[1024];
  const int tid = threadIdx.x;
  const int C = 1024 / E;   // E <= 256: at least 4 chunks
  const int c = tid / E, e = tid % E;
  const int G = gridDim.x, g = blockIdx.x;
  const int r0 = (int)((long long)nblk * g / G), nr = (int)((long long)nblk * (g + 1) / G) - r0;
  part += (size_t)r0 * E;
  out += (size_t)g * E;
  if (c < C) {
    const int b0 = (int)((long long)nr * c / C), b1 = (int)((long long)nr * (c + 1) / C);
    float s = 0.f;
    int b = b0;
    for (; b + 64 <= b1; b += 64) {   // 64 loads in flight, added in block order
      float v[64];
#pragma unroll
      for (int u = 0; u < 64; ++u) v[u] = part[(size_t)(b + u) * E + e];
#pragma unroll
      for (int u = 0; u < 64; ++u) s += v[u];
    }
    for (; b + 8 <= b1; b += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = part[(size_t)(b + u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; b < b1; ++b) s += part[(size_t)b * E + e];
    csum[tid] = s;   // = csum[c * E + e]
  }
  __syncthreads();
  if (tid < E) {
    float t = 0.f;
    for (int q = 0; q < C; ++q) t += csum[q * E + tid];
    out[tid] = t;
  }
}

// ------------------------------------------------------------------ fused router
// When w_gate is small (E <= 16 experts: 128 KB at d = 4096), one workgroup of 16 waves owns a
// block of 16 tokens against every expert over the whole of d, so the logits never leave the CU:
//   1. wave w takes the 16 tokens and the w-th sixteenth of d, all E_pad/16 expert fragments
//      (v_mfma_f32_16x16x32_bf16, fp32 accumulate), loads four 32-column steps ahead; the
//      sixteen partial blocks are added through LDS in wave order (deterministic);
//   2. softmax, top-k and renormalised gates from LDS with the DPP wave reductions of topk.h,
//      one token per wave; the workgroup's probability sums (tokens in wave order) go to its
//      row of psum_part.
// Each block reads w_gate once, from L2, and its 16 x rows once; the split-K path instead writes
// fp32 partial logits for a second launch to add up. With more experts, w_gate re-read per
// 16-token block costs more L2 traffic than the partial logits (measured slower at E = 64).
constexpr int FTB = 16;                 // tokens per fused-router workgroup (one per wave)
constexpr int FMAX_E = 16;              // one expert fragment

__global__ __launch_bounds__(1024) void route_fused_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ w, int T, int d, int E, int k,
    const float* __restrict__ logit_bias, const float* __restrict__ sel_bias,
    int32_t* __restrict__ ids, float* __restrict__ gates, float* __restrict__ psum_part) {
  constexpr int RS = 16 + 4;            // padded logits row
  __shared__ float part[16][FTB * RS];
  __shared__ float pw[16][FMAX_E];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tok0 = blockIdx.x * FTB;
  const int r = lane & 15, kq = (lane >> 4) * 8;
  const int klen = d / 16, kb0 = wave * klen;
  const int t_a = tok0 + r;
  const bool a_ok = t_a < T, b_ok = r < E;
  const bf16_t* ap = x + (size_t)(a_ok ? t_a : 0) * d + kb0 + kq;   // rows past T read row 0
  const bf16_t* bp = w + (size_t)(b_ok ? r : 0) * d + kb0 + kq;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  const bf16x8 z8 = {};
  constexpr int U = 4;
  const int nsteps = klen / 32;         // d % 512 == 0
  int st = 0;
  for (; st + U <= nsteps; st += U) {
    bf16x8 a[U], b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      a[u] = *(const bf16x8*)(ap + (st + u) * 32);
      b[u] = *(const bf16x8*)(bp + (st + u) * 32);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_ok ? a[u] : z8, b_ok ? b[u] : z8, acc, 0, 0,
                                                    0);
  }
  for (; st < nsteps; ++st) {
    const bf16x8 a = *(const bf16x8*)(ap + st * 32);
    const bf16x8 b = *(const bf16x8*)(bp + st * 32);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_ok ? a : z8, b_ok ? b : z8, acc, 0, 0, 0);
  }
  // C layout (16x16): lane holds column (expert) lane%16, rows (tokens) 4*(lane/16)+i
#pragma unroll
  for (int i = 0; i < 4; ++i) part[wave][(4 * (lane >> 4) + i) * RS + r] = acc[i];
  __syncthreads();

  // ---- softmax / top-k, one token per wave; logits = the sixteen parts added in wave order
  const int t = tok0 + wave;
  float pr0 = 0.f;
  if (t < T) {   // uniform
    float lg[4], pr[4];
    bool live[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      live[i] = e < E;
      float v = -INFINITY;
      if (live[i]) {
        v = 0.f;
        for (int wv = 0; wv < 16; ++wv) v += part[wv][wave * RS + e];
        v += logit_bias ? logit_bias[e] : 0.f;
      }
      lg[i] = v;
    }
    int my_e;
    float my_g;
    token_topk(lg, live, sel_bias, k, lane, pr, my_e, my_g);
    pr0 = pr[0];
    if (lane < k) {
      ids[(size_t)t * k + lane] = my_e;
      gates[(size_t)t * k + lane] = my_g;
    }
  }
  if (psum_part) {
    if (lane < FMAX_E) pw[wave][lane] = pr0;
    __syncthreads();
    if (tid < E) {
      float s = 0.f;
      for (int wv = 0; wv < 16; ++wv) s += pw[wv][tid];
      psum_part[(size_t)blockIdx.x * E + tid] = s;
    }
  }
}

}  // namespace

// the fused router: bf16, at most 64 experts, and a batch past the small-batch routing (which
// has its own one-workgroup top-k and grouping)
bool route_fused(const moe_problem& p) {
  return p.dtype == MOE_BF16 && p.E <= FMAX_E && p.d % 512 == 0 && !small_routing(p);
}

static bool route_gemv(const moe_problem& p) {
  return p.dtype == MOE_BF16 && p.T >= 1 && p.T <= 4 && small_routing(p) && p.d % 512 == 0 &&
         p.d <= 4096;
}

int route_ksplit(const moe_problem& p) {
  if (route_gemv(p)) return 1;
  const int E_pad = ceil_div(p.E, 16) * 16;
  const long long base = (long long)ceil_div(p.T, TM) * ceil_div(E_pad, EN);
  int ks = 1;
  // split d while the grid is small and each slice keeps >= 128 columns (a whole 32-column
  // k-step for each of the 4 waves that split a workgroup's slice); at most 16 slices, the
  // most sum_partials adds
  while (base * ks < 512 && ks < 16 && p.d % (ks * 2 * 128) == 0) ks *= 2;
  return ks;
}

size_t route_partial_bytes(const moe_problem& p) {
  const int E_pad = ceil_div(p.E, 16) * 16;
  return (size_t)route_ksplit(p) * p.T * E_pad * sizeof(float);
}

// One token per wave: each wave's logit loads then overlap other waves' top-k on the same CU (four
// tokens per wave, one after the other, left one wave per SIMD waiting on its loads).
int route_topk_tokens(const moe_problem&) { return TOPK_TOK; }
int route_topk_blocks(const moe_problem& p) { return ceil_div(p.T, route_topk_tokens(p)); }

hipError_t launch_route_topk(const moe_problem& p, const float* logits_part,
                             const float* logit_bias, const float* sel_bias, int32_t* ids,
                             float* gates, float* psum_part, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  const int E_pad = ceil_div(p.E, 16) * 16;
  const int KS = route_ksplit(p);
  const int nblk = route_topk_blocks(p);
  hipLaunchKernelGGL(route_topk_kernel<TOPK_TOK>, dim3(nblk), dim3(256), 0, s, logits_part, KS, p.T,
                     p.E, E_pad, p.k, logit_bias, sel_bias, ids, gates, psum_part);
  return hipGetLastError();
}

hipError_t launch_route_logits(const moe_problem& p, const void* x, const void* w_gate,
                               float* logits_part, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  const int E_pad = ceil_div(p.E, 16) * 16;
  const int KS = route_ksplit(p);
  if (route_gemv(p)) {
    hipLaunchKernelGGL(route_logits_gemv_kernel, dim3(ceil_div(E_pad, 4)), dim3(256), 0, s,
                       (const bf16_t*)x, (const bf16_t*)w_gate, p.T, p.d, p.E, E_pad, logits_part);
    return hipGetLastError();
  }
  dim3 grid(ceil_div(p.T, TM), ceil_div(E_pad, EN), KS);
  if (p.dtype == MOE_BF16)
    hipLaunchKernelGGL(route_logits_kernel, grid, dim3(256), 0, s, x, w_gate, p.T, p.d, p.E,
                       E_pad, KS, logits_part);
  else
    hipLaunchKernelGGL(route_logits_f32_kernel,
                       dim3((unsigned)std::min(((long long)KS * p.T * E_pad + 3) / 4, 1ll << 20)),
                       dim3(256), 0, s,
                       (const float*)x, (const float*)w_gate, p.T, p.d, p.E, E_pad, KS,
                       logits_part);
  return hipGetLastError();
}

// One workgroup reads its partials at one CU's rate (1 MB, the skewed shape's 4096 x 64, took
// 12.3 us with 32 or 64 loads in flight); with a stage buffer, many partials go through
// kPsumStage workgroups first (the two launches: 2 x 4.8 us).
hipError_t launch_psum_reduce(const float* psum_part, int nblk, int E, float* prob_sum,
                              hipStream_t s, float* stage) {
  if (stage && nblk >= 8 * kPsumStage) {
    hipLaunchKernelGGL(psum_reduce_kernel, dim3(kPsumStage), dim3(1024), 0, s, psum_part, nblk, E,
                       stage);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    psum_part = stage;
    nblk = kPsumStage;
  }
  hipLaunchKernelGGL(psum_reduce_kernel, dim3(1), dim3(1024), 0, s, psum_part, nblk, E, prob_sum);
  return hipGetLastError();
}

hipError_t launch_route(const moe_problem& p, const void* x, const void* w_gate,
                        const float* logit_bias, const float* sel_bias, int32_t* ids,
                        float* gates, float* prob_sum, float* logits_part, float* psum_part,
                        float* psum_stage, hipStream_t s) {
  if (route_fused(p)) {
    if (p.T == 0) return hipSuccess;
    const int nblk = ceil_div(p.T, FTB);
    hipLaunchKernelGGL(route_fused_kernel, dim3(nblk), dim3(1024), 0, s, (const bf16_t*)x,
                       (const bf16_t*)w_gate, p.T, p.d, p.E, p.k, logit_bias, sel_bias, ids, gates,
                       prob_sum ? psum_part : nullptr);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || !prob_sum) return err;
    return launch_psum_reduce(psum_part, nblk, p.E, prob_sum, s, psum_stage);
  }
  const int nblk = route_topk_blocks(p);
  hipError_t err = launch_route_logits(p, x, w_gate, logits_part, s);
  if (err != hipSuccess) return err;
  err = launch_route_topk(p, logits_part, logit_bias, sel_bias, ids, gates,
                          prob_sum ? psum_part : nullptr, s);
  if (err != hipSuccess) return err;
  if (!prob_sum) return hipSuccess;
  return launch_psum_reduce(psum_part, nblk, p.E, prob_sum, s, psum_stage);
}

}  // namespace moe
