// Decode-sized layers: the down projection and the gate-weighted combine in one launch.
//
// Pages: "MoE Architecture" §1 (y is the sum over the chosen experts of the gate times the
// expert's output) and §3 "Standard MoE" (the expert FFN's down projection); "Mixture of
// experts (MoE)" handbook, "Implementation" (results return to their tokens with their
// weights) and "Inference view" (at decode sizes a step streams the touched experts' weights,
// and fused kernels cut the launch count).
//
// With a handful of tokens, a token's k expert rows are each one row of a different expert,
// so the down GEMM's per-assignment rows exist only to be read back by the combine. Here a
// workgroup owns 16 output features of one token and computes them for all of the token's
// kept slots, then folds the slots into y in slot order. No row goes to HBM and one launch
// (with its start-up latency and its dependent loads) disappears from the step: a decode
// step of one or two tokens is four launches (router logits; top-k with grouping and schedule;
// gate-up; this).
// (Measured and not kept: gate-up tiles found from the top-k ids directly, h by assignment, so
// that neither GEMM looks up the schedule. Decode T = 1 kernel times were the same, and at
// T = 8 the assignments that share an expert each streamed its weights: gate-up 60 -> 62 us.)
//
// The arithmetic is the decode GEMM's and the combine's, operation for operation, so y is
// bit-identical to the two-launch path (down rows, then combine):
//  * each slot's 16 features come from v_mfma_f32_16x16x32_bf16 over four quarters of K, one
//    per wave, with the same k-step order inside a quarter (h row as the A operand, replicated
//    over the 16 A rows; W2 rows as the B columns);
//  * the four quarter sums are added in quarter order, then y = fma(g_j, row_j, y) over the
//    kept slots j in slot order, from 0 (no shared expert on this path).
// Eight waves: waves 4s .. 4s+3 take the slots j with j % 2 == s, so every SIMD streams weights
// of two waves. Each wave's loads run up to eight k-steps ahead, straight into registers.
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kDcFeat = 16;                 // output features per workgroup
constexpr int kDcSG = 2;                    // slot groups (4 waves each)
constexpr int kDcMaxK = 8;                  // slots per token
constexpr int kDcNSW = kDcMaxK / kDcSG;     // slots per wave
constexpr int kDcDepth = 8;                 // k-steps in flight per wave

struct DcArgs {
  const bf16_t* H;             // padded h rows [m-tiles * BM, K] (the gate-up GEMM's output)
  const bf16_t* W2;            // [E, N, K]
  const int32_t* ids;          // [T, k]
  const float* gates;          // [T, k]
  const int32_t* assign_pos;   // [T, k]: row in expert-sorted order, or -1 (dropped)
  const int32_t* grp_off;      // [E]: first sorted row of each expert
  const int32_t* mt_start;     // [E + 1]: first m-tile of each expert
  float* y;                    // [T, N]
  int N, K, k, E, BM;
};

// KTW: 64-wide k-steps per wave (K = 256 * KTW)
template <int KTW>
__global__ __launch_bounds__(256 * kDcSG) void down_combine_dec_kernel(DcArgs a) {
  constexpr int S = kDcNSW * KTW;                       // k-steps per wave over its slots
  constexpr int D = kDcDepth < S ? kDcDepth : S;
  __shared__ float red[4 * kDcSG][kDcNSW][kDcFeat];

  const int t = blockIdx.y, n0 = blockIdx.x * kDcFeat;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = wave & 3, sg = wave >> 2;
  const int r16 = lane & 15, kq = lane >> 4;
  const int K = a.K;
  const int kbase = q * (KTW * 64) + kq * 8;

  // lane j < k: slot j's expert, gate and padded h row (-1: dropped, or an id out of range).
  // Sorted row r of expert e sits at h row mt_start[e] * BM + (r - grp_off[e]).
  int e = 0, srow = -1;
  float g = 0.f;
  if (lane < a.k) {
    const int o = t * a.k + lane;
    e = a.ids[o];
    const int r = a.assign_pos[o];
    g = a.gates[o];
    if (r >= 0 && (unsigned)e < (unsigned)a.E) srow = a.mt_start[e] * a.BM + (r - a.grp_off[e]);
    else e = 0;
  }

  // this wave's slots j = sg + kDcSG * jl; a slot with nothing to add reads expert 0 and h row 0
  // (valid memory) and its sums are never used
  const bf16_t* bp[kDcNSW];
  const bf16_t* ap[kDcNSW];
#pragma unroll
  for (int jl = 0; jl < kDcNSW; ++jl) {
    const int j = sg + kDcSG * jl;
    const int ej = __builtin_amdgcn_readlane(e, j);
    const int rj = __builtin_amdgcn_readlane(srow, j);
    const bool live = j < a.k && rj >= 0;
    bp[jl] = a.W2 + ((size_t)(live ? ej : 0) * a.N + n0 + r16) * K + kbase;
    ap[jl] = a.H + (size_t)(live ? rj : 0) * K + kbase;
  }

  f32x4 acc[kDcNSW];
#pragma unroll
  for (int jl = 0; jl < kDcNSW; ++jl) acc[jl] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 bq[D][2], aq[D][2];
  auto load = [&](int d, int i) {
    const int jl = i / KTW, kt = i % KTW;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bq[d][s] = *(const bf16x8*)(bp[jl] + kt * 64 + s * 32);
      aq[d][s] = *(const bf16x8*)(ap[jl] + kt * 64 + s * 32);
    }
  };
#pragma unroll
  for (int d = 0; d < D; ++d) load(d, d);
#pragma unroll
  for (int i = 0; i < S; ++i) {
    const int d = i % D, jl = i / KTW;
#pragma unroll
    for (int s = 0; s < 2; ++s)
      acc[jl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[d][s], bq[d][s], acc[jl], 0, 0, 0);
    if (i + D < S) load(d, i + D);
    __builtin_amdgcn_sched_barrier(0);
  }
  // every A row is the slot's h row, so row 0 (lanes 0..15, element 0) holds the result
  if (kq == 0) {
#pragma unroll
    for (int jl = 0; jl < kDcNSW; ++jl) red[wave][jl][r16] = acc[jl][0];
  }
  __syncthreads();
  if (tid < kDcFeat) {
    float out = 0.f;
    for (int j = 0; j < a.k; ++j) {
      const int rj = __builtin_amdgcn_readlane(srow, j);
      if (rj < 0) continue;
      const float gj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g), j));
      const int w0 = 4 * (j % kDcSG), jl = j / kDcSG;
      float row = red[w0][jl][tid];
#pragma unroll
      for (int w = 1; w < 4; ++w) row += red[w0 + w][jl][tid];
      out = fmaf(gj, row, out);
    }
    a.y[(size_t)t * a.N + n0 + tid] = out;
  }
}

template <int KTW = 1>
void launch_dc_k(int steps, dim3 grid, hipStream_t s, const DcArgs& a) {
  if constexpr (KTW <= 8) {
    if (steps == KTW)
      hipLaunchKernelGGL((down_combine_dec_kernel<KTW>), grid, dim3(256 * kDcSG), 0, s, a);
    else
      launch_dc_k<KTW + 1>(steps, grid, s, a);
  }
}

}  // namespace

// Decode class (the decode GEMM kernel's shapes), no shared expert, k <= 8 and at most 16
// assignments: with so few tokens the expert rows are each read back once by one token's
// combine, and the grouping has next to nothing to share between tokens. (At T = 8, k = 8 the
// decode down GEMM, since its weights-first prologue, and the combine apart are faster: step
// 108.7 -> 107.3 us; at T = 1 this launch still wins, 31.8 against 33.5 us.)
bool dec_down_combine(const moe_problem& p) {
  return gemm_dec(p) && p.n_shared == 0 && p.k <= kDcMaxK && (long long)p.T * p.k <= 16 &&
         p.d % kDcFeat == 0 && down_ksplit(p) == 1;
}

hipError_t launch_dec_down_combine(const moe_problem& p, const void* h, const void* w2,
                                   const int32_t* ids, const float* gates,
                                   const int32_t* assign_pos, const Schedule& sc, float* y,
                                   hipStream_t s) {
  if (!dec_down_combine(p) || sc.BM != kDecBM) return hipErrorInvalidValue;
  if (p.T == 0) return hipSuccess;
  DcArgs a{};
  a.H = (const bf16_t*)h;
  a.W2 = (const bf16_t*)w2;
  a.ids = ids;
  a.gates = gates;
  a.assign_pos = assign_pos;
  a.grp_off = sc.grp_off;
  a.mt_start = sc.mt_start;
  a.y = y;
  a.N = p.d;
  a.K = p.d_ff;
  a.k = p.k;
  a.E = p.E;
  a.BM = sc.BM;
  launch_dc_k(p.d_ff / 256, dim3(p.d / kDcFeat, p.T), s, a);
  return hipGetLastError();
}

}  // namespace moe
