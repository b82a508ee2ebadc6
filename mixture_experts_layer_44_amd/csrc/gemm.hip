// Grouped expert GEMMs over the per-expert segments.
//
// Pages: "Mixture of experts (MoE)" handbook, "Implementation: token by token vs. grouped
// by expert" (each expert does one matrix multiplication over all its tokens; one grouped
// GEMM covers all experts, and an empty group must be handled); "MoE Architecture" §3
// "Standard MoE" (SwiGLU experts: down(SiLU(gate x) * up x)).
//
// gate-up: for m-tile (group g, rows r0..r0+BM) and n-tile (features n0..n0+BN):
//   u = X_g W1_g^T, v = X_g W3_g^T over the tile, h = SiLU(u) * v -> bf16 H[m-tile rows].
//   X rows are gathered from x by token (sorted_assign / k; identity for the shared group).
// down:    out = H W2_g^T -> fp32 rows in sorted order (routed) or token order (shared).
//
// bf16 tiles: BM = 128 rows x BN = 128 features, BK = 64, 4 waves (2 x 2), each wave a
// 64 x 64 sub-tile of 32x32 MFMA blocks (v_mfma_f32_32x32x16_bf16, fp32 accumulate).
// The gate-up B tile holds the W1 and W3 rows of the same 128 features, so the SwiGLU
// epilogue has u and v of an output in the same lane. Operands are staged through LDS
// with a padded row stride (72 bf16) so the 16-byte fragment reads of 32 consecutive rows
// fall in distinct banks. The next K tile is loaded into registers while the current one
// feeds the MFMAs.
//
// Work order: tiles are numbered group-major, then n-tile, then m-tile, so neighbouring
// tiles share a weight tile (B) or a row block (A). Workgroups are dealt round-robin to
// the 8 XCDs, so workgroup b runs tile (b % 8) * per + b / 8: each XCD walks its own
// contiguous range and its L2 sees the reuse.
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int BM = kGemmBM, BN = 128, BK = 64, LDK = BK + 8;

struct GemmArgs {
  const bf16_t* A;      // gate-up: x [T,K]; down: H [mtiles*BM, K]
  const bf16_t* B0;     // gate-up: w1 [E,N,K]; down: w2 [E,N,K]
  const bf16_t* B1;     // gate-up: w3 [E,N,K]
  const bf16_t* S0;     // shared group: ws1 (gate-up) / ws2 (down) [N,K]
  const bf16_t* S1;     // shared group: ws3
  int N, K, E, k, T;
  const int32_t* sorted_assign;
  Schedule sc;
  bf16_t* H;            // gate-up output
  float* out_rows;      // down output, routed rows (sorted order)
  float* shared_out;    // down output, shared rows (token order)
};

struct TileCoord {
  int g, m_local, n0, mt_global, rows, off;
};

// Tile for this workgroup, or false if it has none. Must be uniform across the workgroup.
__device__ __forceinline__ bool tile_coord(const Schedule& sc, int NT, int bn, TileCoord& tc) {
  const int total = sc.mt_start[sc.G] * NT;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, slot = bid >> 3;
  const int per = (total + 7) >> 3;
  if (slot >= per) return false;
  const int L = xcd * per + slot;
  if (L >= total) return false;
  const int g = sc.mt_group[L / NT];
  const int ms = sc.mt_start[g];
  const int mtg = sc.mt_start[g + 1] - ms;
  const int lp = L - ms * NT;
  const int n_tile = lp / mtg;
  tc.g = g;
  tc.m_local = lp - n_tile * mtg;
  tc.n0 = n_tile * bn;
  tc.mt_global = ms + tc.m_local;
  tc.rows = sc.grp_rows[g];
  tc.off = sc.grp_off[g];
  return true;
}

__device__ __forceinline__ float silu_f(float u) { return u / (1.0f + __expf(-u)); }

template <bool GATEUP>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs args) {
  constexpr int BNB = GATEUP ? 2 * BN : BN;     // B rows per tile
  constexpr int A_LD = BM * BK / 8 / 256;      // 16-byte chunks per thread: 4
  constexpr int B_LD = BNB * BK / 8 / 256;     // 8 (gate-up) or 4 (down)
  __shared__ __attribute__((aligned(16))) bf16_t As[BM * LDK];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[BNB * LDK];

  TileCoord tc;
  if (!tile_coord(args.sc, args.N / BN, BN, tc)) return;
  const bool shared_grp = tc.g >= args.E;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = args.K, N = args.N;

  // ---- per-thread global source rows
  const int crow = tid >> 3, ccol = (tid & 7) * 8;
  const bf16_t* a_src[A_LD];
  bool a_ok[A_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int lr = crow + 32 * i;
    if (GATEUP) {
      const int r = tc.m_local * BM + lr;
      int tok = -1;
      if (r < tc.rows) tok = shared_grp ? r : args.sorted_assign[tc.off + r] / args.k;
      a_ok[i] = (unsigned)tok < (unsigned)args.T;   // rows past the segment (or bad entries) are zero
      a_src[i] = args.A + (size_t)(a_ok[i] ? tok : 0) * K + ccol;
    } else {
      a_ok[i] = true;
      a_src[i] = args.A + (size_t)(tc.mt_global * BM + lr) * K + ccol;
    }
  }
  const bf16_t* b_src[B_LD];
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int br = crow + 32 * i;
    const bf16_t* base;
    int row;
    if (GATEUP) {
      const bool up = br >= BN;
      base = shared_grp ? (up ? args.S1 : args.S0)
                        : (up ? args.B1 : args.B0) + (size_t)tc.g * N * K;
      row = tc.n0 + (up ? br - BN : br);
    } else {
      base = shared_grp ? args.S0 : args.B0 + (size_t)tc.g * N * K;
      row = tc.n0 + br;
    }
    b_src[i] = base + (size_t)row * K + ccol;
  }

  u32x4 ra[A_LD], rb[B_LD];
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) ra[i] = a_ok[i] ? *(const u32x4*)(a_src[i] + k0) : zero4;
#pragma unroll
    for (int i = 0; i < B_LD; ++i) rb[i] = *(const u32x4*)(b_src[i] + k0);
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) *(u32x4*)&As[(crow + 32 * i) * LDK + ccol] = ra[i];
#pragma unroll
    for (int i = 0; i < B_LD; ++i) *(u32x4*)&Bs[(crow + 32 * i) * LDK + ccol] = rb[i];
  };

  const int wm = wave >> 1, wn = wave & 1;
  constexpr int NACC = GATEUP ? 2 : 1;
  f32x16 acc[NACC][2][2];
#pragma unroll
  for (int q = 0; q < NACC; ++q)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[q][i][j][r] = 0.f;

  const int fr = lane & 31, fk = (lane >> 5) * 8;
  const int KT = K / BK;
  gload(0);
  for (int kt = 0; kt < KT; ++kt) {
    __syncthreads();
    lstore();
    __syncthreads();
    if (kt + 1 < KT) gload((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[2], bf[NACC][2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *(const bf16x8*)&As[(wm * 64 + i * 32 + fr) * LDK + ks * 16 + fk];
#pragma unroll
      for (int q = 0; q < NACC; ++q)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          bf[q][j] = *(const bf16x8*)&Bs[(q * BN + wn * 64 + j * 32 + fr) * LDK + ks * 16 + fk];
#pragma unroll
      for (int q = 0; q < NACC; ++q)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[q][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[q][j], acc[q][i][j], 0, 0, 0);
    }
  }

  // ---- epilogue. 32x32 accumulator layout: lane holds column lane%32 and rows
  // 8*(r/4) + 4*(lane/32) + r%4 for r = 0..15.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = tc.n0 + wn * 64 + j * 32 + fr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int lr = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (GATEUP) {
          const float u = acc[0][i][j][r];
          const float v = acc[NACC - 1][i][j][r];
          args.H[(size_t)(tc.mt_global * BM + lr) * N + col] = f32_to_bf16(silu_f(u) * v);
        } else {
          const int rg = tc.m_local * BM + lr;
          if (rg < tc.rows) {
            float* dst = shared_grp ? args.shared_out + (size_t)rg * N
                                    : args.out_rows + (size_t)(tc.off + rg) * N;
            dst[col] = acc[0][i][j][r];
          }
        }
      }
    }
}

// ------------------------------------------------------------------ fp32 path (VALU)
constexpr int BM32 = kGemmBM32, BN32 = 64, BK32 = 16;

struct GemmArgs32 {
  const float* A;
  const float* B0;
  const float* B1;
  const float* S0;
  const float* S1;
  int N, K, E, k, T;
  const int32_t* sorted_assign;
  Schedule sc;
  float* H;
  float* out_rows;
  float* shared_out;
};

template <bool GATEUP>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs32 args) {
  constexpr int NB = GATEUP ? 2 : 1;
  __shared__ float As[BK32][BM32];
  __shared__ float Bs[NB][BK32][BN32];
  __shared__ int tok[BM32];
  TileCoord tc;
  if (!tile_coord(args.sc, (args.N + BN32 - 1) / BN32, BN32, tc)) return;
  const bool shared_grp = tc.g >= args.E;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int K = args.K, N = args.N;
  if (tid < BM32) {
    const int r = tc.m_local * BM32 + tid;
    int t = -1;
    if (GATEUP) {
      if (r < tc.rows) t = shared_grp ? r : args.sorted_assign[tc.off + r] / args.k;
      if (t >= args.T) t = -1;
    } else {
      t = tc.mt_global * BM32 + tid;
    }
    tok[tid] = t;
  }
  const float* Bb[NB];
  Bb[0] = shared_grp ? args.S0 : args.B0 + (size_t)tc.g * N * K;
  if (GATEUP) Bb[NB - 1] = shared_grp ? args.S1 : args.B1 + (size_t)tc.g * N * K;
  float acc[NB][4][4] = {};
  __syncthreads();
  for (int k0 = 0; k0 < K; k0 += BK32) {
    for (int idx = tid; idx < BM32 * BK32; idx += 256) {
      const int r = idx / BK32, kk = idx % BK32;
      const int t = tok[r];
      As[kk][r] = (t >= 0 && k0 + kk < K) ? args.A[(size_t)t * K + k0 + kk] : 0.f;
    }
    for (int q = 0; q < NB; ++q)
      for (int idx = tid; idx < BN32 * BK32; idx += 256) {
        const int c = idx / BK32, kk = idx % BK32;
        const int n = tc.n0 + c;
        Bs[q][kk][c] = (n < N && k0 + kk < K) ? Bb[q][(size_t)n * K + k0 + kk] : 0.f;
      }
    __syncthreads();
    for (int kk = 0; kk < BK32; ++kk) {
      float a[4], b[NB][4];
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
      for (int q = 0; q < NB; ++q)
        for (int j = 0; j < 4; ++j) b[q][j] = Bs[q][kk][tx * 4 + j];
      for (int q = 0; q < NB; ++q)
        for (int i = 0; i < 4; ++i)
          for (int j = 0; j < 4; ++j) acc[q][i][j] = fmaf(a[i], b[q][j], acc[q][i][j]);
    }
    __syncthreads();
  }
  for (int i = 0; i < 4; ++i) {
    const int lr = ty * 4 + i;
    for (int j = 0; j < 4; ++j) {
      const int col = tc.n0 + tx * 4 + j;
      if (col >= N) continue;
      if (GATEUP) {
        const float u = acc[0][i][j], v = acc[NB - 1][i][j];
        args.H[(size_t)(tc.mt_global * BM32 + lr) * N + col] = u / (1.0f + expf(-u)) * v;
      } else {
        const int rg = tc.m_local * BM32 + lr;
        if (rg < tc.rows) {
          float* dst = shared_grp ? args.shared_out + (size_t)rg * N
                                  : args.out_rows + (size_t)(tc.off + rg) * N;
          dst[col] = acc[0][i][j];
        }
      }
    }
  }
}

inline int grid_for(int mtiles, int nt) {
  long long g = (long long)mtiles * nt;
  return (int)((g + 7) / 8 * 8);
}

}  // namespace

hipError_t launch_expert_ffn(const moe_problem& p, const void* x, const void* w1, const void* w3,
                             const void* w2, const void* ws1, const void* ws3, const void* ws2,
                             const int32_t* sorted_assign, const Schedule& sc, void* h,
                             float* out_rows, float* shared_out, hipStream_t s,
                             hipEvent_t between) {
  if (p.dtype == MOE_BF16) {
    GemmArgs a{};
    a.A = (const bf16_t*)x;
    a.B0 = (const bf16_t*)w1;
    a.B1 = (const bf16_t*)w3;
    a.S0 = (const bf16_t*)ws1;
    a.S1 = (const bf16_t*)ws3;
    a.N = p.d_ff;
    a.K = p.d;
    a.E = p.E;
    a.k = p.k;
    a.T = p.T;
    a.sorted_assign = sorted_assign;
    a.sc = sc;
    a.H = (bf16_t*)h;
    hipLaunchKernelGGL(gemm_bf16_kernel<true>, dim3(grid_for(sc.max_mtiles, p.d_ff / BN)),
                       dim3(256), 0, s, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (between && (err = hipEventRecord(between, s)) != hipSuccess) return err;
    GemmArgs b{};
    b.A = (const bf16_t*)h;
    b.B0 = (const bf16_t*)w2;
    b.S0 = (const bf16_t*)ws2;
    b.N = p.d;
    b.K = p.d_ff;
    b.E = p.E;
    b.k = p.k;
    b.T = p.T;
    b.sorted_assign = sorted_assign;
    b.sc = sc;
    b.out_rows = out_rows;
    b.shared_out = shared_out;
    hipLaunchKernelGGL(gemm_bf16_kernel<false>, dim3(grid_for(sc.max_mtiles, p.d / BN)), dim3(256),
                       0, s, b);
    return hipGetLastError();
  }
  GemmArgs32 a{};
  a.A = (const float*)x;
  a.B0 = (const float*)w1;
  a.B1 = (const float*)w3;
  a.S0 = (const float*)ws1;
  a.S1 = (const float*)ws3;
  a.N = p.d_ff;
  a.K = p.d;
  a.E = p.E;
  a.k = p.k;
  a.T = p.T;
  a.sorted_assign = sorted_assign;
  a.sc = sc;
  a.H = (float*)h;
  hipLaunchKernelGGL(gemm_f32_kernel<true>, dim3(grid_for(sc.max_mtiles, ceil_div(p.d_ff, BN32))),
                     dim3(256), 0, s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (between && (err = hipEventRecord(between, s)) != hipSuccess) return err;
  GemmArgs32 b{};
  b.A = (const float*)h;
  b.B0 = (const float*)w2;
  b.S0 = (const float*)ws2;
  b.N = p.d;
  b.K = p.d_ff;
  b.E = p.E;
  b.k = p.k;
  b.T = p.T;
  b.sorted_assign = sorted_assign;
  b.sc = sc;
  b.out_rows = out_rows;
  b.shared_out = shared_out;
  hipLaunchKernelGGL(gemm_f32_kernel<false>, dim3(grid_for(sc.max_mtiles, ceil_div(p.d, BN32))),
                     dim3(256), 0, s, b);
  return hipGetLastError();
}

}  // namespace moe
