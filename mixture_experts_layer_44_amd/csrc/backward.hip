// Layer backward: the gradient of <dy, y> + dL * L_balance with respect to x, the router
// weight (and logit offset) and every expert weight, for bf16 storage.
//
// Pages: "MoE (Mixture of Experts) Deep Dive", "Load Balancing Loss Derivation" (F is a
// post-hoc count with no gradient, P carries it); "MoE Architecture" §2 "Gating Function"
// (softmax, top-k, renormalised gates) and "Load Balancing" (L = alpha * E * sum f_i p_i);
// §3 "Standard MoE" (SwiGLU experts); "Mixture of experts (MoE)" handbook, "Implementation:
// token by token vs. grouped by expert" (grouped expert GEMMs). The selection is held fixed:
// top-k and capacity drops have no gradient.
//
// Per kept row r of expert e (token t, gate g): d o = g dy_t, d g = <dy_t, o>,
//   dh = W2^T d o, du = dh * v * SiLU'(u), dv = dh * SiLU(u), d x_t += W1^T du + W3^T dv,
//   dW2 += d o h^T, dW1 += du x^T, dW3 += dv x^T.
// Router: d l = (softmax over the selected logits)' d g + the balance term through p;
//   dx += d l W_gate, dW_gate = d l^T x, d logit_bias = column sums of d l.
//
// Storage. Every per-row activation lives in "storage rows": group g's rows r = 0..rows_g-1
// at row mt_start[g] * SB + r of a [m-tiles * SB, width] buffer, where SB and mt_start are the
// forward's own m-tile schedule (the shared expert is group E). The recompute of the gate-up
// GEMM (the forward's kernel, tile for tile) writes
// h (bf16) and u, v (fp32) there; a prep kernel writes g * dy (bf16) and the gathered x rows
// (bf16) there, and dy once in bf16 in token order.
//
// GEMMs (bf16 MFMA 32x32x16, fp32 accumulation, BK 64, direct global->LDS loads):
//   dgrad-down  [rows x d_ff] = dy_tok [rows x d] . W2_e [d x d_ff]   + SwiGLU backward epilogue
//   dgrad-x     [rows x d]    = (du|dv) [rows x 2 d_ff] . (W1_e;W3_e) [2 d_ff x d]
//   router      dx_r [T x d]  = d l [T x E] . W_gate [E x d]
//     -- row-tiled (bwd_gemm_kernel): 256 x BN tiles, 8 waves of 64 x 128, staggered rings
//        (the register-staged ring on the wide class), ragged last tiles
//   wgrad-down  dW2_e [d x d_ff]     = (g dy)^T [d x rows] . h [rows x d_ff]
//   wgrad-up    (dW1_e;dW3_e) [2 d_ff x d] = (du|dv)^T . x_gathered [rows x d]
//     -- persistent (bwd_wgrad_kernel): 128 x 128 tiles streamed through a 2-slot ring
//   router      dW_gate = d l^T x  (K = T) -- bwd_gemm_kernel's weights mode
// Every weight and activation stays in its forward layout in HBM. An operand whose contraction
// index is its row index ("transposed": the weights in dgrad, everything in wgrad) is staged
// into LDS as [k][m] rows, as it lies in memory, and read with ds_read_b64_tr_b16: within each
// 16-lane group, lane i points at row k0 + i/4, columns m0 + 4 (i%4) .. +3, and lane j receives
// column m0 + j at rows k0 .. k0+3 -- half of an MFMA operand; two such reads make the 8 k
// values a 32x32x16 fragment takes. Such [k][m] rows are XOR-swizzled in 16-byte chunks by
// 4 * (k % 4), so the 4 rows x 2 chunks of a 16-lane group (and the 4 x 4 of 32 lanes) hit
// distinct bank groups. Contraction rows past a segment's end read a zero row.
#include <type_traits>

#include "moe_internal.h"
#include "mfma_tiles.h"
#include "topk.h"

namespace moe {

namespace {

typedef short v4s __attribute__((ext_vector_type(4)));

constexpr int BBM = 128;   // rows of a weight-gradient m-tile (rows of the weight matrix)
// The router's weight gradient (K = T) runs as a launched 128 x 128 tile with a 2-stage ring
// (64 KB of LDS, two workgroups per CU). The experts' weight gradients use the persistent
// kernel (bwd_wgrad_kernel).
constexpr int kWgradStages = 2;
constexpr int kWgradBN = 128;
constexpr int kRowsBM = 256;      // m-tile of the row-tiled GEMMs
constexpr int ZERO_ELEMS = 256;

enum AKind : int { A_TOKEN, A_STORE, A_IDENT, AT_STORE, AT_IDENT };
enum BKind : int { B_W2, B_W13, B_WGATE, BT_STORE, BT_IDENT };
enum EpiKind : int { EPI_DDOWN, EPI_ROWS, EPI_WF32 };
enum ModeKind : int { M_ROWS, M_WEIGHTS };

struct BwdArgs {
  const bf16_t* A;          // A_TOKEN: dy (bf16, token rows); A_STORE / AT_STORE: storage rows;
  int lda;                  // A_IDENT / AT_IDENT: d l rows [T, lda]
  const bf16_t* B0;         // routed weights (B_W2: w2; B_W13: w1; B_WGATE: w_gate) or row source
  const bf16_t* B1;         // B_W13: w3
  const bf16_t* S0;         // shared expert's weights (B_W2: ws2; B_W13: ws1)
  const bf16_t* S1;         // B_W13: ws3
  int ldb;
  const bf16_t* zero;       // ZERO_ELEMS zero bf16: contraction rows past a segment's end
  int M, N, K;              // K: rows mode only (weights mode: each group's rows)
  int E, k, T;
  int ident;                // 1: one group of ident_rows rows in identity order (router)
  int ident_rows;
  int ident_split;          // weights mode with ident: that group cut into this many groups of
  int ident_chunk;          // ident_chunk consecutive rows (the last one shorter), each writing
                            // its own [Mvalid, N] slice of Wf
  int Kvalid;               // B_WGATE: rows of B that exist (E)
  const int32_t* sorted_assign;
  Schedule sc;              // rows mode: the row-tile schedule; weights mode: the storage one
  const int32_t* stor_start;   // the storage schedule's m-tile starts
  int stor_bm;                 // its m-tile height: group g's row r is storage row
                               // stor_start[g] * stor_bm + r
  float* out;               // EPI_ROWS: routed rows (sorted order) or identity rows
  float* out_shared;        // EPI_ROWS: the shared expert's rows (token order)
  bf16_t* W0;               // bf16 weight gradient (persistent kernel): routed, rows < Msplit
  bf16_t* W1;               //            routed dW, output rows >= Msplit
  bf16_t* SW0;              //            shared expert, rows < Msplit
  bf16_t* SW1;              //            shared expert, rows >= Msplit
  int Msplit;
  float* Wf;                // EPI_WF32: [Mvalid, N]
  int Mvalid;
  const float* U;           // EPI_DDOWN: u, v (fp32 storage rows, width N, fragment order)
  const float* V;
  const float* topk_w;
  bf16_t* DUV;              //            du | dv (bf16 storage rows, width 2N)
  float* dgate_part;        //            [rows, NT] per-n-tile partial sums of d g (routed)
  int NT;
};

// Physical offset of logical element (row, col) of a swizzled [k][W] tile (transposed stage).
template <int W>
__device__ __forceinline__ int tr_off(int row, int col) {
  return row * W + ((((col >> 3) ^ ((row & 3) << 2))) << 3) + (col & 7);
}

// MFMA operands from a transposed [k][W] stage: for each of NF operand blocks (first column
// base-derived, see tr_base), lane l gets rows ks*16 + 8*(l/32) .. +7 of column mb + l%32, as
// two 4-row ds_read_b64_tr_b16 reads. All of a sub-step's reads are one asm block that ends with
// its own lgkmcnt wait, so its outputs are complete when it ends; they are early-clobber, since
// a read may return while a later read of the block has not yet taken its address.
// (With the compiler's ds_read_tr16_b64 builtin, the compiler put a full vmcnt(0) wait before
// the first read of every K step: it cannot tell the read from the stages that the in-flight
// global->LDS loads fill, so every step drained the ring. The ring's own waits and barriers
// already order the stage writes before these reads.)
__device__ __forceinline__ uint32_t lds_byte_addr(const bf16_t* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const bf16_t*)p;
}
template <int W, int NF>
__device__ __forceinline__ void tr_frags(const bf16_t* st, const int (&base)[NF], int ks,
                                         bf16x8 (&out)[NF]) {
  static_assert(NF == 1 || NF == 2 || NF == 4, "1, 2 or 4 operand blocks");
  constexpr int O0 = 0, O1 = 4 * W * 2;       // byte offsets of the two 4-row reads
  const int kofs = ks * 16 * W;
  v4s r[2 * NF];
  uint32_t ad[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) ad[f] = lds_byte_addr(st + base[f] + kofs);
  if constexpr (NF == 1) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %2 offset:%3\n\t"
        "ds_read_b64_tr_b16 %1, %2 offset:%4\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1])
        : "v"(ad[0]), "i"(O0), "i"(O1));
  } else if constexpr (NF == 2) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4 offset:%6\n\t"
        "ds_read_b64_tr_b16 %1, %4 offset:%7\n\t"
        "ds_read_b64_tr_b16 %2, %5 offset:%6\n\t"
        "ds_read_b64_tr_b16 %3, %5 offset:%7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(ad[0]), "v"(ad[1]), "i"(O0), "i"(O1));
  } else {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:%12\n\t"
        "ds_read_b64_tr_b16 %1, %8 offset:%13\n\t"
        "ds_read_b64_tr_b16 %2, %9 offset:%12\n\t"
        "ds_read_b64_tr_b16 %3, %9 offset:%13\n\t"
        "ds_read_b64_tr_b16 %4, %10 offset:%12\n\t"
        "ds_read_b64_tr_b16 %5, %10 offset:%13\n\t"
        "ds_read_b64_tr_b16 %6, %11 offset:%12\n\t"
        "ds_read_b64_tr_b16 %7, %11 offset:%13\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
          "=&v"(r[7])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "i"(O0), "i"(O1));
  }
#pragma unroll
  for (int f = 0; f < NF; ++f)
    out[f] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r[2 * f], r[2 * f + 1], 0, 1, 2,
                                                                3, 4, 5, 6, 7));
}

// The same reads through the compiler builtin, for kernels with no global->LDS loads in flight
// (register-staged rings): the compiler then places the LDS waits itself, and the reads of one
// sub-step can overlap the MFMAs of the previous one.
template <int W, int NF>
__device__ __forceinline__ void tr_frags_bi(const bf16_t* st, const int (&base)[NF], int ks,
                                            bf16x8 (&out)[NF]) {
  typedef __attribute__((address_space(3))) v4s lds_v4s;
  const int kofs = ks * 16 * W;
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const __attribute__((address_space(3))) bf16_t* p =
        (const __attribute__((address_space(3))) bf16_t*)(st + base[f] + kofs);
    const v4s r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p);
    const v4s r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p + 4 * W));
    out[f] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
  }
}

// This lane's element offset, in a transposed [k][W] stage, of the first of the 4 rows it
// points at for the operand block whose first column is mb (sub-step 0, first read):
// lane i of each 16-lane group points at row 8*(group/2) + i/4, column mb + 16*(group%2) + 4*(i%4).
template <int W>
__device__ __forceinline__ int tr_base(int lane, int mb) {
  const int g16 = lane >> 4, i = lane & 15;
  const int row = 8 * (g16 >> 1) + (i >> 2);
  const int col = mb + 16 * (g16 & 1) + 4 * (i & 3);
  return tr_off<W>(row, col);
}

// The GEMM. BM x BN tiles, WM x WN waves, each a (BM/WM) x (BN/WN) block of 32x32 fragments.
// Row fragments are dealt to the waves interleaved: fragment i of wave row wm covers tile rows
// (i*WM + wm)*32 .. +32, so a ragged tile's rows with data spread over all SIMDs.
// ST >= 2: a ring of ST stages of both operands, ST-1 steps in flight (weights mode).
// ST == 0: staggered rings (rows mode): A, the rows, in 2 slots one step ahead; B, the
// weights, in 3 slots two steps ahead; A issued first in each step so that the step's wait
// leaves only B's latest loads in flight. The A row groups past a tile's last row with data
// are then not loaded at all, and a wave skips the fragments that are all padding.
// RS (rows mode, ST == 2): both operands go through registers instead, each lane storing its
// 16-byte pieces of step k+1 at the places the direct loads fill while step k computes; the
// weight fragments are then read with the transpose builtin (with direct loads in flight the
// compiler drains them before every builtin read). Same padding skip as staggered.
template <int BM, int BN, int WM, int WN, int MODE, int AK, int BKIND, int EPI, int ST,
          bool RS = false>
__global__ __launch_bounds__(WM * WN * 64) void bwd_gemm_kernel(BwdArgs a) {
  constexpr int BK = 64, NW = WM * WN, NKS = BK / 16;
  constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 32, FN = TN / 32;
  constexpr bool ATR = AK == AT_STORE || AK == AT_IDENT;
  constexpr bool STAG = ST == 0;
  constexpr int ASZ = BM * BK, BSZ = BN * BK;
  // ring slots of A and B (staggered: the deep operand has 3, the shallow one 2)
  constexpr int NA = STAG ? 2 : ST, NB = STAG ? 3 : ST;   // RS: ST = 2
  constexpr int DMA_A = ASZ * 2 / 1024 / NW, DMA_B = BSZ * 2 / 1024 / NW;
  static_assert(DMA_A * 1024 * NW == ASZ * 2 && DMA_B * 1024 * NW == BSZ * 2, "even split");
  static_assert(FM >= 1 && FN >= 1 && FM <= 3, "wave tile covers whole fragments");
  static_assert(!STAG || (MODE == M_ROWS && !ATR), "staggered rings: rows mode only");
  static_assert(!RS || (ST == 2 && MODE == M_ROWS && !ATR), "register staging: rows mode, 2 slots");
  constexpr bool SKIPA = STAG || RS;   // A row groups past the data are skipped
  static_assert((NA * ASZ + NB * BSZ) * 2 <= 160 * 1024, "rings fit in LDS");
  static_assert(EPI != EPI_DDOWN || (NA * ASZ + NB * BSZ) * 2 >= (WN + 1) * BM * 4,
                "the ring holds the epilogue's row sums");
  __shared__ __attribute__((aligned(1024))) bf16_t smem[NA * ASZ + NB * BSZ];
  bf16_t* const As = smem;
  bf16_t* const Bs = smem + NA * ASZ;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

  // ---- tile
  int g = 0, rows = 0, off = 0, m_local = 0, mt_global = 0, n0 = 0, m0 = 0, sbase = 0;
  if (MODE == M_ROWS) {
    if (a.ident) {
      const int MT = (a.ident_rows + BM - 1) / BM, NTt = a.N / BN, total = MT * NTt;
      const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, per = (total + 7) >> 3;
      if (slot >= per) return;
      const int L = xcd * per + slot;
      if (L >= total) return;
      const int nt = L / MT;
      m_local = L - nt * MT;
      mt_global = m_local;
      n0 = nt * BN;
      rows = a.ident_rows;
    } else {
      TileCoord tc;
      if (!tile_coord(a.sc, a.N / BN, BN, tc)) return;
      g = tc.g;
      m_local = tc.m_local;
      mt_global = tc.mt_global;
      n0 = tc.n0;
      rows = tc.rows;
      off = tc.off;
    }
    // rows of this group are stored from storage row sbase (the storage schedule)
    sbase = a.ident ? 0 : a.stor_start[g] * a.stor_bm;
  } else {
    const int G = a.ident ? a.ident_split : a.sc.G;
    const int MT = a.M / BM, NTt = a.N / BN, total = G * MT * NTt;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, per = (total + 7) >> 3;
    if (slot >= per) return;
    const int L = xcd * per + slot;
    if (L >= total) return;
    g = L / (MT * NTt);
    const int rem = L - g * MT * NTt;
    const int mt = rem / NTt;
    m0 = mt * BM;
    n0 = (rem - mt * NTt) * BN;
    if (a.ident) {
      sbase = g * a.ident_chunk;
      rows = max(0, min(a.ident_chunk, a.ident_rows - sbase));
    } else {
      rows = a.sc.grp_rows[g];
      sbase = a.stor_start[g] * a.stor_bm;
    }
  }
  const bool shared_grp = !a.ident && g >= a.E;
  const int KT = MODE == M_ROWS ? a.K / BK : (rows + BK - 1) / BK;
  // rows of this tile that hold data (rows mode)
  const int rows_here =
      MODE == M_ROWS ? __builtin_amdgcn_readfirstlane(min(BM, rows - m_local * BM)) : BM;

  // ---- A loads
  // non-transposed [BM][BK] stage (rows mode): load i of this wave fills rows q*8 .. q*8+7
  // (q = wave*DMA_A + i); lane l fetches the logical chunk that the swizzle puts at physical
  // chunk l%8 of row q*8 + l/8. Row sources are fixed for the whole tile.
  // transposed [BK][BM] stage (weights mode): load i fills k-rows q*4 .. q*4+3; lane l writes
  // physical chunk l%16 of k-row q*4 + l/16.
  uint32_t aoff[DMA_A];
  int akrow[DMA_A], alch[DMA_A];
#pragma unroll
  for (int i = 0; i < DMA_A; ++i) {
    const int q = wave * DMA_A + i;
    if (!ATR) {
      const int row = q * 8 + lane / 8;
      const int lchunk = (swz<BK>(row, lane % 8) - row * BK) >> 3;
      const int rg = m_local * BM + row;
      const int rc = rg < rows ? rg : 0;       // padding rows read the group's first row
      int src;
      if (AK == A_TOKEN) {
        src = shared_grp ? rc : a.sorted_assign[off + rc] / a.k;
        src = (unsigned)src < (unsigned)a.T ? src : 0;
      } else if (AK == A_STORE) {
        src = sbase + rc;
      } else {
        src = rc;
      }
      aoff[i] = (uint32_t)src * (uint32_t)a.lda + lchunk * 8;
    } else {
      akrow[i] = q * 4 + lane / 16;
      alch[i] = (lane % 16) ^ ((akrow[i] & 3) << 2);
    }
  }
  auto issue_a = [&](int kt, int slot) {
    bf16_t* dst = As + slot * ASZ;
#pragma unroll
    for (int i = 0; i < DMA_A; ++i) {
      const bf16_t* src;
      if (!ATR) {
        if (SKIPA && (wave * DMA_A + i) * 8 >= rows_here) continue;   // wave-uniform
        src = a.A + aoff[i] + kt * BK;
      } else {
        const int r = kt * BK + akrow[i];
        src = r < rows ? a.A + (uint32_t)(sbase + r) * (uint32_t)a.lda + m0 + alch[i] * 8
                       : a.zero + alch[i] * 8;
      }
      __builtin_amdgcn_global_load_lds((const void*)src,
                                       (lds_ptr_t)(dst + (wave * DMA_A + i) * 512), 16, 0, 0);
    }
  };

  // ---- B loads: transposed [BK][BN] stage; load i fills k-rows q*RB .. (q = wave*DMA_B + i)
  constexpr int CPR = BN / 8, RB = 64 / CPR;   // 16-byte chunks per k-row, k-rows per load
  int bkrow[DMA_B], blch[DMA_B];
#pragma unroll
  for (int i = 0; i < DMA_B; ++i) {
    const int q = wave * DMA_B + i;
    bkrow[i] = q * RB + lane / CPR;
    blch[i] = (lane % CPR) ^ ((bkrow[i] & 3) << 2);
  }
  const bf16_t* bmat0 = nullptr;   // B_W2 / B_W13: this group's matrices
  const bf16_t* bmat1 = nullptr;
  if (BKIND == B_W2) {
    bmat0 = shared_grp ? a.S0 : a.B0 + (size_t)g * a.K * a.N;
  } else if (BKIND == B_W13) {
    const size_t msz = (size_t)(a.K / 2) * a.N;
    bmat0 = shared_grp ? a.S0 : a.B0 + (size_t)g * msz;
    bmat1 = shared_grp ? a.S1 : a.B1 + (size_t)g * msz;
  }
  // source of B load i of step kt
  auto b_src = [&](int i, int kt) -> const bf16_t* {
    const int r = kt * BK + bkrow[i];
    if (BKIND == B_W2) {
      return bmat0 + (uint32_t)r * (uint32_t)a.ldb + n0 + blch[i] * 8;
    } else if (BKIND == B_W13) {
      const int half = a.K / 2;
      return r < half ? bmat0 + (uint32_t)r * (uint32_t)a.ldb + n0 + blch[i] * 8
                      : bmat1 + (uint32_t)(r - half) * (uint32_t)a.ldb + n0 + blch[i] * 8;
    } else if (BKIND == B_WGATE) {
      return r < a.Kvalid ? a.B0 + (uint32_t)r * (uint32_t)a.ldb + n0 + blch[i] * 8
                          : a.zero + blch[i] * 8;
    } else {
      return r < rows ? a.B0 + (uint32_t)(sbase + r) * (uint32_t)a.ldb + n0 + blch[i] * 8
                      : a.zero + blch[i] * 8;
    }
  };
  auto issue_b = [&](int kt, int slot) {
    bf16_t* dst = Bs + slot * BSZ;
#pragma unroll
    for (int i = 0; i < DMA_B; ++i)
      __builtin_amdgcn_global_load_lds((const void*)b_src(i, kt),
                                       (lds_ptr_t)(dst + (wave * DMA_B + i) * 512), 16, 0, 0);
  };

  // ---- fragment offsets
  const int fr = lane & 31, fkc = lane >> 5;
  int aoffs[NKS], abase[FM], bbase[FN];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
    aoffs[ks] = (wm * 32 + fr) * BK + ((((2 * ks + fkc) ^ ((fr >> 1) & 7))) << 3);
#pragma unroll
  for (int i = 0; i < FM; ++i) abase[i] = tr_base<BM>(lane, (i * WM + wm) * 32);
#pragma unroll
  for (int j = 0; j < FN; ++j) bbase[j] = tr_base<BN>(lane, wn * TN + j * 32);

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // the K loop for a wave whose first NF row fragments hold data
  auto k_loop = [&](auto nf_tag) {
    constexpr int NF = decltype(nf_tag)::value;
    auto compute = [&](const bf16_t* Ast, const bf16_t* Bst) {
      if constexpr (NF == 0) return;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        bf16x8 af[FM], bfv[FN];
        if constexpr (ATR) {
          tr_frags<BM, FM>(Ast, abase, ks, af);
        } else {
#pragma unroll
          for (int i = 0; i < NF; ++i) af[i] = *(const bf16x8*)&Ast[aoffs[ks] + i * WM * 32 * BK];
        }
        if constexpr (RS) tr_frags_bi<BN, FN>(Bst, bbase, ks, bfv);
        else tr_frags<BN, FN>(Bst, bbase, ks, bfv);
#pragma unroll
        for (int i = 0; i < NF; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfv[j], acc[i][j], 0, 0, 0);
      }
    };
    if constexpr (RS) {
      u32x4 ra[DMA_A], rb[DMA_B];
      auto load_regs = [&](int kt) {
#pragma unroll
        for (int i = 0; i < DMA_A; ++i) {
          if ((wave * DMA_A + i) * 8 >= rows_here) continue;   // wave-uniform
          ra[i] = *(const u32x4*)(a.A + aoff[i] + kt * BK);
        }
#pragma unroll
        for (int i = 0; i < DMA_B; ++i) rb[i] = *(const u32x4*)b_src(i, kt);
      };
      auto write_regs = [&](int slot) {
#pragma unroll
        for (int i = 0; i < DMA_A; ++i) {
          if ((wave * DMA_A + i) * 8 >= rows_here) continue;
          *(u32x4*)(As + slot * ASZ + (wave * DMA_A + i) * 512 + lane * 8) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < DMA_B; ++i)
          *(u32x4*)(Bs + slot * BSZ + (wave * DMA_B + i) * 512 + lane * 8) = rb[i];
      };
      load_regs(0);
      write_regs(0);
      load_regs(KT > 1 ? 1 : 0);
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's stores are in LDS
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      for (int kt = 0; kt < KT; ++kt) {
        compute(As + (kt & 1) * ASZ, Bs + (kt & 1) * BSZ);
        write_regs((kt + 1) & 1);            // step kt+1 (past the end: a copy nobody reads)
        load_regs(kt + 2 < KT ? kt + 2 : KT - 1);
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if constexpr (STAG) {
      issue_a(0, 0);
      issue_b(0, 0);
      issue_b(KT > 1 ? 1 : 0, 1);
      for (int kt = 0; kt < KT; ++kt) {
        __builtin_amdgcn_s_waitcnt(wait_vm(DMA_B));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        issue_a(kt + 1 < KT ? kt + 1 : KT - 1, (kt + 1) & 1);
        issue_b(kt + 2 < KT ? kt + 2 : KT - 1, (kt + 2) % 3);
        compute(As + (kt & 1) * ASZ, Bs + (kt % 3) * BSZ);
      }
    } else {
#pragma unroll
      for (int s0 = 0; s0 < ST - 1; ++s0) {
        const int ld = s0 < KT ? s0 : KT - 1;
        issue_a(ld, s0);
        issue_b(ld, s0);
      }
      for (int kt = 0; kt < KT; ++kt) {
        __builtin_amdgcn_s_waitcnt(wait_vm((ST - 2) * (DMA_A + DMA_B)));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        const int nxt = kt + ST - 1, ld = nxt < KT ? nxt : KT - 1;
        issue_a(ld, nxt % ST);
        issue_b(ld, nxt % ST);
        compute(As + (kt % ST) * ASZ, Bs + (kt % ST) * BSZ);
      }
    }
  };
  if (KT > 0) {
    // wave-uniform count of this wave's row fragments that hold data (rows mode, staggered)
    const int nf = SKIPA ? min(FM, max(0, (rows_here - wm * 32 + WM * 32 - 1) / (WM * 32))) : FM;
    if (nf >= FM) k_loop(std::integral_constant<int, FM>{});
    else if (nf == 2) k_loop(std::integral_constant<int, (FM > 2 ? 2 : 0)>{});
    else if (nf == 1) k_loop(std::integral_constant<int, (FM > 1 ? 1 : 0)>{});
    else k_loop(std::integral_constant<int, 0>{});
    __builtin_amdgcn_s_waitcnt(wait_vm(0));
  }

  // ---- epilogues. 32x32 accumulator layout: lane holds column lane%32 and rows
  // 8*(r/4) + 4*(lane/32) + r%4 for r = 0..15 of each fragment.
  __syncthreads();                         // every wave is done with the ring
  if (EPI == EPI_DDOWN) {
    float* red = (float*)smem;             // [WN][BM] per-wave row sums of the gate gradient
    float* gate_s = red + WN * BM;         // [BM] gate of each tile row
    for (int r = tid; r < BM; r += NW * 64) {
      const int rg = m_local * BM + r;
      float gv = 1.f;
      if (!shared_grp && rg < rows) gv = a.topk_w[a.sorted_assign[off + rg]];
      gate_s[r] = gv;
    }
    __syncthreads();
    const int N = a.N;
    float part[FM][16];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) part[i][r] = 0.f;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = n0 + wn * TN + j * 32 + fr;
        const int fr0 = m_local * BM + (i * WM + wm) * 32;   // the fragment's first tile row
        if (fr0 >= rows) continue;                           // all padding (wave-uniform)
        // this lane's 16 values of u and v, in fragment order
        f32x4 uq[4], vq[4];
        const size_t o = uv_frag(sbase + fr0, col - fr, N, lane);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uq[q] = *(const f32x4*)(a.U + o + 256 * q);
          vq[q] = *(const f32x4*)(a.V + o + 256 * q);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int lr = (i * WM + wm) * 32 + 8 * (r >> 2) + 4 * fkc + (r & 3);
          if (m_local * BM + lr < rows) {
            const size_t s = (size_t)(sbase + m_local * BM + lr);
            const float u = uq[r >> 2][r & 3], v = vq[r >> 2][r & 3];
            const float dh = acc[i][j][r];
            const float sig = __builtin_amdgcn_rcpf(1.0f + __expf(-u));
            const float sl = u * sig;                           // SiLU(u), as the forward
            const float h = bf16_to_f32(f32_to_bf16(sl * v));   // the forward's stored h
            part[i][r] += dh * h;
            const float gdh = gate_s[lr] * dh;
            a.DUV[s * 2 * N + col] = f32_to_bf16(gdh * v * sig * (1.0f + u * (1.0f - sig)));
            a.DUV[s * 2 * N + N + col] = f32_to_bf16(gdh * sl);
          }
        }
      }
    // row sums over this wave's columns: the 32 lanes of each half share their rows
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = part[i][r];
        v += __shfl_xor(v, 16, 32);
        v += __shfl_xor(v, 8, 32);
        v += __shfl_xor(v, 4, 32);
        v += __shfl_xor(v, 2, 32);
        v += __shfl_xor(v, 1, 32);
        if (fr == 0) red[wn * BM + (i * WM + wm) * 32 + 8 * (r >> 2) + 4 * fkc + (r & 3)] = v;
      }
    __syncthreads();
    if (!shared_grp)
      for (int r = tid; r < BM; r += NW * 64) {
        const int rg = m_local * BM + r;
        if (rg < rows) {
          float sum = 0.f;
#pragma unroll
          for (int w = 0; w < WN; ++w) sum += red[w * BM + r];
          a.dgate_part[(size_t)(off + rg) * a.NT + n0 / BN] = sum;
        }
      }
    return;
  }

#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + wn * TN + j * 32 + fr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int lr = (i * WM + wm) * 32 + 8 * (r >> 2) + 4 * fkc + (r & 3);
        const float val = acc[i][j][r];
        if (EPI == EPI_ROWS) {
          const int rg = m_local * BM + lr;
          if (rg < rows) {
            float* dst = a.ident         ? a.out + (size_t)rg * a.N
                         : shared_grp     ? a.out_shared + (size_t)rg * a.N
                                          : a.out + (size_t)(off + rg) * a.N;
            dst[col] = val;
          }
        } else {
          const int m = m0 + lr;
          if (m < a.Mvalid) a.Wf[((size_t)g * a.Mvalid + m) * a.N + col] = val;
        }
      }
    }
}

// Persistent weight-gradient GEMM (bf16 output, storage-row operands): workgroup run r takes
// output tiles (group, 128-row m-tile, 128-column n-tile) r, r + nwg, r + 2 nwg, ... (so every
// workgroup gets a mix of long and short segments, and at any moment the workgroups of one XCD
// work on consecutive tiles that share their row operand in L2), and walks all of their K
// steps (a segment's rows, 64 at a time) as one stream through a 4-slot ring, three steps in
// flight across tile boundaries. A tile's last step is followed by its epilogue:
// the tile goes through a dedicated LDS buffer and out in 16-byte row pieces. A tile whose
// group has no rows still takes one step of zero rows (its gradient is zero).

struct WTile {
  int g, m0, n0, rows, sbase, kt_n;
};

__device__ __forceinline__ WTile wgrad_tile(const BwdArgs& a, int L, int MT, int NT) {
  WTile t;
  t.g = L / (MT * NT);
  const int rem = L - t.g * MT * NT;
  const int mt = rem / NT;
  t.m0 = mt * BBM;
  t.n0 = (rem - mt * NT) * 128;
  t.rows = a.sc.grp_rows[t.g];
  t.sbase = a.stor_start[t.g] * a.stor_bm;
  t.kt_n = max(1, (t.rows + 63) / 64);
  return t;
}

// WG_SLOTS = 4: three steps in flight, the output stage in its own 32 KB (160 KB, one
// workgroup per CU). WG_SLOTS = 2: one step in flight, the output staged in the slot the
// tile's last step just used (64 KB, two workgroups per CU).
template <int WG_SLOTS>
__global__ __launch_bounds__(512) void bwd_wgrad_kernel(BwdArgs a) {
  constexpr int BM = BBM, BN = 128, BK = 64, WM = 2, WN = 4, NW = 8, NKS = BK / 16;
  constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 32, FN = TN / 32;
  constexpr int ASZ = BM * BK, BSZ = BN * BK, SLOT = ASZ + BSZ;
  constexpr int DMA_A = ASZ * 2 / 1024 / NW, DMA_B = BSZ * 2 / 1024 / NW;
  constexpr bool OWN_STAGE = WG_SLOTS > 2;
  static_assert(SLOT >= BM * BN, "a ring slot holds the output tile");
  static_assert((WG_SLOTS * SLOT + (OWN_STAGE ? BM * BN : 0)) * 2 <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) bf16_t smem[WG_SLOTS * SLOT + (OWN_STAGE ? BM * BN : 0)];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int MT = a.M / BM, NT = a.N / BN, total = a.sc.G * MT * NT;
  // workgroup b runs on XCD b % 8; run (b % 8) * per + b / 8 keeps an XCD's runs consecutive
  const int nwg = gridDim.x, per = nwg >> 3;
  const int L0 = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (L0 >= total) return;

  // per-lane load geometry (transposed [64 k][128] stages for both operands)
  int akrow[DMA_A], alch[DMA_A], bkrow[DMA_B], blch[DMA_B];
#pragma unroll
  for (int i = 0; i < DMA_A; ++i) {
    akrow[i] = (wave * DMA_A + i) * 4 + lane / 16;
    alch[i] = (lane % 16) ^ ((akrow[i] & 3) << 2);
  }
#pragma unroll
  for (int i = 0; i < DMA_B; ++i) {
    bkrow[i] = (wave * DMA_B + i) * 4 + lane / 16;
    blch[i] = (lane % 16) ^ ((bkrow[i] & 3) << 2);
  }
  auto issue = [&](const WTile& t, int kt, int slot) {
    bf16_t* dA = smem + slot * SLOT;
    bf16_t* dB = dA + ASZ;
#pragma unroll
    for (int i = 0; i < DMA_A; ++i) {
      const int r = kt * BK + akrow[i];
      const bf16_t* src = r < t.rows
          ? a.A + (uint32_t)(t.sbase + r) * (uint32_t)a.lda + t.m0 + alch[i] * 8
          : a.zero + alch[i] * 8;
      __builtin_amdgcn_global_load_lds((const void*)src,
                                       (lds_ptr_t)(dA + (wave * DMA_A + i) * 512), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < DMA_B; ++i) {
      const int r = kt * BK + bkrow[i];
      const bf16_t* src = r < t.rows
          ? a.B0 + (uint32_t)(t.sbase + r) * (uint32_t)a.ldb + t.n0 + blch[i] * 8
          : a.zero + blch[i] * 8;
      __builtin_amdgcn_global_load_lds((const void*)src,
                                       (lds_ptr_t)(dB + (wave * DMA_B + i) * 512), 16, 0, 0);
    }
  };

  int abase[FM], bbase[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) abase[i] = tr_base<BM>(lane, (i * WM + wm) * 32);
#pragma unroll
  for (int j = 0; j < FN; ++j) bbase[j] = tr_base<BN>(lane, wn * TN + j * 32);
  const int fr = lane & 31, fkc = lane >> 5;

  f32x16 acc[FM][FN];
  auto zero_acc = [&]() {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  };
  zero_acc();

  // issue side: tile iL, step ikt (past the last tile: repeat the last step into a dead slot)
  int iL = L0, ikt = 0;
  WTile it = wgrad_tile(a, iL, MT, NT);
  WTile last_it = it;
  int last_kt = 0;
  auto issue_next = [&](int slot) {
    if (iL < total) {
      issue(it, ikt, slot);
      last_it = it;
      last_kt = ikt;
      if (++ikt == it.kt_n) {
        ikt = 0;
        iL += nwg;
        if (iL < total) it = wgrad_tile(a, iL, MT, NT);
      }
    } else {
      issue(last_it, last_kt, slot);
    }
  };
#pragma unroll
  for (int s = 0; s < WG_SLOTS - 1; ++s) issue_next(s);

  // compute side
  int cL = L0, ckt = 0;
  WTile ct = wgrad_tile(a, cL, MT, NT);
  for (int step = 0; cL < total; ++step) {
    __builtin_amdgcn_s_waitcnt(wait_vm((WG_SLOTS - 2) * (DMA_A + DMA_B)));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue_next((step + WG_SLOTS - 1) % WG_SLOTS);
    const bf16_t* As = smem + (step % WG_SLOTS) * SLOT;
    const bf16_t* Bs = As + ASZ;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      bf16x8 af[FM], bfv[FN];
      tr_frags<BM, FM>(As, abase, ks, af);
      tr_frags<BN, FN>(Bs, bbase, ks, bfv);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfv[j], acc[i][j], 0, 0, 0);
    }
    if (++ckt < ct.kt_n) continue;
    // ---- epilogue of tile cL: bf16 through the output stage, then 16-byte row pieces.
    // (The previous epilogue's reads of the stage finished before this step's barrier. With the
    // stage in this step's slot, every wave must first be done with its MFMA reads of it; the
    // slot is loaded again only after the next step's barrier.)
    bf16_t* const outst = OWN_STAGE ? smem + WG_SLOTS * SLOT : smem + (step % WG_SLOTS) * SLOT;
    if (!OWN_STAGE) __syncthreads();
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int lr = (i * WM + wm) * 32 + 8 * (r >> 2) + 4 * fkc + (r & 3);
          outst[lr * BN + wn * TN + j * 32 + fr] = f32_to_bf16(acc[i][j][r]);
        }
    zero_acc();
    __syncthreads();
    const bool shared_grp = ct.g >= a.E;
    const bool second = ct.m0 >= a.Msplit;
    const int mm0 = second ? ct.m0 - a.Msplit : ct.m0;
    bf16_t* base = shared_grp ? (second ? a.SW1 : a.SW0)
                              : (second ? a.W1 : a.W0) + (size_t)ct.g * a.Msplit * a.N;
    // non-temporal: the gradients are not read again here (DeepSeek-V3 shape: 22.6 GB of them)
    for (int idx = tid; idx < BM * BN / 8; idx += NW * 64) {
      const int row = idx / (BN / 8), ch = idx % (BN / 8);
      __builtin_nontemporal_store(*(const u32x4*)(outst + row * BN + ch * 8),
                                  (u32x4*)(base + (size_t)(mm0 + row) * a.N + ct.n0 + ch * 8));
    }
    ckt = 0;
    cL += nwg;
    if (cL < total) ct = wgrad_tile(a, cL, MT, NT);
  }
  __builtin_amdgcn_s_waitcnt(wait_vm(0));   // the dead loads past the last step
}

// ------------------------------------------------------------------ small kernels
// Items 0..T-1: dy row t -> bf16. Items T..: storage rows s of the grouped layout: routed row
// (group g, row r) -> assignment a = sorted_assign[off + r], token t = a / k, gate g_a:
// DO[s] = bf16(g_a dy_t), XS[s] = x_t; shared rows: DO[s] = bf16(dy_r), XS[s] = x_r. Padding
// rows are skipped. The first workgroup also clears the zero row.
// four bf16 (round to nearest even) in one 8-byte word, element 0 lowest
__device__ __forceinline__ uint2 pack_bf16x4(float a, float b, float c, float d) {
  return uint2{(uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16),
               (uint32_t)f32_to_bf16(c) | ((uint32_t)f32_to_bf16(d) << 16)};
}

__global__ __launch_bounds__(256) void bwd_prep_kernel(const float* __restrict__ dy,
                                                       const bf16_t* __restrict__ x,
                                                       const int32_t* __restrict__ sorted_assign,
                                                       const float* __restrict__ topk_w,
                                                       Schedule sc, int T, int d, int k, int E,
                                                       bf16_t* __restrict__ dyb,
                                                       bf16_t* __restrict__ DO,
                                                       bf16_t* __restrict__ XS,
                                                       bf16_t* __restrict__ zero) {
  if (blockIdx.x == 0 && threadIdx.x < ZERO_ELEMS) zero[threadIdx.x] = 0;
  const int SB = sc.BM;                 // storage rows per m-tile
  const int total = T + sc.mt_start[sc.G] * SB;
  const int d4 = d >> 2;
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    if (item < T) {
      const f32x4* src = (const f32x4*)(dy + (size_t)item * d);
      for (int c = threadIdx.x; c < d4; c += 256) {
        const f32x4 v = src[c];
        *(uint2*)(dyb + (size_t)item * d + 4 * c) = pack_bf16x4(v[0], v[1], v[2], v[3]);
      }
      continue;
    }
    const int s = item - T;
    const int mt = s / SB, g = sc.mt_group[mt];
    const int r = (mt - sc.mt_start[g]) * SB + s % SB;
    if (r >= sc.grp_rows[g]) continue;
    int t = r;
    float gate = 1.f;
    if (g < E) {
      const int asg = sorted_assign[sc.grp_off[g] + r];
      t = asg / k;
      gate = topk_w[asg];
    }
    const f32x4* src = (const f32x4*)(dy + (size_t)t * d);
    const uint2* xs = (const uint2*)(x + (size_t)t * d);
    for (int c = threadIdx.x; c < d4; c += 256) {
      const f32x4 v = src[c];
      *(uint2*)(DO + (size_t)s * d + 4 * c) =
          pack_bf16x4(gate * v[0], gate * v[1], gate * v[2], gate * v[3]);
      ((uint2*)(XS + (size_t)s * d))[c] = xs[c];
    }
  }
}

// Router backward, one wave per token (each wave takes RT_TOK tokens in turn, so a workgroup
// covers 4 * RT_TOK). Lane e (+64 i) recomputes the logit and the softmax probability of expert
// e exactly as the forward's router does; lanes j < k hold slot j's gate gradient (the sum of
// its per-n-tile partials, 0 if the slot was dropped).
// d l[e] = sum over slots j choosing e of g_j (dg_j - sum_j' g_j' dg_j')          (gates)
//        + p_e (w_e - sum_e' p_e' w_e'),  w_e = dL alpha E counts_pre[e] / (T k T)  (balance)
// Writes d l in bf16 ([T, E_pad], zero past E) and per-workgroup column sums (fp32, tokens in
// order within each wave, then the waves in order) for the logit offset's gradient.
constexpr int RT_TOK = 1;   // 4 in turn left one wave per SIMD waiting on its loads

__global__ __launch_bounds__(256) void bwd_router_kernel(
    const float* __restrict__ part, int KS, int T, int E, int E16, int k,
    const float* __restrict__ logit_bias, const int32_t* __restrict__ ids,
    const float* __restrict__ topk_w, const int32_t* __restrict__ assign_pos,
    const float* __restrict__ dgate_part, int NT, const int32_t* __restrict__ counts_pre,
    float bal_coef, int E_pad, bf16_t* __restrict__ dlog, float* __restrict__ dlb_part) {
  __shared__ float colsum[4][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float csum[4] = {0.f, 0.f, 0.f, 0.f};
  for (int tt = 0; tt < RT_TOK; ++tt) {
    const int t = (blockIdx.x * 4 + wave) * RT_TOK + tt;
    if (t >= T) break;                  // uniform across the wave
    float dl[4] = {0.f, 0.f, 0.f, 0.f};
    float lg[4];
    bool live[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      live[i] = e < E;
      lg[i] = live[i] ? sum_partials(part, KS, T, E16, t, e) + (logit_bias ? logit_bias[e] : 0.f)
                      : -INFINITY;
    }
    const float m = wave_max_f(fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3])));
    float ex[4], loc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ex[i] = live[i] ? expf(lg[i] - m) : 0.f;
      loc += ex[i];
    }
    const float inv = 1.0f / wave_sum_f(loc);
    // slots
    float dg = 0.f, gj = 0.f;
    int ej = -1;
    if (lane < k) {
      const int asg = t * k + lane;
      const int pos = assign_pos[asg];
      if (pos >= 0)
        for (int n = 0; n < NT; ++n) dg += dgate_part[(size_t)pos * NT + n];
      gj = topk_w[asg];
      ej = ids[asg];
    }
    const float inner = wave_sum_f(lane < k ? gj * dg : 0.f);
    const float cj = gj * (dg - inner);
    for (int j = 0; j < k; ++j) {
      const int e = __builtin_amdgcn_readlane(ej, j);
      const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cj), j));
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lane + 64 * i == e) dl[i] += c;
    }
    if (bal_coef != 0.f) {
      float w[4], pw = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w[i] = live[i] ? bal_coef * (float)counts_pre[lane + 64 * i] : 0.f;
        pw += ex[i] * inv * w[i];
      }
      pw = wave_sum_f(pw);
#pragma unroll
      for (int i = 0; i < 4; ++i) dl[i] += ex[i] * inv * (w[i] - pw);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      if (e < E_pad) dlog[(size_t)t * E_pad + e] = f32_to_bf16(live[i] ? dl[i] : 0.f);
      csum[i] += dl[i];
    }
  }
  if (!dlb_part) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) colsum[wave][lane + 64 * i] = csum[i];
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256)
    dlb_part[(size_t)blockIdx.x * E + e] =
        ((colsum[0][e] + colsum[1][e]) + colsum[2][e]) + colsum[3][e];
}

// dx[t] = router share + shared expert's rows + the kept slots' rows in slot order.
__global__ __launch_bounds__(256) void bwd_dx_kernel(const float* __restrict__ dx_router,
                                                     const float* __restrict__ dx_shared,
                                                     const float* __restrict__ dx_rows,
                                                     const int32_t* __restrict__ assign_pos,
                                                     int k, int d, float* __restrict__ dx) {
  __shared__ int pos[16];
  const int t = blockIdx.x;
  if (threadIdx.x < k) pos[threadIdx.x] = assign_pos[(size_t)t * k + threadIdx.x];
  __syncthreads();
  const int d4 = d >> 2;
  for (int c = threadIdx.x; c < d4; c += 256) {
    f32x4 acc = *(const f32x4*)(dx_router + (size_t)t * d + 4 * c);
    if (dx_shared) {
      const f32x4 v = *(const f32x4*)(dx_shared + (size_t)t * d + 4 * c);
      acc[0] += v[0];
      acc[1] += v[1];
      acc[2] += v[2];
      acc[3] += v[3];
    }
    for (int j = 0; j < k; ++j) {
      if (pos[j] < 0) continue;
      const f32x4 v = *(const f32x4*)(dx_rows + (size_t)pos[j] * d + 4 * c);
      acc[0] += v[0];
      acc[1] += v[1];
      acc[2] += v[2];
      acc[3] += v[3];
    }
    *(f32x4*)(dx + (size_t)t * d + 4 * c) = acc;
  }
}

// Row-tiled GEMMs (dgrads, router dgrad): 256 x BN tiles, 8 waves (4 x 2); the register-staged
// ring when `staged`, else the staggered rings.
template <int BN, int AK, int BKIND, int EPI>
hipError_t launch_rows(const BwdArgs& a, int tiles, bool staged, hipStream_t s) {
  if (tiles <= 0) return hipSuccess;
  if (staged)
    hipLaunchKernelGGL((bwd_gemm_kernel<kRowsBM, BN, 4, 2, M_ROWS, AK, BKIND, EPI, 2, true>),
                       dim3((tiles + 7) / 8 * 8), dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_gemm_kernel<kRowsBM, BN, 4, 2, M_ROWS, AK, BKIND, EPI, 0>),
                       dim3((tiles + 7) / 8 * 8), dim3(512), 0, s, a);
  return hipGetLastError();
}
// The router's weight-gradient GEMM: 128 x kWgradBN tiles, 8 waves (2 x 4), a kWgradStages ring.
// out[i] = sum over the S splits, in split order, of part[s][i] (float4 per thread)
__global__ __launch_bounds__(256) void bwd_split_sum_kernel(const float* __restrict__ part, int S,
                                                           long long n4, float* __restrict__ out) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n4;
       i += (long long)gridDim.x * 256) {
    f32x4 acc = ((const f32x4*)part)[i];
    for (int sp = 1; sp < S; ++sp) {
      const f32x4 v = ((const f32x4*)part)[(size_t)sp * n4 + i];
      acc[0] += v[0];
      acc[1] += v[1];
      acc[2] += v[2];
      acc[3] += v[3];
    }
    ((f32x4*)out)[i] = acc;
  }
}

template <int AK, int BKIND, int EPI>
hipError_t launch_weights(const BwdArgs& a, int tiles, hipStream_t s) {
  if (tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_gemm_kernel<BBM, kWgradBN, 2, 4, M_WEIGHTS, AK, BKIND, EPI,
                                      kWgradStages>),
                     dim3((tiles + 7) / 8 * 8), dim3(512), 0, s, a);
  return hipGetLastError();
}

// Persistent weight-gradient GEMM: kWgradPerCU workgroups per CU.
constexpr int kWgradPerCU = 2;
hipError_t launch_wgrad(const BwdArgs& a, hipStream_t s) {
  constexpr int kCUs = 256;                 // MI355X compute units
  const long long total = (long long)a.sc.G * (a.M / BBM) * (a.N / 128);
  if (total <= 0) return hipSuccess;
  const int nwg = (int)std::min<long long>(kCUs * kWgradPerCU, (total + 7) / 8 * 8);
  if (kWgradPerCU == 1)
    hipLaunchKernelGGL(bwd_wgrad_kernel<4>, dim3(nwg), dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL(bwd_wgrad_kernel<2>, dim3(nwg), dim3(512), 0, s, a);
  return hipGetLastError();
}

// BN for an output width: 256 when it divides, else 128
inline int bn_for(int n) { return n % 256 == 0 ? 256 : 128; }


}  // namespace

// ------------------------------------------------------------------ workspace
BwdLayout backward_layout(const moe_problem& p) {
  BwdLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + (bytes ? bytes : 1), 256);
    return o;
  };
  const size_t n = (size_t)p.T * p.k;
  const int G = p.E + p.n_shared;
  L.E_pad = ceil_div(p.E, 128) * 128;
  // storage rows follow the forward's own m-tile class, so the recompute is the forward's
  // gate-up GEMM, tile for tile
  L.stor_bm = gemm_bm(p);
  L.max_mt = max_mtiles((long long)n, p.T, p.E, p.n_shared, L.stor_bm);
  const size_t srows = (size_t)L.max_mt * L.stor_bm;
  L.NT_down = p.d_ff / bn_for(p.d_ff);
  L.nblk_router = ceil_div(p.T, 4 * RT_TOK);
  L.grp_rows = take((size_t)G * 4);
  L.grp_off = take((size_t)G * 4);
  L.mt_start = take((size_t)(G + 1) * 4);
  L.mt_group = take((size_t)L.max_mt * 4);
  L.max_mt_rows = max_mtiles((long long)n, p.T, p.E, p.n_shared, kRowsBM);
  L.r_grp_rows = take((size_t)G * 4);
  L.r_grp_off = take((size_t)G * 4);
  L.r_mt_start = take((size_t)(G + 1) * 4);
  L.r_mt_group = take((size_t)L.max_mt_rows * 4);
  L.logits_part = take(route_partial_bytes(p));
  L.dlb_part = take((size_t)L.nblk_router * p.E * 4);
  L.zero = take(ZERO_ELEMS * 2);
  L.H = take(srows * p.d_ff * 2);
  L.U = take(srows * p.d_ff * 4);
  L.V = take(srows * p.d_ff * 4);
  L.DUV = take(srows * 2 * p.d_ff * 2);
  L.DO = take(srows * p.d * 2);
  L.XS = take(srows * p.d * 2);
  L.dyb = take((size_t)p.T * p.d * 2);
  L.dgate_part = take(n * L.NT_down * 4);
  L.dx_rows = take(n * p.d * 4);
  L.dx_shared = take((size_t)p.n_shared * p.T * p.d * 4);
  L.dlog = take((size_t)p.T * L.E_pad * 2);
  L.dx_router = take((size_t)p.T * p.d * 4);
  // The router weight gradient (K = T) has only (E_pad/128) x (d/128) output tiles: its K is
  // cut into splits of whole 64-row steps, enough for ~256 workgroups, at least 512 rows each;
  // the splits' fp32 partials are added in split order.
  {
    const int tiles = (L.E_pad / BBM) * (p.d / kWgradBN);
    int split = std::max(1, std::min(ceil_div(256, std::max(tiles, 1)), p.T / 512));
    L.wgate_rows = ceil_div(std::max(p.T, 1), split * 64) * 64;
    L.wgate_split = ceil_div(std::max(p.T, 1), L.wgate_rows);
    L.wgate_part = take(L.wgate_split > 1 ? (size_t)L.wgate_split * p.E * p.d * 4 : 0);
  }
  L.total = off;
  return L;
}

// ------------------------------------------------------------------ the pass
hipError_t launch_backward(const moe_problem& p, const BwdLayout& L, void* ws, const void* x,
                           const void* w_gate, const float* logit_bias, const void* w1,
                           const void* w3, const void* w2, const void* ws1, const void* ws3,
                           const void* ws2, const int32_t* topk_ids, const float* topk_w,
                           const int32_t* counts_pre, const int32_t* offsets,
                           const int32_t* sorted_assign, const int32_t* assign_pos,
                           const float* dy, float alpha, float dL, float* dx, float* dw_gate,
                           float* dlogit_bias, void* dw1, void* dw3, void* dw2, void* dws1,
                           void* dws3, void* dws2, hipStream_t s, hipEvent_t* ev) {
  char* base = (char*)ws;
  auto at = [&](size_t o) { return (void*)(base + o); };
  const int G = p.E + p.n_shared;
  Schedule sc;
  sc.grp_rows = (int32_t*)at(L.grp_rows);
  sc.grp_off = (int32_t*)at(L.grp_off);
  sc.mt_start = (int32_t*)at(L.mt_start);
  sc.mt_group = (int32_t*)at(L.mt_group);
  sc.max_mtiles = L.max_mt;
  sc.G = G;
  sc.BM = L.stor_bm;
  Schedule sr;                        // row tiles of the row-tiled GEMMs
  sr.grp_rows = (int32_t*)at(L.r_grp_rows);
  sr.grp_off = (int32_t*)at(L.r_grp_off);
  sr.mt_start = (int32_t*)at(L.r_mt_start);
  sr.mt_group = (int32_t*)at(L.r_mt_group);
  sr.max_mtiles = L.max_mt_rows;
  sr.G = G;
  sr.BM = kRowsBM;
  bf16_t* H = (bf16_t*)at(L.H);
  float* U = (float*)at(L.U);
  float* V = (float*)at(L.V);
  bf16_t* DUV = (bf16_t*)at(L.DUV);
  bf16_t* DO = (bf16_t*)at(L.DO);
  bf16_t* XS = (bf16_t*)at(L.XS);
  bf16_t* dyb = (bf16_t*)at(L.dyb);
  bf16_t* zero = (bf16_t*)at(L.zero);
  float* dgate_part = (float*)at(L.dgate_part);
  float* dx_rows = (float*)at(L.dx_rows);
  float* dx_shared = p.n_shared ? (float*)at(L.dx_shared) : nullptr;
  bf16_t* dlog = (bf16_t*)at(L.dlog);
  float* dx_router = (float*)at(L.dx_router);
  float* logits_part = (float*)at(L.logits_part);
  float* dlb_part = (float*)at(L.dlb_part);

  hipError_t err;
  int stage = 0;
  auto mark = [&]() { return ev ? hipEventRecord(ev[stage++], s) : hipSuccess; };
#define MOE_TRY(call)                  \
  do {                                 \
    if ((err = (call)) != hipSuccess) \
      return err;                      \
  } while (0)
  // 1. schedules (storage = the forward's class; 256-row tiles) and the gate-up recompute
  //    (h, u, v in storage rows)
  MOE_TRY(mark());
  MOE_TRY(launch_schedule(p, offsets, sc, s));
  MOE_TRY(launch_schedule(p, offsets, sr, s));
  MOE_TRY(launch_expert_ffn(p, x, w1, w3, w2, ws1, ws3, ws2, sorted_assign, sc, H, nullptr,
                            nullptr, nullptr, s, nullptr, 0, U, V));
  MOE_TRY(mark());
  // 2. dy in bf16, g dy and the gathered x rows in storage rows
  hipLaunchKernelGGL(bwd_prep_kernel, dim3(std::min(p.T + L.max_mt * L.stor_bm, 16384)), dim3(256), 0,
                     s, dy, (const bf16_t*)x, sorted_assign, topk_w, sc, p.T, p.d, p.k, p.E, dyb,
                     DO, XS, zero);
  MOE_TRY(hipGetLastError());
  MOE_TRY(mark());

  BwdArgs c{};
  c.E = p.E;
  c.k = p.k;
  c.T = p.T;
  c.sorted_assign = sorted_assign;
  c.sc = sc;
  c.stor_start = sc.mt_start;
  c.stor_bm = L.stor_bm;
  c.zero = zero;
  BwdArgs cr = c;                     // row-tiled GEMMs walk the row-tile schedule
  cr.sc = sr;
  // register-staged ring when the weight tiles are shared in L2 by several m-tiles (the
  // forward's wide class); the staggered rings otherwise
  const bool staged = gemm_wide(p);
  // 3. dgrad-down + SwiGLU backward: d h' = dy_t W2, then du, dv, d g partials
  {
    BwdArgs a = cr;
    a.A = dyb;
    a.lda = p.d;
    a.B0 = (const bf16_t*)w2;
    a.S0 = (const bf16_t*)ws2;
    a.ldb = p.d_ff;
    a.M = 0;
    a.N = p.d_ff;
    a.K = p.d;
    a.U = U;
    a.V = V;
    a.topk_w = topk_w;
    a.DUV = DUV;
    a.dgate_part = dgate_part;
    a.NT = L.NT_down;
    const int tiles = L.max_mt_rows * L.NT_down;
    err = (L.NT_down * 256 == p.d_ff) ? launch_rows<256, A_TOKEN, B_W2, EPI_DDOWN>(a, tiles, staged, s)
                                      : launch_rows<128, A_TOKEN, B_W2, EPI_DDOWN>(a, tiles, staged, s);
    MOE_TRY(err);
  }
  MOE_TRY(mark());
  // 4. dgrad-x: (du | dv) (W1; W3) -> per-row dx (sorted order) and the shared rows
  {
    BwdArgs a = cr;
    a.A = DUV;
    a.lda = 2 * p.d_ff;
    a.B0 = (const bf16_t*)w1;
    a.B1 = (const bf16_t*)w3;
    a.S0 = (const bf16_t*)ws1;
    a.S1 = (const bf16_t*)ws3;
    a.ldb = p.d;
    a.N = p.d;
    a.K = 2 * p.d_ff;
    a.out = dx_rows;
    a.out_shared = dx_shared;
    const int bn = bn_for(p.d);
    const int tiles = L.max_mt_rows * (p.d / bn);
    err = (bn == 256) ? launch_rows<256, A_STORE, B_W13, EPI_ROWS>(a, tiles, staged, s)
                      : launch_rows<128, A_STORE, B_W13, EPI_ROWS>(a, tiles, staged, s);
    MOE_TRY(err);
  }
  MOE_TRY(mark());
  // 5. wgrad-down: dW2_g = (g dy)^T h over the group's rows
  {
    BwdArgs a = c;
    a.A = DO;
    a.lda = p.d;
    a.B0 = H;
    a.ldb = p.d_ff;
    a.M = p.d;
    a.N = p.d_ff;
    a.W0 = (bf16_t*)dw2;
    a.SW0 = (bf16_t*)dws2;
    a.Msplit = p.d;
    err = launch_wgrad(a, s);
    MOE_TRY(err);
  }
  MOE_TRY(mark());
  // 6. wgrad-up: (dW1_g; dW3_g) = (du | dv)^T x_rows
  {
    BwdArgs a = c;
    a.A = DUV;
    a.lda = 2 * p.d_ff;
    a.B0 = XS;
    a.ldb = p.d;
    a.M = 2 * p.d_ff;
    a.N = p.d;
    a.W0 = (bf16_t*)dw1;
    a.W1 = (bf16_t*)dw3;
    a.SW0 = (bf16_t*)dws1;
    a.SW1 = (bf16_t*)dws3;
    a.Msplit = p.d_ff;
    err = launch_wgrad(a, s);
    MOE_TRY(err);
  }
  MOE_TRY(mark());
  // 7. router: logits again, then d l per token (gates + balance), then its column sums
  if (p.T > 0) {
    MOE_TRY(launch_route_logits(p, x, w_gate, logits_part, s));
    const float coef = dL * alpha * (float)p.E / ((float)p.T * (float)p.k * (float)p.T);
    hipLaunchKernelGGL(bwd_router_kernel, dim3(L.nblk_router), dim3(256), 0, s, logits_part,
                       route_ksplit(p), p.T, p.E, ceil_div(p.E, 16) * 16, p.k, logit_bias,
                       topk_ids, topk_w, assign_pos, dgate_part, L.NT_down, counts_pre, coef,
                       L.E_pad, dlog, dlogit_bias ? dlb_part : nullptr);
    MOE_TRY(hipGetLastError());
  }
  if (dlogit_bias) MOE_TRY(launch_psum_reduce(dlb_part, p.T > 0 ? L.nblk_router : 0, p.E, dlogit_bias, s));
  MOE_TRY(mark());
  // 8. router dgrad: dx_router = d l W_gate (K = E_pad; rows of W_gate past E read zeros)
  {
    BwdArgs a = c;
    a.A = dlog;
    a.lda = L.E_pad;
    a.B0 = (const bf16_t*)w_gate;
    a.ldb = p.d;
    a.N = p.d;
    a.K = L.E_pad;
    a.Kvalid = p.E;
    a.ident = 1;
    a.ident_rows = p.T;
    a.out = dx_router;
    const int bn = bn_for(p.d);
    const int tiles = ceil_div(p.T, kRowsBM) * (p.d / bn);
    err = (bn == 256) ? launch_rows<256, A_IDENT, B_WGATE, EPI_ROWS>(a, tiles, true, s)
                      : launch_rows<128, A_IDENT, B_WGATE, EPI_ROWS>(a, tiles, true, s);
    MOE_TRY(err);
  }
  MOE_TRY(mark());
  // 9. router wgrad: dW_gate = d l^T x (K = T)
  {
    BwdArgs a = c;
    a.A = dlog;
    a.lda = L.E_pad;
    a.B0 = (const bf16_t*)x;
    a.ldb = p.d;
    a.M = L.E_pad;
    a.N = p.d;
    a.ident = 1;
    a.ident_rows = p.T;
    a.ident_split = L.wgate_split;
    a.ident_chunk = L.wgate_rows;
    float* part = L.wgate_split > 1 ? (float*)at(L.wgate_part) : dw_gate;
    a.Wf = part;
    a.Mvalid = p.E;
    const int tiles = L.wgate_split * (L.E_pad / BBM) * (p.d / kWgradBN);
    // (T = 0: one split whose K loop is empty, so every tile writes zeros)
    err = launch_weights<AT_IDENT, BT_IDENT, EPI_WF32>(a, tiles, s);
    MOE_TRY(err);
    if (L.wgate_split > 1) {
      const long long n4 = (long long)p.E * p.d / 4;
      hipLaunchKernelGGL(bwd_split_sum_kernel, dim3((unsigned)std::min<long long>(ceil_div(n4, 256), 1024)),
                         dim3(256), 0, s, part, L.wgate_split, n4, dw_gate);
      MOE_TRY(hipGetLastError());
    }
  }
  MOE_TRY(mark());
  // 10. dx
  if (p.T > 0) {
    hipLaunchKernelGGL(bwd_dx_kernel, dim3(p.T), dim3(256), 0, s, dx_router, dx_shared, dx_rows,
                       assign_pos, p.k, p.d, dx);
    MOE_TRY(hipGetLastError());
  }
  MOE_TRY(mark());
#undef MOE_TRY
  return hipSuccess;
}

}  // namespace moe
