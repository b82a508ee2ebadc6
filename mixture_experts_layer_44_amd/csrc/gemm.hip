// Grouped expert GEMMs over the per-expert segments.
//
// Pages: "Mixture of experts (MoE)" handbook, "Implementation: token by token vs. grouped
// by expert" (each expert does one matrix multiplication over all its tokens; one grouped
// GEMM covers all experts, and an empty group must be handled); "MoE Architecture" §3
// "Standard MoE" (SwiGLU experts: down(SiLU(gate x) * up x)).
//
// gate-up: for m-tile (group g, rows r0..r0+BM) and n-tile (features n0..n0+BNB/2):
//   u = X_g W1_g^T, v = X_g W3_g^T over the tile, h = SiLU(u) * v -> bf16 H[m-tile rows].
//   X rows are gathered from x by token (sorted_assign / k; identity for the shared group).
// down:    out = H W2_g^T (n-tile = BNB features) -> fp32 rows in sorted order (routed) or
//          token order (shared).
//
// Tile classes, chosen on the host per problem from the expected rows per expert r:
//   decode  (r <= 48, d and d_ff multiples of 256 up to 2048) gemm_bf16_dec_kernel: 32-row
//                         m-tiles x 32 (gate-up) / 64 (down) features, the 4 waves splitting K
//                         and streaming their operands straight into registers.
//   small   (r <= 48, other d / d_ff) gemm_bf16_kernel, BM=32, BNB=256 / 128, BK=64, 4-stage
//                         ring, 4 waves (1x4): many workgroups stream the touched experts' weights.
//   ragged  (48 < r < 768) gemm_bf16_st_kernel, BM=128 / 192 (8 waves, 2x4) or 256 (4x2),
//                         BNB=256, BK=64; B in the deep ring, A in the shallow one; the rows of
//                         a tile past its segment's end are neither loaded nor multiplied.
//   wide    (r >= 768)    gemm_bf16_w4_kernel, BM=256, BNB=256, 4 waves of 128 x 128 (one per
//                         SIMD), 2 LDS stages filled from two register sets (the weight tiles
//                         are shared in L2 by several m-tiles; the loads run faster through
//                         registers than straight to LDS). Shapes whose x or h reach 2 GiB take
//                         gemm_bf16_kernel with 8 waves (4x2) and one register set.
//   d % 256 != 0          gemm_bf16_kernel, BM=128, BNB=256 / 128, BK=64, 3-stage ring.
// Except in the decode and wide classes, each wave owns a block of 32x32 MFMA tiles
// (v_mfma_f32_32x32x16_bf16, fp32 accumulators), two waves per SIMD: while one waits for its
// LDS fragments the other issues MFMAs.
// BNB counts B rows: the gate-up B tile holds the W1 rows and then the W3 rows of the same
// BNB/2 features, and each wave reads the u and v fragments of the same features, so the
// SwiGLU epilogue has u and v of an output in the same lane.
//
// Main loop of gemm_bf16_kernel: a ring of STAGES LDS buffers, each one K step of BK for all
// BM + BNB rows, filled by direct global->LDS loads (global_load_lds_dwordx4, 16 bytes per
// lane, 1 KB per instruction). STAGES-1 steps are in flight while the MFMAs consume one; each
// step is one wait for this wave's loads of the step, one barrier, the loads of step
// kt+STAGES-1 into the buffer freed by step kt-1, and the MFMAs of step kt. Past the last step
// the loads repeat the last step into a buffer nobody reads again, so the loop has no
// branches. With RS (register staging, 2 stages) the same 16-byte pieces go through registers
// instead: loaded during step kt, stored into the other stage at its end. Each LDS row is
// BK*2 bytes (BK/8 chunks of 16); chunk c of row r sits in a swizzled slot (see swz) so 16
// consecutive rows at one logical chunk cover all 16 16-byte bank groups of a 256-byte LDS
// cycle.
//
// In gemm_bf16_kernel, rows of an m-tile past the end of its segment are loaded from the
// segment's first row; their results land only in padding rows of H (gate-up) or are not
// stored (down). The eight-wave wide variant keeps loading them on purpose: with every tile the
// same length, the m-tiles that share a weight tile stay in step and meet in L2 (skipping the
// padding loads of a segment's last tile doubled FETCH_SIZE at unchanged time); it skips only the
// LDS reads and MFMAs of row fragments that are all padding. The four-wave wide kernel does the
// same, except that its padding rows' loads fall outside the buffer range and return zeros
// without a memory access (the loads and barriers still run, so the pace is unchanged).
//
// Work order: tiles are numbered group-major, then n-tile, then m-tile, so neighbouring
// tiles share a weight tile (B) or a row block (A). Workgroups are dealt round-robin to
// the 8 XCDs, so workgroup b runs tile (b % 8) * per + b / 8: each XCD walks its own
// contiguous range and its L2 sees the reuse.
#include <type_traits>

#include "moe_internal.h"
#include "mfma_tiles.h"

namespace moe {

namespace {

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
  float* out_rows_b;    // down with K split in two: the second half's routed rows
  int ksplit;           // 1, or 2 for the down GEMM (routed groups only, no shared expert)
  float* U;             // gate-up, or null: also store u and v (fp32 storage rows, fragment order)
  float* V;
};

// RS: 1 = register-staged (2 stages), 0 = direct global->LDS ring
template <int BM, int BNB, int WM, int WN, int BK, int STAGES, bool GATEUP, int RS = 0>
__global__ __launch_bounds__(WM * WN * 64) void gemm_bf16_kernel(GemmArgs args) {
  constexpr int NW = WM * WN;
  constexpr int CHUNKS = BK / 8;                   // 16-byte chunks per row per stage
  constexpr int RPI = 64 / CHUNKS;                 // rows covered by one 1 KB load
  constexpr int TM = BM / WM, TNB = BNB / WN;      // wave tile: rows x B rows
  constexpr int FM = TM / 32, FN = TNB / 32;       // 32x32 fragments per wave
  constexpr int ROWS = BM + BNB;                   // A rows then B rows in one stage
  constexpr int STAGE = ROWS * BK;                 // bf16 elements per stage
  constexpr int DMA_WAVE = ROWS * CHUNKS / 64 / NW; // 1 KB loads per wave per stage
  static_assert(DMA_WAVE * 64 * NW == ROWS * CHUNKS, "loads split evenly over the waves");
  static_assert((STAGES - 1) * DMA_WAVE <= 63, "the loads in flight fit the vmcnt counter");
  constexpr int FEAT = GATEUP ? BNB / 2 : BNB;     // output features per n-tile
  static_assert(!GATEUP || FN % 2 == 0, "u and v fragments pair up");
  static_assert(BM % RPI == 0 && (BNB / 2) % RPI == 0, "a 1 KB load covers rows of one matrix");
  __shared__ __attribute__((aligned(1024))) bf16_t smem[STAGES * STAGE];

  // with the K range split in two (down GEMM only), work unit = (half, tile), as in the
  // staggered kernel below
  const int S = GATEUP ? 1 : args.ksplit;
  TileCoord tc;
  int half = 0;
  if (!tile_coord(args.sc, args.N / FEAT, FEAT, tc, S, &half)) return;
  const bool shared_grp = tc.g >= args.E;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = args.K, N = args.N;

  // ---- load sources. Load i of this wave fills stage rows q*RPI .. q*RPI+RPI-1 with
  // q = wave*DMA_WAVE+i; lane l writes 16-byte slot l of the 1 KB: row q*RPI + l/CHUNKS,
  // physical slot l%CHUNKS, so it fetches the logical chunk that the swizzle puts there.
  const bf16_t* src_base[DMA_WAVE];
  uint32_t src_off[DMA_WAVE];
  // The assignment ids of this lane's gathered rows are loaded together, before the first wait
  // (loaded one by one, each behind the branch on its load's matrix, they were serial round
  // trips at the start of every tile). Loads of B rows read a valid entry and discard it.
  int sa[DMA_WAVE];
#pragma unroll
  for (int i = 0; i < DMA_WAVE; ++i) {
    const int r = tc.m_local * BM + (wave * DMA_WAVE + i) * RPI + lane / CHUNKS;
    const bool gathered = !shared_grp && (wave * DMA_WAVE + i) * RPI < BM;
    sa[i] = GATEUP ? args.sorted_assign[tc.off + (gathered && r < tc.rows ? r : 0)] : 0;
  }
#pragma unroll
  for (int i = 0; i < DMA_WAVE; ++i) {
    const int q = wave * DMA_WAVE + i;
    const int row = q * RPI + lane / CHUNKS;
    const int lchunk = (swz<BK>(row, lane % CHUNKS) - row * BK) >> 3;  // the swizzle is an involution
    if (q * RPI < BM) {
      int srow;
      if (GATEUP) {
        const int r = tc.m_local * BM + row;
        const int rr = r < tc.rows ? r : 0;             // padding rows repeat the first row
        int tok = shared_grp ? rr : sa[i] / args.k;
        srow = (unsigned)tok < (unsigned)args.T ? tok : 0;
      } else {
        srow = tc.mt_global * BM + row;
      }
      src_base[i] = args.A;
      src_off[i] = (uint32_t)srow * (uint32_t)K + lchunk * 8;
    } else {
      const int br = row - BM;
      const bool second = GATEUP && br >= BNB / 2;
      const bf16_t* mat;
      if (GATEUP)
        mat = shared_grp ? (second ? args.S1 : args.S0)
                         : (second ? args.B1 : args.B0) + (size_t)tc.g * N * K;
      else
        mat = shared_grp ? args.S0 : args.B0 + (size_t)tc.g * N * K;
      src_base[i] = mat + (size_t)tc.n0 * K;
      src_off[i] = (uint32_t)(second ? br - BNB / 2 : br) * (uint32_t)K + lchunk * 8;
    }
  }
  const int KT = K / BK / S;                       // steps of this work unit
  const int k0 = half * KT * BK;                    // its first K element
  auto issue = [&](int kt, int st) {
    bf16_t* dst = smem + st * STAGE;
    const int kk = k0 + kt * BK;
#pragma unroll
    for (int i = 0; i < DMA_WAVE; ++i) {
      const int q = wave * DMA_WAVE + i;
      __builtin_amdgcn_global_load_lds((const void*)(src_base[i] + src_off[i] + kk),
                                       (lds_ptr_t)(dst + q * RPI * BK), 16, 0, 0);
    }
  };

  const int wm = wave / WN, wn = wave % WN;
  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // stage rows of this lane's fragments
  const int fr = lane & 31, fkc = lane >> 5;
  int arow[FM], brow[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) arow[i] = wm * TM + i * 32 + fr;
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    if (GATEUP) {
      const int fw = BNB / 2 / WN;   // features per wave
      const int jj = j % (FN / 2);
      brow[j] = BM + (j < FN / 2 ? 0 : BNB / 2) + wn * fw + jj * 32 + fr;
    } else {
      brow[j] = BM + wn * TNB + j * 32 + fr;
    }
  }

  // One K stage of MFMAs. Fragments are double-buffered across the k16 steps so the reads for
  // step ks+1 can be in flight while the MFMAs of step ks run; iglp_opt(1) asks the backend
  // scheduler for its DS-read/MFMA interleaving strategy (measured best of the options).
  auto compute = [&](const bf16_t* buf, auto nf_tag) {
    constexpr int NF = decltype(nf_tag)::value;
    if constexpr (NF == 0) return;
    constexpr int NKS = BK / 16;
    __builtin_amdgcn_iglp_opt(1);
    bf16x8 af[2][FM], bfr[2][FN];
#pragma unroll
    for (int i = 0; i < NF; ++i) af[0][i] = *(const bf16x8*)&buf[swz<BK>(arow[i], fkc)];
#pragma unroll
    for (int j = 0; j < FN; ++j) bfr[0][j] = *(const bf16x8*)&buf[swz<BK>(brow[j], fkc)];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int cur = ks & 1, nxt = cur ^ 1;
      if (ks + 1 < NKS) {
#pragma unroll
        for (int i = 0; i < NF; ++i)
          af[nxt][i] = *(const bf16x8*)&buf[swz<BK>(arow[i], 2 * (ks + 1) + fkc)];
#pragma unroll
        for (int j = 0; j < FN; ++j)
          bfr[nxt][j] = *(const bf16x8*)&buf[swz<BK>(brow[j], 2 * (ks + 1) + fkc)];
      }
#pragma unroll
      for (int i = 0; i < NF; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][i], bfr[cur][j], acc[i][j],
                                                              0, 0, 0);
    }
  };

  if constexpr (RS == 1) {
    // Register-staged: each lane loads its 16-byte pieces of step kt+1 into registers while
    // step kt computes, then stores them (ds_write_b128, the same places the direct loads
    // fill) into the other stage; one barrier per step.
    static_assert(STAGES == 2, "two stages: compute one while the other is written");
    u32x4 stg[DMA_WAVE];
    auto load_regs = [&](int kt) {
#pragma unroll
      for (int i = 0; i < DMA_WAVE; ++i)
        stg[i] = *(const u32x4*)(src_base[i] + src_off[i] + k0 + kt * BK);
    };
    auto write_regs = [&](int st) {
      bf16_t* dst = smem + st * STAGE;
#pragma unroll
      for (int i = 0; i < DMA_WAVE; ++i)
        *(u32x4*)(dst + (wave * DMA_WAVE + i) * RPI * BK + lane * 8) = stg[i];
    };
    auto rs_loop = [&](auto nf_tag) {
      load_regs(0);
      write_regs(0);
      load_regs(KT > 1 ? 1 : 0);
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's stores are in LDS
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      for (int kt = 0; kt < KT; ++kt) {
        compute(smem + (kt & 1) * STAGE, nf_tag);
        write_regs((kt + 1) & 1);            // step kt+1 (past the end: a copy nobody reads)
        load_regs(kt + 2 < KT ? kt + 2 : KT - 1);
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // Row fragments of this wave that hold rows of the segment: a segment's last m-tile is
    // often mostly padding (Mixtral-shaped: 4 of 36 m-tiles hold 7-31 rows). The LDS reads and
    // MFMAs of the other fragments are skipped; the loads and barriers stay, so the tile keeps
    // the pace of the m-tiles that share its weight tiles in L2 (gate-up 1.88 -> 1.85 ms).
    static_assert(FM <= 2, "dispatch covers up to two row fragments per wave");
    const int live_rows = __builtin_amdgcn_readfirstlane(tc.rows - tc.m_local * BM - wm * TM);
    if (live_rows > 32 || (FM == 1 && live_rows > 0)) rs_loop(std::integral_constant<int, FM>{});
    else if (live_rows > 0) rs_loop(std::integral_constant<int, 1>{});
    else rs_loop(std::integral_constant<int, 0>{});
  } else {
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s) issue(s < KT ? s : KT - 1, s);
    for (int kt = 0; kt < KT; ++kt) {
      // this wave's loads of step kt are done once at most STAGES-2 steps remain in flight;
      // then one barrier makes every wave's part visible and retires step kt-1's buffer. (A
      // bare s_barrier: a release fence here would also drain the loads still in flight.)
      __builtin_amdgcn_s_waitcnt(wait_vm((STAGES - 2) * DMA_WAVE));
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      const int nxt = kt + STAGES - 1;
      issue(nxt < KT ? nxt : KT - 1, nxt % STAGES);
      compute(smem + (kt % STAGES) * STAGE, std::integral_constant<int, FM>{});
    }
  }
  __builtin_amdgcn_s_waitcnt(wait_vm(0));

  // ---- epilogue. 32x32 accumulator layout: lane holds column lane%32 and rows
  // 8*(r/4) + 4*(lane/32) + r%4 for r = 0..15.
  constexpr int FO = GATEUP ? FN / 2 : FN;   // output fragments along n
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FO; ++j) {
      const int col = tc.n0 + wn * (FEAT / WN) + j * 32 + fr;
      if (GATEUP && args.U && tc.m_local * BM + wm * TM + i * 32 < tc.rows) {
        const size_t o = uv_frag(tc.mt_global * BM + wm * TM + i * 32, col - fr, N, lane);
        uv_store(args.U + o, acc[i][j]);
        uv_store(args.V + o, acc[i][j + FN / 2]);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int lr = wm * TM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (GATEUP) {
          if (tc.m_local * BM + lr < tc.rows) {   // padding rows of H are never read
            const float u = acc[i][j][r];
            const float v = acc[i][j + FN / 2][r];
            args.H[(size_t)(tc.mt_global * BM + lr) * N + col] = f32_to_bf16(silu_f(u) * v);
          }
        } else {
          const int rg = tc.m_local * BM + lr;
          if (rg < tc.rows) {
            float* dst = shared_grp ? args.shared_out + (size_t)rg * N
                                    : (half ? args.out_rows_b : args.out_rows) +
                                          (size_t)(tc.off + rg) * N;
            dst[col] = acc[i][j][r];
          }
        }
      }
    }
}

// ------------------------------------------------------------------ wide class, four waves
// 256 x 256 tiles (gate-up: 128 features of W1 and of W3), four waves of 128 x 128, one wave
// per SIMD with its 16 accumulator fragments (256 registers) in the accumulation registers.
// Against eight waves of 64 x 128, a K step reads a third fewer LDS bytes (8 fragment reads
// per 16 MFMAs instead of 6 per 8).
// Both operands go through registers in two sets: set s holds the steps of parity s. During
// step kt, piece p of the set holding step kt+1 is written to LDS and then reloaded with step
// kt+3, so every load has about two steps to land before its write. The writes, the loads and
// the fragment reads of the next sub-step are interleaved with the MFMAs
// (sched_group_barrier): with one wave per SIMD, no other wave covers them.
// Each thread moves 16 pieces of 16 bytes per step: piece p is stage row p*32 + tid/8 (rows
// 0..255 A, 256..511 B), physical slot tid%8, so one wave's write of a piece is 1 KB contiguous
// and its load of a piece covers 8 whole 128-byte row segments. In a [rows][64] stage the
// swizzle of row r depends on (r/2)%8 only, so all 16 pieces of a thread fetch one logical chunk.
template <bool GATEUP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_w4_kernel(GemmArgs args) {
  constexpr int BM = 256, BNB = 256, BK = 64, WN = 2;
  constexpr int STAGE = (BM + BNB) * BK;            // bf16 elements per stage
  constexpr int FM = 4, FN = 4, NKS = BK / 16;
  constexpr int FEAT = GATEUP ? BNB / 2 : BNB;
  __shared__ __attribute__((aligned(1024))) bf16_t smem[2 * STAGE];

  const int S = GATEUP ? 1 : args.ksplit;
  TileCoord tc;
  int half = 0;
  if (!tile_coord(args.sc, args.N / FEAT, FEAT, tc, S, &half)) return;
  const bool shared_grp = tc.g >= args.E;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = args.K, N = args.N;
  const int KT = K / BK / S;
  const int k0 = half * KT * BK;

  const int prow = tid >> 3, slot = tid & 7;
  const int lchunk = slot ^ ((prow >> 1) & 7);
  // A pieces: gathered rows, byte offsets from x (gate-up) or h (down) in 32 bits (the launch
  // takes this kernel only when x and the padded h rows stay below 2 GiB). Padding rows (past
  // the segment's end) get an offset past the buffer's 2 GiB range, so their loads return zeros
  // without a memory access; their results are never stored.
  int sa[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int r = tc.m_local * BM + p * 32 + prow;
    sa[p] = GATEUP ? args.sorted_assign[tc.off + (!shared_grp && r < tc.rows ? r : 0)] : 0;
  }
  constexpr uint32_t kARange = 0x80000000u;
  uint32_t aoff[8];
  // (gate-up: computed in the prologue after the first steps' weight loads are out, since the
  // gathered rows' offsets wait for the ids above and the weights' do not: Mixtral-shaped
  // gate-up 1.801 -> 1.783 ms over three paired runs)
  auto make_aoff = [&]() {
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int r = tc.m_local * BM + p * 32 + prow;
      int srow;
      if (GATEUP) {
        const int tok = shared_grp ? r : sa[p] / args.k;
        srow = (unsigned)tok < (unsigned)args.T ? tok : 0;
      } else {
        srow = tc.mt_global * BM + p * 32 + prow;
      }
      aoff[p] = r < tc.rows ? ((uint32_t)srow * (uint32_t)K + lchunk * 8) * 2 : kARange;
    }
  };
  if (!GATEUP) make_aoff();
  // B pieces: weight rows n0 + q*32 + tid/8 (gate-up: W1 for q < 4, W3 for q >= 4; down: W2
  // rows n0 + q*32 + tid/8), one lane offset for all eight, the row block in the scalar offset
  const bf16_t* bm0;
  const bf16_t* bm1;
  if (GATEUP) {
    bm0 = shared_grp ? args.S0 : args.B0 + (size_t)tc.g * N * K;
    bm1 = shared_grp ? args.S1 : args.B1 + (size_t)tc.g * N * K;
  } else {
    bm0 = shared_grp ? args.S0 : args.B0 + (size_t)tc.g * N * K;
    bm1 = bm0 + (size_t)128 * K;
  }
  bm0 += (size_t)tc.n0 * K;
  bm1 += (size_t)tc.n0 * K;
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc((void*)args.A, (short)0, (int)kARange, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb0 = __builtin_amdgcn_make_buffer_rsrc((void*)bm0, (short)0, -1, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb1 = __builtin_amdgcn_make_buffer_rsrc((void*)bm1, (short)0, -1, 0x00020000);
  const uint32_t boff = ((uint32_t)prow * (uint32_t)K + lchunk * 8) * 2;

  auto gload = [&](u32x4* st, int p, int kt) {
    const int kb = (k0 + kt * BK) * 2;
    if (p < 8) {
      st[p] = __builtin_amdgcn_raw_buffer_load_b128(ra, aoff[p], kb, 0);
    } else {
      const int q = p - 8;
      st[p] = __builtin_amdgcn_raw_buffer_load_b128(q < 4 ? rb0 : rb1, boff, (q & 3) * 64 * K + kb, 0);
    }
  };
  // LDS (bytes): A of stage s at s*32K, B of stage s at 64K + s*32K, each [256 rows][128 B]
  // swizzled; piece p of this thread lands at tid*16 + (p%8)*4K in its matrix's region, so
  // every LDS access below is one of a few base registers plus an immediate offset.
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
  typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
  typedef __attribute__((address_space(3))) char lds_char;
  lds_char* const lds = (lds_char*)smem;
  constexpr int ASTG = 32768, BREG = 65536;
  auto lwrite = [&](const u32x4* st, int p, int stg) {
    *(lds_u32x4*)(lds + (p < 8 ? 0 : BREG) + stg * ASTG + (p & 7) * 4096 + tid * 16) = st[p];
  };

  const int wm = wave / WN, wn = wave % WN;
  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int fr = lane & 31, fkc = lane >> 5;
  // Fragment rows are (multiples of 32) + lane%32, so all of this lane's fragments share one
  // swizzle, ((lane%32)/2)%8: per sub-step one A and one B base register serve the eight reads.
  bf16x8 af[2][FM], bfr[2][FN];
  const int sx = (fr >> 1) & 7;
  const int bw = GATEUP ? wn * 64 : wn * 128;   // first B row of this wave
  uint32_t rdA[NKS], rdB[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const int c = ((2 * ks + fkc) ^ sx) << 4;
    rdA[ks] = (wm * 128 + fr) * BK * 2 + c;
    rdB[ks] = BREG + (bw + fr) * BK * 2 + c;
  }
  auto fread = [&](int buf, int stg, int ks) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
      af[buf][i] = *(const lds_bf16x8*)(lds + rdA[ks] + stg * ASTG + i * 32 * BK * 2);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int rb = GATEUP ? (j < FN / 2 ? 0 : BNB / 2) + (j % (FN / 2)) * 32 : j * 32;
      bfr[buf][j] = *(const lds_bf16x8*)(lds + rdB[ks] + stg * ASTG + rb * BK * 2);
    }
  };
  // Gate-up: the weights are the MFMA's first operand, so each accumulator holds a transposed
  // 32 x 32 block: lane l has row (token) l%32 of fragment i and, at r = 0..15, feature
  // 8*(r/4) + 4*(l/32) + r%4 of fragment j, and the epilogue stores four consecutive h values
  // (8 bytes) at a time. Down: the usual layout (lane l has feature l%32 and rows
  // 8*(r/4) + 4*(l/32) + r%4), so each fp32 store instruction writes two whole 128-byte row
  // segments (transposed, 16-byte pieces of 32 rows: down 0.92 -> 0.94 ms).
  auto mfma = [&](int buf, int m) {
    const int i = m >> 2, j = m & 3;
    acc[i][j] = GATEUP
        ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[buf][j], af[buf][i], acc[i][j], 0, 0, 0)
        : __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[buf][i], bfr[buf][j], acc[i][j], 0, 0, 0);
  };

  // pieces written (and reloaded) in sub-step ks: [PW[ks], PW[ks+1]); MFMAs of the last sub-step
  // issued before the barrier that publishes the next stage: PRE (the rest cover the first
  // fragment reads of the next step). Measured on the Mixtral-shaped layer against reading the
  // fragments first in each sub-step, and against 4 or 8 MFMAs before the barrier.
  constexpr int PW[NKS + 1] = {0, 4, 8, 12, 16};
  constexpr int PRE = 12;
  u32x4 st0[16], st1[16];
  // one K step: MFMAs of step kt from stage kt&1 over the first NF row fragments of this wave;
  // the set W (step kt+1) goes to the other stage and is reloaded with step kt+3 (past the
  // end: the last step again, never read)
  auto step = [&](auto cs_tag, auto nf_tag, int kt, u32x4* W) {
    constexpr int cs = decltype(cs_tag)::value, ns = cs ^ 1;
    constexpr int NF = decltype(nf_tag)::value;
    constexpr int NM = NF * FN, NR = NF ? NF + FN : 0;
    const int rl = kt + 3 < KT ? kt + 3 : KT - 1;
    auto fread_nf = [&](int buf, int stg, int ks) {
      if constexpr (NF > 0) {
#pragma unroll
        for (int i = 0; i < NF; ++i)
          af[buf][i] = *(const lds_bf16x8*)(lds + rdA[ks] + stg * ASTG + i * 32 * BK * 2);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int rb = GATEUP ? (j < FN / 2 ? 0 : BNB / 2) + (j % (FN / 2)) * 32 : j * 32;
          bfr[buf][j] = *(const lds_bf16x8*)(lds + rdB[ks] + stg * ASTG + rb * BK * 2);
        }
      }
    };
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < NKS) fread_nf(cur ^ 1, cs, ks + 1);
#pragma unroll
      for (int p = PW[ks]; p < PW[ks + 1]; ++p) {
        lwrite(W, p, ns);
        gload(W, p, rl);
      }
      const int nm = ks + 1 < NKS ? NM : (PRE < NM ? PRE : NM);
#pragma unroll
      for (int m = 0; m < nm; ++m) mfma(cur, m);
      const int nr = ks + 1 < NKS ? NR : 0, np = PW[ks + 1] - PW[ks];
      // per 4 MFMAs: 2 fragment reads, then 1 LDS write and 1 load
      for (int r = 0; r < 16; ++r) {
        if (r < nm) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (r < nr) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if ((r & 3) == 1 && r / 4 < np) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
        if ((r & 3) == 3 && r / 4 < np) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // the barrier that publishes the next stage, then its first fragment reads under the
    // remaining MFMAs of the last sub-step
    constexpr int cur = (NKS - 1) & 1;
    constexpr int pre = PRE < NM ? PRE : NM;
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's writes are in LDS
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    fread_nf(cur ^ 1, ns, 0);
#pragma unroll
    for (int m = pre; m < NM; ++m) mfma(cur, m);
    for (int r = 0; r < NR; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (r + pre < NM) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  auto main_loop = [&](auto nf_tag) {
    // prologue: steps 0 and 1 loaded (gate-up: the weight pieces first), step 0 written, set 0
    // reloaded with step 2
    if constexpr (GATEUP) {
#pragma unroll
      for (int p = 8; p < 16; ++p) gload(st0, p, 0);
#pragma unroll
      for (int p = 8; p < 16; ++p) gload(st1, p, KT > 1 ? 1 : 0);
      __builtin_amdgcn_sched_barrier(0);
      make_aoff();
#pragma unroll
      for (int p = 0; p < 8; ++p) gload(st0, p, 0);
#pragma unroll
      for (int p = 0; p < 8; ++p) gload(st1, p, KT > 1 ? 1 : 0);
    } else {
#pragma unroll
      for (int p = 0; p < 16; ++p) gload(st0, p, 0);
#pragma unroll
      for (int p = 0; p < 16; ++p) gload(st1, p, KT > 1 ? 1 : 0);
    }
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      lwrite(st0, p, 0);
      gload(st0, p, KT > 2 ? 2 : KT - 1);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    constexpr int NF = decltype(nf_tag)::value;
    if constexpr (NF > 0) fread(0, 0, 0);
    // NKS = 4 sub-steps: a step starts and ends with its fragments in buffer 0. KT is even (the
    // launch checks it), so the loop body is two whole steps.
    static_assert(NKS % 2 == 0, "fragment buffers alternate within a step");
    for (int kt = 0; kt < KT; kt += 2) {
      step(std::integral_constant<int, 0>{}, nf_tag, kt, st1);
      step(std::integral_constant<int, 1>{}, nf_tag, kt + 1, st0);
    }
  };
  // Row fragments of this wave that hold rows of the segment: a segment's last m-tile is often
  // mostly padding. The LDS reads and MFMAs of the other fragments are skipped; the loads and
  // barriers stay, so the tile keeps the pace of the m-tiles that share its weight tiles in L2.
  const int live_rows = __builtin_amdgcn_readfirstlane(tc.rows - tc.m_local * BM - wm * 128);
  if (live_rows > 32) main_loop(std::integral_constant<int, FM>{});
  else if (live_rows > 0) main_loop(std::integral_constant<int, 1>{});
  else main_loop(std::integral_constant<int, 0>{});
  __builtin_amdgcn_s_waitcnt(wait_vm(0));

  // ---- epilogue: h = SiLU(u) * v as bf16 (round to nearest even), or the fp32 rows
  constexpr int FO = GATEUP ? FN / 2 : FN;
  if constexpr (GATEUP) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int lr = wm * 128 + i * 32 + fr;   // this lane's row of the tile
      if (tc.m_local * BM + lr >= tc.rows) continue;   // padding rows are never stored
#pragma unroll
      for (int j = 0; j < FO; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = tc.n0 + wn * (FEAT / WN) + j * 32 + 8 * q + 4 * (lane >> 5);
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          bf16x4 h;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            h[e] = (__bf16)(silu_f(acc[i][j][4 * q + e]) * acc[i][j + FN / 2][4 * q + e]);
          *(bf16x4*)(args.H + (size_t)(tc.mt_global * BM + lr) * N + col) = h;
        }
    }
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FO; ++j) {
        const int col = tc.n0 + wn * (FEAT / WN) + j * 32 + fr;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rg = tc.m_local * BM + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (rg < tc.rows) {
            float* dst = shared_grp ? args.shared_out + (size_t)rg * N
                                    : (half ? args.out_rows_b : args.out_rows) + (size_t)(tc.off + rg) * N;
            dst[col] = acc[i][j][r];
          }
        }
      }
  }
}

// ------------------------------------------------------------------ staggered rings
// The ragged classes: each weight tile streams from HBM for about one m-tile, so the weights
// (B) need more latency tolerance than a 2-stage ring gives, and a third full stage does not
// fit in 160 KB of LDS. Both operands go straight to LDS, in two rings of different depth: the
// gathered rows (A, "shallow") in 2 slots, issued one step ahead, and the weights (B, "deep")
// in 3 slots, issued two steps ahead.
//   step kt: wait until only this wave's B loads issued in step kt-1 are outstanding (so the A
//            loads of step kt, issued before them, and the B loads of step kt, issued earlier,
//            have landed); barrier; issue A(kt+1) and then B(kt+2); MFMAs of step kt.
// Vector-memory loads retire in order, so issuing A first is what lets the wait leave the B
// loads in flight; the same ordering is why a deeper ring would not help: every wait retires
// all loads issued before that step's A loads. Every slot written in step kt was last read in
// step kt-1, which all waves finished before this step's barrier.
// NTR (down only): the fp32 rows go out with the non-temporal hint
template <int BM, int BNB, int WM, int WN, bool GATEUP, bool NTR = false, bool TR = GATEUP>
__global__ __launch_bounds__(WM * WN * 64) void gemm_bf16_st_kernel(GemmArgs args) {
  constexpr int BK = 64, NKS = BK / 16;
  constexpr int NW = WM * WN;
  constexpr int CHUNKS = BK / 8, RPI = 64 / CHUNKS;
  constexpr int TM = BM / WM, TNB = BNB / WN;
  constexpr int FM = TM / 32, FN = TNB / 32;
  constexpr int ASLOT = BM * BK, BSLOT = BNB * BK;   // bf16 elements
  constexpr int DMA_A = BM * CHUNKS / 64 / NW;       // 1 KB A loads per wave per step
  constexpr int DMA_B = BNB * CHUNKS / 64 / NW;      // 1 KB B loads per wave per step
  static_assert(DMA_A * 64 * NW == BM * CHUNKS && DMA_B * 64 * NW == BNB * CHUNKS, "even split");
  constexpr int FEAT = GATEUP ? BNB / 2 : BNB;
  static_assert(!GATEUP || FN % 2 == 0, "u and v fragments pair up");
  static_assert((BNB / 2) % RPI == 0, "a B row group stays within one matrix");
  constexpr int DS = 3;                                     // slots of the deep ring
  constexpr int NA = 2, NB = DS;                            // ring slots of A and B
  static_assert((NA * ASLOT + NB * BSLOT) * 2 <= 160 * 1024, "rings fit in LDS");
  __shared__ __attribute__((aligned(1024))) bf16_t smem[NA * ASLOT + NB * BSLOT];
  bf16_t* const As = smem;
  bf16_t* const Bs = smem + NA * ASLOT;

  // with the K range split in two (down GEMM only), work unit = (half, tile): half h runs
  // steps [h*KT/2, (h+1)*KT/2) and writes its partial rows to its own buffer
  const int S = GATEUP ? 1 : args.ksplit;
  TileCoord tc;
  int half = 0;
  if (!tile_coord(args.sc, args.N / FEAT, FEAT, tc, S, &half)) return;
  const bool shared_grp = tc.g >= args.E;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = args.K, N = args.N;
  const int KT = K / BK / S;                          // steps of this work unit
  const int k0 = half * KT * BK;                      // its first K element

  // A load i of this wave fills slot rows q*RPI.. (q = wave*DMA_A + i): lane l writes physical
  // 16-byte chunk l%CHUNKS of row q*RPI + l/CHUNKS and so fetches the logical chunk that the
  // swizzle puts there (the swizzle is an involution).
  // (32-bit element offsets from the matrix base keep the register count down; the entry
  // points reject every shape whose x, expert matrices or padded h rows reach 2^32 elements)
  // (the assignment ids of the gathered rows are loaded together, before the first wait)
  int sa[DMA_A];
#pragma unroll
  for (int i = 0; i < DMA_A; ++i) {
    const int r = tc.m_local * BM + (wave * DMA_A + i) * RPI + lane / CHUNKS;
    sa[i] = GATEUP ? args.sorted_assign[tc.off + (!shared_grp && r < tc.rows ? r : 0)] : 0;
  }
  uint32_t aoff[DMA_A];
#pragma unroll
  for (int i = 0; i < DMA_A; ++i) {
    const int q = wave * DMA_A + i;
    const int row = q * RPI + lane / CHUNKS;
    const int lchunk = (swz<BK>(row, lane % CHUNKS) - row * BK) >> 3;
    int srow;
    if (GATEUP) {
      const int r = tc.m_local * BM + row;
      const int rr = r < tc.rows ? r : 0;             // padding rows repeat the first row
      const int tok = shared_grp ? rr : sa[i] / args.k;
      srow = (unsigned)tok < (unsigned)args.T ? tok : 0;
    } else {
      srow = tc.mt_global * BM + row;
    }
    aoff[i] = (uint32_t)srow * (uint32_t)K + lchunk * 8;
  }
  // B load i of this wave fills B slot rows q*RPI.. (q = wave*DMA_B + i) the same way; the
  // rows of one load lie in one matrix, so its base is wave-uniform.
  const bf16_t* bmat[DMA_B];
  uint32_t boff[DMA_B];
#pragma unroll
  for (int i = 0; i < DMA_B; ++i) {
    const int q = wave * DMA_B + i;
    const int br = q * RPI + lane / CHUNKS;
    const int lchunk = (swz<BK>(br, lane % CHUNKS) - br * BK) >> 3;
    const bool second = GATEUP && q * RPI >= BNB / 2;
    const bf16_t* mat;
    if (GATEUP)
      mat = shared_grp ? (second ? args.S1 : args.S0)
                       : (second ? args.B1 : args.B0) + (size_t)tc.g * N * K;
    else
      mat = shared_grp ? args.S0 : args.B0 + (size_t)tc.g * N * K;
    bmat[i] = mat;
    boff[i] = (uint32_t)(tc.n0 + (second ? br - BNB / 2 : br)) * (uint32_t)K + lchunk * 8;
  }

  // Rows of this tile that hold data (the last tile of a segment is ragged). With A as the
  // shallow operand, A row groups past them are not loaded at all: the step's wait leaves only
  // the deep B loads of later steps in flight, whatever number of A loads was issued before
  // them. Their LDS rows keep stale bits, which reach only padding rows of the results.
  const int rows_here = __builtin_amdgcn_readfirstlane(min(BM, tc.rows - tc.m_local * BM));
  auto issue_a = [&](int kt, int slot) {
    bf16_t* dst = As + slot * ASLOT;
#pragma unroll
    for (int i = 0; i < DMA_A; ++i) {
      if ((wave * DMA_A + i) * RPI >= rows_here) continue;   // wave-uniform
      __builtin_amdgcn_global_load_lds((const void*)(args.A + aoff[i] + k0 + kt * BK),
                                       (lds_ptr_t)(dst + (wave * DMA_A + i) * RPI * BK), 16, 0, 0);
    }
  };
  // A weight tile that only one m-tile of its group reads is streamed from HBM once: it goes in
  // with the non-temporal hint, so it does not push out of L2 the lines that are reused -- the
  // gathered x rows, shared by the expert's n-tiles, and the weight tiles of groups with several
  // m-tiles (a capped expert, the shared expert), shared by those m-tiles. DeepSeek-V3-shaped
  // gate-up 3.41 -> 3.08 ms and down 1.93 -> 1.82 ms; skewed gate-up 0.45 -> 0.42 ms. (The hint on
  // every weight tile: gate-up 3.21 ms.)
  const bool b_stream = tc.mtg == 1;   // uniform
  auto issue_b = [&](int kt, int slot) {
    bf16_t* dst = Bs + slot * BSLOT;
    if (b_stream) {
#pragma unroll
      for (int i = 0; i < DMA_B; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(bmat[i] + boff[i] + k0 + kt * BK),
                                         (lds_ptr_t)(dst + (wave * DMA_B + i) * RPI * BK), 16, 0,
                                         2 /* nt */);
    } else {
#pragma unroll
      for (int i = 0; i < DMA_B; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(bmat[i] + boff[i] + k0 + kt * BK),
                                         (lds_ptr_t)(dst + (wave * DMA_B + i) * RPI * BK), 16, 0,
                                         0);
    }
  };

  const int wm = wave / WN, wn = wave % WN;
  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Row fragments are dealt to the waves interleaved: fragment i of wave row wm covers tile
  // rows (i*WM + wm)*32 .. +32, so the fragments of a ragged tile that hold data are spread
  // over all wave rows (and SIMDs) rather than piled on the first ones.
  // Fragment reads. Lane l reads row (block base + l%32) at 16-byte chunk 2*ks + l/32. Every
  // fragment block starts at a multiple of 16 rows, so a lane's swizzle key ((row/2) % 8) is the
  // same for all its rows: the address is one per-lane offset per sub-step plus a
  // compile-time offset per fragment.
  static_assert(BK == 64 && TM % 32 == 0 && (GATEUP ? BNB / 2 / WN : TNB) % 32 == 0,
                "fragment row blocks start at multiples of 32 rows");
  const int fr = lane & 31, fkc = lane >> 5;
  const int sw = (fr >> 1) & (CHUNKS - 1);
  const int fw = GATEUP ? BNB / 2 / WN : TNB;        // B rows per wave and matrix half
  int aoffs[NKS], boffs[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const int ch = ((2 * ks + fkc) ^ sw) << 3;
    aoffs[ks] = (wm * 32 + fr) * BK + ch;
    boffs[ks] = (wn * fw + fr) * BK + ch;
  }
  auto bconst = [](int j) {   // compile-time B row of fragment j relative to the wave's rows
    return GATEUP ? (j < FN / 2 ? 0 : BNB / 2) + (j % (FN / 2)) * 32 : j * 32;
  };

  // prologue: shallow(0), deep(0), deep(1)
  auto issue_shallow = [&](int kt) { issue_a(kt, kt & 1); };
  auto issue_deep = [&](int kt) { issue_b(kt, kt % DS); };
  constexpr int DEEP_OPS = DMA_B;
  // The K loop for a wave whose first NF row fragments hold data: the others are all padding
  // rows, so their LDS reads and MFMAs are skipped (NF = 0: the wave only loads and waits).
  auto k_loop = [&](auto nf_tag) {
    constexpr int NF = decltype(nf_tag)::value;
    issue_shallow(0);
#pragma unroll
    for (int s = 0; s < DS - 1; ++s) issue_deep(s < KT ? s : KT - 1);
    for (int kt = 0; kt < KT; ++kt) {
      __builtin_amdgcn_s_waitcnt(wait_vm(DEEP_OPS));
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      issue_shallow(kt + 1 < KT ? kt + 1 : KT - 1);
      issue_deep(kt + DS - 1 < KT ? kt + DS - 1 : KT - 1);
      if (NF == 0) continue;
      const bf16_t* a = As + (kt % NA) * ASLOT;
      const bf16_t* b = Bs + (kt % NB) * BSLOT;
      __builtin_amdgcn_iglp_opt(1);
      bf16x8 af[2][FM], bfr[2][FN];
#pragma unroll
      for (int i = 0; i < NF; ++i) af[0][i] = *(const bf16x8*)&a[aoffs[0] + i * WM * 32 * BK];
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[0][j] = *(const bf16x8*)&b[boffs[0] + bconst(j) * BK];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int cur = ks & 1, nxt = cur ^ 1;
        if (ks + 1 < NKS) {
#pragma unroll
          for (int i = 0; i < NF; ++i)
            af[nxt][i] = *(const bf16x8*)&a[aoffs[ks + 1] + i * WM * 32 * BK];
#pragma unroll
          for (int j = 0; j < FN; ++j)
            bfr[nxt][j] = *(const bf16x8*)&b[boffs[ks + 1] + bconst(j) * BK];
        }
#pragma unroll
        for (int i = 0; i < NF; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = TR ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[cur][j], af[cur][i],
                                                                     acc[i][j], 0, 0, 0)
                           : __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][i], bfr[cur][j],
                                                                     acc[i][j], 0, 0, 0);
      }
    }
  };
  static_assert(FM <= 3, "the K-loop dispatch covers up to three row fragments per wave");
  const int nf = min(FM, max(0, (rows_here - wm * 32 + WM * 32 - 1) / (WM * 32)));
  if (nf >= FM) k_loop(std::integral_constant<int, FM>{});
  else if (nf == 2) k_loop(std::integral_constant<int, (FM > 2 ? 2 : 0)>{});
  else if (nf == 1) k_loop(std::integral_constant<int, (FM > 1 ? 1 : 0)>{});
  else k_loop(std::integral_constant<int, 0>{});
  __builtin_amdgcn_s_waitcnt(wait_vm(0));

  // ---- epilogue
  constexpr int FO = GATEUP ? FN / 2 : FN;
  if constexpr (TR) {
    // TR: the weights were the MFMA's first operand, so lane l holds row (token) l%32 of row
    // fragment i and, at r = 0..15, feature 8*(r/4) + 4*(l/32) + r%4 of fragment j: four
    // consecutive features go out as one 8-byte (h) or 16-byte (fp32 row) store. (Not used for
    // the fp32 rows: 16-byte pieces of 32 rows per instruction, instead of two whole 128-byte
    // row segments, made the DeepSeek-V3-shaped down GEMM 1.77 -> 1.90 ms.)
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int lr = (i * WM + wm) * 32 + fr;
      if (lr >= rows_here) continue;   // padding rows of H feed only padding rows of the down
      const int rg = tc.m_local * BM + lr;
#pragma unroll
      for (int j = 0; j < FO; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = tc.n0 + wn * (FEAT / WN) + j * 32 + 8 * q + 4 * (lane >> 5);
          if (GATEUP) {
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            bf16x4 h;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              h[e] = (__bf16)(silu_f(acc[i][j][4 * q + e]) * acc[i][j + FN / 2][4 * q + e]);
            *(bf16x4*)(args.H + (size_t)(tc.mt_global * BM + lr) * N + col) = h;
          } else {
            float* dst = shared_grp ? args.shared_out + (size_t)rg * N
                                    : (half ? args.out_rows_b : args.out_rows) + (size_t)(tc.off + rg) * N;
            const f32x4 o{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                          acc[i][j][4 * q + 3]};
            if (NTR) __builtin_nontemporal_store(o, (f32x4*)(dst + col));
            else *(f32x4*)(dst + col) = o;
          }
        }
    }
    return;
  }
  // !TR (the backward's gate-up recompute, which also stores u and v in this layout): lane l
  // holds column l%32 and rows 8*(r/4) + 4*(l/32) + r%4, as in gemm_bf16_kernel
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FO; ++j) {
      const int col = tc.n0 + wn * (FEAT / WN) + j * 32 + fr;
      if (GATEUP && args.U && (i * WM + wm) * 32 < rows_here) {
        const size_t o = uv_frag(tc.mt_global * BM + (i * WM + wm) * 32, col - fr, N, lane);
        uv_store(args.U + o, acc[i][j]);
        uv_store(args.V + o, acc[i][j + FN / 2]);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int lr = (i * WM + wm) * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (GATEUP) {
          if (lr < rows_here) {          // padding rows of H feed only padding rows of the down
            const float u = acc[i][j][r];
            const float v = acc[i][j + FN / 2][r];
            args.H[(size_t)(tc.mt_global * BM + lr) * N + col] = f32_to_bf16(silu_f(u) * v);
          }
        } else {
          const int rg = tc.m_local * BM + lr;
          if (rg < tc.rows) {
            float* dst = shared_grp ? args.shared_out + (size_t)rg * N
                                    : (half ? args.out_rows_b : args.out_rows) +
                                          (size_t)(tc.off + rg) * N;
            if (NTR) __builtin_nontemporal_store(acc[i][j][r], dst + col);
            else dst[col] = acc[i][j][r];
          }
        }
      }
    }
}

// ------------------------------------------------------------------ decode class
// With a few rows per expert the layer streams each touched expert's weights once, and its
// pace is set by HBM latency times the bytes in flight, not by MFMA work. A workgroup takes
// one m-tile of up to 32 rows (a second 16-row fragment only when it holds rows) and 32
// (gate-up) or 64 (down) output features. Its four waves split K in four: each wave streams
// its quarter of the tile's weight rows (and the A rows) straight into registers, several
// steps of 64 ahead, with no LDS ring and no barrier, and accumulates its own partial sums
// with v_mfma_f32_16x16x32_bf16. The four partials are added through LDS in wave order
// (deterministic), then the SwiGLU (gate-up) or the fp32 store (down) follows.
// MFMA 16x16x32 operands: lane l holds row (A) or column (B) l%16 and k = 8*(l/16) .. +7 of
// the 32-wide block, so one 16-byte load per lane reads 16 rows x 64 contiguous bytes. The
// result: lane l holds column l%16, rows 4*(l/16) .. +3.
// KTW, the steps per wave (K / 256), is a template argument: the K loop is unrolled whole, so
// the ring slots and the last loads are fixed at compile time and the compiler's vmcnt waits
// are exact (with a rolled loop it drained every load at the loop head).
constexpr int kDecMaxSteps = 8;
// output features per workgroup: gate-up 32 (16-row blocks W1, W1, W3, W3), down 64
constexpr int dec_feat(bool gateup) { return gateup ? 32 : 64; }
// steps in flight: as many as about 200 VGPRs of operands hold (40 per step with one A
// fragment, 48 with two)
constexpr int dec_depth(int nf, int steps) {
  const int d = nf == 1 ? 5 : 4;
  return d < steps ? d : steps;
}

template <bool GATEUP, int KTW>
__global__ __launch_bounds__(256) void gemm_bf16_dec_kernel(GemmArgs args) {
  constexpr int NBLK = 4;                    // 16-row B blocks: gate-up W1, W1, W3, W3; down W2
  constexpr int FEAT = dec_feat(GATEUP);
  constexpr int RS = NBLK * 16 + 4;          // padded fp32 row of a wave's partial sums in LDS
  __shared__ float red[4][kDecBM * RS];

  // tiles in identity order: the tile is known one round trip after the start (each tile
  // streams its own weight rows, so the XCD-contiguous walk buys little here)
  TileCoord tc;
  if (!tile_coord<true>(args.sc, args.N / FEAT, FEAT, tc)) return;
  const bool shared_grp = tc.g >= args.E;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = args.K, N = args.N;          // K == KTW * 256 (checked by the launcher)
  const int rows_here = __builtin_amdgcn_readfirstlane(min(kDecBM, tc.rows - tc.m_local * kDecBM));
  const int r16 = lane & 15, kq = lane >> 4;
  const int kbase = wave * (KTW * 64) + kq * 8;   // this wave's K range starts at wave*K/4

  const bf16_t* bp[NBLK];
#pragma unroll
  for (int b = 0; b < NBLK; ++b) {
    const bool second = GATEUP && b >= 2;
    const bf16_t* mat;
    if (GATEUP)
      mat = shared_grp ? (second ? args.S1 : args.S0)
                       : (second ? args.B1 : args.B0) + (size_t)tc.g * N * K;
    else
      mat = shared_grp ? args.S0 : args.B0 + (size_t)tc.g * N * K;
    const int row = tc.n0 + (GATEUP ? (b & 1) : b) * 16 + r16;
    bp[b] = mat + (size_t)row * K + kbase;
  }
  // (the assignment ids of the gathered rows are loaded together, before the first wait)
  int sa[kDecBM / 16];
#pragma unroll
  for (int f = 0; f < kDecBM / 16; ++f) {
    const int r = tc.m_local * kDecBM + f * 16 + r16;
    sa[f] = GATEUP ? args.sorted_assign[tc.off + (!shared_grp && r < tc.rows ? r : 0)] : 0;
  }
  const bf16_t* ap[kDecBM / 16];
  auto make_ap = [&]() {
#pragma unroll
    for (int f = 0; f < kDecBM / 16; ++f) {
      int srow;
      if (GATEUP) {
        const int r = tc.m_local * kDecBM + f * 16 + r16;
        const int rr = r < tc.rows ? r : 0;             // padding rows repeat the first row
        const int tok = shared_grp ? rr : sa[f] / args.k;
        srow = (unsigned)tok < (unsigned)args.T ? tok : 0;
      } else {
        srow = tc.mt_global * kDecBM + f * 16 + r16;     // padding rows: results not stored
      }
      ap[f] = args.A + (size_t)srow * K + kbase;
    }
  };
  if (GATEUP) make_ap();

  auto run = [&](auto nf_tag) {
    constexpr int NF = decltype(nf_tag)::value;
    constexpr int D = dec_depth(NF, KTW);
    f32x4 acc[NF][NBLK];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int b = 0; b < NBLK; ++b) acc[f][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    // A and B of a step are issued together, D steps ahead: vector-memory loads retire in
    // order, so an A load issued after a later step's B loads would make its wait cover them.
    // The down GEMM issues its first D steps as all weights, then all h rows: decode T = 128
    // down 83 -> 78 us, T = 32 67.5 -> 64.5 us. (The same for the gate-up, with its row addresses computed after the
    // weight loads went out, made it slower: T = 1 13.5 -> 15.1 us, T = 128 139 -> 150 us.)
    bf16x8 bq[D][NBLK][2], aq[D][NF][2];
    auto load_b = [&](int d, int kt) {
#pragma unroll
      for (int b = 0; b < NBLK; ++b)
#pragma unroll
        for (int s = 0; s < 2; ++s) bq[d][b][s] = *(const bf16x8*)(bp[b] + kt * 64 + s * 32);
    };
    auto load_a = [&](int d, int kt) {
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int s = 0; s < 2; ++s) aq[d][f][s] = *(const bf16x8*)(ap[f] + kt * 64 + s * 32);
    };
    auto load = [&](int d, int kt) {
      load_b(d, kt);
      load_a(d, kt);
    };
    if constexpr (GATEUP) {
#pragma unroll
      for (int d = 0; d < D; ++d) load(d, d);
    } else {
#pragma unroll
      for (int d = 0; d < D; ++d) load_b(d, d);
      __builtin_amdgcn_sched_barrier(0);
      make_ap();
#pragma unroll
      for (int d = 0; d < D; ++d) load_a(d, d);
    }
#pragma unroll
    for (int kt = 0; kt < KTW; ++kt) {
      const int d = kt % D;
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
          for (int b = 0; b < NBLK; ++b)
            acc[f][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[d][f][s], bq[d][b][s], acc[f][b],
                                                                0, 0, 0);
      if (kt + D < KTW) load(d, kt + D);
      __builtin_amdgcn_sched_barrier(0);
    }
    float* my = red[wave];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int b = 0; b < NBLK; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) my[(f * 16 + 4 * kq + i) * RS + b * 16 + r16] = acc[f][b][i];
  };
  static_assert(kDecBM == 32, "one or two 16-row fragments");
  if (rows_here > 16) run(std::integral_constant<int, 2>{});
  else run(std::integral_constant<int, 1>{});
  __syncthreads();

  // the four partials, added in wave order; thread t takes output feature t%FEAT of rows
  // t/FEAT + (256/FEAT)*i
  const int col = tid % FEAT;
  for (int row = tid / FEAT; row < rows_here; row += 256 / FEAT) {
    const float* r0 = &red[0][row * RS];
    if (GATEUP) {
      float u = r0[col], v = r0[32 + col];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        u += red[w][row * RS + col];
        v += red[w][row * RS + 32 + col];
      }
      const int srow = tc.mt_global * kDecBM + row;
      args.H[(size_t)srow * N + tc.n0 + col] = f32_to_bf16(silu_f(u) * v);
      if (args.U) {
        const size_t o = uv_elem(srow, tc.n0 + col, N);
        args.U[o] = u;
        args.V[o] = v;
      }
    } else {
      float y = r0[col];
#pragma unroll
      for (int w = 1; w < 4; ++w) y += red[w][row * RS + col];
      const int rg = tc.m_local * kDecBM + row;
      float* dst = shared_grp ? args.shared_out + (size_t)rg * N
                              : args.out_rows + (size_t)(tc.off + rg) * N;
      dst[tc.n0 + col] = y;
    }
  }
}

// ------------------------------------------------------------------ fp32 path (VALU)
constexpr int BM32 = kGemmBM32, BN32 = 64, BK32 = 32;

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
  constexpr int RM = BM32 / 16;   // rows per thread (16 x 16 threads over BM32 x 64)
  float acc[NB][RM][4] = {};
  __syncthreads();
  // This thread's elements of one K chunk, loaded into registers one chunk ahead (the loads of
  // chunk k0 + BK32 are in flight while chunk k0 is multiplied), then stored to LDS.
  constexpr int LA = BM32 * BK32 / 256, LB = BN32 * BK32 / 256;
  static_assert(LA * 256 == BM32 * BK32 && LB * 256 == BN32 * BK32, "even split");
  float ra[LA], rb[NB][LB];
  auto load = [&](int k0) {
#pragma unroll
    for (int u = 0; u < LA; ++u) {
      const int idx = tid + 256 * u, r = idx / BK32, kk = idx % BK32;
      const int t = tok[r];
      ra[u] = (t >= 0 && k0 + kk < K) ? args.A[(size_t)t * K + k0 + kk] : 0.f;
    }
#pragma unroll
    for (int q = 0; q < NB; ++q)
#pragma unroll
      for (int u = 0; u < LB; ++u) {
        const int idx = tid + 256 * u, c = idx / BK32, kk = idx % BK32;
        const int n = tc.n0 + c;
        rb[q][u] = (n < N && k0 + kk < K) ? Bb[q][(size_t)n * K + k0 + kk] : 0.f;
      }
  };
  load(0);
  for (int k0 = 0; k0 < K; k0 += BK32) {
#pragma unroll
    for (int u = 0; u < LA; ++u) {
      const int idx = tid + 256 * u;
      As[idx % BK32][idx / BK32] = ra[u];
    }
#pragma unroll
    for (int q = 0; q < NB; ++q)
#pragma unroll
      for (int u = 0; u < LB; ++u) {
        const int idx = tid + 256 * u;
        Bs[q][idx % BK32][idx / BK32] = rb[q][u];
      }
    __syncthreads();
    if (k0 + BK32 < K) load(k0 + BK32);
#pragma unroll 8
    for (int kk = 0; kk < BK32; ++kk) {
      float a[RM], b[NB][4];
      for (int i = 0; i < RM; ++i) a[i] = As[kk][ty * RM + i];
      for (int q = 0; q < NB; ++q)
        for (int j = 0; j < 4; ++j) b[q][j] = Bs[q][kk][tx * 4 + j];
      for (int q = 0; q < NB; ++q)
        for (int i = 0; i < RM; ++i)
          for (int j = 0; j < 4; ++j) acc[q][i][j] = fmaf(a[i], b[q][j], acc[q][i][j]);
    }
    __syncthreads();
  }
  for (int i = 0; i < RM; ++i) {
    const int lr = ty * RM + i;
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

}  // namespace

int grid_for(int mtiles, int nt, int xcd_chunk) {
  const long long g = (long long)mtiles * nt, q = xcd_chunk ? 8 * kXcdChunk : 8;
  return (int)((g + q - 1) / q * q);
}

// expected kept rows per expert: T*k/E, or the capacity if that is smaller
static double expected_rows(const moe_problem& p) {
  double rows = (double)p.T * p.k / p.E;
  if (p.capacity_factor > 0) rows = std::min(rows, std::ceil(p.capacity_factor * rows));
  return rows;
}

// Row-tile classes between the small and the wide one (bf16, d % 256 == 0). All use ragged
// tiles (the staggered kernel skips the A loads, LDS reads and MFMAs of padding rows), so a
// taller tile costs little extra MFMA work and streams each weight tile once for more rows.
// The height, by the expected rows per expert r, is the one measured fastest on MI355X for
// DeepSeek-V3-like routing (segment sizes spread about +-13% around r):
//   r <= 100: 128;  (100, 176]: 192;  (176, 288]: 256;  (288, 448]: 192;  (448, 768): 256.
// With a capacity limit the routing is usually skewed (a few segments at the cap, many tiny
// ones) and 128 was fastest throughout.
int gemm_bm(const moe_problem& p) {
  if (p.dtype != MOE_BF16) return kGemmBM32;
  if (gemm_wide(p)) return 256;
  if (gemm_small(p)) return gemm_dec(p) ? kDecBM : 32;
  if (p.d % 256 || p.capacity_factor > 0) return 128;
  const double r = expected_rows(p);
  if (r <= 100.0) return 128;
  if (r <= 176.0 || (r > 288.0 && r <= 448.0)) return 192;
  return 256;
}

// Expert-choice routing: every segment holds exactly C rows, so take the height with the
// fewest tiles per segment, the shortest of those on a tie.
int gemm_bm_exact(const moe_problem& p, int C) {
  if (p.dtype != MOE_BF16) return kGemmBM32;
  if (gemm_wide(p)) return 256;
  if (gemm_small(p)) return gemm_dec(p) ? kDecBM : 32;
  if (p.d % 256) return 128;
  int best = 128, tiles = ceil_div(C, 128);
  for (int bm : {192, 256})
    if (ceil_div(C, bm) < tiles) {
      best = bm;
      tiles = ceil_div(C, bm);
    }
  return best;
}

bool gemm_wide(const moe_problem& p) {
  return p.dtype == MOE_BF16 && p.d % 256 == 0 && expected_rows(p) >= 768.0;
}

// The down GEMM of the wide class has few tiles (d/256 per 256-row m-tile); when they fill
// the 256 CUs in a poor number of rounds (e.g. 576 tiles = 2.25 rounds), split K in two so the
// half-tiles fill the rounds better. The halves go to two buffers that the combine adds.
int down_ksplit(const moe_problem& p) {
  if (!gemm_wide(p) || p.n_shared) return 1;
  constexpr double kCUs = 256.0;                        // MI355X compute units
  const double mtiles = p.E * (expected_rows(p) / 256.0 + 0.5);   // +1/2 tile of padding
  const double tiles = std::ceil(mtiles) * (p.d / 256);
  const double r1 = std::ceil(tiles / kCUs), r2 = std::ceil(2.0 * tiles / kCUs) / 2.0;
  return r2 < 0.9 * r1 ? 2 : 1;
}

bool gemm_small(const moe_problem& p) { return p.dtype == MOE_BF16 && expected_rows(p) <= 48.0; }

// the small class takes the decode kernel when both K ranges split into four whole 64-steps,
// at most kDecMaxSteps each
bool gemm_dec(const moe_problem& p) {
  return gemm_small(p) && p.d % 256 == 0 && p.d_ff % 256 == 0 && p.d <= 256 * kDecMaxSteps &&
         p.d_ff <= 256 * kDecMaxSteps;
}

// the decode kernel for K = steps * 256, steps in 1 .. kDecMaxSteps
template <bool GATEUP, int STEPS = 1>
void launch_dec_k(int steps, dim3 grid, hipStream_t s, const GemmArgs& a) {
  if constexpr (STEPS <= kDecMaxSteps) {
    if (steps == STEPS)
      hipLaunchKernelGGL((gemm_bf16_dec_kernel<GATEUP, STEPS>), grid, dim3(256), 0, s, a);
    else
      launch_dec_k<GATEUP, STEPS + 1>(steps, grid, s, a);
  }
}

hipError_t launch_dec(const moe_problem& p, const GemmArgs& a, const GemmArgs& b, hipStream_t s,
                      hipEvent_t between, bool up_only) {
  if (!gemm_dec(p) || a.sc.BM != kDecBM) return hipErrorInvalidValue;
  launch_dec_k<true>(p.d / 256, dim3(grid_for(a.sc.max_mtiles, p.d_ff / dec_feat(true), a.sc.xcd_chunk)), s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || up_only) return err;
  if (between && (err = hipEventRecord(between, s)) != hipSuccess) return err;
  launch_dec_k<false>(p.d_ff / 256, dim3(grid_for(b.sc.max_mtiles, p.d / dec_feat(false), b.sc.xcd_chunk)), s, b);
  return hipGetLastError();
}

template <int BM, int BNB_UP, int WM_UP, int WN_UP, int BNB_DN, int WM_DN, int WN_DN, int BK, int ST,
          int RS = 0>
hipError_t launch_bf16(const moe_problem& p, const GemmArgs& a, const GemmArgs& b, hipStream_t s,
                       hipEvent_t between, bool up_only) {
  if (p.d_ff % (BNB_UP / 2) || p.d % BNB_DN) return hipErrorInvalidValue;   // n-tiles cover N
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BNB_UP, WM_UP, WN_UP, BK, ST, true, RS>),
                     dim3(grid_for(a.sc.max_mtiles, p.d_ff / (BNB_UP / 2), a.sc.xcd_chunk)), dim3(WM_UP * WN_UP * 64),
                     0, s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || up_only) return err;
  if (between && (err = hipEventRecord(between, s)) != hipSuccess) return err;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BNB_DN, WM_DN, WN_DN, BK, ST, false, RS>),
                     dim3(grid_for(b.sc.max_mtiles * b.ksplit, p.d / BNB_DN, b.sc.xcd_chunk)),
                     dim3(WM_DN * WN_DN * 64), 0, s, b);
  return hipGetLastError();
}

template <int BM, int BNB_UP, int WM_UP, int WN_UP, int BNB_DN, int WM_DN, int WN_DN>
hipError_t launch_bf16_st(const moe_problem& p, const GemmArgs& a, const GemmArgs& b,
                          hipStream_t s, hipEvent_t between, bool up_only) {
  if (p.d_ff % (BNB_UP / 2) || p.d % BNB_DN) return hipErrorInvalidValue;   // n-tiles cover N
  const dim3 gup(grid_for(a.sc.max_mtiles, p.d_ff / (BNB_UP / 2), a.sc.xcd_chunk));
  if (up_only)   // the backward's recompute keeps u and v in the untransposed accumulator layout
    hipLaunchKernelGGL((gemm_bf16_st_kernel<BM, BNB_UP, WM_UP, WN_UP, true, false, false>), gup,
                       dim3(WM_UP * WN_UP * 64), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_bf16_st_kernel<BM, BNB_UP, WM_UP, WN_UP, true>), gup,
                       dim3(WM_UP * WN_UP * 64), 0, s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || up_only) return err;
  if (between && (err = hipEventRecord(between, s)) != hipSuccess) return err;
  const dim3 gdn(grid_for(b.sc.max_mtiles * b.ksplit, p.d / BNB_DN, b.sc.xcd_chunk));
  // Rows the combine reads once. When they outgrow the 256 MB memory-side cache (at most T*k
  // rows of d fp32), they go out with the non-temporal hint: DeepSeek-V3-shaped step
  // 5.11 -> 5.07 ms (940 MB of rows; down 1.84 -> 1.80 ms). Smaller sets stay cacheable: with
  // the hint the combine after them read slower (skewed shape 72 -> 83 us).
  if ((double)p.T * p.k * p.d * 4.0 * b.ksplit > 512.0 * 1048576.0)
    hipLaunchKernelGGL((gemm_bf16_st_kernel<BM, BNB_DN, WM_DN, WN_DN, false, true>), gdn,
                       dim3(WM_DN * WN_DN * 64), 0, s, b);
  else
    hipLaunchKernelGGL((gemm_bf16_st_kernel<BM, BNB_DN, WM_DN, WN_DN, false>), gdn,
                       dim3(WM_DN * WN_DN * 64), 0, s, b);
  return hipGetLastError();
}

// The four-wave wide kernel addresses x and h with byte offsets below 2^31 and runs whole pairs
// of K steps; other wide shapes, and the backward's gate-up recompute (which also stores u and v in
// the accumulator layout), take the eight-wave register-staged kernel.
static bool wide_w4_ok(const moe_problem& p, const Schedule& sc, int ksplit) {
  return (double)p.T * p.d * 2.0 < 2147483648.0 &&
         (double)sc.max_mtiles * 256.0 * p.d_ff * 2.0 < 2147483648.0 && p.d % 128 == 0 &&
         p.d_ff % (128 * ksplit) == 0;
}

hipError_t launch_bf16_w4(const moe_problem& p, const GemmArgs& a, const GemmArgs& b, hipStream_t s,
                          hipEvent_t between, bool up_only) {
  if (p.d_ff % 128 || p.d % 256) return hipErrorInvalidValue;   // n-tiles cover N
  hipLaunchKernelGGL(gemm_bf16_w4_kernel<true>,
                     dim3(grid_for(a.sc.max_mtiles, p.d_ff / 128, a.sc.xcd_chunk)), dim3(256), 0, s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || up_only) return err;
  if (between && (err = hipEventRecord(between, s)) != hipSuccess) return err;
  hipLaunchKernelGGL(gemm_bf16_w4_kernel<false>,
                     dim3(grid_for(b.sc.max_mtiles * b.ksplit, p.d / 256, b.sc.xcd_chunk)), dim3(256), 0,
                     s, b);
  return hipGetLastError();
}

hipError_t launch_dec_gate_up(const moe_problem& p, const void* x, const void* w1, const void* w3,
                              const int32_t* sorted_assign, const Schedule& sc, void* h,
                              hipStream_t s) {
  if (!gemm_dec(p) || sc.BM != kDecBM || p.n_shared) return hipErrorInvalidValue;
  if (p.T == 0) return hipSuccess;
  GemmArgs a{};
  a.A = (const bf16_t*)x;
  a.B0 = (const bf16_t*)w1;
  a.B1 = (const bf16_t*)w3;
  a.N = p.d_ff;
  a.K = p.d;
  a.E = p.E;
  a.k = p.k;
  a.T = p.T;
  a.sorted_assign = sorted_assign;
  a.sc = sc;
  a.H = (bf16_t*)h;
  a.ksplit = 1;
  launch_dec_k<true>(p.d / 256, dim3(grid_for(sc.max_mtiles, p.d_ff / dec_feat(true), sc.xcd_chunk)), s, a);
  return hipGetLastError();
}

hipError_t launch_expert_ffn(const moe_problem& p, const void* x, const void* w1, const void* w3,
                             const void* w2, const void* ws1, const void* ws3, const void* ws2,
                             const int32_t* sorted_assign, const Schedule& sc, void* h,
                             float* out_rows, float* out_rows_b, float* shared_out, hipStream_t s,
                             hipEvent_t between, int row_div, float* U, float* V) {
  const bool up_only = U != nullptr;   // the backward's recompute: gate-up with u and v kept
  const int kdiv = row_div > 0 ? row_div : p.k;
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
    a.k = kdiv;
    a.T = p.T;
    a.sorted_assign = sorted_assign;
    a.sc = sc;
    a.H = (bf16_t*)h;
    a.U = U;
    a.V = V;
    GemmArgs b{};
    b.A = (const bf16_t*)h;
    b.B0 = (const bf16_t*)w2;
    b.S0 = (const bf16_t*)ws2;
    b.N = p.d;
    b.K = p.d_ff;
    b.E = p.E;
    b.k = kdiv;
    b.T = p.T;
    b.sorted_assign = sorted_assign;
    b.sc = sc;
    b.out_rows = out_rows;
    b.shared_out = shared_out;
    a.ksplit = 1;
    b.ksplit = down_ksplit(p);
    b.out_rows_b = out_rows_b;
    if (!up_only && b.ksplit == 2 && !out_rows_b) return hipErrorInvalidValue;
    if (sc.BM == 256 && gemm_wide(p))
      return wide_w4_ok(p, sc, b.ksplit) && !up_only
                 ? launch_bf16_w4(p, a, b, s, between, up_only)
                 : launch_bf16<256, 256, 4, 2, 256, 4, 2, 64, 2, 1>(p, a, b, s, between, up_only);
    if (sc.BM == 256) return launch_bf16_st<256, 256, 4, 2, 256, 4, 2>(p, a, b, s, between, up_only);
    if (sc.BM == 192) return launch_bf16_st<192, 256, 2, 4, 256, 2, 4>(p, a, b, s, between, up_only);
    if (sc.BM == kDecBM && gemm_dec(p)) return launch_dec(p, a, b, s, between, up_only);
    if (sc.BM == 32) return launch_bf16<32, 256, 1, 4, 128, 1, 4, 64, 4>(p, a, b, s, between, up_only);
    // down tiles of 256 output features need d % 256 == 0 (the entry points accept d % 128)
    if (p.d % 256 == 0) return launch_bf16_st<128, 256, 2, 4, 256, 2, 4>(p, a, b, s, between, up_only);
    return launch_bf16<128, 256, 2, 4, 128, 2, 4, 64, 3>(p, a, b, s, between, up_only);
  }
  if (up_only) return hipErrorInvalidValue;   // the backward runs on bf16 storage only
  GemmArgs32 a{};
  a.A = (const float*)x;
  a.B0 = (const float*)w1;
  a.B1 = (const float*)w3;
  a.S0 = (const float*)ws1;
  a.S1 = (const float*)ws3;
  a.N = p.d_ff;
  a.K = p.d;
  a.E = p.E;
  a.k = kdiv;
  a.T = p.T;
  a.sorted_assign = sorted_assign;
  a.sc = sc;
  a.H = (float*)h;
  hipLaunchKernelGGL(gemm_f32_kernel<true>, dim3(grid_for(sc.max_mtiles, ceil_div(p.d_ff, BN32), sc.xcd_chunk)),
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
  b.k = kdiv;
  b.T = p.T;
  b.sorted_assign = sorted_assign;
  b.sc = sc;
  b.out_rows = out_rows;
  b.shared_out = shared_out;
  hipLaunchKernelGGL(gemm_f32_kernel<false>, dim3(grid_for(sc.max_mtiles, ceil_div(p.d, BN32), sc.xcd_chunk)),
                     dim3(256), 0, s, b);
  return hipGetLastError();
}

}  // namespace moe
