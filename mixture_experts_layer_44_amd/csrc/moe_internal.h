// Internal declarations shared by the HIP translation units of libmoe_mi355x.
// Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <algorithm>
#include <cmath>
#include <stdint.h>

#include "../../include/moe_mi355x.h"

namespace moe {

typedef uint16_t bf16_t;  // raw bf16 storage
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t v) { return __uint_as_float((uint32_t)v << 16); }

// u and v kept by the backward's gate-up recompute (fp32, storage rows x N columns, N a multiple
// of 32) lie in MFMA fragment order: each 32 x 32 block of (storage row, column) is 1024
// contiguous floats holding the 32x32 accumulator layout (lane c + 32h holds column c and rows
// 8*(r/4) + 4h + r%4 at r = 0..15) as four quads, quad q = lanes' values r = 4q..4q+3, lane-major
// inside the quad. A wave then writes or reads a fragment with four 16-byte accesses per lane,
// each instruction covering 1 KB contiguous. Offset of lane `lane`'s first quad in the block at
// (srow0, col0), both multiples of 32 (quad q at + 256 q):
__device__ __forceinline__ size_t uv_frag(int srow0, int col0, int N, int lane) {
  return ((size_t)(srow0 >> 5) * (size_t)(N >> 5) + (size_t)(col0 >> 5)) * 1024 + (size_t)lane * 4;
}
// offset of element (srow, col)
__device__ __forceinline__ size_t uv_elem(int srow, int col, int N) {
  const int rb = srow & 31, c = col & 31;
  return uv_frag(srow & ~31, col & ~31, N, c + 32 * ((rb >> 2) & 1)) + 256 * (rb >> 3) + (rb & 3);
}
__device__ __forceinline__ void uv_store(float* dst, const f32x16& v) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *(f32x4*)(dst + 256 * q) = f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
}

// fp32 -> bf16, round to nearest even (NaN stays NaN): the hardware conversion
// (v_cvt_pk_bf16_f32), one instruction instead of the integer rounding sequence.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, (__bf16)f);
}

// ---------------------------------------------------------------- tiling constants
constexpr int kAlignChunk = 1024;    // assignments per align workgroup
constexpr int kGemmBM = 128;         // rows per grouped-GEMM m-tile (bf16 path)
constexpr int kGemmBM32 = 16;        // rows per m-tile (fp32 path; its tiles are VALU-bound)
constexpr int kDecBM = 32;           // rows per m-tile of the decode-class GEMM kernels

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---------------------------------------------------------------- schedule
// Grouped-GEMM work list built on the device from the align offsets. Groups
// 0..E-1 are the routed experts, group E the shared expert (if any).
struct Schedule {
  int32_t* grp_rows;   // [G]   rows (kept assignments, or T for the shared expert)
  int32_t* grp_off;    // [G]   first row in sorted order (routed), 0 for shared
  int32_t* mt_start;   // [G+1] exclusive prefix of ceil(rows/BM); mt_start[G] = total m-tiles
  int32_t* mt_group;   // [max_mtiles] group of each m-tile
  // [max_mtiles][8] or null: per m-tile slot m, {g, mt_start[g], m-tiles of g, grp_rows[g],
  // grp_off[g], 0, 0, 0}, so that a workgroup finds its tile with one load instead of a chain
  int32_t* mt_info = nullptr;
  int max_mtiles;
  int G;
  int BM;
  int xcd_chunk = 0;   // 1: tiles dealt to the XCDs in chunks of kXcdChunk (capacity-limited routing)
};
constexpr int kXcdChunk = 16;

// m-tiles that n_rows routed rows (in E segments) plus the shared expert's T rows can need
int max_mtiles(long long n_rows, int T, int E, int n_shared, int BM);
// grouped-GEMM tile shape class from the expected rows per expert: wide (256-row m-tiles),
// narrow (128) or small (32)
bool gemm_wide(const moe_problem& p);
bool gemm_small(const moe_problem& p);
bool gemm_dec(const moe_problem& p);     // small class on the decode kernel (32-row m-tiles)
int gemm_bm(const moe_problem& p);
int gemm_bm_exact(const moe_problem& p, int C);   // all segments of exactly C rows
// workgroups for up to mtiles * nt tiles (a whole number of XCD chunks when chunked)
int grid_for(int mtiles, int nt, int xcd_chunk = 0);

// ---------------------------------------------------------------- launchers
// router: d-slices of the logits GEMM, scratch bytes for its fp32 partial logits, and the
// number of top-k workgroups (rows of the per-workgroup probability sums)
int route_ksplit(const moe_problem& p);
size_t route_partial_bytes(const moe_problem& p);
int route_topk_blocks(const moe_problem& p);

hipError_t launch_route_logits(const moe_problem& p, const void* x, const void* w_gate,
                               float* logits_part, hipStream_t s);

// small batches (T*k <= 1024): top-k, probability sums, grouping and GEMM schedule in one
// single-workgroup launch after the logits
bool small_routing(const moe_problem& p);
hipError_t launch_route_align_small(const moe_problem& p, int cap, const float* logits_part,
                                    const float* logit_bias, const float* sel_bias, int32_t* ids,
                                    float* gates, float* prob_sum, float* psum_part,
                                    int32_t* counts_pre, int32_t* counts, int32_t* offsets,
                                    int32_t* sorted_assign, int32_t* assign_pos, const Schedule& sc,
                                    hipStream_t s);

// top-k + grouping + GEMM schedule in one workgroup after the logits kernel (T <= 16,
// T*k <= 1024); without do_align only the top-k (ids, gates, prob_sum)
bool small_topk_fused(const moe_problem& p);
hipError_t launch_topk_align_small(const moe_problem& p, int cap, const float* logits_part,
                                   const float* logit_bias, const float* sel_bias, int32_t* ids,
                                   float* gates, float* prob_sum, bool do_align,
                                   int32_t* counts_pre, int32_t* counts, int32_t* offsets,
                                   int32_t* sorted_assign, int32_t* assign_pos, const Schedule& sc,
                                   hipStream_t s);

// top-k of every token from the logits partials; per-workgroup probability sums to psum_part
// (when not null)
hipError_t launch_route_topk(const moe_problem& p, const float* logits_part,
                             const float* logit_bias, const float* sel_bias, int32_t* ids,
                             float* gates, float* psum_part, hipStream_t s);

// psum_stage: [kPsumStage][E] floats for the probability-sum reduction, or null
hipError_t launch_route(const moe_problem& p, const void* x, const void* w_gate,
                        const float* logit_bias, const float* sel_bias, int32_t* ids,
                        float* gates, float* prob_sum, float* logits_part, float* psum_part,
                        float* psum_stage, hipStream_t s);

hipError_t launch_align(const moe_problem& p, int cap, const int32_t* ids, int32_t* counts_pre,
                        int32_t* counts, int32_t* offsets, int32_t* sorted_assign,
                        int32_t* assign_pos, int32_t* blk_counts, int32_t* blk_base, hipStream_t s);

// n_rows: rows the routed segments can span (T*k when negative)
hipError_t launch_schedule(const moe_problem& p, const int32_t* offsets, const Schedule& sc,
                           hipStream_t s, long long n_rows = -1);

// 2 when the down GEMM runs with its K range split in two (second half -> out_rows_b)
int down_ksplit(const moe_problem& p);

// out_rows_b: [T*k, d] second-half partial rows, required when down_ksplit(p) == 2.
// row_div: a routed row r gathers token sorted_assign[r] / row_div (0: k).
// U, V (bf16 storage only): when given, only the gate-up GEMM runs, and it also stores u and v
// in fp32, in fragment order over H's storage rows (uv_frag; the backward's recompute).
hipError_t launch_expert_ffn(const moe_problem& p, const void* x, const void* w1, const void* w3,
                             const void* w2, const void* ws1, const void* ws3, const void* ws2,
                             const int32_t* sorted_assign, const Schedule& sc, void* h,
                             float* out_rows, float* out_rows_b, float* shared_out, hipStream_t s,
                             hipEvent_t between = nullptr, int row_div = 0, float* U = nullptr,
                             float* V = nullptr);

// Decode-sized layers without a shared expert (k <= 8, T*k <= 16): the gate-up GEMM alone
// (decode class, h out), then the down GEMM and the combine in one launch, y bit-identical to
// launch_expert_ffn's rows followed by launch_combine.
hipError_t launch_dec_gate_up(const moe_problem& p, const void* x, const void* w1, const void* w3,
                              const int32_t* sorted_assign, const Schedule& sc, void* h,
                              hipStream_t s);
bool dec_down_combine(const moe_problem& p);
hipError_t launch_dec_down_combine(const moe_problem& p, const void* h, const void* w2,
                                   const int32_t* ids, const float* gates,
                                   const int32_t* assign_pos, const Schedule& sc, float* y,
                                   hipStream_t s);

// out_rows_b may be null; when given, each expert row is out_rows + out_rows_b
hipError_t launch_combine(const moe_problem& p, const float* out_rows, const float* out_rows_b,
                          const int32_t* assign_pos, const float* topk_w, const float* shared_out,
                          float* y, hipStream_t s);

// out_rows[r] += out_rows_b[r] for the first offsets[E] rows
hipError_t launch_add_rows(const moe_problem& p, float* out_rows, const float* out_rows_b,
                           const int32_t* offsets, hipStream_t s);

hipError_t launch_balance(const moe_problem& p, const int32_t* counts_pre, const float* prob_sum,
                          float alpha, float* f, float* P, float* L, hipStream_t s);

// prob_sum[e] = sum over the nblk per-workgroup partials, a fixed tree (run-to-run identical).
// stage: [kPsumStage][E] floats, or null (one workgroup reads every partial).
constexpr int kPsumStage = 64;
hipError_t launch_psum_reduce(const float* psum_part, int nblk, int E, float* prob_sum,
                              hipStream_t s, float* stage = nullptr);

// ---- expert-choice routing (expert_choice.hip)
int ec_probs_blocks(const moe_problem& p);
// router probabilities, expert-major probsT [E][T]; per-workgroup sums when psum_part != null
hipError_t launch_ec_probs(const moe_problem& p, const float* logits_part, const float* logit_bias,
                           float* probsT, float* psum_part, hipStream_t s);
// buckets: tokens / gates [E*C] (expert e at e*C, ascending tokens), pos_table [T][E] (row of
// (t,e) or -1), offsets [E+1] = e*C
hipError_t launch_ec_select(const moe_problem& p, int C, const float* probsT, int32_t* tokens,
                            float* gates, int32_t* pos_table, int32_t* offsets, hipStream_t s);
hipError_t launch_ec_combine(const moe_problem& p, const int32_t* pos_table, const float* gates,
                             const float* out_rows, const float* out_rows_b,
                             const float* shared_out, float* y, hipStream_t s);

hipError_t launch_bias_update(const moe_problem& p, const int32_t* counts_pre, float gamma,
                              float* sel_bias, hipStream_t s);

// ---------------------------------------------------------------- backward
// Workspace of the layer backward (byte offsets; bf16 storage only).
struct BwdLayout {
  size_t grp_rows, grp_off, mt_start, mt_group, logits_part, dlb_part, zero;
  size_t r_grp_rows, r_grp_off, r_mt_start, r_mt_group;   // the row-tile schedule
  size_t H, U, V, DUV, DO, XS, dyb, dgate_part, dx_rows, dx_shared, dlog, dx_router;
  size_t wgate_part;   // the router weight gradient's per-split fp32 partials (wgate_split > 1)
  size_t total;
  int max_mt, max_mt_rows, E_pad, NT_down, nblk_router, stor_bm;
  int wgate_split, wgate_rows;   // token splits of that GEMM's K, and the rows of each
};
BwdLayout backward_layout(const moe_problem& p);
hipError_t launch_backward(const moe_problem& p, const BwdLayout& L, void* ws, const void* x,
                           const void* w_gate, const float* logit_bias, const void* w1,
                           const void* w3, const void* w2, const void* ws1, const void* ws3,
                           const void* ws2, const int32_t* topk_ids, const float* topk_w,
                           const int32_t* counts_pre, const int32_t* offsets,
                           const int32_t* sorted_assign, const int32_t* assign_pos,
                           const float* dy, float alpha, float dL, float* dx, float* dw_gate,
                           float* dlogit_bias, void* dw1, void* dw3, void* dw2, void* dws1,
                           void* dws3, void* dws2, hipStream_t s, hipEvent_t* ev = nullptr);

}  // namespace moe
