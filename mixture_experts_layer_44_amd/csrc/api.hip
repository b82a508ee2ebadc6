// C ABI of libmoe_mi355x: argument validation, workspace layout and the stream-ordered
// launch sequence route -> align -> schedule -> gate-up GEMM -> down GEMM -> combine.
// Validation never touches the GPU, so invalid calls return before anything is enqueued.
#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <mutex>

#include "moe_internal.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

// Workspace of moe_forward_noalloc: one copy per GPU, held until the process ends. Host code
// never passes this name to a kernel (on the host it is only a stand-in for the symbol); it uses
// the device address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace moe {
namespace {

struct Layout {
  size_t logits_part, psum_part, psum_stage, blk_counts, blk_base, grp_rows, grp_off, mt_start,
      mt_group, h;
  size_t mt_info;
  size_t ids, gates, prob_sum, counts_pre, counts, offsets, sorted_assign, assign_pos;
  size_t out_rows, out_rows_b, shared_out;
  size_t probsT, pos_table;   // expert choice only
  size_t total;
  int max_mt, BM;
};

// bucket size of expert-choice routing: ceil(cf * T*k / E) (cf = 1 when unset), at most T
int ec_capacity(const moe_problem& p) {
  const double cf = p.capacity_factor > 0 ? p.capacity_factor : 1.0;
  const double c = std::ceil(cf * (double)((long long)p.T * p.k) / (double)p.E);
  return c >= (double)p.T ? p.T : (int)c;
}

// Workspace of the token-choice path, or (ec) of the expert-choice path, whose routed rows are
// the E*C bucket slots.
Layout layout(const moe_problem& p, bool ec = false) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + (bytes ? bytes : 1), 256);
    return o;
  };
  const size_t n = ec ? std::max((size_t)p.T * p.k, (size_t)p.E * ec_capacity(p))
                      : (size_t)p.T * p.k;
  const int G = p.E + p.n_shared;
  const int nblk_route = ec ? std::max(route_topk_blocks(p), ec_probs_blocks(p)) : route_topk_blocks(p);
  const int nblk_align = ceil_div((int)n, kAlignChunk);
  L.BM = ec ? gemm_bm_exact(p, ec_capacity(p)) : gemm_bm(p);
  L.max_mt = max_mtiles((long long)n, p.T, p.E, p.n_shared, L.BM);
  const size_t esz = p.dtype == MOE_BF16 ? 2 : 4;
  L.logits_part = take(route_partial_bytes(p));
  L.psum_part = take((size_t)nblk_route * p.E * 4);
  L.psum_stage = take((size_t)kPsumStage * p.E * 4);
  L.blk_counts = take((size_t)nblk_align * p.E * 4);
  L.blk_base = take((size_t)nblk_align * p.E * 4);
  L.grp_rows = take((size_t)G * 4);
  L.grp_off = take((size_t)G * 4);
  L.mt_start = take((size_t)(G + 1) * 4);
  L.mt_group = take((size_t)L.max_mt * 4);
  L.mt_info = take((size_t)L.max_mt * 32);
  L.h = take((size_t)L.max_mt * L.BM * p.d_ff * esz);
  L.ids = take(n * 4);
  L.gates = take(n * 4);
  L.prob_sum = take((size_t)p.E * 4);
  L.counts_pre = take((size_t)p.E * 4);
  L.counts = take((size_t)p.E * 4);
  L.offsets = take((size_t)(p.E + 1) * 4);
  L.sorted_assign = take(n * 4);
  L.assign_pos = take(n * 4);
  L.out_rows = take(n * p.d * 4);
  L.out_rows_b = take(down_ksplit(p) == 2 ? n * p.d * 4 : 0);
  L.shared_out = take((size_t)p.n_shared * p.T * p.d * 4);
  L.probsT = ec ? take((size_t)p.E * p.T * 4) : 0;
  L.pos_table = ec ? take((size_t)p.T * p.E * 4) : 0;
  L.total = off;
  return L;
}

template <typename T>
T* at(void* ws, size_t off) {
  return (T*)((char*)ws + off);
}

Schedule schedule_in(const moe_problem& p, const Layout& L, void* ws) {
  Schedule sc;
  sc.grp_rows = at<int32_t>(ws, L.grp_rows);
  sc.grp_off = at<int32_t>(ws, L.grp_off);
  sc.mt_start = at<int32_t>(ws, L.mt_start);
  sc.mt_group = at<int32_t>(ws, L.mt_group);
  sc.mt_info = at<int32_t>(ws, L.mt_info);
  sc.max_mtiles = L.max_mt;
  sc.G = p.E + p.n_shared;
  sc.BM = L.BM;
  // under a capacity limit a few segments sit at the cap: spread their tiles over the XCDs
  // (skewed layer: gate-up 0.49 -> 0.47 ms)
  sc.xcd_chunk = p.capacity_factor > 0 ? 1 : 0;
  return sc;
}

// cap as used by the kernels: -1 = none; clamped to T*k (an equivalent limit)
int kernel_cap(const moe_problem& p) {
  if (!(p.capacity_factor > 0)) return -1;
  const double c = std::ceil(p.capacity_factor * (double)((long long)p.T * p.k) / (double)p.E);
  const long long n = (long long)p.T * p.k;
  return c >= (double)n ? (int)n : (int)c;
}

// The GEMM loaders address each matrix as a 64-bit base plus a 32-bit element offset
// (row * row length + column), so every matrix they read must hold fewer than 2^32 elements:
// x [T, d], each expert matrix [d_ff, d], and the padded row table h [m-tiles * BM, d_ff]
// (for the expert-choice layout, its E*C bucket rows). With the backward, also its storage
// rows times the widest row it addresses (2*d_ff for du|dv, d for the row copies).
constexpr long long kAddr32 = 1ll << 32;

bool forward_addr32_ok(const moe_problem& p, bool ec) {
  if ((long long)p.T * p.d >= kAddr32 || (long long)p.d * p.d_ff >= kAddr32) return false;
  const Layout L = layout(p, ec);
  return (long long)L.max_mt * L.BM * p.d_ff < kAddr32;
}

bool backward_addr32_ok(const moe_problem& p) {
  if (!forward_addr32_ok(p, false)) return false;
  const BwdLayout L = backward_layout(p);
  const long long rows = std::max((long long)L.max_mt * L.stor_bm, (long long)p.T);
  const long long width = std::max({(long long)p.d, 2ll * p.d_ff, (long long)L.E_pad});
  return rows * width < kAddr32;
}

moe_status check_ws(const moe_problem& p, const void* ws, size_t ws_bytes, bool ec = false) {
  const size_t need = layout(p, ec).total;
  if (ws_bytes < need) return MOE_EWORKSPACE;
  if (!ws) return MOE_EINVAL;
  return MOE_OK;
}

inline moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

}  // namespace
}  // namespace moe

using namespace moe;

MOE_API const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported shape";
    case MOE_EWORKSPACE: return "workspace too small";
    case MOE_EHIP: return "HIP launch or runtime error";
    default: return "unknown status";
  }
}

MOE_API moe_status moe_validate(const moe_problem* p) {
  if (!p) return MOE_EINVAL;
  if (p->T < 0 || p->d <= 0 || p->E <= 0 || p->k <= 0 || p->d_ff <= 0) return MOE_EINVAL;
  if (p->dtype != MOE_F32 && p->dtype != MOE_BF16) return MOE_EINVAL;
  if (p->n_shared < 0 || p->d_ff_shared < 0) return MOE_EINVAL;
  if (!std::isfinite(p->capacity_factor)) return MOE_EINVAL;
  if (p->E > 256 || p->k > p->E || p->k > 32) return MOE_EUNSUPPORTED;
  if (p->n_shared > 1) return MOE_EUNSUPPORTED;
  if (p->n_shared == 1 && p->d_ff_shared != p->d_ff) return MOE_EUNSUPPORTED;
  if ((long long)p->T * p->k >= (long long)INT_MAX - 4096) return MOE_EUNSUPPORTED;
  if (p->dtype == MOE_BF16 && (p->d % 128 || p->d_ff % 128)) return MOE_EUNSUPPORTED;
  if (p->dtype == MOE_F32 && p->d % 4) return MOE_EUNSUPPORTED;
  if (!forward_addr32_ok(*p, false)) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

MOE_API moe_status moe_capacity(const moe_problem* p, int32_t* cap_out) {
  moe_status st = moe_validate(p);
  if (st != MOE_OK) return st;
  if (!cap_out) return MOE_EINVAL;
  if (!(p->capacity_factor > 0)) {
    *cap_out = -1;
    return MOE_OK;
  }
  const double c = std::ceil(p->capacity_factor * (double)((long long)p->T * p->k) / (double)p->E);
  *cap_out = c >= (double)INT_MAX ? INT_MAX : (int32_t)c;
  return MOE_OK;
}

MOE_API moe_status moe_workspace_bytes(const moe_problem* p, size_t* bytes_out) {
  moe_status st = moe_validate(p);
  if (st != MOE_OK) return st;
  if (!bytes_out) return MOE_EINVAL;
  *bytes_out = layout(*p).total;
  return MOE_OK;
}

MOE_API moe_status moe_expert_choice_capacity(const moe_problem* p, int32_t* c_out) {
  moe_status st = moe_validate(p);
  if (st != MOE_OK) return st;
  if (!c_out) return MOE_EINVAL;
  *c_out = ec_capacity(*p);
  return MOE_OK;
}

MOE_API moe_status moe_expert_choice_workspace_bytes(const moe_problem* p, size_t* bytes_out) {
  moe_status st = moe_validate(p);
  if (st != MOE_OK) return st;
  if (!bytes_out) return MOE_EINVAL;
  if (!forward_addr32_ok(*p, true)) return MOE_EUNSUPPORTED;
  *bytes_out = layout(*p, true).total;
  return MOE_OK;
}

MOE_API moe_status moe_forward_expert_choice(const moe_problem* p, const void* x,
                                             const void* w_gate, const float* logit_bias,
                                             const void* w1, const void* w3, const void* w2,
                                             const void* ws1, const void* ws3, const void* ws2,
                                             float* y, int32_t* tokens_out, float* gates_out,
                                             float* prob_sum, void* ws, size_t ws_bytes,
                                             hipStream_t stream) {
  moe_status st = moe_validate(p);
  if (st != MOE_OK) return st;
  const bool hasT = p->T > 0;
  if (!w_gate || !w1 || !w3 || !w2 || (hasT && (!x || !y))) return MOE_EINVAL;
  if (p->n_shared && (!ws1 || !ws3 || !ws2)) return MOE_EINVAL;
  if (!forward_addr32_ok(*p, true)) return MOE_EUNSUPPORTED;
  if ((st = check_ws(*p, ws, ws_bytes, true)) != MOE_OK) return st;
  const Layout L = layout(*p, true);
  const int C = ec_capacity(*p);
  int32_t* tokens = tokens_out ? tokens_out : at<int32_t>(ws, L.sorted_assign);
  float* gates = gates_out ? gates_out : at<float>(ws, L.gates);
  int32_t* offs = at<int32_t>(ws, L.offsets);
  float* out_rows = at<float>(ws, L.out_rows);
  float* out_b = down_ksplit(*p) == 2 ? at<float>(ws, L.out_rows_b) : nullptr;
  float* shared_out = p->n_shared ? at<float>(ws, L.shared_out) : nullptr;
  float* probsT = at<float>(ws, L.probsT);
  int32_t* pos = at<int32_t>(ws, L.pos_table);
  float* psum_part = at<float>(ws, L.psum_part);
  const Schedule sc = schedule_in(*p, L, ws);
  hipError_t e = launch_route_logits(*p, x, w_gate, at<float>(ws, L.logits_part), stream);
  if (e == hipSuccess)
    e = launch_ec_probs(*p, at<float>(ws, L.logits_part), logit_bias, probsT,
                        prob_sum ? psum_part : nullptr, stream);
  if (e == hipSuccess && prob_sum)
    e = launch_psum_reduce(psum_part, hasT ? ec_probs_blocks(*p) : 0, p->E, prob_sum, stream,
                           at<float>(ws, L.psum_stage));
  if (e == hipSuccess) e = launch_ec_select(*p, C, probsT, tokens, gates, pos, offs, stream);
  if (e == hipSuccess) e = launch_schedule(*p, offs, sc, stream, (long long)p->E * C);
  if (e == hipSuccess)
    e = launch_expert_ffn(*p, x, w1, w3, w2, ws1, ws3, ws2, tokens, sc, at<void>(ws, L.h), out_rows,
                          out_b, shared_out, stream, nullptr, 1);
  if (e == hipSuccess) e = launch_ec_combine(*p, pos, gates, out_rows, out_b, shared_out, y, stream);
  return hip_status(e);
}

MOE_API moe_status moe_route(const moe_problem* p, const void* x, const void* w_gate,
                             const float* logit_bias, const float* sel_bias, int32_t* topk_ids,
                             float* topk_w, float* prob_sum, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  moe_status st = moe_validate(p);
  if (st != MOE_OK) return st;
  const bool hasT = p->T > 0;
  if (!w_gate || (hasT && (!x || !topk_ids || !topk_w))) return MOE_EINVAL;
  if ((st = check_ws(*p, ws, ws_bytes)) != MOE_OK) return st;
  const Layout L = layout(*p);
  if (small_topk_fused(*p)) {   // the same kernels (and bits) as moe_forward at these sizes
    hipError_t e = launch_route_logits(*p, x, w_gate, at<float>(ws, L.logits_part), stream);
    if (e == hipSuccess)
      e = launch_topk_align_small(*p, -1, at<float>(ws, L.logits_part), logit_bias, sel_bias,
                                  topk_ids, topk_w, prob_sum, false, nullptr, nullptr, nullptr,
                                  nullptr, nullptr, schedule_in(*p, L, ws), stream);
    return hip_status(e);
  }
  return hip_status(launch_route(*p, x, w_gate, logit_bias, sel_bias, topk_ids, topk_w, prob_sum,
                                 at<float>(ws, L.logits_part), at<float>(ws, L.psum_part),
                                 at<float>(ws, L.psum_stage), stream));
}

MOE_API moe_status moe_align(const moe_problem* p, const int32_t* topk_ids, int32_t* counts_pre,
                             int32_t* counts, int32_t* offsets, int32_t* sorted_assign,
                             int32_t* assign_pos, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = moe_validate(p);
  if (st != MOE_OK) return st;
  const bool hasT = p->T > 0;
  if (!counts_pre || !counts || !offsets) return MOE_EINVAL;
  if (hasT && (!topk_ids || !sorted_assign || !assign_pos)) return MOE_EINVAL;
  if ((st = check_ws(*p, ws, ws_bytes)) != MOE_OK) return st;
  const Layout L = layout(*p);
  return hip_status(launch_align(*p, kernel_cap(*p), topk_ids, counts_pre, counts, offsets,
                                 sorted_assign, assign_pos, at<int32_t>(ws, L.blk_counts),
                                 at<int32_t>(ws, L.blk_base), stream));
}

MOE_API moe_status moe_expert_ffn(const moe_problem* p, const void* x, const void* w1,
                                  const void* w3, const void* w2, const void* ws1, const void* ws3,
                                  const void* ws2, const int32_t* sorted_assign,
                                  const int32_t* offsets, float* out_rows, float* shared_out,
                                  void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = moe_validate(p);
  if (st != MOE_OK) return st;
  const bool hasT = p->T > 0;
  if (!w1 || !w3 || !w2 || !offsets) return MOE_EINVAL;
  if (hasT && (!x || !sorted_assign || !out_rows)) return MOE_EINVAL;
  if (p->n_shared && (!ws1 || !ws3 || !ws2 || (hasT && !shared_out))) return MOE_EINVAL;
  if ((st = check_ws(*p, ws, ws_bytes)) != MOE_OK) return st;
  const Layout L = layout(*p);
  const Schedule sc = schedule_in(*p, L, ws);
  hipError_t e = launch_schedule(*p, offsets, sc, stream);
  if (e != hipSuccess) return MOE_EHIP;
  float* out_b = down_ksplit(*p) == 2 ? at<float>(ws, L.out_rows_b) : nullptr;
  e = launch_expert_ffn(*p, x, w1, w3, w2, ws1, ws3, ws2, sorted_assign, sc, at<void>(ws, L.h),
                        out_rows, out_b, shared_out, stream);
  if (e == hipSuccess && out_b) e = launch_add_rows(*p, out_rows, out_b, offsets, stream);
  return hip_status(e);
}

MOE_API moe_status moe_combine(const moe_problem* p, const float* out_rows,
                               const int32_t* assign_pos, const float* topk_w,
                               const float* shared_out, float* y, hipStream_t stream) {
  moe_status st = moe_validate(p);
  if (st != MOE_OK) return st;
  if (p->T > 0 && (!out_rows || !assign_pos || !topk_w || !y)) return MOE_EINVAL;
  if (p->T > 0 && p->n_shared && !shared_out) return MOE_EINVAL;
  return hip_status(launch_combine(*p, out_rows, nullptr, assign_pos, topk_w, shared_out, y, stream));
}

MOE_API moe_status moe_balance(const moe_problem* p, const int32_t* counts_pre,
                               const float* prob_sum, float alpha, float* f, float* P, float* L,
                               hipStream_t stream) {
  moe_status st = moe_validate(p);
  if (st != MOE_OK) return st;
  if (!counts_pre || !prob_sum || !f || !P || !L) return MOE_EINVAL;
  if (!std::isfinite(alpha)) return MOE_EINVAL;
  return hip_status(launch_balance(*p, counts_pre, prob_sum, alpha, f, P, L, stream));
}

MOE_API moe_status moe_bias_update(const moe_problem* p, const int32_t* counts_pre, float gamma,
                                   float* sel_bias, hipStream_t stream) {
  moe_status st = moe_validate(p);
  if (st != MOE_OK) return st;
  if (!counts_pre || !sel_bias) return MOE_EINVAL;
  if (!std::isfinite(gamma) || gamma < 0.f) return MOE_EINVAL;
  return hip_status(launch_bias_update(*p, counts_pre, gamma, sel_bias, stream));
}

MOE_API moe_status moe_backward_workspace_bytes(const moe_problem* p, size_t* bytes_out) {
  moe_status st = moe_validate(p);
  if (st != MOE_OK) return st;
  if (!bytes_out) return MOE_EINVAL;
  if (p->dtype != MOE_BF16 || p->k > 16 || !backward_addr32_ok(*p)) return MOE_EUNSUPPORTED;
  *bytes_out = backward_layout(*p).total;
  return MOE_OK;
}

static moe_status backward_impl(const moe_problem* p, const void* x, const void* w_gate,
                                const float* logit_bias, const void* w1, const void* w3,
                                const void* w2, const void* ws1, const void* ws3, const void* ws2,
                                const int32_t* topk_ids, const float* topk_w,
                                const int32_t* counts_pre, const int32_t* offsets,
                                const int32_t* sorted_assign, const int32_t* assign_pos,
                                const float* dy, float alpha, float dL, float* dx, float* dw_gate,
                                float* dlogit_bias, void* dw1, void* dw3, void* dw2, void* dws1,
                                void* dws3, void* dws2, void* ws, size_t ws_bytes,
                                hipStream_t stream, hipEvent_t* ev) {
  moe_status st = moe_validate(p);
  if (st != MOE_OK) return st;
  if (p->dtype != MOE_BF16 || p->k > 16 || !backward_addr32_ok(*p)) return MOE_EUNSUPPORTED;
  const bool hasT = p->T > 0;
  if (!w_gate || !w1 || !w3 || !w2 || !counts_pre || !offsets || !dw_gate || !dw1 || !dw3 || !dw2)
    return MOE_EINVAL;
  if (hasT && (!x || !topk_ids || !topk_w || !sorted_assign || !assign_pos || !dy || !dx))
    return MOE_EINVAL;
  if (p->n_shared && (!ws1 || !ws3 || !ws2 || !dws1 || !dws3 || !dws2)) return MOE_EINVAL;
  if (!std::isfinite(alpha) || !std::isfinite(dL)) return MOE_EINVAL;
  const BwdLayout L = backward_layout(*p);
  if (ws_bytes < L.total) return MOE_EWORKSPACE;
  if (!ws) return MOE_EINVAL;
  return hip_status(launch_backward(*p, L, ws, x, w_gate, logit_bias, w1, w3, w2, ws1, ws3, ws2,
                                    topk_ids, topk_w, counts_pre, offsets, sorted_assign,
                                    assign_pos, dy, alpha, dL, dx, dw_gate, dlogit_bias, dw1, dw3,
                                    dw2, dws1, dws3, dws2, stream, ev));
}

MOE_API moe_status moe_backward(const moe_problem* p, const void* x, const void* w_gate,
                                const float* logit_bias, const void* w1, const void* w3,
                                const void* w2, const void* ws1, const void* ws3, const void* ws2,
                                const int32_t* topk_ids, const float* topk_w,
                                const int32_t* counts_pre, const int32_t* offsets,
                                const int32_t* sorted_assign, const int32_t* assign_pos,
                                const float* dy, float alpha, float dL, float* dx, float* dw_gate,
                                float* dlogit_bias, void* dw1, void* dw3, void* dw2, void* dws1,
                                void* dws3, void* dws2, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  return backward_impl(p, x, w_gate, logit_bias, w1, w3, w2, ws1, ws3, ws2, topk_ids, topk_w,
                       counts_pre, offsets, sorted_assign, assign_pos, dy, alpha, dL, dx, dw_gate,
                       dlogit_bias, dw1, dw3, dw2, dws1, dws3, dws2, ws, ws_bytes, stream, nullptr);
}

MOE_API moe_status moe_backward_staged(
    const moe_problem* p, const void* x, const void* w_gate, const float* logit_bias,
    const void* w1, const void* w3, const void* w2, const void* ws1, const void* ws3,
    const void* ws2, const int32_t* topk_ids, const float* topk_w, const int32_t* counts_pre,
    const int32_t* offsets, const int32_t* sorted_assign, const int32_t* assign_pos,
    const float* dy, float alpha, float dL, float* dx, float* dw_gate, float* dlogit_bias,
    void* dw1, void* dw3, void* dw2, void* dws1, void* dws3, void* dws2, void* ws,
    size_t ws_bytes, hipStream_t stream, hipEvent_t* stage_events) {
  if (!stage_events) return MOE_EINVAL;
  for (int i = 0; i < MOE_BWD_STAGE_EVENTS; ++i)
    if (!stage_events[i]) return MOE_EINVAL;
  return backward_impl(p, x, w_gate, logit_bias, w1, w3, w2, ws1, ws3, ws2, topk_ids, topk_w,
                       counts_pre, offsets, sorted_assign, assign_pos, dy, alpha, dL, dx, dw_gate,
                       dlogit_bias, dw1, dw3, dw2, dws1, dws3, dws2, ws, ws_bytes, stream,
                       stage_events);
}

namespace {

moe_status forward_impl(const moe_problem* p, const void* x, const void* w_gate,
                        const float* logit_bias, const float* sel_bias, const void* w1,
                        const void* w3, const void* w2, const void* ws1, const void* ws3,
                        const void* ws2, float* y, int32_t* topk_ids, float* topk_w,
                        float* prob_sum, int32_t* counts_pre, int32_t* counts, int32_t* offsets,
                        int32_t* sorted_assign, int32_t* assign_pos, void* ws, size_t ws_bytes,
                        hipStream_t stream, hipEvent_t* ev) {
  moe_status st = moe_validate(p);
  if (st != MOE_OK) return st;
  const bool hasT = p->T > 0;
  if (!w_gate || !w1 || !w3 || !w2 || (hasT && (!x || !y))) return MOE_EINVAL;
  if (p->n_shared && (!ws1 || !ws3 || !ws2)) return MOE_EINVAL;
  if ((st = check_ws(*p, ws, ws_bytes)) != MOE_OK) return st;
  const Layout L = layout(*p);
  int32_t* ids = topk_ids ? topk_ids : at<int32_t>(ws, L.ids);
  float* gates = topk_w ? topk_w : at<float>(ws, L.gates);
  int32_t* cpre = counts_pre ? counts_pre : at<int32_t>(ws, L.counts_pre);
  int32_t* cnt = counts ? counts : at<int32_t>(ws, L.counts);
  int32_t* offs = offsets ? offsets : at<int32_t>(ws, L.offsets);
  int32_t* sa = sorted_assign ? sorted_assign : at<int32_t>(ws, L.sorted_assign);
  int32_t* ap = assign_pos ? assign_pos : at<int32_t>(ws, L.assign_pos);
  float* out_rows = at<float>(ws, L.out_rows);
  float* out_b = down_ksplit(*p) == 2 ? at<float>(ws, L.out_rows_b) : nullptr;
  float* shared_out = p->n_shared ? at<float>(ws, L.shared_out) : nullptr;
  auto mark = [&](int i) { return ev ? hipEventRecord(ev[i], stream) : hipSuccess; };
  if (mark(0) != hipSuccess) return MOE_EHIP;
  const Schedule sc = schedule_in(*p, L, ws);
  hipError_t e;
  if (small_topk_fused(*p)) {
    // decode-sized: the logits, then top-k, grouping and schedule in one launch
    e = launch_route_logits(*p, x, w_gate, at<float>(ws, L.logits_part), stream);
    if (e != hipSuccess || mark(1) != hipSuccess) return MOE_EHIP;
    e = launch_topk_align_small(*p, kernel_cap(*p), at<float>(ws, L.logits_part), logit_bias,
                                sel_bias, ids, gates, prob_sum, true, cpre, cnt, offs, sa, ap, sc,
                                stream);
    if (e != hipSuccess || mark(2) != hipSuccess || mark(3) != hipSuccess) return MOE_EHIP;
  } else if (small_routing(*p)) {
    // small batches: logits, top-k, then grouping + schedule in one launch
    e = launch_route_logits(*p, x, w_gate, at<float>(ws, L.logits_part), stream);
    if (e != hipSuccess || mark(1) != hipSuccess) return MOE_EHIP;
    e = launch_route_align_small(*p, kernel_cap(*p), at<float>(ws, L.logits_part), logit_bias,
                                 sel_bias, ids, gates, prob_sum, at<float>(ws, L.psum_part), cpre,
                                 cnt, offs, sa, ap, sc, stream);
    if (e != hipSuccess || mark(2) != hipSuccess || mark(3) != hipSuccess) return MOE_EHIP;
  } else {
    e = launch_route(*p, x, w_gate, logit_bias, sel_bias, ids, gates, prob_sum,
                     at<float>(ws, L.logits_part), at<float>(ws, L.psum_part),
                     at<float>(ws, L.psum_stage), stream);
    if (e != hipSuccess || mark(1) != hipSuccess) return MOE_EHIP;
    e = launch_align(*p, kernel_cap(*p), ids, cpre, cnt, offs, sa, ap,
                     at<int32_t>(ws, L.blk_counts), at<int32_t>(ws, L.blk_base), stream);
    if (e != hipSuccess || mark(2) != hipSuccess) return MOE_EHIP;
    if (launch_schedule(*p, offs, sc, stream) != hipSuccess || mark(3) != hipSuccess)
      return MOE_EHIP;
  }
  if (dec_down_combine(*p) && sc.BM == kDecBM) {
    // decode-sized: gate-up, then the down GEMM and the combine in one launch (same bits as
    // the rows-then-combine path below; the "combine" stage is empty)
    e = launch_dec_gate_up(*p, x, w1, w3, sa, sc, at<void>(ws, L.h), stream);
    if (e != hipSuccess || (ev && hipEventRecord(ev[4], stream) != hipSuccess)) return MOE_EHIP;
    e = launch_dec_down_combine(*p, at<void>(ws, L.h), w2, ids, gates, ap, sc, y, stream);
    if (e != hipSuccess || mark(5) != hipSuccess || mark(6) != hipSuccess) return MOE_EHIP;
    return MOE_OK;
  }
  e = launch_expert_ffn(*p, x, w1, w3, w2, ws1, ws3, ws2, sa, sc, at<void>(ws, L.h), out_rows,
                        out_b, shared_out, stream, ev ? ev[4] : nullptr);
  if (e != hipSuccess || mark(5) != hipSuccess) return MOE_EHIP;
  e = launch_combine(*p, out_rows, out_b, ap, gates, shared_out, y, stream);
  if (e != hipSuccess || mark(6) != hipSuccess) return MOE_EHIP;
  return MOE_OK;
}

}  // namespace

MOE_API moe_status moe_forward(const moe_problem* p, const void* x, const void* w_gate,
                               const float* logit_bias, const float* sel_bias, const void* w1,
                               const void* w3, const void* w2, const void* ws1, const void* ws3,
                               const void* ws2, float* y, int32_t* topk_ids, float* topk_w,
                               float* prob_sum, int32_t* counts_pre, int32_t* counts,
                               int32_t* offsets, int32_t* sorted_assign, int32_t* assign_pos,
                               void* ws, size_t ws_bytes, hipStream_t stream) {
  return forward_impl(p, x, w_gate, logit_bias, sel_bias, w1, w3, w2, ws1, ws3, ws2, y, topk_ids,
                      topk_w, prob_sum, counts_pre, counts, offsets, sorted_assign, assign_pos, ws,
                      ws_bytes, stream, nullptr);
}

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device, looked up once per device (with that device
// current, as the lookup requires) and kept for the rest of the process.
moe_status scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_EUNSUPPORTED;
  void* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch[dev].load(std::memory_order_relaxed);
    if (!ptr) {
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MOE_EHIP;
      g_scratch[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return MOE_OK;
}

}  // namespace

MOE_API moe_status moe_forward_noalloc(const moe_problem* p, const void* x, const void* w_gate,
                                       const float* logit_bias, const float* sel_bias,
                                       const void* w1, const void* w3, const void* w2,
                                       const void* ws1, const void* ws3, const void* ws2, float* y,
                                       int32_t* topk_ids, float* topk_w, float* prob_sum,
                                       int32_t* counts_pre, int32_t* counts, int32_t* offsets,
                                       int32_t* sorted_assign, int32_t* assign_pos,
                                       hipStream_t stream) {
  moe_status st = moe_validate(p);
  if (st != MOE_OK) return st;
  if (layout(*p).total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_EWORKSPACE;
  void* ws = nullptr;
  if ((st = scratch_ptr(&ws)) != MOE_OK) return st;
  return forward_impl(p, x, w_gate, logit_bias, sel_bias, w1, w3, w2, ws1, ws3, ws2, y, topk_ids,
                      topk_w, prob_sum, counts_pre, counts, offsets, sorted_assign, assign_pos, ws,
                      (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

MOE_API moe_status moe_forward_staged(const moe_problem* p, const void* x, const void* w_gate,
                                      const float* logit_bias, const float* sel_bias,
                                      const void* w1, const void* w3, const void* w2,
                                      const void* ws1, const void* ws3, const void* ws2, float* y,
                                      void* ws, size_t ws_bytes, hipStream_t stream,
                                      hipEvent_t* stage_events) {
  if (!stage_events) return MOE_EINVAL;
  for (int i = 0; i < MOE_STAGE_EVENTS; ++i)
    if (!stage_events[i]) return MOE_EINVAL;
  return forward_impl(p, x, w_gate, logit_bias, sel_bias, w1, w3, w2, ws1, ws3, ws2, y, nullptr,
                      nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, ws, ws_bytes,
                      stream, stage_events);
}
