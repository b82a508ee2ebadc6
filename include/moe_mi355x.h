/*
 * moe_mi355x.h -- C ABI of the sparse top-k MoE layer forward on one MI355X (gfx950).
 *
 * The layer (pages cited by title and section):
 *   router scores x . W_gate, softmax, top-k with renormalised gates and an
 *   optional selection-only per-expert bias ("MoE Architecture" §2 "The
 *   Router"; "Mixture of experts (MoE)" handbook, "Structure" and "Load
 *   balancing"); grouping of the T*k assignments by expert with an optional
 *   capacity limit that drops overflow (handbook, "Implementation: token by
 *   token vs. grouped by expert"; "MoE Architecture" §2 "Expert capacity and
 *   token dropping"); one SwiGLU FFN per expert over its contiguous segment
 *   ("MoE Architecture" §3 "Standard MoE"); the gate-weighted combine back to
 *   token order plus an always-on shared expert ("MoE Architecture" §1 and §3
 *   "Shared Experts (DeepSeek)").
 *
 * Conventions for every call below:
 *   - Every array argument is a DEVICE pointer owned by the caller; the
 *     library never allocates or frees device memory and keeps no pointer
 *     after returning. Row-major, densely packed.
 *   - Weights use the "out x in" layout of a linear layer: w_gate [E,d],
 *     w1 (gate proj, through SiLU) and w3 (up proj) [E,d_ff,d], w2 (down
 *     proj) [E,d,d_ff]; the shared expert's ws1/ws3 [d_ff_shared,d] and ws2
 *     [d,d_ff_shared].
 *   - x and all weights are stored in problem->dtype (bf16 or fp32);
 *     accumulation is fp32; gates, probabilities, expert output rows and y
 *     are fp32; ids, counts and positions are int32.
 *   - Flat assignment index a = t*k + j (token t, slot j).
 *   - All work is enqueued on `stream` in order; nothing synchronises the host.
 *   - Argument errors return before anything is enqueued. MOE_EHIP means a
 *     launch failed. Faults inside kernels surface at the caller's next
 *     synchronisation. The library is stateless: calls on different streams
 *     with different workspaces may run concurrently.
 *   - `ws` is caller-provided device scratch of at least
 *     moe_workspace_bytes() bytes (any 256-byte-aligned buffer); its contents
 *     on entry are ignored.
 *   - Limits (else MOE_EUNSUPPORTED): 1 <= k <= E <= 256, k <= 32; T >= 0 and
 *     T*k < 2^31; n_shared in {0,1} with d_ff_shared == d_ff when 1; bf16:
 *     d and d_ff multiples of 128; fp32: d a multiple of 4.
 *     Addressing: the kernels index each matrix with 32-bit element offsets, so
 *     T*d, d*d_ff and (padded expert rows)*d_ff must each stay below 2^32. The
 *     padded rows are T*k (or E*C for expert choice) plus at most one row tile
 *     per expert and the shared expert's T rows; a Mixtral-shaped layer (d=4096,
 *     d_ff=14336, k=2) accepts about 148k tokens per call. moe_backward also
 *     needs (padded rows)*max(d, 2*d_ff) below 2^32.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,        /* null pointer where one is required, negative size, bad enum */
  MOE_EUNSUPPORTED = 2,  /* a shape outside the limits above */
  MOE_EWORKSPACE = 3,    /* ws_bytes smaller than moe_workspace_bytes() */
  MOE_EHIP = 4           /* a HIP launch or runtime call failed */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef struct {
  int32_t T;               /* tokens */
  int32_t d;               /* hidden size */
  int32_t E;               /* routed experts */
  int32_t k;               /* experts per token */
  int32_t d_ff;            /* routed-expert intermediate size */
  int32_t n_shared;        /* always-on shared experts: 0 or 1 */
  int32_t d_ff_shared;     /* shared-expert intermediate size (== d_ff when n_shared = 1) */
  int32_t dtype;           /* moe_dtype: storage of x and every weight */
  double capacity_factor;  /* <= 0: no limit; else cap = ceil(capacity_factor * (T*k) / E),
                              evaluated in IEEE double in that order */
} moe_problem;

/* Host-only helpers (no HIP call, no GPU needed). */
const char* moe_status_str(int status);
/* Checks every field against the limits above. */
moe_status moe_validate(const moe_problem* p);
/* Capacity limit in assignments per expert, or -1 for no limit
   ("Mixture of Experts" notes, "How it works": capacity factor times the
   average load per expert; the average with top-k routing is T*k/E). */
moe_status moe_capacity(const moe_problem* p, int32_t* cap_out);
/* Scratch bytes any entry point below may need for problem p (the maximum
   over all of them, moe_forward included). */
moe_status moe_workspace_bytes(const moe_problem* p, size_t* bytes_out);

/* Router: logits l = x . w_gate^T (+ logit_bias), p = softmax(l) over the E
   experts, keys = l (+ sel_bias), the k largest keys per token in descending
   order (equal keys: lower expert index first), gates = p at those experts
   divided by their sum ("MoE (Mixture of Experts) Deep Dive", "Router Network
   Computation" and "Weighted Sum Output"; "MoE Architecture" §2 "Gating
   Function"). sel_bias only chooses experts, never enters gates or p
   (handbook "Load balancing": the DeepSeek-V3 bias).
     x [T,d] dtype; w_gate [E,d] dtype; logit_bias [E] fp32 or NULL;
     sel_bias [E] fp32 or NULL;
     topk_ids [T,k] int32 out; topk_w [T,k] fp32 out;
     prob_sum [E] fp32 out or NULL: sum over tokens of p[t,e]. */
moe_status moe_route(const moe_problem* p, const void* x, const void* w_gate,
                     const float* logit_bias, const float* sel_bias,
                     int32_t* topk_ids, float* topk_w, float* prob_sum,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/* Grouping by expert (handbook "Implementation: token by token vs. grouped
   by expert": per-expert count is a histogram, segment starts a prefix sum,
   assignments sorted stably by expert). Assignment a is kept iff fewer than
   cap earlier assignments (smaller a) chose its expert; dropped assignments
   contribute nothing ("MoE Architecture" §2 "Expert capacity and token
   dropping"). Bit-exact and deterministic.
     topk_ids [T,k] int32 in, each in [0,E) (an id outside that range is
       treated as dropped and counted nowhere);
     counts_pre [E] out: assignments per expert before dropping;
     counts [E] out: kept per expert; offsets [E+1] out: exclusive prefix of counts;
     sorted_assign [T*k] out: flat a of kept assignments, expert-major,
       ascending a inside an expert; the first offsets[E] entries are valid;
     assign_pos [T*k] out: row of a in sorted order, -1 if dropped. */
moe_status moe_align(const moe_problem* p, const int32_t* topk_ids,
                     int32_t* counts_pre, int32_t* counts, int32_t* offsets,
                     int32_t* sorted_assign, int32_t* assign_pos,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/* Expert FFNs: for each kept assignment row r of expert e (token t =
   sorted_assign[r] / k), out_rows[r] = w2_e (SiLU(w1_e x_t) * (w3_e x_t))
   ("MoE Architecture" §3 "Standard MoE": SwiGLU experts; handbook Expert:
   gate, up and down projections). With a shared expert, shared_out[t] is the
   same FFN with ws1/ws3/ws2 on every token ("MoE Architecture" §3 "Shared
   Experts (DeepSeek)").
     x [T,d]; w1,w3 [E,d_ff,d]; w2 [E,d,d_ff]; ws1,ws3,ws2 or NULL (n_shared=0);
     sorted_assign, offsets as produced by moe_align;
     out_rows [T*k,d] fp32 out (rows >= offsets[E] untouched);
     shared_out [T,d] fp32 out, or NULL when n_shared = 0. */
moe_status moe_expert_ffn(const moe_problem* p, const void* x,
                          const void* w1, const void* w3, const void* w2,
                          const void* ws1, const void* ws3, const void* ws2,
                          const int32_t* sorted_assign, const int32_t* offsets,
                          float* out_rows, float* shared_out,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/* Combine: y[t] = sum over slots j with assign_pos[t*k+j] >= 0 of
   topk_w[t*k+j] * out_rows[assign_pos[t*k+j]], plus shared_out[t] if given
   ("MoE Architecture" §1: y is the gate-weighted sum of the chosen experts;
   dropped slots add nothing and the remaining gates are not renormalised).
     y [T,d] fp32 out. */
moe_status moe_combine(const moe_problem* p, const float* out_rows, const int32_t* assign_pos,
                       const float* topk_w, const float* shared_out, float* y,
                       hipStream_t stream);

/* Balance statistics: f[e] = counts_pre[e] / (T*k), P[e] = prob_sum[e] / T,
   L = alpha * E * sum_e f[e] * P[e] ("MoE Architecture" §2 "Load Balancing";
   the Deep Dive's "Load Balancing Loss Derivation" has the same form).
     f [E], P [E], L [1] fp32 out. */
moe_status moe_balance(const moe_problem* p, const int32_t* counts_pre, const float* prob_sum,
                       float alpha, float* f, float* P, float* L, hipStream_t stream);

/* Auxiliary-loss-free balancing step ("MoE Architecture" §2 "Auxiliary-loss-free
   balancing"; handbook "Load balancing"): the per-expert selection bias (the sel_bias
   argument of moe_route / moe_forward, which only chooses experts) is lowered for an
   overloaded expert and raised for an underloaded one. An expert is overloaded when
   its count before capacity dropping exceeds the mean load T*k/E (compared exactly as
   E*counts_pre[e] against T*k) and underloaded when below; at the mean it keeps its
   bias. In fp32: sel_bias[e] += gamma * sign(T*k - E*counts_pre[e]).
     counts_pre [E] as produced by moe_align / moe_forward (device);
     sel_bias [E] fp32, updated in place (device);
     gamma: step, finite and >= 0 (the pages give no value). EINVAL otherwise. */
moe_status moe_bias_update(const moe_problem* p, const int32_t* counts_pre, float gamma,
                           float* sel_bias, hipStream_t stream);

/* Expert-choice routing ("One Deep Concept #04", "Expert Choice -- Reverse Who Selects
   Whom": the experts choose the tokens, with fixed bucket sizes, so a token may get any
   number of experts). Scores are the router probabilities p = softmax over experts of
   x * w_gate^T (+ logit_bias) ("MoE Architecture" §2 "Gating Function"). Expert e takes
   the C tokens with the largest p[t,e], equal scores going to the lower token, and
   y[t] = shared(x[t]) + sum over the experts e that took t, in expert order, of
   p[t,e] * Expert_e(x[t]); nothing is renormalised.
   Bucket size: C = ceil(cf * T*k / E) evaluated in double (cf = capacity_factor, or 1
   when it is <= 0), at most T; k is the mean number of experts per token. */
moe_status moe_expert_choice_capacity(const moe_problem* p, int32_t* c_out);

/* Workspace bytes of moe_forward_expert_choice (host-only). */
moe_status moe_expert_choice_workspace_bytes(const moe_problem* p, size_t* bytes_out);

/* The expert-choice layer.
     x, w_gate, logit_bias, w1/w3/w2, ws1/ws3/ws2: as for moe_forward (no selection bias);
     y [T,d] fp32 out;
     tokens_out [E*C] int32 out or NULL: expert e's bucket at e*C, ascending token ids;
     gates_out [E*C] fp32 out or NULL: p[t,e] of each bucket slot;
     prob_sum [E] fp32 out or NULL: sum over tokens of p[t,e];
     ws: moe_expert_choice_workspace_bytes bytes. Errors as moe_forward. */
moe_status moe_forward_expert_choice(const moe_problem* p, const void* x, const void* w_gate,
                                     const float* logit_bias, const void* w1, const void* w3,
                                     const void* w2, const void* ws1, const void* ws3,
                                     const void* ws2, float* y, int32_t* tokens_out,
                                     float* gates_out, float* prob_sum, void* ws,
                                     size_t ws_bytes, hipStream_t stream);

/* The whole layer in one call: route -> align -> expert FFNs -> combine.
   y [T,d] fp32 out (required). Every routing output pointer may be NULL, in
   which case it lives in ws; when given, it receives the same values the
   separate calls above would produce (prob_sum: the same sum, possibly added
   in a different order when T*k <= 1024, where routing runs in one launch). */
moe_status moe_forward(const moe_problem* p, const void* x, const void* w_gate,
                       const float* logit_bias, const float* sel_bias,
                       const void* w1, const void* w3, const void* w2,
                       const void* ws1, const void* ws3, const void* ws2,
                       float* y,
                       int32_t* topk_ids, float* topk_w, float* prob_sum,
                       int32_t* counts_pre, int32_t* counts, int32_t* offsets,
                       int32_t* sorted_assign, int32_t* assign_pos,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_forward without a workspace argument, for callers that cannot allocate device memory
   (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). It
   allocates nothing: its scratch is one library-owned array of MOE_NOALLOC_SCRATCH_BYTES per
   GPU, held from the first call on that GPU until the process ends. Same arguments, outputs
   and errors as moe_forward, plus MOE_EWORKSPACE when the problem's moe_workspace_bytes()
   exceeds MOE_NOALLOC_SCRATCH_BYTES (for example a decode-sized layer with d = 2048, E = 128,
   k = 8, d_ff = 768 fits up to T = 256). Runs on the current device, which must be the
   stream's. Every call on one GPU shares that GPU's array: calls that overlap in time on one
   GPU (different streams, or threads) race and give wrong results; calls ordered on one stream
   are safe. Nothing in the array needs to start at any value. */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
moe_status moe_forward_noalloc(const moe_problem* p, const void* x, const void* w_gate,
                               const float* logit_bias, const float* sel_bias,
                               const void* w1, const void* w3, const void* w2,
                               const void* ws1, const void* ws3, const void* ws2,
                               float* y,
                               int32_t* topk_ids, float* topk_w, float* prob_sum,
                               int32_t* counts_pre, int32_t* counts, int32_t* offsets,
                               int32_t* sorted_assign, int32_t* assign_pos,
                               hipStream_t stream);

/* Per-stage timing of moe_forward, for measurement tools. Same computation and
   kernels as moe_forward (routing outputs stay in ws), and additionally records
   caller-created HIP events on `stream`: stage_events[0] before the router,
   then one after each stage -- [1] route, [2] align, [3] GEMM schedule,
   [4] gate-up GEMM (+SwiGLU), [5] down GEMM, [6] combine. The caller owns
   the events (hipEventCreate) and reads them with hipEventElapsedTime after
   synchronising. Returns MOE_EINVAL if stage_events or any of its
   MOE_STAGE_EVENTS entries is NULL. */
#define MOE_STAGE_EVENTS 7
moe_status moe_forward_staged(const moe_problem* p, const void* x, const void* w_gate,
                              const float* logit_bias, const float* sel_bias,
                              const void* w1, const void* w3, const void* w2,
                              const void* ws1, const void* ws3, const void* ws2, float* y,
                              void* ws, size_t ws_bytes, hipStream_t stream,
                              hipEvent_t* stage_events);

/* Workspace bytes of moe_backward (host-only). MOE_EUNSUPPORTED unless dtype is
   MOE_BF16 and k <= 16. */
moe_status moe_backward_workspace_bytes(const moe_problem* p, size_t* bytes_out);

/* Layer backward: the gradient of J = sum_t <dy_t, y_t> + dL * L_balance with respect to
   every input of the layer, for the routing a moe_forward call produced.
   The selection (top-k ids, capacity drops) is held fixed -- it has no gradient -- and f_i
   is its count, a constant in L_balance = alpha * E * sum_i f_i P_i, so the balance term
   reaches the router only through P ("MoE (Mixture of Experts) Deep Dive", "Load
   Balancing Loss Derivation"; "MoE Architecture" §2 "Load Balancing"). The gates are a
   softmax over the k selected logits ("Weighted Sum Output"; §2 "Gating Function"), so a
   gate's gradient reaches only the selected logits; a dropped slot has a zero gate
   gradient but stays in its token's renormalising sum. SwiGLU experts as in §3.
     x, w_gate, logit_bias, w1/w3/w2, ws1/ws3/ws2: the forward's inputs (bf16 storage);
     topk_ids, topk_w, counts_pre, offsets, sorted_assign, assign_pos: the forward's
       routing outputs, unchanged (device);
     dy [T,d] fp32: gradient of y; alpha: the balance loss's alpha; dL: gradient of
       L_balance (0 leaves the balance term out); both finite;
     dx [T,d] fp32 out; dw_gate [E,d] fp32 out; dlogit_bias [E] fp32 out or NULL;
     dw1, dw3 [E,d_ff,d] and dw2 [E,d,d_ff] out, bf16 (the weights' storage type; an
       expert with no kept rows gets zeros); dws1/dws3/dws2 likewise for the shared
       expert (required when n_shared = 1);
     ws: moe_backward_workspace_bytes bytes, caller-owned scratch.
   Rounding: dy, g*dy, du, dv and the router's logit gradient enter the MFMA products as
   bf16 (fp32 accumulation); u and v are recomputed with the forward's own gate-up GEMM.
   Errors: MOE_EINVAL for a NULL required pointer or a non-finite alpha / dL,
   MOE_EUNSUPPORTED for fp32 storage or k > 16, MOE_EWORKSPACE, MOE_EHIP. */
moe_status moe_backward(const moe_problem* p, const void* x, const void* w_gate,
                        const float* logit_bias, const void* w1, const void* w3, const void* w2,
                        const void* ws1, const void* ws3, const void* ws2,
                        const int32_t* topk_ids, const float* topk_w, const int32_t* counts_pre,
                        const int32_t* offsets, const int32_t* sorted_assign,
                        const int32_t* assign_pos, const float* dy, float alpha, float dL,
                        float* dx, float* dw_gate, float* dlogit_bias, void* dw1, void* dw3,
                        void* dw2, void* dws1, void* dws3, void* dws2, void* ws,
                        size_t ws_bytes, hipStream_t stream);

/* Per-stage timing of moe_backward, for measurement tools: the same computation, and
   additionally records caller-created HIP events on `stream`: stage_events[0] before the
   first kernel, then one after each stage -- [1] gate-up recompute, [2] row preparation
   (bf16 dy, g*dy, gathered x), [3] dgrad-down + SwiGLU backward, [4] dgrad-x, [5] wgrad-down,
   [6] wgrad-up, [7] router logit gradient, [8] router dgrad, [9] router wgrad, [10] dx
   gather. MOE_EINVAL if stage_events or any of its entries is NULL. */
#define MOE_BWD_STAGE_EVENTS 11
moe_status moe_backward_staged(const moe_problem* p, const void* x, const void* w_gate,
                               const float* logit_bias, const void* w1, const void* w3,
                               const void* w2, const void* ws1, const void* ws3, const void* ws2,
                               const int32_t* topk_ids, const float* topk_w,
                               const int32_t* counts_pre, const int32_t* offsets,
                               const int32_t* sorted_assign, const int32_t* assign_pos,
                               const float* dy, float alpha, float dL, float* dx,
                               float* dw_gate, float* dlogit_bias, void* dw1, void* dw3,
                               void* dw2, void* dws1, void* dws3, void* dws2, void* ws,
                               size_t ws_bytes, hipStream_t stream, hipEvent_t* stage_events);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
