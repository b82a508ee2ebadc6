"""Plain fp64 CPU oracle for the sparse top-k MoE layer: forward and backward.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this module:
only the tests, the smoke check and the benchmark's CPU-baseline leg may call
it. It shares no code with the HIP path (no kernels, tables, helpers or pre-
and post-processing); both sides only share the seeded input generator.

Everything is float64 NumPy, written as the plain definition of each step so a
reader can check it against the pages by eye. Library primitives (matmul, a
stable argsort, bincount, exp) serve as single steps; there is no blocking,
fusion or reordering beyond what the definitions state.

Pages cited (by title, then section):
  [Deep Dive]  "MoE (Mixture of Experts) Deep Dive: Principles, Formulas, and
               Implementation" (kongchang.com)
  [Arch]       "MoE Architecture" (infra.bea.ai guide)
  [Notes]      "Mixture of Experts" (avinashkadimisetty.com ML-algorithm notes)
  [Handbook]   "Mixture of experts (MoE)" (ai-infra-handbooks)
  [Concept]    "One Deep Concept #04 -- Mixture of Experts" (Miniblog)

Readings taken where the pages are silent or disagree (each also listed in the
design notes): router weight stored [E, d] (a linear layer's weight); top-k on
the logits plus the selection bias, equal keys broken toward the lower expert
index, slots in descending key order; the selection bias never reaches the
gates or p_i; gates always renormalised over the kept k; capacity
ceil(cf * T*k / E) in IEEE double; overflow dropped first-come in ascending
flat assignment order a = t*k + j with no gate renormalisation afterwards;
f_i counted before dropping over T*k assignments; alpha inside L_balance.

bias_update follows the pages' direction rule; its threshold (the mean load)
and step (a caller parameter) are readings.

moe_backward is the chain rule through the same forward, with the selection
held fixed (top-k and capacity drops have no gradient) and f_i a constant in
the balance loss, as the [Deep Dive] derivation prescribes.

Pin status: every function below is pinned by a `-m "not gpu"` test against
values the pages print, closed forms, library special cases or brute force,
except the readings themselves (drop order, the Zipf offset, what the
selection bias is added to), which no page fixes beyond plausibility.
"""
from __future__ import annotations

import math
from typing import Callable, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "router_logits", "softmax", "selection_keys", "select_topk", "renormalised_gates",
    "route", "capacity", "align", "silu", "swiglu_expert", "moe_forward",
    "moe_forward_naive", "token_output", "token_outputs", "balance", "expert_table",
    "bias_update", "expert_choice_capacity", "expert_choice_route", "moe_forward_expert_choice",
    "sigmoid", "silu_grad", "swiglu_expert_backward", "gate_logit_grad", "balance_logit_grad",
    "moe_backward", "moe_backward_sampled",
]

ExpertFn = Callable[[int], Tuple[np.ndarray, np.ndarray, np.ndarray]]


# ----------------------------------------------------------------------------- router
def router_logits(x: np.ndarray, w_gate: np.ndarray,
                  logit_bias: Optional[np.ndarray] = None) -> np.ndarray:
    """Router scores, one per (token, expert).

    [Arch] §2 "Gating Function" writes the scores as x times W_gate with
    W_gate of shape d x E; [Notes] "Routing math" writes W_g x with W_g of
    shape N x d. Here w_gate is stored [E, d] (the second form), so the
    scores are x @ w_gate.T -- the same numbers as x @ W_gate with
    W_gate = w_gate.T. An optional per-expert offset is part of the logits
    (it enters the softmax, the selection and p_i)."""
    x = np.asarray(x, dtype=np.float64)
    w_gate = np.asarray(w_gate, dtype=np.float64)
    logits = x @ w_gate.T
    if logit_bias is not None:
        logits = logits + np.asarray(logit_bias, dtype=np.float64)[None, :]
    return logits


def softmax(logits: np.ndarray) -> np.ndarray:
    """Softmax over the experts of each token ([Deep Dive] "Router Network
    Computation"; [Arch] §2; [Concept] §4), shifted by the row maximum so no
    exponential overflows (the shift cancels in the ratio)."""
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    return e / e.sum(axis=1, keepdims=True)


def selection_keys(logits: np.ndarray, sel_bias: Optional[np.ndarray] = None) -> np.ndarray:
    """The values top-k selects on: the logits, plus the per-expert balancing
    bias if one is given. [Handbook] "Load balancing" and [Arch] §2 describe
    that bias as used only to choose the experts, never in the weights;
    [Notes] adds it to the router logits."""
    if sel_bias is None:
        return logits
    return logits + np.asarray(sel_bias, dtype=np.float64)[None, :]


def select_topk(keys: np.ndarray, k: int) -> np.ndarray:
    """Each token's k experts with the largest keys, largest first
    ([Arch] §2 route(); [Handbook] "Structure" step 2). Equal keys go to the
    lower expert index (a stable sort of the negated keys keeps index order
    among equals). Selecting on logits rather than probabilities selects the
    same set, since softmax is increasing."""
    order = np.argsort(-keys, axis=1, kind="stable")
    return order[:, :k].astype(np.int64)


def renormalised_gates(probs: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """The kept probabilities divided by their sum, so each token's k gates
    add to 1 ([Deep Dive] "Weighted Sum Output": 0.55 and 0.3 are divided by
    0.85; [Handbook] "Structure"). This equals [Arch]'s softmax over the k
    selected scores."""
    sel = np.take_along_axis(probs, ids, axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def route(x, w_gate, k: int, logit_bias=None, sel_bias=None):
    """Router forward: returns (ids [T,k], gates [T,k], probs [T,E], keys [T,E])."""
    logits = router_logits(x, w_gate, logit_bias)
    probs = softmax(logits)
    keys = selection_keys(logits, sel_bias)
    ids = select_topk(keys, k)
    gates = renormalised_gates(probs, ids)
    return ids, gates, probs, keys


# ----------------------------------------------------------------------------- grouping
def capacity(capacity_factor: float, T: int, k: int, E: int) -> Optional[int]:
    """Per-expert limit on kept assignments, or None for no limit.

    [Notes] "How it works" sizes each expert's buffer as the capacity factor
    times the average load per expert; [Arch] §2 calls it 1.0-1.5x of the
    average. With top-k routing the average is T*k/E assignments, so the limit
    is ceil(cf * (T*k) / E), evaluated in IEEE double in that order."""
    if capacity_factor is None or capacity_factor <= 0:
        return None
    return int(math.ceil(float(capacity_factor) * float(T * k) / float(E)))


def align(ids: np.ndarray, E: int, cap: Optional[int] = None) -> dict:
    """Group the T*k assignments by expert ([Handbook] "Implementation: token
    by token vs. grouped by expert": flatten, stable sort by expert, count,
    segment starts by prefix sum).

    Assignment a = t*k + j goes to expert ids[t, j]. Within an expert the
    assignments keep ascending a. With a capacity limit, assignment a is kept
    iff fewer than `cap` earlier assignments went to its expert; a dropped
    assignment contributes nothing ([Arch] §2 "Expert capacity and token
    dropping"; [Handbook] "Load balancing").

    Returns int64 arrays: counts_pre [E] (before dropping), counts [E] (kept),
    offsets [E+1], sorted_assign [offsets[E]] (flat a, expert-major), and
    assign_pos [T*k] (row of a in sorted order, or -1 if dropped)."""
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    n = flat.size
    counts_pre = np.bincount(flat, minlength=E).astype(np.int64)
    order = np.argsort(flat, kind="stable")          # expert-major, ascending a inside
    starts = np.concatenate([[0], np.cumsum(counts_pre)[:-1]])
    rank = np.empty(n, dtype=np.int64)
    rank[order] = np.arange(n, dtype=np.int64) - starts[flat[order]]
    kept = np.ones(n, dtype=bool) if cap is None else rank < cap
    counts = counts_pre.copy() if cap is None else np.minimum(counts_pre, cap)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    assign_pos = np.where(kept, offsets[flat] + rank, -1).astype(np.int64)
    sorted_assign = np.empty(int(offsets[-1]), dtype=np.int64)
    sorted_assign[assign_pos[kept]] = np.nonzero(kept)[0]
    return dict(counts_pre=counts_pre, counts=counts, offsets=offsets,
                sorted_assign=sorted_assign, assign_pos=assign_pos)


# ----------------------------------------------------------------------------- experts
def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z), evaluated without overflow: for z < 0 the
    sigmoid is written exp(z) / (1 + exp(z))."""
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = z[pos] / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = z[~pos] * ez / (1.0 + ez)
    return out


def swiglu_expert(rows: np.ndarray, w1: np.ndarray, w3: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """One SwiGLU expert on a batch of rows: W2 (SiLU(W1 x) * (W3 x)).

    [Arch] §3 "Standard MoE" makes each expert a SwiGLU FFN with 3*d*d_ff
    parameters; [Handbook]'s expert has a gate projection (through SiLU), an
    up projection and a down projection. w1 = gate [d_ff, d], w3 = up
    [d_ff, d], w2 = down [d, d_ff], all "out x in"."""
    rows = np.asarray(rows, dtype=np.float64)
    u = rows @ np.asarray(w1, dtype=np.float64).T
    v = rows @ np.asarray(w3, dtype=np.float64).T
    h = silu(u) * v
    return h @ np.asarray(w2, dtype=np.float64).T


def expert_table(w1, w3, w2) -> ExpertFn:
    """Wrap stacked [E, ...] arrays as an expert lookup e -> (w1_e, w3_e, w2_e) in fp64."""
    def get(e: int):
        return (np.asarray(w1[e], dtype=np.float64), np.asarray(w3[e], dtype=np.float64),
                np.asarray(w2[e], dtype=np.float64))
    return get


def _shared_sum(x: np.ndarray, shared: Sequence[Tuple[np.ndarray, np.ndarray, np.ndarray]]) -> np.ndarray:
    """Always-on shared experts, ungated and added to the routed sum
    ([Deep Dive] "Shared Experts"; [Arch] §3 "Shared Experts (DeepSeek)")."""
    out = np.zeros((x.shape[0], x.shape[1]), dtype=np.float64)
    for (s1, s3, s2) in shared:
        out += swiglu_expert(x, s1, s3, s2)
    return out


# ----------------------------------------------------------------------------- forward
def moe_forward(x, w_gate, experts: ExpertFn, E: int, k: int, logit_bias=None, sel_bias=None,
                shared: Sequence = (), capacity_factor: float = 0.0, ids=None):
    """Grouped forward ([Handbook] "Implementation": group by expert, one
    batched expert call per non-empty segment, weighted scatter back).

    y[t] = sum over kept slots j of g[t,j] * Expert_{ids[t,j]}(x[t]) + shared(x[t])
    ([Arch] §1; [Notes] "Routing math"). If `ids` is given, routing uses those
    ids and the oracle's own probabilities (gates renormalised over them).
    Returns (y [T,d], info dict with ids, gates, probs, keys and the align
    outputs)."""
    x = np.asarray(x, dtype=np.float64)
    T, d = x.shape
    r_ids, gates, probs, keys = route(x, w_gate, k, logit_bias, sel_bias)
    if ids is not None:
        r_ids = np.asarray(ids, dtype=np.int64)
        gates = renormalised_gates(probs, r_ids)
    cap = capacity(capacity_factor, T, k, E)
    al = align(r_ids, E, cap)
    flat_gates = gates.reshape(-1)
    y = np.zeros((T, d), dtype=np.float64)
    for e in range(E):
        seg = al["sorted_assign"][al["offsets"][e]:al["offsets"][e + 1]]
        if seg.size == 0:                         # an empty group does nothing
            continue
        tok = seg // k
        out = swiglu_expert(x[tok], *experts(e))
        np.add.at(y, tok, flat_gates[seg][:, None] * out)
    y += _shared_sum(x, shared)
    info = dict(ids=r_ids, gates=gates, probs=probs, keys=keys, cap=cap, **al)
    return y, info


def token_output(x_t: np.ndarray, ids_t, gates_t, kept_t, experts: ExpertFn,
                 shared: Sequence = ()) -> np.ndarray:
    """One token's output, slot by slot ([Deep Dive] "Code Implementation
    Essentials" item 3: for each token, for each chosen expert, add the
    gate-weighted expert output), plus the shared experts."""
    x_t = np.asarray(x_t, dtype=np.float64).reshape(1, -1)
    y = np.zeros(x_t.shape[1], dtype=np.float64)
    for j in range(len(ids_t)):
        if kept_t[j]:
            y += float(gates_t[j]) * swiglu_expert(x_t, *experts(int(ids_t[j])))[0]
    y += _shared_sum(x_t, shared)[0]
    return y


def token_outputs(x_rows: np.ndarray, ids_rows, gates_rows, kept_rows, experts: ExpertFn,
                  shared: Sequence = ()) -> np.ndarray:
    """Outputs of a chosen subset of tokens, given each one's routing (ids,
    gates, kept flags): the same weighted sum as token_output, visiting each
    expert once for all the rows that chose it (so one expert's weights are
    fetched once). Used to check sampled rows of a full-size layer."""
    x_rows = np.asarray(x_rows, dtype=np.float64)
    ids_rows = np.asarray(ids_rows, dtype=np.int64)
    gates_rows = np.asarray(gates_rows, dtype=np.float64)
    kept_rows = np.asarray(kept_rows, dtype=bool)
    y = np.zeros_like(x_rows)
    for e in np.unique(ids_rows[kept_rows]):
        rows, slots = np.nonzero((ids_rows == e) & kept_rows)   # a row chooses e at most once
        out = swiglu_expert(x_rows[rows], *experts(int(e)))
        y[rows] += gates_rows[rows, slots][:, None] * out
    y += _shared_sum(x_rows, shared)
    return y


def moe_forward_naive(x, w_gate, experts: ExpertFn, E: int, k: int, logit_bias=None,
                      sel_bias=None, shared: Sequence = (), capacity_factor: float = 0.0):
    """Token-by-token forward ([Handbook] forward_naive's method). The
    capacity rule is applied with a running per-expert counter in ascending
    (t, j) order, a formulation independent of align()'s stable sort."""
    x = np.asarray(x, dtype=np.float64)
    T, d = x.shape
    ids, gates, _, _ = route(x, w_gate, k, logit_bias, sel_bias)
    cap = capacity(capacity_factor, T, k, E)
    used = np.zeros(E, dtype=np.int64)
    y = np.zeros((T, d), dtype=np.float64)
    for t in range(T):
        kept = []
        for j in range(k):
            e = int(ids[t, j])
            ok = cap is None or used[e] < cap
            used[e] += 1
            kept.append(ok)
        y[t] = token_output(x[t], ids[t], gates[t], kept, experts, shared)
    return y


# ----------------------------------------------------------------------------- statistics
def balance(counts_pre: np.ndarray, probs: np.ndarray, T: int, k: int, alpha: float = 0.01):
    """Load statistics and the auxiliary balance loss.

    f_i: share of the T*k routed assignments that chose expert i (counted
    before capacity dropping; [Handbook] "Load balancing" divides the top-k id
    histogram by the number of ids). P_i: mean router probability of expert i
    over the tokens. L = alpha * E * sum_i f_i * P_i ([Arch] §2 "Load
    Balancing"; [Notes] gives alpha ~ 0.01; [Deep Dive] "Load Balancing Loss
    Derivation" has the same N * sum F_i P_i form). Returns (f, P, L)."""
    counts_pre = np.asarray(counts_pre, dtype=np.float64)
    E = counts_pre.size
    f = counts_pre / float(T * k)
    P = np.asarray(probs, dtype=np.float64).mean(axis=0)
    L = float(alpha) * E * float(np.sum(f * P))
    return f, P, L


# ----------------------------------------------------------------------------- bias update
def bias_update(counts_pre: np.ndarray, sel_bias: np.ndarray, gamma: float, T: int,
                k: int) -> np.ndarray:
    """One step of the auxiliary-loss-free balancing bias.

    [Arch] §2 "Auxiliary-loss-free balancing" and [Handbook] "Load balancing":
    a per-expert bias that only enters the top-k choice is lowered for an
    overloaded expert and raised for an idle one, from the observed load.
    The pages give the direction only. Reading: an expert is overloaded when
    its assignment count before capacity dropping exceeds the mean load
    T*k/E and underloaded when it is below it (compared exactly, as
    E*c_e against T*k); the bias moves by the caller's step gamma, and an
    expert at exactly the mean keeps its bias. The bias is an fp32 tensor, so
    the step is taken in fp32: b + gamma * sign(T*k - E*c_e), rounded once.
    """
    c = np.asarray(counts_pre, dtype=np.int64)
    E = c.size
    direction = np.sign(np.int64(T) * np.int64(k) - np.int64(E) * c)   # +1 under, -1 over
    b = np.asarray(sel_bias, dtype=np.float32)
    return (b + np.float32(gamma) * direction.astype(np.float32)).astype(np.float32)


# ----------------------------------------------------------------------------- expert choice
def expert_choice_capacity(capacity_factor: float, T: int, k: int, E: int) -> int:
    """Bucket size C of expert-choice routing.

    [Concept] "Expert Choice -- Reverse Who Selects Whom": experts choose the
    tokens, with fixed bucket sizes. Reading: the bucket is the capacity of
    the token-choice layer, ceil(cf * T*k / E) (k = the average number of
    experts per token), with cf = 1 when no factor is given, and at most T."""
    cf = 1.0 if capacity_factor is None or capacity_factor <= 0 else float(capacity_factor)
    return min(T, int(math.ceil(cf * float(T * k) / float(E))))


def expert_choice_route(x, w_gate, E: int, C: int, logit_bias=None):
    """Each expert picks its C tokens ([Concept] "Expert Choice").

    Scores: the router probabilities p = softmax over experts of the logits
    (the same gate as token choice, [Arch] §2 "Gating Function"). Expert e
    takes the C tokens with the largest p[t, e], equal scores going to the
    lower token index; its bucket lists them in ascending token order. The
    weight of (t, e) is p[t, e] itself: a token may get any number of experts
    (0 to E) and nothing is renormalised over them. Returns
    (tokens [E, C], gates [E, C], probs [T, E])."""
    logits = router_logits(x, w_gate, logit_bias)
    probs = softmax(logits)
    T = probs.shape[0]
    tokens = np.zeros((E, C), dtype=np.int64)
    gates = np.zeros((E, C), dtype=np.float64)
    for e in range(E):
        best = np.argsort(-probs[:, e], kind="stable")[:C]    # stable: ties -> lower t
        tok = np.sort(best)
        tokens[e] = tok
        gates[e] = probs[tok, e]
    return tokens, gates, probs


def moe_forward_expert_choice(x, w_gate, experts: ExpertFn, E: int, C: int, logit_bias=None,
                              shared: Sequence = (), tokens=None):
    """y[t] = sum over experts e whose bucket holds t of p[t,e] * Expert_e(x[t]),
    plus the shared experts, added in expert order. With `tokens` given, the
    buckets are those ([E, C]) and the weights the oracle's own p.
    Returns (y [T,d], info dict with tokens, gates, probs)."""
    x = np.asarray(x, dtype=np.float64)
    T, d = x.shape
    r_tok, gates, probs = expert_choice_route(x, w_gate, E, C, logit_bias)
    if tokens is not None:
        r_tok = np.asarray(tokens, dtype=np.int64)
        gates = np.take_along_axis(probs.T, r_tok, axis=1)
    y = np.zeros((T, d), dtype=np.float64)
    for e in range(E):
        if C == 0:
            break
        tok = r_tok[e]
        out = swiglu_expert(x[tok], *experts(e))
        np.add.at(y, tok, gates[e][:, None] * out)
    y += _shared_sum(x, shared)
    return y, dict(tokens=r_tok, gates=gates, probs=probs)



# ----------------------------------------------------------------------------- backward
# The layer's gradient, written step by step from the chain rule. The objective is
#   J = sum_t <dy_t, y_t> + dL * L_balance,
# where dy is the upstream gradient of the output and dL that of the balance loss. The
# selection (top-k ids, capacity drops) is a discrete decision with no gradient; f_i is the
# count of that decision and is held constant, so the balance loss reaches the router only
# through P_i ([Deep Dive] "Load Balancing Loss Derivation": F is a post-hoc statistic with
# no gradient, P is the differentiable proxy that carries it; [Arch] §2 "Load Balancing").
def sigmoid(z: np.ndarray) -> np.ndarray:
    """1 / (1 + exp(-z)), written as exp(z) / (1 + exp(z)) for z < 0 (no overflow)."""
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def silu_grad(z: np.ndarray) -> np.ndarray:
    """d/dz [z * sigmoid(z)] = sigmoid(z) * (1 + z * (1 - sigmoid(z)))."""
    s = sigmoid(z)
    return s * (1.0 + np.asarray(z, dtype=np.float64) * (1.0 - s))


def swiglu_expert_backward(rows, w1, w3, w2, d_out):
    """Backward of one SwiGLU expert o = W2 (SiLU(W1 x) * (W3 x)) over a batch of rows.

    d_out [n, d] is the gradient of the n output rows. Returns (d_rows [n, d], dw1 [d_ff, d],
    dw3 [d_ff, d], dw2 [d, d_ff], o [n, d]) -- o, the forward output, is what a gate's
    gradient is taken against."""
    rows = np.asarray(rows, dtype=np.float64)
    w1 = np.asarray(w1, dtype=np.float64)
    w3 = np.asarray(w3, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    u = rows @ w1.T
    v = rows @ w3.T
    s = silu(u)
    h = s * v
    o = h @ w2.T
    dw2 = d_out.T @ h                     # o = h W2^T
    dh = d_out @ w2
    du = dh * v * silu_grad(u)            # h = SiLU(u) * v
    dv = dh * s
    dw1 = du.T @ rows                     # u = x W1^T
    dw3 = dv.T @ rows                     # v = x W3^T
    d_rows = du @ w1 + dv @ w3
    return d_rows, dw1, dw3, dw2, o


def gate_logit_grad(gates: np.ndarray, dgate: np.ndarray) -> np.ndarray:
    """Gradient of the k renormalised gates of each token w.r.t. the logits of its selected
    experts. The gates are the selected probabilities over their sum, which is a softmax over
    the k selected logits ([Deep Dive] "Weighted Sum Output"; [Arch] §2 "Gating Function"), so
    d g_j / d l_m = g_j (delta_jm - g_m) for selected m and 0 for the rest. Returns [T, k]:
    the gradient of each selected logit."""
    inner = (gates * dgate).sum(axis=1, keepdims=True)
    return gates * (dgate - inner)


def balance_logit_grad(probs: np.ndarray, counts_pre: np.ndarray, T: int, k: int,
                       alpha: float, dL: float) -> np.ndarray:
    """Gradient of dL * L_balance w.r.t. the router logits, with f held constant.

    L = alpha * E * sum_i f_i P_i and P_i = mean over tokens of p[t, i], so
    dJ/dp[t, i] = dL * alpha * E * f_i / T; the softmax then gives
    dJ/dl[t, e] = p[t, e] * (dJ/dp[t, e] - sum_i p[t, i] dJ/dp[t, i]). Returns [T, E]."""
    probs = np.asarray(probs, dtype=np.float64)
    E = probs.shape[1]
    f = np.asarray(counts_pre, dtype=np.float64) / float(T * k)
    w = float(dL) * float(alpha) * E * f / float(T)
    return probs * (w[None, :] - (probs * w[None, :]).sum(axis=1, keepdims=True))


def moe_backward(x, w_gate, experts: ExpertFn, E: int, k: int, dy, logit_bias=None,
                 sel_bias=None, shared: Sequence = (), capacity_factor: float = 0.0, ids=None,
                 alpha: float = 0.01, dL: float = 0.0):
    """Gradients of J = sum_t <dy_t, y_t> + dL * L_balance w.r.t. every input of the layer.

    The forward is moe_forward's (with `ids` given, routing uses those ids, as there). Each
    kept assignment (t, j) to expert e adds g_tj * o_tj to y_t with o_tj = Expert_e(x_t):
      d g_tj = <dy_t, o_tj>; the expert's rows get d o = g_tj * dy_t;
      a dropped assignment adds nothing, so its d g is 0 (it still sits in the renormalising
      sum of the gates);
      the shared experts take dy_t with gate 1.
    The router: d l = gate part (selected logits) + balance part; dx gets d l W_gate,
    dW_gate = d l^T x, d logit_bias = column sums of d l. sel_bias has no gradient.
    Returns a dict: dx [T,d], dw_gate [E,d], dlogit_bias [E], dw1/dw3 [E,d_ff,d],
    dw2 [E,d,d_ff], dshared (list of (ds1, ds3, ds2)), dgate [T,k], dlogits [T,E], and the
    routing (ids, gates, probs, align outputs)."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    T, d = x.shape
    r_ids, gates, probs, keys = route(x, w_gate, k, logit_bias, sel_bias)
    if ids is not None:
        r_ids = np.asarray(ids, dtype=np.int64)
        gates = renormalised_gates(probs, r_ids)
    cap = capacity(capacity_factor, T, k, E)
    al = align(r_ids, E, cap)
    flat_gates = gates.reshape(-1)
    dx = np.zeros((T, d), dtype=np.float64)
    dgate = np.zeros(T * k, dtype=np.float64)
    dw1, dw3, dw2 = [], [], []
    for e in range(E):
        w1_e, w3_e, w2_e = experts(e)
        seg = al["sorted_assign"][al["offsets"][e]:al["offsets"][e + 1]]
        if seg.size == 0:                         # an expert with no kept rows: zero gradient
            dw1.append(np.zeros_like(w1_e))
            dw3.append(np.zeros_like(w3_e))
            dw2.append(np.zeros_like(w2_e))
            continue
        tok = seg // k
        g = flat_gates[seg]
        d_rows, g1, g3, g2, o = swiglu_expert_backward(x[tok], w1_e, w3_e, w2_e,
                                                       g[:, None] * dy[tok])
        dgate[seg] = (dy[tok] * o).sum(axis=1)
        np.add.at(dx, tok, d_rows)
        dw1.append(g1)
        dw3.append(g3)
        dw2.append(g2)
    dshared = []
    for (s1, s3, s2) in shared:
        d_rows, g1, g3, g2, _ = swiglu_expert_backward(x, s1, s3, s2, dy)
        dx += d_rows
        dshared.append((g1, g3, g2))
    dgate = dgate.reshape(T, k)
    dlogits = np.zeros((T, E), dtype=np.float64)
    if T:
        sel_grad = gate_logit_grad(gates, dgate)
        np.add.at(dlogits, (np.repeat(np.arange(T), k), r_ids.reshape(-1)), sel_grad.reshape(-1))
        if dL:
            dlogits += balance_logit_grad(probs, al["counts_pre"], T, k, alpha, dL)
    w_gate64 = np.asarray(w_gate, dtype=np.float64)
    dx += dlogits @ w_gate64
    return dict(dx=dx, dw_gate=dlogits.T @ x, dlogit_bias=dlogits.sum(axis=0),
                dw1=np.stack(dw1) if E else np.zeros((0,)), dw3=np.stack(dw3) if E else np.zeros((0,)),
                dw2=np.stack(dw2) if E else np.zeros((0,)), dshared=dshared, dgate=dgate,
                dlogits=dlogits, ids=r_ids, gates=gates, probs=probs, cap=cap, **al)


def moe_backward_sampled(x, w_gate, experts: ExpertFn, E: int, k: int, dy, ids, tokens,
                         sample_experts, logit_bias=None, shared: Sequence = (),
                         capacity_factor: float = 0.0, alpha: float = 0.01, dL: float = 0.0):
    """The parts of moe_backward that can be computed one by one on a full-size layer: dx of
    the given tokens and the weight gradients of the given experts, for the batch's routing
    `ids` [T, k] (the whole batch's ids fix the capacity drops and f_i). The same steps as
    moe_backward, restricted: each sampled token's gate gradients come from its own expert
    outputs; an expert's weight gradient sums over all of its kept rows.
    Returns dict(dx [S, d], dlogits [S, E], dgate [S, k], wgrads {e: (dw1, dw3, dw2)})."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    ids = np.asarray(ids, dtype=np.int64)
    T, d = x.shape
    cap = capacity(capacity_factor, T, k, E)
    al = align(ids, E, cap)
    kept = (al["assign_pos"] >= 0).reshape(T, k)
    tokens = np.asarray(tokens, dtype=np.int64)
    xs, dys, ids_s, kept_s = x[tokens], dy[tokens], ids[tokens], kept[tokens]
    probs = softmax(router_logits(xs, w_gate, logit_bias))
    gates = renormalised_gates(probs, ids_s)
    S = tokens.size
    dx = np.zeros((S, d), dtype=np.float64)
    dgate = np.zeros((S, k), dtype=np.float64)
    for e in np.unique(ids_s[kept_s]):
        rows, slots = np.nonzero((ids_s == e) & kept_s)   # a token chooses e at most once
        d_rows, _, _, _, o = swiglu_expert_backward(xs[rows], *experts(int(e)),
                                                    gates[rows, slots][:, None] * dys[rows])
        dgate[rows, slots] = (dys[rows] * o).sum(axis=1)
        np.add.at(dx, rows, d_rows)
    for (s1, s3, s2) in shared:
        d_rows, *_ = swiglu_expert_backward(xs, s1, s3, s2, dys)
        dx += d_rows
    dlogits = np.zeros((S, E), dtype=np.float64)
    if S:
        sel_grad = gate_logit_grad(gates, dgate)
        np.add.at(dlogits, (np.repeat(np.arange(S), k), ids_s.reshape(-1)), sel_grad.reshape(-1))
        if dL:
            dlogits += balance_logit_grad(probs, al["counts_pre"], T, k, alpha, dL)
    dx += dlogits @ np.asarray(w_gate, dtype=np.float64)
    wgrads = {}
    for e in sample_experts:
        seg = al["sorted_assign"][al["offsets"][e]:al["offsets"][e + 1]]
        tok, slot = seg // k, seg % k
        g = renormalised_gates(softmax(router_logits(x[tok], w_gate, logit_bias)), ids[tok])
        _, g1, g3, g2, _ = swiglu_expert_backward(x[tok], *experts(int(e)),
                                                  g[np.arange(tok.size), slot][:, None] * dy[tok])
        wgrads[int(e)] = (g1, g3, g2)
    return dict(dx=dx, dlogits=dlogits, dgate=dgate, wgrads=wgrads)
