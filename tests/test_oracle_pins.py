"""Pins for the fp64 oracle: values the pages print, closed forms, special
cases that reduce to library routines, invariants and brute force on tiny
inputs. CPU only (no GPU marker).

Each pin is a plain function that raises AssertionError; the same functions
are re-run against deliberately broken copies of the oracle (planted
mistakes) at the bottom of this file, to show that a plausible slip anywhere
in the oracle fails at least one pin."""
import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.moe_oracle as O
import workloads
from util import golden, oracle_inputs

RNG = np.random.default_rng(1234)


def _experts(rng, E, d, d_ff, std=0.3):
    w1 = rng.normal(0, std, (E, d_ff, d))
    w3 = rng.normal(0, std, (E, d_ff, d))
    w2 = rng.normal(0, std, (E, d, d_ff))
    return w1, w3, w2


def _torch_swiglu(x, w1, w3, w2):
    """Dense SwiGLU FFN from torch's library ops, fp64 CPU."""
    xt = torch.from_numpy(np.ascontiguousarray(x))
    return F.linear(F.silu(F.linear(xt, torch.from_numpy(w1))) * F.linear(xt, torch.from_numpy(w3)),
                    torch.from_numpy(w2)).numpy()


# ============================================================================ pins
def pin_gates_worked_example():
    """[Deep Dive] 'Weighted Sum Output': 0.55 and 0.3 divided by 0.85."""
    g = golden("gate_renorm_deep_dive.json")
    p = np.array(g["probs"])
    # d = 1, x = 1 and w_gate[e] = ln p_e makes the logits ln p, whose softmax is p.
    ids, gates, probs, _ = O.route(np.ones((1, 1)), np.log(p)[:, None], g["k"])
    assert ids[0].tolist() == g["expected_ids"], ids
    np.testing.assert_allclose(probs[0], p, rtol=1e-14, atol=0)
    np.testing.assert_allclose(gates[0], g["expected_gates"], rtol=1e-14, atol=0)


def pin_gates_flowchart():
    """[Notes] flowchart: experts 3 and 7 kept with 0.7 / 0.3; y = 0.7 E3 + 0.3 E7."""
    g = golden("gate_flowchart_notes.json")
    E, k = g["E"], g["k"]
    rng = np.random.default_rng(7)
    d, d_ff = 6, 10
    w1, w3, w2 = _experts(rng, E, d, d_ff)
    x = rng.normal(0, 1, (1, d))
    # logits: ln 0.7 and ln 0.3 on experts 3 and 7, far lower elsewhere
    target = np.full(E, -40.0)
    target[3], target[7] = math.log(0.7), math.log(0.3)
    # w_gate = outer(target, x) / |x|^2 makes x @ w_gate.T == target
    w_gate = np.outer(target, x[0]) / float(x[0] @ x[0])
    y, info = O.moe_forward(x, w_gate, O.expert_table(w1, w3, w2), E, k)
    assert info["ids"][0].tolist() == g["expected_ids"]
    np.testing.assert_allclose(info["gates"][0], g["expected_gates"], rtol=1e-12)
    want = 0.7 * _torch_swiglu(x, w1[3], w3[3], w2[3]) + 0.3 * _torch_swiglu(x, w1[7], w3[7], w2[7])
    np.testing.assert_allclose(y, want, rtol=1e-10, atol=1e-12)


def _brute_topk(keys_row, k):
    """Max-sum k-subset; ties between subsets -> lexicographically smallest ids;
    inside the subset: descending key, equal keys by lower index."""
    best, best_sum = None, None
    for comb in itertools.combinations(range(len(keys_row)), k):   # lexicographic order
        s = sum(keys_row[list(comb)])
        if best is None or s > best_sum:
            best, best_sum = comb, s
    return sorted(best, key=lambda e: (-keys_row[e], e))


def pin_topk_brute_force():
    rng = np.random.default_rng(11)
    for trial in range(300):
        T, E = rng.integers(1, 7), rng.integers(1, 7)
        k = int(rng.integers(1, min(E, 3) + 1))
        # integer-valued keys so that ties are common and sums are exact
        keys = rng.integers(-2, 3, (T, E)).astype(np.float64)
        ids = O.select_topk(keys, k)
        for t in range(T):
            assert ids[t].tolist() == _brute_topk(keys[t], k), (keys[t], ids[t])


def pin_zero_input():
    """x = 0: all logits tie at 0, so ids are 0..k-1 (lower index wins), each
    gate is 1/k, and SiLU(0) = 0 makes the output exactly 0."""
    rng = np.random.default_rng(3)
    E, k, d, d_ff, T = 7, 3, 5, 9, 4
    w1, w3, w2 = _experts(rng, E, d, d_ff)
    w_gate = rng.normal(0, 1, (E, d))
    y, info = O.moe_forward(np.zeros((T, d)), w_gate, O.expert_table(w1, w3, w2), E, k)
    assert (info["ids"] == np.arange(k)[None, :]).all()
    np.testing.assert_array_equal(info["gates"], np.full((T, k), 1.0 / k))
    np.testing.assert_array_equal(y, 0.0)


def pin_gates_sum_to_one():
    rng = np.random.default_rng(5)
    x, w = rng.normal(0, 1, (40, 12)), rng.normal(0, 1, (9, 12))
    for k in (1, 2, 5, 9):
        _, gates, probs, _ = O.route(x, w, k)
        np.testing.assert_allclose(gates.sum(1), 1.0, rtol=0, atol=1e-14)
        np.testing.assert_allclose(probs.sum(1), 1.0, rtol=0, atol=1e-14)
        # k = E: renormalised gates are the plain softmax weights, in key order
        if k == 9:
            ids, _, _, _ = O.route(x, w, k)
            np.testing.assert_allclose(gates, np.take_along_axis(probs, ids, 1), rtol=1e-14)


def pin_softmax_library():
    """Softmax equals torch's, including on logits large enough to overflow exp."""
    rng = np.random.default_rng(9)
    logits = rng.normal(0, 50, (30, 11)) + 800.0
    np.testing.assert_allclose(O.softmax(logits), torch.softmax(torch.from_numpy(logits), 1).numpy(),
                               rtol=1e-12, atol=1e-300)


def pin_selection_bias_only_selects():
    """[Handbook] 'Load balancing': the bias chooses experts but never weights
    them. With x = 0 every probability is 1/E, so whichever experts the bias
    picks, each gate must be exactly 1/k; and p_i stays 1/E."""
    E, k, d = 8, 3, 4
    sel = np.zeros(E)
    sel[[6, 1, 4]] = [0.5, 0.9, 0.2]
    ids, gates, probs, keys = O.route(np.zeros((2, d)), np.ones((E, d)), k, sel_bias=sel)
    assert ids.tolist() == [[1, 6, 4]] * 2
    np.testing.assert_array_equal(gates, np.full((2, k), 1.0 / k))
    np.testing.assert_array_equal(probs, np.full((2, E), 1.0 / E))


def pin_logit_bias_enters_softmax():
    """A logit offset of ln q on zero scores makes the router probabilities
    exactly q (closed form), and the gates q renormalised over the top-k."""
    q = np.array([0.05, 0.4, 0.1, 0.25, 0.2])
    ids, gates, probs, _ = O.route(np.zeros((3, 2)), np.zeros((5, 2)), 2, logit_bias=np.log(q))
    np.testing.assert_allclose(probs, np.tile(q, (3, 1)), rtol=1e-14)
    assert ids.tolist() == [[1, 3]] * 3
    np.testing.assert_allclose(gates, np.tile([0.4 / 0.65, 0.25 / 0.65], (3, 1)), rtol=1e-14)


def pin_dense_swiglu_E1():
    """E = 1, k = 1: the layer is a dense SwiGLU FFN (torch library ops)."""
    rng = np.random.default_rng(13)
    d, d_ff, T = 6, 11, 9
    w1, w3, w2 = _experts(rng, 1, d, d_ff)
    x = rng.normal(0, 1.5, (T, d))
    y, _ = O.moe_forward(x, rng.normal(0, 1, (1, d)), O.expert_table(w1, w3, w2), 1, 1)
    np.testing.assert_allclose(y, _torch_swiglu(x, w1[0], w3[0], w2[0]), rtol=1e-11, atol=1e-13)


def pin_k_equals_E():
    """k = E, no capacity: y = sum_e softmax(x W_gate)_e * FFN_e(x), with the
    softmax and the FFNs from torch's library ops."""
    rng = np.random.default_rng(17)
    E, d, d_ff, T = 5, 7, 6, 8
    w1, w3, w2 = _experts(rng, E, d, d_ff)
    wg = rng.normal(0, 1, (E, d))
    x = rng.normal(0, 1, (T, d))
    y, _ = O.moe_forward(x, wg, O.expert_table(w1, w3, w2), E, E)
    p = torch.softmax(torch.from_numpy(x) @ torch.from_numpy(wg).T, dim=1).numpy()
    want = sum(p[:, e:e + 1] * _torch_swiglu(x, w1[e], w3[e], w2[e]) for e in range(E))
    np.testing.assert_allclose(y, want, rtol=1e-11, atol=1e-13)


def pin_naive_equals_grouped_handbook():
    """[Handbook] 'Implementation': token-by-token and grouped-by-expert agree
    (the page checks fp32 to 1e-5 at d=64, d_ff=128, E=16, k=4, 50 tokens, one
    shared expert; in fp64 they must agree to rounding)."""
    w = workloads.get("handbook_fp32")
    inp = oracle_inputs(workloads.generate(w))
    ex = O.expert_table(inp["w1"], inp["w3"], inp["w2"])
    shared = [(inp["ws1"][0], inp["ws3"][0], inp["ws2"][0])]
    a, _ = O.moe_forward(inp["x"], inp["w_gate"], ex, w.E, w.k, shared=shared)
    b = O.moe_forward_naive(inp["x"], inp["w_gate"], ex, w.E, w.k, shared=shared)
    assert np.linalg.norm(a - b) <= 1e-12 * np.linalg.norm(b)


def pin_naive_equals_grouped_capacity():
    rng = np.random.default_rng(19)
    E, k, d, d_ff, T = 6, 2, 5, 8, 30
    w1, w3, w2 = _experts(rng, E, d, d_ff)
    wg = rng.normal(0, 1, (E, d))
    wg[0] += 2.0                       # skew toward expert 0 so the cap bites
    x = rng.normal(0, 1, (T, d)) + 0.5
    ex = O.expert_table(w1, w3, w2)
    for cf in (0.5, 1.0, 1.25):
        a, info = O.moe_forward(x, wg, ex, E, k, capacity_factor=cf)
        assert (info["assign_pos"] < 0).any()
        b = O.moe_forward_naive(x, wg, ex, E, k, capacity_factor=cf)
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


def _brute_align(ids, E, cap):
    """O(E*T*k): scan experts in order, then assignments in order."""
    T, k = ids.shape
    flat = ids.reshape(-1)
    counts_pre, counts, sorted_assign, assign_pos = [], [], [], [-1] * flat.size
    for e in range(E):
        c = 0
        for a in range(flat.size):
            if flat[a] == e:
                if cap is None or c < cap:
                    assign_pos[a] = len(sorted_assign)
                    sorted_assign.append(a)
                c += 1
        counts_pre.append(c)
        counts.append(c if cap is None else min(c, cap))
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    return dict(counts_pre=counts_pre, counts=counts, offsets=offsets,
                sorted_assign=sorted_assign, assign_pos=assign_pos)


def pin_align_brute_force():
    rng = np.random.default_rng(23)
    for trial in range(200):
        E = int(rng.integers(1, 9))
        k = int(rng.integers(1, E + 1))
        T = int(rng.integers(0, 12))
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]) if T else np.zeros((0, k), int)
        cap = [None, 1, 2, 3, 7][trial % 5]
        got = O.align(ids, E, cap)
        want = _brute_align(ids, E, cap)
        for key in want:
            assert np.asarray(got[key]).tolist() == want[key], (key, ids, cap)


def pin_align_invariants():
    rng = np.random.default_rng(29)
    E, k, T = 16, 4, 300
    ids = np.stack([rng.choice(E, k, replace=False, p=np.arange(1, E + 1) / (E * (E + 1) / 2))
                    for _ in range(T)])
    for cap in (None, 10, 75, 10_000):
        al = O.align(ids, E, cap)
        flat = ids.reshape(-1)
        kept = al["assign_pos"] >= 0
        assert sorted(al["sorted_assign"].tolist()) == np.nonzero(kept)[0].tolist()
        assert (al["assign_pos"][al["sorted_assign"]] == np.arange(al["offsets"][-1])).all()
        for e in range(E):
            seg = al["sorted_assign"][al["offsets"][e]:al["offsets"][e + 1]]
            assert (flat[seg] == e).all() and (np.diff(seg) > 0).all()
        assert al["offsets"][-1] == T * k - (~kept).sum()
        if cap is None or cap >= T:
            assert kept.all()
    big = O.align(ids, E, 10_000)
    none = O.align(ids, E, None)
    for key in none:
        assert (np.asarray(big[key]) == np.asarray(none[key])).all()


def pin_capacity_values():
    """ceil(cf * T*k / E): the skewed workload's limit is exactly 640; no
    capacity factor means no limit."""
    w = workloads.get("skew_cap")
    assert O.capacity(*workloads.capacity_inputs(w)) == 640
    assert O.capacity(0.0, 10, 2, 4) is None
    assert O.capacity(1.0, 10, 2, 4) == 5
    assert O.capacity(1.0, 10, 2, 3) == 7          # ceil(20/3)
    assert O.capacity(1.25, 4096, 8, 256) == 160


def pin_silu():
    z = np.array([-1000.0, -30.0, -1.0, 0.0, 1e-300, 1.0, 30.0, 1000.0])
    with np.errstate(over="raise", invalid="raise"):
        s = O.silu(z)
    assert s[3] == 0.0 and s[0] == 0.0 and s[-1] == 1000.0
    # z*sig(z) - (-z)*sig(-z) = z, since sig(z) + sig(-z) = 1
    np.testing.assert_allclose(s - O.silu(-z), z, rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(s, F.silu(torch.from_numpy(z)).numpy(), rtol=1e-15, atol=1e-300)


def pin_balance_uniform():
    """f = P = 1/E gives L = alpha (and E * sum f P = 1 without alpha)."""
    E, T, k = 16, 64, 4
    ids = np.array([[(t * k + j) % E for j in range(k)] for t in range(T)])
    counts_pre = O.align(ids, E)["counts_pre"]
    f, P, L = O.balance(counts_pre, np.full((T, E), 1.0 / E), T, k, alpha=0.01)
    np.testing.assert_allclose(f, 1.0 / E, rtol=1e-15)
    assert abs(L - 0.01) < 1e-15 and abs(f.sum() - 1) < 1e-15


def pin_balance_handbook():
    """[Handbook] simulation: ~1 balanced (alpha excluded); all tokens on the
    first 4 of 16 experts with probability 0.25 each gives 4."""
    g = golden("aux_loss_handbook.json")
    E, k, T = g["E"], g["k"], g["tokens"]
    skew_p = np.zeros((T, E))
    skew_p[:, :k] = 0.25
    bad_ids = np.tile(np.arange(k), (T, 1))
    _, _, L = O.balance(O.align(bad_ids, E)["counts_pre"], skew_p, T, k, alpha=1.0)
    assert abs(L - g["skewed_without_alpha"]) < 1e-14
    _, _, La = O.balance(O.align(bad_ids, E)["counts_pre"], skew_p, T, k, alpha=g["alpha"])
    assert abs(La - g["alpha"] * g["skewed_without_alpha"]) < 1e-15
    # a random router on many tokens is close to balanced: L / alpha ~ 1
    rng = np.random.default_rng(31)
    x, wg = rng.normal(0, 1, (4000, 32)), rng.normal(0, 0.02, (E, 32))
    ids, _, probs, _ = O.route(x, wg, k)
    _, _, Lr = O.balance(O.align(ids, E)["counts_pre"], probs, 4000, k, alpha=1.0)
    assert abs(Lr - g["balanced_without_alpha"]) < 0.02 and Lr < g["skewed_without_alpha"]


def pin_sum_sq():
    """[Deep Dive]: sum of squared frequencies, 1 for (1, 0) and 0.5 for (0.5, 0.5)."""
    g = golden("sum_sq_deep_dive.json")
    T = 10
    for case, ids in zip(g["cases"], (np.zeros((T, 1), int), np.array([[t % 2] for t in range(T)]))):
        f, _, _ = O.balance(O.align(ids, 2)["counts_pre"], np.full((T, 2), 0.5), T, 1)
        np.testing.assert_allclose(f, case["F"])
        assert abs(float((f ** 2).sum()) - case["sum_sq"]) < 1e-15


def pin_equivariance_and_scaling():
    """No capacity: permuting tokens permutes y; scaling every W2 by c scales
    the routed output by c (shared expert absent)."""
    rng = np.random.default_rng(37)
    E, k, d, d_ff, T = 6, 2, 5, 7, 20
    w1, w3, w2 = _experts(rng, E, d, d_ff)
    wg, x = rng.normal(0, 1, (E, d)), rng.normal(0, 1, (T, d))
    y, _ = O.moe_forward(x, wg, O.expert_table(w1, w3, w2), E, k)
    perm = rng.permutation(T)
    yp, _ = O.moe_forward(x[perm], wg, O.expert_table(w1, w3, w2), E, k)
    np.testing.assert_allclose(yp, y[perm], rtol=1e-13, atol=1e-15)
    yc, _ = O.moe_forward(x, wg, O.expert_table(w1, w3, 2.5 * w2), E, k)
    np.testing.assert_allclose(yc, 2.5 * y, rtol=1e-13, atol=1e-15)


def pin_token_outputs_equal_grouped():
    """The per-subset combine used for sampled rows equals the grouped forward
    (with a capacity limit, a shared expert and a selection bias)."""
    rng = np.random.default_rng(41)
    E, k, d, d_ff, T = 7, 3, 6, 5, 40
    w1, w3, w2 = _experts(rng, E, d, d_ff)
    s1, s3, s2 = _experts(rng, 1, d, d_ff)
    wg, x = rng.normal(0, 1, (E, d)), rng.normal(0, 1, (T, d))
    sb = rng.uniform(-0.5, 0.5, E)
    ex = O.expert_table(w1, w3, w2)
    shared = [(s1[0], s3[0], s2[0])]
    y, info = O.moe_forward(x, wg, ex, E, k, sel_bias=sb, shared=shared, capacity_factor=0.8)
    kept = (info["assign_pos"] >= 0).reshape(T, k)
    assert not kept.all()
    sub = np.array([0, 3, 17, 39, 22])
    ys = O.token_outputs(x[sub], info["ids"][sub], info["gates"][sub], kept[sub], ex, shared)
    np.testing.assert_allclose(ys, y[sub], rtol=1e-13, atol=1e-15)
    for t in sub:
        yt = O.token_output(x[t], info["ids"][t], info["gates"][t], kept[t], ex, shared)
        np.testing.assert_allclose(yt, y[t], rtol=1e-13, atol=1e-15)


def pin_bias_update_direction():
    """[Arch] §2 / [Handbook] "Load balancing": an overloaded expert's bias goes down, an idle or
    underloaded one's goes up; at exactly the mean load (T*k/E) it stays. Hand-computed case:
    T=6, k=2, E=4 -> mean 3."""
    counts = np.array([0, 3, 5, 4])
    b = np.array([0.5, -0.25, 0.0, 1.0], dtype=np.float32)
    out = O.bias_update(counts, b, 0.125, T=6, k=2)
    assert out.dtype == np.float32
    np.testing.assert_array_equal(out, np.array([0.625, -0.25, -0.125, 0.875], dtype=np.float32))
    # a mean that is not an integer (T*k/E = 2.5): 2 is under, 3 is over
    out = O.bias_update(np.array([2, 3, 2, 3]), np.zeros(4, np.float32), 1.0, T=5, k=2)
    np.testing.assert_array_equal(out, np.array([1, -1, 1, -1], dtype=np.float32))


def pin_bias_update_balances():
    """The pages' purpose of the bias: repeated updates from the observed load even out a
    router that strongly prefers some experts. Routing here is the oracle's own top-k on
    logits + bias (the bias only selects); a log-Zipf logit offset makes the router skewed."""
    rng = np.random.default_rng(7)
    T, d, E, k = 2048, 16, 16, 2
    x = rng.normal(size=(T, d))
    w = rng.normal(scale=0.3, size=(E, d))
    offset = -1.1 * np.log(np.arange(E) + 1.0)
    bias = np.zeros(E, dtype=np.float32)

    def imbalance(b):
        logits = O.router_logits(x, w, offset)
        ids = O.select_topk(O.selection_keys(logits, b.astype(np.float64)), k)
        counts = np.bincount(ids.reshape(-1), minlength=E)
        return counts, counts.max() / (T * k / E)

    counts, start = imbalance(bias)
    for _ in range(300):
        bias = O.bias_update(counts, bias, 0.02, T, k)
        counts, _ = imbalance(bias)
    _, end = imbalance(bias)
    assert start > 3.0, start
    assert end < 1.35, end


def pin_expert_choice_all_tokens_is_softmax_mixture():
    """With C = T every expert takes every token: y = sum_e p[t,e] Expert_e(x_t), which is also
    the token-choice layer with k = E (its renormalised gates are p itself)."""
    rng = np.random.default_rng(41)
    T, d, E, d_ff = 9, 6, 4, 5
    x = rng.normal(size=(T, d))
    w_gate = rng.normal(size=(E, d))
    w1, w3, w2 = _experts(rng, E, d, d_ff)
    ex = O.expert_table(w1, w3, w2)
    y_ec, info = O.moe_forward_expert_choice(x, w_gate, ex, E, T)
    y_tc, _ = O.moe_forward(x, w_gate, ex, E, E)
    np.testing.assert_allclose(y_ec, y_tc, rtol=1e-12, atol=1e-14)
    assert (info["tokens"] == np.arange(T)[None, :]).all()


def pin_expert_choice_brute_force():
    """Buckets against a plain sort key (-p, t) per expert, with exact ties (repeated tokens),
    and y against a direct per-token sum over the experts that chose the token."""
    rng = np.random.default_rng(42)
    T, d, E, d_ff, C = 8, 5, 3, 4, 3
    x = rng.normal(size=(T, d))
    x[5] = x[1]                                    # tokens 1 and 5 tie for every expert
    x[7] = x[2]
    w_gate = rng.normal(size=(E, d))
    w1, w3, w2 = _experts(rng, E, d, d_ff)
    ex = O.expert_table(w1, w3, w2)
    y, info = O.moe_forward_expert_choice(x, w_gate, ex, E, C)
    p = info["probs"]
    for e in range(E):
        want = sorted(sorted(range(T), key=lambda t: (-p[t, e], t))[:C])
        assert list(info["tokens"][e]) == want, (e, list(info["tokens"][e]), want)
        np.testing.assert_array_equal(info["gates"][e], p[want, e])
    for t in range(T):
        acc = np.zeros(d)
        for e in range(E):
            if t in info["tokens"][e]:
                acc += p[t, e] * O.swiglu_expert(x[t:t + 1], w1[e], w3[e], w2[e])[0]
        np.testing.assert_allclose(y[t], acc, rtol=1e-12, atol=1e-14)
    # fixed buckets: E*C slots, variable experts per token
    per_token = np.bincount(info["tokens"].reshape(-1), minlength=T)
    assert per_token.sum() == E * C


def pin_expert_choice_single_expert():
    """E = 1: p = 1 for every token, so the bucket is the first C tokens (ties -> lower t) and
    only they get the expert's output."""
    rng = np.random.default_rng(43)
    T, d, d_ff, C = 6, 4, 3, 4
    x = rng.normal(size=(T, d))
    w_gate = rng.normal(size=(1, d))
    w1, w3, w2 = _experts(rng, 1, d, d_ff)
    y, info = O.moe_forward_expert_choice(x, w_gate, O.expert_table(w1, w3, w2), 1, C)
    assert list(info["tokens"][0]) == [0, 1, 2, 3]
    np.testing.assert_allclose(y[:C], O.swiglu_expert(x[:C], w1[0], w3[0], w2[0]), rtol=1e-13)
    assert (y[C:] == 0).all()


def pin_expert_choice_capacity():
    """Bucket size: the token-choice capacity ceil(cf*T*k/E), cf = 1 when unset, at most T."""
    assert O.expert_choice_capacity(0.0, 4096, 2, 8) == 1024
    assert O.expert_choice_capacity(1.25, 16384, 2, 64) == 640
    assert O.expert_choice_capacity(0.0, 300, 3, 7) == 129          # ceil(900 / 7)
    assert O.expert_choice_capacity(0.0, 10, 8, 2) == 10            # 40 capped at T
    assert O.expert_choice_capacity(0.0, 0, 2, 8) == 0


PINS = [pin_token_outputs_equal_grouped, pin_gates_worked_example, pin_gates_flowchart, pin_topk_brute_force, pin_zero_input,
        pin_gates_sum_to_one, pin_softmax_library, pin_selection_bias_only_selects,
        pin_logit_bias_enters_softmax, pin_dense_swiglu_E1, pin_k_equals_E,
        pin_naive_equals_grouped_handbook, pin_naive_equals_grouped_capacity,
        pin_align_brute_force, pin_align_invariants, pin_capacity_values, pin_silu,
        pin_balance_uniform, pin_balance_handbook, pin_sum_sq, pin_equivariance_and_scaling,
        pin_bias_update_direction, pin_bias_update_balances,
        pin_expert_choice_all_tokens_is_softmax_mixture, pin_expert_choice_brute_force,
        pin_expert_choice_single_expert, pin_expert_choice_capacity]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# ============================================================================ planted mistakes
def _mut_no_renorm(p, ids):
    return np.take_along_axis(p, ids, axis=1)


def _mut_topk_ascending(keys, k):
    return np.argsort(keys, axis=1, kind="stable")[:, :k]


def _mut_tie_high(keys, k):
    E = keys.shape[1]
    rev = np.argsort(-keys[:, ::-1], axis=1, kind="stable")
    return (E - 1 - rev)[:, :k]


def _mut_relu(z):
    return np.maximum(np.asarray(z, dtype=np.float64), 0.0)


def _mut_swap_gate_up(rows, w1, w3, w2):
    u, v = rows @ w1.T, rows @ w3.T
    return (O.silu(v) * u) @ w2.T


def _mut_sel_bias_in_gates(x, w_gate, k, logit_bias=None, sel_bias=None):
    logits = O.router_logits(x, w_gate, logit_bias)
    keys = O.selection_keys(logits, sel_bias)
    probs = O.softmax(keys)
    ids = O.select_topk(keys, k)
    return ids, O.renormalised_gates(probs, ids), probs, keys


def _mut_drop_latest_first(ids, E, cap=None):
    # keep the *last* cap assignments of each expert instead of the first
    out = _orig_align(ids[::-1], E, cap)
    T, k = ids.shape
    n = T * k
    rev = np.arange(n).reshape(T, k)[::-1].reshape(-1)
    out["sorted_assign"] = rev[out["sorted_assign"]]
    return out


def _mut_no_alpha(counts_pre, probs, T, k, alpha=0.01):
    return _orig_balance(counts_pre, probs, T, k, 1.0)


def _mut_f_over_T(counts_pre, probs, T, k, alpha=0.01):
    f, P, _ = _orig_balance(counts_pre, probs, T, k, alpha)
    f = f * k
    return f, P, alpha * f.size * float((f * P).sum())


def _mut_softmax_no_shift(logits):
    e = np.exp(logits)
    return e / e.sum(axis=1, keepdims=True)


def _mut_bias_sign_flipped(counts_pre, sel_bias, gamma, T, k):
    return _orig_bias_update(counts_pre, sel_bias, -gamma, T, k)


def _mut_ec_smallest(x, w_gate, E, C, logit_bias=None):
    tok, gates, probs = _orig_ec_route(x, w_gate, E, C, logit_bias)
    for e in range(E):
        t = np.sort(np.argsort(probs[:, e], kind="stable")[:C])
        tok[e], gates[e] = t, probs[t, e]
    return tok, gates, probs


def _mut_ec_ties_high(x, w_gate, E, C, logit_bias=None):
    tok, gates, probs = _orig_ec_route(x, w_gate, E, C, logit_bias)
    T = probs.shape[0]
    for e in range(E):
        rev = np.argsort(-probs[::-1, e], kind="stable")[:C]
        t = np.sort(T - 1 - rev)
        tok[e], gates[e] = t, probs[t, e]
    return tok, gates, probs


def _mut_ec_renormalised(x, w_gate, experts, E, C, logit_bias=None, shared=(), tokens=None):
    y, info = _orig_ec_forward(x, w_gate, experts, E, C, logit_bias, shared, tokens)
    T = y.shape[0]
    tot = np.zeros(T)
    for e in range(E):
        np.add.at(tot, info["tokens"][e], info["gates"][e])
    y2 = np.zeros_like(y)
    xx = np.asarray(x, dtype=np.float64)
    for e in range(E):
        tok = info["tokens"][e]
        out = O.swiglu_expert(xx[tok], *experts(e))
        np.add.at(y2, tok, (info["gates"][e] / tot[tok])[:, None] * out)
    return y2, info


_orig_align = O.align
_orig_balance = O.balance
_orig_bias_update = O.bias_update
_orig_ec_route = O.expert_choice_route
_orig_ec_forward = O.moe_forward_expert_choice

MUTATIONS = {
    "gates_not_renormalised": ("renormalised_gates", _mut_no_renorm),
    "topk_ascending": ("select_topk", _mut_topk_ascending),
    "ties_to_higher_index": ("select_topk", _mut_tie_high),
    "relu_instead_of_silu": ("silu", _mut_relu),
    "gate_and_up_swapped": ("swiglu_expert", _mut_swap_gate_up),
    "selection_bias_in_gates": ("route", _mut_sel_bias_in_gates),
    "drop_latest_first": ("align", _mut_drop_latest_first),
    "alpha_missing": ("balance", _mut_no_alpha),
    "f_over_tokens_not_assignments": ("balance", _mut_f_over_T),
    "softmax_without_shift": ("softmax", _mut_softmax_no_shift),
    "bias_update_sign_flipped": ("bias_update", _mut_bias_sign_flipped),
    "expert_choice_takes_smallest": ("expert_choice_route", _mut_ec_smallest),
    "expert_choice_ties_to_higher_token": ("expert_choice_route", _mut_ec_ties_high),
    "expert_choice_gates_renormalised": ("moe_forward_expert_choice", _mut_ec_renormalised),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, FloatingPointError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name!r} passed every pin"
