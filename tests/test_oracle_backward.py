"""Pins for the fp64 oracle's layer backward (CPU only).

The backward is checked against things it does not share code with:
central finite differences of the (separately pinned) oracle forward plus
balance loss, torch's autograd through an independent torch forward, and
invariants the chain rule fixes. Planted mistakes at the bottom show that a
plausible slip in any backward step fails at least one pin."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.moe_oracle as O


def _problem(seed, T, d, E, k, d_ff, n_shared=0, cf=0.0, std=0.4, logit_bias=True, sel_bias=True):
    rng = np.random.default_rng(seed)
    P = dict(
        x=rng.normal(0, 1, (T, d)),
        w_gate=rng.normal(0, 0.5, (E, d)),
        w1=rng.normal(0, std, (E, d_ff, d)),
        w3=rng.normal(0, std, (E, d_ff, d)),
        w2=rng.normal(0, std, (E, d, d_ff)),
        shared=[tuple(rng.normal(0, std, s) for s in ((d_ff, d), (d_ff, d), (d, d_ff)))
                for _ in range(n_shared)],
        logit_bias=rng.normal(0, 0.3, E) if logit_bias else None,
        sel_bias=rng.uniform(-0.1, 0.1, E) if sel_bias else None,
        dy=rng.normal(0, 1, (T, d)),
        E=E, k=k, cf=cf,
    )
    return P


def _objective(P, ids, alpha, dL, **over):
    """J = <dy, y> + dL * L_balance through the oracle forward, routing fixed to `ids`."""
    Q = dict(P)
    Q.update(over)
    y, info = O.moe_forward(Q["x"], Q["w_gate"], O.expert_table(Q["w1"], Q["w3"], Q["w2"]), Q["E"],
                            Q["k"], Q["logit_bias"], Q["sel_bias"], Q["shared"], Q["cf"], ids=ids)
    T = Q["x"].shape[0]
    _, _, L = O.balance(info["counts_pre"], info["probs"], T, Q["k"], alpha)
    return float((Q["dy"] * y).sum()) + dL * L


def _backward(P, alpha, dL, ids=None):
    return O.moe_backward(P["x"], P["w_gate"], O.expert_table(P["w1"], P["w3"], P["w2"]), P["E"],
                          P["k"], P["dy"], P["logit_bias"], P["sel_bias"], P["shared"], P["cf"],
                          ids=ids, alpha=alpha, dL=dL)


def _fd(P, ids, alpha, dL, name, index, eps=1e-5):
    def at(delta):
        if name.startswith("shared"):
            s, m = int(name[6]), int(name[8])
            sh = [list(t) for t in P["shared"]]
            arr = sh[s][m].copy()
            arr[index] += delta
            sh[s][m] = arr
            return _objective(P, ids, alpha, dL, shared=[tuple(t) for t in sh])
        arr = P[name].copy()
        arr[index] += delta
        return _objective(P, ids, alpha, dL, **{name: arr})
    return (at(eps) - at(-eps)) / (2 * eps)


# ============================================================================ pins
def pin_bwd_finite_differences():
    """Every gradient entry against a central difference of J (routing held at the base ids,
    which is what the selection's zero gradient means; f moves only with the ids)."""
    P = _problem(11, T=7, d=5, E=4, k=2, d_ff=3, n_shared=1, cf=0.75)
    alpha, dL = 0.05, 1.7
    g = _backward(P, alpha, dL)
    ids = g["ids"]
    assert (g["assign_pos"] < 0).any(), "the capacity must drop something here"
    checks = {"x": g["dx"], "w_gate": g["dw_gate"], "logit_bias": g["dlogit_bias"],
              "w1": g["dw1"], "w3": g["dw3"], "w2": g["dw2"],
              "shared0_0": g["dshared"][0][0], "shared0_1": g["dshared"][0][1],
              "shared0_2": g["dshared"][0][2]}
    for name, grad in checks.items():
        for index in np.ndindex(grad.shape):
            num = _fd(P, ids, alpha, dL, name, index)
            assert abs(num - grad[index]) <= 1e-7 * (1.0 + abs(num)), (name, index, num, grad[index])


def _torch_grads(P, ids, kept, alpha, dL):
    """Independent forward in torch (fp64, autograd): softmax, gates over the given ids,
    SwiGLU experts slot by slot, balance loss with f from the ids (a constant tensor)."""
    t = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    x, wg = t(P["x"]), t(P["w_gate"])
    w1, w3, w2 = t(P["w1"]), t(P["w3"]), t(P["w2"])
    lb = t(P["logit_bias"])
    sh = [tuple(t(a) for a in s) for s in P["shared"]]
    E, k = P["E"], P["k"]
    T = P["x"].shape[0]
    logits = x @ wg.T + lb
    p = torch.softmax(logits, dim=1)
    idx = torch.tensor(ids)
    sel = torch.gather(p, 1, idx)
    gates = sel / sel.sum(dim=1, keepdim=True)
    rows = []
    for tt in range(T):
        acc = torch.zeros(P["x"].shape[1], dtype=torch.float64)
        for j in range(k):
            if kept[tt, j]:
                e = int(ids[tt, j])
                h = F.silu(w1[e] @ x[tt]) * (w3[e] @ x[tt])
                acc = acc + gates[tt, j] * (w2[e] @ h)
        for (s1, s3, s2) in sh:
            acc = acc + s2 @ (F.silu(s1 @ x[tt]) * (s3 @ x[tt]))
        rows.append(acc)
    y = torch.stack(rows)
    f = torch.tensor(np.bincount(ids.reshape(-1), minlength=E) / float(T * k))
    L = alpha * E * (f * p.mean(dim=0)).sum()
    J = (torch.tensor(P["dy"]) * y).sum() + dL * L
    J.backward()
    out = dict(dx=x.grad, dw_gate=wg.grad, dlogit_bias=lb.grad, dw1=w1.grad, dw3=w3.grad,
               dw2=w2.grad)
    for i, s in enumerate(sh):
        for m in range(3):
            out[f"ds{i}{m}"] = s[m].grad
    return {a: b.numpy() for a, b in out.items()}


def pin_bwd_autograd():
    """Every gradient against torch autograd through an independent torch forward."""
    P = _problem(12, T=24, d=10, E=6, k=3, d_ff=8, n_shared=1, cf=0.9)
    alpha, dL = 0.01, 3.0
    g = _backward(P, alpha, dL)
    kept = (g["assign_pos"] >= 0).reshape(g["ids"].shape)
    assert not kept.all()
    ref = _torch_grads(P, g["ids"], kept, alpha, dL)
    mine = dict(dx=g["dx"], dw_gate=g["dw_gate"], dlogit_bias=g["dlogit_bias"], dw1=g["dw1"],
                dw3=g["dw3"], dw2=g["dw2"], ds00=g["dshared"][0][0], ds01=g["dshared"][0][1],
                ds02=g["dshared"][0][2])
    for name, val in mine.items():
        np.testing.assert_allclose(val, ref[name], rtol=1e-10, atol=1e-12, err_msg=name)


def pin_bwd_logit_rows_sum_to_zero():
    """A softmax's logit gradient sums to zero over the experts, for the gate part (softmax
    over the selected logits) and the balance part alike; so does d logit_bias."""
    P = _problem(13, T=40, d=6, E=8, k=3, d_ff=4, cf=1.0)
    for dL in (0.0, 2.5):
        g = _backward(P, 0.01, dL)
        np.testing.assert_allclose(g["dlogits"].sum(axis=1), 0.0, atol=1e-13)
        assert abs(g["dlogit_bias"].sum()) <= 1e-12
        assert np.abs(g["dlogits"]).max() > 1e-3


def pin_bwd_linear_in_upstream():
    """The gradient is linear in (dy, dL)."""
    P = _problem(14, T=16, d=6, E=5, k=2, d_ff=4, n_shared=1)
    rng = np.random.default_rng(5)
    dy1, dy2 = rng.normal(0, 1, P["dy"].shape), rng.normal(0, 1, P["dy"].shape)
    P1, P2, P3 = dict(P, dy=dy1), dict(P, dy=dy2), dict(P, dy=dy1 + 2.0 * dy2)
    g1, g2, g3 = _backward(P1, 0.01, 1.0), _backward(P2, 0.01, 0.5), _backward(P3, 0.01, 2.0)
    for key in ("dx", "dw_gate", "dw1", "dw3", "dw2", "dgate"):
        np.testing.assert_allclose(g3[key], g1[key] + 2.0 * g2[key], rtol=1e-10, atol=1e-11,
                                   err_msg=key)


def pin_bwd_single_expert_is_dense_swiglu():
    """E = 1, k = 1: the gate is identically 1 and p identically 1, so the router gets no
    gradient at all and dx is the dense SwiGLU backward (torch's autograd of F.silu/linear)."""
    P = _problem(15, T=9, d=6, E=1, k=1, d_ff=5, sel_bias=False)
    g = _backward(P, 0.01, 1.0)
    assert np.abs(g["dw_gate"]).max() == 0.0 and np.abs(g["dlogit_bias"]).max() == 0.0
    x = torch.tensor(P["x"], requires_grad=True)
    w1, w3, w2 = (torch.tensor(P[n][0], requires_grad=True) for n in ("w1", "w3", "w2"))
    y = F.linear(F.silu(F.linear(x, w1)) * F.linear(x, w3), w2)
    (torch.tensor(P["dy"]) * y).sum().backward()
    np.testing.assert_allclose(g["dx"], x.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g["dw1"][0], w1.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g["dw3"][0], w3.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g["dw2"][0], w2.grad.numpy(), rtol=1e-11, atol=1e-12)


def pin_bwd_unused_and_dropped():
    """An expert nobody keeps gets exactly zero weight gradient; a dropped assignment has a
    zero gate gradient; a token whose every assignment was dropped gets only the router's and
    the shared expert's share of dx."""
    P = _problem(16, T=30, d=6, E=6, k=2, d_ff=4, n_shared=1, cf=0.34)
    P["logit_bias"] = np.array([0.0, 0.0, 0.0, 0.0, 0.0, -50.0])
    P["sel_bias"] = None
    g = _backward(P, 0.01, 1.0)
    assert (g["ids"] != 5).all()
    assert np.abs(g["dw1"][5]).max() == 0 and np.abs(g["dw2"][5]).max() == 0
    kept = (g["assign_pos"] >= 0).reshape(g["ids"].shape)
    assert (g["dgate"][~kept] == 0).all() and (~kept).any()
    full = np.nonzero(~kept.any(axis=1))[0]
    assert full.size, "some token must have lost every assignment"
    t = full[0]
    s1, s3, s2 = P["shared"][0]
    d_rows, *_ = O.swiglu_expert_backward(P["x"][t:t + 1], s1, s3, s2, P["dy"][t:t + 1])
    want = d_rows[0] + g["dlogits"][t] @ P["w_gate"]
    np.testing.assert_allclose(g["dx"][t], want, rtol=1e-12, atol=1e-13)


def pin_bwd_sampled_equals_full():
    """moe_backward_sampled (dx of chosen tokens, weight gradients of chosen experts) equals
    the corresponding parts of moe_backward, with drops, a shared expert and dL != 0."""
    P = _problem(17, T=40, d=8, E=6, k=2, d_ff=6, n_shared=1, cf=0.8)
    g = _backward(P, 0.02, 1.3)
    tokens = [0, 3, 17, 39, 22]
    sample = [1, 4]
    s = O.moe_backward_sampled(P["x"], P["w_gate"], O.expert_table(P["w1"], P["w3"], P["w2"]),
                               P["E"], P["k"], P["dy"], g["ids"], tokens, sample, P["logit_bias"],
                               P["shared"], P["cf"], alpha=0.02, dL=1.3)
    np.testing.assert_allclose(s["dx"], g["dx"][tokens], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(s["dlogits"], g["dlogits"][tokens], rtol=1e-12, atol=1e-14)
    for e in sample:
        for m, key in enumerate(("dw1", "dw3", "dw2")):
            np.testing.assert_allclose(s["wgrads"][e][m], g[key][e], rtol=1e-12, atol=1e-13)


PINS = [pin_bwd_sampled_equals_full, pin_bwd_finite_differences, pin_bwd_autograd, pin_bwd_logit_rows_sum_to_zero,
        pin_bwd_linear_in_upstream, pin_bwd_single_expert_is_dense_swiglu,
        pin_bwd_unused_and_dropped]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# ============================================================================ planted mistakes
_orig = {n: getattr(O, n) for n in ("silu_grad", "swiglu_expert_backward", "gate_logit_grad",
                                    "balance_logit_grad", "sigmoid")}


def _mut_silu_grad_is_sigmoid(z):
    return _orig["sigmoid"](z)


def _mut_swiglu_no_up_branch(rows, w1, w3, w2, d_out):
    d_rows, dw1, dw3, dw2, o = _orig["swiglu_expert_backward"](rows, w1, w3, w2, d_out)
    u = rows @ w1.T
    v = rows @ w3.T
    du = (d_out @ w2) * v * O.silu_grad(u)
    return du @ w1, dw1, dw3, dw2, o


def _mut_swiglu_du_dv_swapped(rows, w1, w3, w2, d_out):
    d_rows, dw1, dw3, dw2, o = _orig["swiglu_expert_backward"](rows, w1, w3, w2, d_out)
    return d_rows, dw3, dw1, dw2, o


def _mut_gate_grad_no_coupling(gates, dgate):
    return gates * dgate


def _mut_gate_grad_wrong_sign(gates, dgate):
    return -_orig["gate_logit_grad"](gates, dgate)


def _mut_balance_no_softmax_centering(probs, counts_pre, T, k, alpha, dL):
    f = np.asarray(counts_pre, dtype=np.float64) / float(T * k)
    return probs * (float(dL) * alpha * probs.shape[1] * f / float(T))[None, :]


def _mut_balance_missing_E(probs, counts_pre, T, k, alpha, dL):
    return _orig["balance_logit_grad"](probs, counts_pre, T, k, alpha, dL) / probs.shape[1]


MUTATIONS = {
    "silu_grad_is_sigmoid": ("silu_grad", _mut_silu_grad_is_sigmoid),
    "swiglu_drops_up_branch_of_dx": ("swiglu_expert_backward", _mut_swiglu_no_up_branch),
    "swiglu_dw1_dw3_swapped": ("swiglu_expert_backward", _mut_swiglu_du_dv_swapped),
    "gate_grad_without_renorm_coupling": ("gate_logit_grad", _mut_gate_grad_no_coupling),
    "gate_grad_sign_flipped": ("gate_logit_grad", _mut_gate_grad_wrong_sign),
    "balance_grad_not_centred": ("balance_logit_grad", _mut_balance_no_softmax_centering),
    "balance_grad_missing_E": ("balance_logit_grad", _mut_balance_missing_E),
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
