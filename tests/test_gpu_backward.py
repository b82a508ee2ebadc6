"""Layer backward on the GPU (moe_backward, through the C ABI) against the fp64 oracle.

Both sides differentiate the same selection: the GPU forward's top-k ids are handed to the
oracle (the selection has no gradient, and near-ties are the forward tests' business).

Tolerance. The HIP path rounds dy, g*dy, du, dv and the router's logit gradient to bf16
before its MFMA products (fp32 accumulation), and writes the expert weight gradients in
bf16; each rounding is a relative error of at most 2^-9 per element, and the products over
K terms of random sign keep a normwise error of the same order. Every gradient tensor must
be within 1e-2 relative Frobenius error of the oracle's, and no element may be off by more
than 3e-2 of the tensor's largest magnitude."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import workloads
from util import f64

pytestmark = pytest.mark.gpu

W = workloads.Workload
REL_F = 1e-2
REL_MAX = 3e-2


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dy(w, scale=1.0):
    g = torch.Generator()
    g.manual_seed(workloads.tensor_seed(w.seed, "x", 7))
    return (torch.randn((w.T, w.d), generator=g, dtype=torch.float32) * scale)


def _compare(name, got, ref):
    got = f64(got)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    if ref.size == 0:
        return 0.0, 0.0
    scale = np.abs(ref).max()
    err = np.abs(got - ref)
    den = np.linalg.norm(ref)
    relf = float(np.linalg.norm(got - ref) / den) if den > 0 else float(np.linalg.norm(got))
    relmax = float(err.max() / scale) if scale > 0 else float(err.max())
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    if den > 0:
        assert relf <= REL_F, f"{name}: relative Frobenius error {relf:.3e} > {REL_F}"
        assert relmax <= REL_MAX, f"{name}: max error {relmax:.3e} of max|ref| > {REL_MAX}"
    else:
        assert err.max() == 0.0, f"{name}: expected exact zeros"
    return relf, relmax


def run_backward(w, alpha=0.01, dL=1.0, dy_scale=1.0):
    import mixture_experts_layer_44_amd as moe
    inp = workloads.generate(w)
    g = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    p = moe.problem_for(w)
    y, r = moe.forward(p, g["x"], g["w_gate"], g["w1"], g["w3"], g["w2"],
                       logit_bias=g["logit_bias"], sel_bias=g["sel_bias"], ws1=g["ws1"],
                       ws3=g["ws3"], ws2=g["ws2"], return_routing=True)
    dy = _dy(w, dy_scale)
    grads = moe.backward(p, g["x"], g["w_gate"], g["w1"], g["w3"], g["w2"], r, dy.cuda(),
                         logit_bias=g["logit_bias"], ws1=g["ws1"], ws3=g["ws3"], ws2=g["ws2"],
                         alpha=alpha, dL=dL, want_dlogit_bias=True)
    torch.cuda.synchronize()
    ids = r["topk_ids"].cpu().numpy().astype(np.int64)
    shared = [] if not w.n_shared else [(f64(inp["ws1"][0]), f64(inp["ws3"][0]), f64(inp["ws2"][0]))]
    ref = O.moe_backward(f64(inp["x"]), f64(inp["w_gate"]),
                         O.expert_table(f64(inp["w1"]), f64(inp["w3"]), f64(inp["w2"])), w.E, w.k,
                         f64(dy), f64(inp["logit_bias"]), None, shared, w.capacity_factor, ids=ids,
                         alpha=alpha, dL=dL)
    return grads, ref, r


CASES = [
    W("bwd_basic", T=300, d=256, E=16, k=4, d_ff=384, seed=501),
    W("bwd_shared_sel_cap", T=257, d=384, E=32, k=8, d_ff=256, seed=502, n_shared=1,
      d_ff_shared=256, sel_bias=True, capacity_factor=1.0),
    W("bwd_zipf_cap", T=500, d=256, E=16, k=2, d_ff=256, seed=503, capacity_factor=1.0, zipf_s=1.1),
    W("bwd_E1", T=200, d=256, E=1, k=1, d_ff=512, seed=504),
    W("bwd_many_small", T=600, d=256, E=128, k=8, d_ff=256, seed=505, n_shared=1,
      d_ff_shared=256, sel_bias=True),
    W("bwd_E256", T=64, d=256, E=256, k=8, d_ff=128, seed=506),
    W("bwd_long_segments", T=1600, d=512, E=4, k=2, d_ff=384, seed=507, n_shared=1,
      d_ff_shared=384),
    W("bwd_k_eq_E", T=100, d=128, E=8, k=8, d_ff=128, seed=508),
    # ~150 rows per expert: the recompute runs the forward's ragged 192-row class
    W("bwd_mid192", T=600, d=512, E=8, k=2, d_ff=384, seed=511, n_shared=1, d_ff_shared=384),
    # the router weight gradient's K (T = 4096) cut into 8 token splits
    W("bwd_router_split", T=4096, d=256, E=8, k=2, d_ff=128, seed=512, zipf_s=1.1),
]


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_backward_parity(w):
    _say(f"[backward] {w}")
    grads, ref, r = run_backward(w)
    report = {}
    for name in ("dx", "dw_gate", "dlogit_bias", "dw1", "dw3", "dw2"):
        report[name] = _compare(name, grads[name], ref[name])
    if w.n_shared:
        for m, name in enumerate(("dws1", "dws3", "dws2")):
            report[name] = _compare(name, grads[name][0], ref["dshared"][0][m])
    _say(f"{w.name}: " + ", ".join(f"{k}=({a:.1e},{b:.1e})" for k, (a, b) in report.items()))
    if w.capacity_factor:
        assert (r["assign_pos"][: w.T * w.k] < 0).any()


def test_backward_balance_term_only():
    """dy = 0: only the balance loss drives the router; the expert weights get exactly zero."""
    w = W("bwd_balance_only", T=400, d=256, E=16, k=2, d_ff=256, seed=509, zipf_s=1.1,
          capacity_factor=1.25)
    grads, ref, _ = run_backward(w, alpha=0.01, dL=50.0, dy_scale=0.0)
    for name in ("dx", "dw_gate", "dlogit_bias"):
        _compare(name, grads[name], ref[name])
    for name in ("dw1", "dw3", "dw2"):
        assert torch.count_nonzero(grads[name]).item() == 0, name
    assert np.abs(ref["dw_gate"]).max() > 0


def test_backward_empty_batch():
    """T = 0: every weight gradient is exactly zero."""
    import mixture_experts_layer_44_amd as moe
    w = W("bwd_empty", T=0, d=256, E=8, k=2, d_ff=256, seed=510, n_shared=1, d_ff_shared=256)
    inp = {k: (None if v is None else v.cuda()) for k, v in workloads.generate(w).items()}
    p = moe.problem_for(w)
    y, r = moe.forward(p, inp["x"], inp["w_gate"], inp["w1"], inp["w3"], inp["w2"], ws1=inp["ws1"],
                       ws3=inp["ws3"], ws2=inp["ws2"], return_routing=True)
    grads = moe.backward(p, inp["x"], inp["w_gate"], inp["w1"], inp["w3"], inp["w2"], r,
                         torch.zeros((0, w.d), device="cuda"), ws1=inp["ws1"], ws3=inp["ws3"],
                         ws2=inp["ws2"], want_dlogit_bias=True,
                         out={n: torch.full(s, 7.0, device="cuda", dtype=dt) for n, s, dt in (
                             ("dw_gate", (w.E, w.d), torch.float32),
                             ("dw1", (w.E, w.d_ff, w.d), torch.bfloat16),
                             ("dws2", (1, w.d, w.d_ff), torch.bfloat16))})
    torch.cuda.synchronize()
    for name in ("dw_gate", "dlogit_bias", "dw1", "dw3", "dw2", "dws1", "dws3", "dws2"):
        assert torch.count_nonzero(grads[name]).item() == 0, name


def test_backward_deterministic():
    """Two runs give the same bits (no atomics anywhere in the backward)."""
    import mixture_experts_layer_44_amd as moe
    w = CASES[1]
    inp = {k: (None if v is None else v.cuda()) for k, v in workloads.generate(w).items()}
    p = moe.problem_for(w)
    _, r = moe.forward(p, inp["x"], inp["w_gate"], inp["w1"], inp["w3"], inp["w2"],
                       sel_bias=inp["sel_bias"], ws1=inp["ws1"], ws3=inp["ws3"], ws2=inp["ws2"],
                       return_routing=True)
    dy = _dy(w).cuda()
    outs = [moe.backward(p, inp["x"], inp["w_gate"], inp["w1"], inp["w3"], inp["w2"], r, dy,
                         ws1=inp["ws1"], ws3=inp["ws3"], ws2=inp["ws2"], dL=1.0) for _ in range(2)]
    torch.cuda.synchronize()
    for name in outs[0]:
        assert torch.equal(outs[0][name], outs[1][name]), name


FULL = [("mixtral_prefill", 16, 2), ("dsv3_fine", 8, 3), ("skew_cap", 16, 3)]


@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,n_tok,n_exp", FULL, ids=[f[0] for f in FULL])
def test_full_size_backward_sampled(name, n_tok, n_exp):
    """Full-size layer, in the launch configuration the benchmark times: dx of sampled tokens
    and the weight gradients of sampled experts (the most and least loaded touched ones and a
    random one) against the oracle computed one by one."""
    import mixture_experts_layer_44_amd as moe
    w = workloads.get(name)
    _say(f"[backward] full {w} tokens={n_tok} experts={n_exp}")
    g = workloads.generate(w, device="cuda")
    p = moe.problem_for(w)
    _, r = moe.forward(p, g["x"], g["w_gate"], g["w1"], g["w3"], g["w2"], logit_bias=g["logit_bias"],
                       sel_bias=g["sel_bias"], ws1=g["ws1"], ws3=g["ws3"], ws2=g["ws2"],
                       return_routing=True)
    dy = _dy(w).cuda()
    grads = moe.backward(p, g["x"], g["w_gate"], g["w1"], g["w3"], g["w2"], r, dy,
                         logit_bias=g["logit_bias"], ws1=g["ws1"], ws3=g["ws3"], ws2=g["ws2"],
                         alpha=0.01, dL=1.0)
    torch.cuda.synchronize()
    ids = r["topk_ids"].cpu().numpy().astype(np.int64)
    counts = r["counts"].cpu().numpy()
    rng = np.random.default_rng(w.seed)
    tokens = np.sort(rng.choice(w.T, size=n_tok, replace=False))
    touched = np.nonzero(counts > 0)[0]
    picks = [int(touched[np.argmax(counts[touched])]), int(touched[np.argmin(counts[touched])])]
    rest = [e for e in touched if e not in picks]
    picks += [int(e) for e in rng.choice(rest, size=max(0, n_exp - 2), replace=False)]

    def experts(e):
        return f64(g["w1"][e]), f64(g["w3"][e]), f64(g["w2"][e])

    shared = [] if not w.n_shared else [(f64(g["ws1"][0]), f64(g["ws3"][0]), f64(g["ws2"][0]))]
    ref = O.moe_backward_sampled(f64(g["x"]), f64(g["w_gate"]), experts, w.E, w.k, f64(dy), ids,
                                 tokens, picks, f64(g["logit_bias"]), shared, w.capacity_factor,
                                 alpha=0.01, dL=1.0)
    rep = {"dx": _compare("dx", grads["dx"][torch.from_numpy(tokens).cuda()], ref["dx"])}
    for e in picks:
        for m, key in enumerate(("dw1", "dw3", "dw2")):
            rep[f"{key}[{e}]"] = _compare(f"{key}[{e}]", grads[key][e], ref["wgrads"][e][m])
    _say(f"{name}: experts {picks} rows {[int(counts[e]) for e in picks]}: " +
         ", ".join(f"{k}=({a:.1e},{b:.1e})" for k, (a, b) in rep.items()))
    del grads, g
    torch.cuda.empty_cache()
