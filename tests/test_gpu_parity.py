"""HIP path vs the fp64 oracle, through the C ABI (needs an MI355X).

Every case, the full-size workloads included, is compared on every routing
output (ids by the gap rule, grouping bit-exact, gates) and on every row of
y; the full-size workloads run in the same launch configuration the
benchmark times."""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle as O
import workloads
from parity import run_parity
from util import f64

pytestmark = pytest.mark.gpu

W = workloads.Workload


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


SMALL = [
    workloads.get("tiny_fp32"),
    workloads.get("handbook_fp32"),
    W("bf16_ragged", T=300, d=256, E=16, k=4, d_ff=384, seed=101),
    W("bf16_shared_selbias", T=257, d=384, E=32, k=8, d_ff=256, seed=102, n_shared=1,
      d_ff_shared=256, sel_bias=True),
    W("bf16_cap_zipf", T=500, d=256, E=16, k=2, d_ff=256, seed=103, capacity_factor=1.0, zipf_s=1.1),
    W("bf16_dense_E1", T=200, d=256, E=1, k=1, d_ff=512, seed=104),
    W("bf16_k_eq_E", T=100, d=128, E=8, k=8, d_ff=128, seed=105),
    W("bf16_E256_T1", T=1, d=256, E=256, k=8, d_ff=128, seed=106),
    W("bf16_empty", T=0, d=256, E=8, k=2, d_ff=256, seed=107),
    W("bf16_cap1", T=64, d=128, E=4, k=2, d_ff=128, seed=108, capacity_factor=0.01),
    W("bf16_many_tiles", T=1500, d=512, E=4, k=2, d_ff=640, seed=109, n_shared=1, d_ff_shared=640),
    W("f32_ragged", T=77, d=100, E=5, k=3, d_ff=70, seed=110, dtype="f32", capacity_factor=0.9,
      n_shared=1, d_ff_shared=70),
    # many small segments with the multi-launch routing path (T*k > 1024)
    W("bf16_many_small", T=600, d=256, E=128, k=8, d_ff=256, seed=111, n_shared=1,
      d_ff_shared=256, sel_bias=True),
    # small segments, one-launch routing, capacity limit and a logit offset
    W("bf16_small_cap", T=96, d=512, E=64, k=6, d_ff=384, seed=112, capacity_factor=1.0,
      zipf_s=1.1),
    # wide tiles (expected >= 768 rows per expert) on a small problem
    W("bf16_wide", T=1600, d=512, E=4, k=2, d_ff=384, seed=113, n_shared=1, d_ff_shared=384),
    # wide tiles with the down GEMM's K range split in two (few down tiles, no shared expert)
    W("bf16_wide_ksplit", T=2048, d=1024, E=4, k=2, d_ff=1024, seed=114),
    # wide tiles under a steep logit offset: segments of 2048, 1820, 200 and 28 rows, so the
    # four-wave kernel's waves run with all, one and no live row fragments
    W("bf16_wide_skew", T=2048, d=512, E=4, k=2, d_ff=512, seed=131, zipf_s=2.0),
    # wide tiles under a capacity limit (overflow dropped, tiles dealt to the XCDs in chunks,
    # the down GEMM's K range split in two)
    W("bf16_wide_cap", T=2048, d=512, E=4, k=2, d_ff=512, seed=133, capacity_factor=0.9,
      zipf_s=0.5),
    # one token: routing, grouping and schedule in one wave, with a shared expert (a group of
    # its own after the routed ones), a selection bias and a capacity limit
    W("bf16_T1_shared_selbias", T=1, d=512, E=64, k=6, d_ff=256, seed=132, n_shared=1,
      d_ff_shared=256, sel_bias=True, capacity_factor=1.0),
    # ragged 192-row tiles: ~150 rows per expert (one tile), the shared group 600 rows (four)
    W("bf16_mid192", T=600, d=512, E=8, k=2, d_ff=384, seed=115, n_shared=1, d_ff_shared=384),
    # ragged 192-row tiles, ~350 rows per expert (two tiles each)
    W("bf16_mid192_two", T=1400, d=256, E=8, k=2, d_ff=256, seed=116),
    # ragged 256-row tiles (~230 rows per expert) with a selection bias
    W("bf16_mid256", T=920, d=256, E=8, k=2, d_ff=256, seed=117, sel_bias=True),
    # decode class (<= 48 rows per expert, d and d_ff multiples of 256): K split over the four
    # waves; segments of 1..32 rows and longer ones (several 32-row m-tiles) under Zipf routing,
    # one or two 16-row fragments, a shared expert of T rows, and K of 1, 3 and 8 wave steps
    W("bf16_dec_zipf", T=200, d=512, E=32, k=4, d_ff=768, seed=118, zipf_s=1.1),
    W("bf16_dec_shared", T=70, d=2048, E=64, k=2, d_ff=256, seed=119, n_shared=1, d_ff_shared=256,
      sel_bias=True),
    W("bf16_dec_cap", T=96, d=256, E=16, k=4, d_ff=512, seed=120, capacity_factor=1.0, zipf_s=1.1),
    # the remaining per-wave step counts of the decode kernel: 4, 5, 6 and 7 (gate-up K = d)
    # with 6, 4, 7 and 5 (down K = d_ff)
    W("bf16_dec_k4", T=24, d=1024, E=16, k=2, d_ff=1536, seed=121),
    W("bf16_dec_k5", T=24, d=1280, E=16, k=2, d_ff=1024, seed=122, n_shared=1, d_ff_shared=1024),
    W("bf16_dec_k6", T=40, d=1536, E=16, k=4, d_ff=1792, seed=123),
    W("bf16_dec_k7", T=40, d=1792, E=16, k=4, d_ff=1280, seed=124, capacity_factor=1.0),
    # the fused router (E <= 16, d % 512 == 0, T*k > 1024): E not a multiple of 16, T not a
    # multiple of 16, logit offset, selection bias and a capacity limit
    W("bf16_fused_router", T=1101, d=512, E=12, k=3, d_ff=256, seed=125, sel_bias=True,
      zipf_s=1.1, capacity_factor=1.25),
    # top-k, grouping and schedule in one workgroup (T <= 16) with a capacity limit, a selection
    # bias and a shared expert
    W("bf16_small16_cap", T=16, d=256, E=32, k=4, d_ff=256, seed=126, capacity_factor=0.5,
      sel_bias=True, n_shared=1, d_ff_shared=256),
    # router logits one expert per wave (T <= 4, d a multiple of 512): three 512-column pieces
    # per lane, E_pad = 48 (the last workgroup's waves past E write zeros), offset, selection
    # bias, shared expert
    W("bf16_gemv_T3", T=3, d=1536, E=40, k=5, d_ff=256, seed=128, sel_bias=True, zipf_s=0.7,
      n_shared=1, d_ff_shared=256),
    # the same with the widest row it takes (d = 4096: eight pieces per lane) and T = 4
    W("bf16_gemv_T4", T=4, d=4096, E=24, k=3, d_ff=512, seed=129, capacity_factor=1.0),
    # multi-launch routing with E_pad = 208 (the router's last 64-expert group is partly
    # padding), T not a multiple of the 64-token logits block, a logit offset and a selection bias
    W("bf16_E200", T=300, d=384, E=200, k=6, d_ff=256, seed=127, sel_bias=True,
      zipf_s=0.5),
    # decode down GEMM + combine in one launch (T*k <= 16, k <= 8, no shared expert): dropped
    # slots under a capacity limit (one row per expert), and an odd k (the second slot group one
    # slot short) with K = d_ff of eight wave steps
    W("bf16_dec_fused_cap", T=2, d=512, E=16, k=8, d_ff=512, seed=130, capacity_factor=0.5,
      zipf_s=1.1),
    # just past the merged launch's limit (18 assignments): the down GEMM and the combine apart
    W("bf16_dec_T3_k6", T=3, d=1024, E=32, k=6, d_ff=512, seed=134, sel_bias=True),
    # the same shape at T = 8 (64 assignments): the down GEMM and the combine apart
    W("bf16_dec_cap_T8", T=8, d=512, E=16, k=8, d_ff=512, seed=130, capacity_factor=0.5,
      zipf_s=1.1),
    W("bf16_dec_fused_k5", T=3, d=768, E=32, k=5, d_ff=2048, seed=131, sel_bias=True),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_small_parity(w):
    _say(f"[parity] {w}")
    rep = run_parity(w, gen_device="cpu")
    _say(str(rep))
    assert rep.ok(w.dtype), str(rep)


DECODE = [workloads.get(f"decode_T{T}") for T in (1, 8, 32, 128)]


@pytest.mark.parametrize("w", DECODE, ids=[w.name for w in DECODE])
def test_decode_parity(w):
    _say(f"[parity] {w}")
    rep = run_parity(w, gen_device="cuda")
    _say(str(rep))
    assert rep.ok(w.dtype), str(rep)


FULL = ["mixtral_prefill", "skew_cap", "dsv3_fine"]


@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL)
def test_full_size_parity(name):
    # every output row of the full-size layer, in the launch configuration the benchmark times;
    # the oracle visits each expert once for all of its rows (host BLAS threads)
    w = workloads.get(name)
    _say(f"[parity] full {w}, every row")
    rep = run_parity(w, gen_device="cuda", sample=None)
    _say(str(rep) + f" timings={ {k: round(v, 1) for k, v in rep.timings.items()} }")
    assert rep.rows_checked == w.T
    assert rep.ok(w.dtype), str(rep)
    if w.capacity_factor:
        assert rep.dropped > 0
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------- align alone
ALIGN_CASES = [
    # (T, E, k, capacity_factor, skew)
    (64, 8, 2, 0.0, 0.0),
    (4096, 8, 2, 0.0, 0.0),
    (4096, 256, 8, 0.0, 0.0),
    (4096, 256, 8, 1.25, 1.0),
    (1, 128, 8, 0.0, 0.0),
    (8, 128, 8, 0.0, 0.0),
    (128, 128, 8, 1.0, 0.5),
    (16384, 64, 2, 1.25, 1.1),
    (16384, 64, 2, 0.05, 1.1),
    (1000, 1, 1, 0.0, 0.0),
    (777, 13, 5, 0.7, 0.8),
    (3, 256, 1, 0.0, 0.0),
]


def _ids(T, E, k, skew, seed):
    rng = np.random.default_rng(seed)
    pr = (np.arange(1, E + 1, dtype=np.float64) ** -skew)
    pr /= pr.sum()
    # distinct experts per token drawn from a skewed prior (Gumbel top-k)
    g = np.log(pr)[None, :] + rng.gumbel(size=(T, E))
    return np.argsort(-g, axis=1, kind="stable")[:, :k].astype(np.int32)


@pytest.mark.parametrize("case", ALIGN_CASES, ids=[str(c) for c in ALIGN_CASES])
def test_align_bit_exact_given_ids(case):
    import mixture_experts_layer_44_amd as moe
    T, E, k, cf, skew = case
    _say(f"[align] T={T} E={E} k={k} cf={cf} skew={skew}")
    ids = _ids(T, E, k, skew, seed=T * 31 + E)
    p = moe.make_problem(T, 128, E, k, 128, capacity_factor=cf)
    got = moe.align(p, torch.from_numpy(ids).cuda())
    want = O.align(ids, E, O.capacity(cf, T, k, E))
    n_kept = int(want["offsets"][-1])
    for key in want:
        a = got[key].cpu().numpy().astype(np.int64)
        if key == "sorted_assign":          # only the first offsets[E] entries are defined
            a = a[:n_kept]
        assert np.array_equal(a, want[key]), (key, a[:10], want[key][:10])
    # determinism: repeated runs give identical bytes
    for _ in range(4):
        again = moe.align(p, torch.from_numpy(ids).cuda())
        for key in got:
            a, b = again[key], got[key]
            if key == "sorted_assign":
                a, b = a[:n_kept], b[:n_kept]
            assert torch.equal(a, b)


def test_align_ignores_out_of_range_ids():
    """An id outside [0, E) is documented as dropped and counted nowhere."""
    import mixture_experts_layer_44_amd as moe
    T, E, k = 300, 16, 2
    ids = _ids(T, E, k, 0.0, seed=5)
    bad = ids.copy()
    bad[::7, 1] = E + 3
    bad[::11, 0] = -1
    p = moe.make_problem(T, 128, E, k, 128)
    got = moe.align(p, torch.from_numpy(bad).cuda())
    flat = bad.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    ap = got["assign_pos"].cpu().numpy()
    assert (ap[~valid] == -1).all()
    assert got["offsets"][-1].item() == int(valid.sum())
    # the valid assignments are grouped exactly as if the invalid ones were absent
    cnt = np.bincount(flat[valid], minlength=E)
    assert np.array_equal(got["counts_pre"].cpu().numpy(), cnt)
    sa = got["sorted_assign"].cpu().numpy()[:valid.sum()]
    assert np.array_equal(flat[sa], np.repeat(np.arange(E), cnt))
    assert all((np.diff(sa[o:o2]) > 0).all() for o, o2 in zip(np.r_[0, np.cumsum(cnt)[:-1]], np.cumsum(cnt)))


# ---------------------------------------------------------------------------- composition
COMPOSE = [
    W("compose", T=333, d=256, E=24, k=3, d_ff=384, seed=201, n_shared=1, d_ff_shared=384,
      sel_bias=True, capacity_factor=1.1),
    # wide tiles, down GEMM split in K: expert_ffn sums the halves itself, forward in the combine
    W("compose_ksplit", T=2048, d=1024, E=4, k=2, d_ff=1024, seed=202, capacity_factor=0.9),
    # T <= 16: top-k, grouping and schedule in one workgroup after the logits
    W("compose_small16", T=12, d=256, E=16, k=4, d_ff=256, seed=203, sel_bias=True,
      capacity_factor=0.8),
    # decode-sized: moe_forward runs the down GEMM and the combine as one launch; expert_ffn +
    # combine run them apart. Same bits.
    W("compose_dec_fused_cap", T=2, d=512, E=16, k=8, d_ff=512, seed=204, capacity_factor=0.5),
    W("compose_dec_T1", T=1, d=2048, E=128, k=8, d_ff=768, seed=205),
    W("compose_dec_k3", T=2, d=256, E=8, k=3, d_ff=2048, seed=206, sel_bias=True),
]


@pytest.mark.parametrize("w", COMPOSE, ids=[w.name for w in COMPOSE])
def test_entry_points_compose_to_forward(w):
    """route -> align -> expert_ffn -> combine gives the same bits as moe_forward."""
    import mixture_experts_layer_44_amd as moe
    inp = {k: (None if v is None else v.cuda()) for k, v in workloads.generate(w).items()}
    p = moe.problem_for(w)
    y, r = moe.forward(p, inp["x"], inp["w_gate"], inp["w1"], inp["w3"], inp["w2"],
                       sel_bias=inp["sel_bias"], ws1=inp["ws1"], ws3=inp["ws3"], ws2=inp["ws2"],
                       return_routing=True)
    ids, gates, psum = moe.route(p, inp["x"], inp["w_gate"], sel_bias=inp["sel_bias"])
    al = moe.align(p, ids)
    out_rows, shared_out = moe.expert_ffn(p, inp["x"], inp["w1"], inp["w3"], inp["w2"],
                                          al["sorted_assign"], al["offsets"], inp["ws1"], inp["ws3"],
                                          inp["ws2"])
    y2 = moe.combine(p, out_rows, al["assign_pos"], gates, shared_out)
    torch.cuda.synchronize()
    assert torch.equal(ids, r["topk_ids"]) and torch.equal(gates, r["topk_w"])
    # prob_sum is the same sum; small batches add it in another order (fp32 rounding only)
    torch.testing.assert_close(psum, r["prob_sum"], rtol=1e-6, atol=1e-6)
    n_kept = int(al["offsets"][-1].item())
    if w.capacity_factor:
        assert n_kept < w.T * w.k                 # the capacity limit dropped something
    for key in al:
        a, b = al[key], r[key]
        if key == "sorted_assign":                # only the first offsets[E] entries are defined
            a, b = a[:n_kept], b[:n_kept]
        assert torch.equal(a, b), key
    assert torch.equal(y, y2)


def test_balance_statistics():
    import mixture_experts_layer_44_amd as moe
    w = W("balance", T=2000, d=256, E=64, k=2, d_ff=128, seed=202, capacity_factor=1.25, zipf_s=1.1)
    inp = workloads.generate(w)
    g = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    p = moe.problem_for(w)
    _, r = moe.forward(p, g["x"], g["w_gate"], g["w1"], g["w3"], g["w2"], logit_bias=g["logit_bias"],
                       return_routing=True)
    f, P, L = moe.balance(p, r["counts_pre"], r["prob_sum"], 0.01)
    _, _, probs, _ = O.route(f64(inp["x"]), f64(inp["w_gate"]), w.k, f64(inp["logit_bias"]))
    f_o, P_o, L_o = O.balance(O.align(r["topk_ids"].cpu().numpy(), w.E)["counts_pre"], probs, w.T,
                              w.k, 0.01)
    np.testing.assert_allclose(f.cpu().numpy(), f_o, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(P.cpu().numpy(), P_o, rtol=1e-4, atol=1e-6)
    assert abs(L.item() - L_o) <= 1e-4 * abs(L_o)
    assert L_o > 0.01        # a skewed router is above the balanced value alpha


def test_prepared_forward_balance_statistics():
    """The timed step with balance outputs (PreparedForward(balance_alpha=...)): y as the plain
    forward, f / P / L as the oracle, also with many top-k workgroups (T = 16384 rows of partial
    probability sums, the tree reduction's chunks longer than its 8-load batches)."""
    import mixture_experts_layer_44_amd as moe
    for w in (W("bal_prepared", T=2000, d=256, E=64, k=2, d_ff=128, seed=205,
                capacity_factor=1.25, zipf_s=1.1),
              W("bal_prepared_big", T=16384, d=128, E=24, k=2, d_ff=128, seed=206, zipf_s=1.1)):
        inp = workloads.generate(w)
        g = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
        p = moe.problem_for(w)
        fwd = moe.PreparedForward(p, g["x"], g["w_gate"], g["w1"], g["w3"], g["w2"],
                                  logit_bias=g["logit_bias"], balance_alpha=0.01)
        y = fwd().clone()
        y_ref, r = moe.forward(p, g["x"], g["w_gate"], g["w1"], g["w3"], g["w2"],
                               logit_bias=g["logit_bias"], return_routing=True)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref)
        assert torch.equal(fwd.counts_pre, r["counts_pre"])
        _, _, probs, _ = O.route(f64(inp["x"]), f64(inp["w_gate"]), w.k, f64(inp["logit_bias"]))
        f_o, P_o, L_o = O.balance(O.align(r["topk_ids"].cpu().numpy(), w.E)["counts_pre"], probs,
                                  w.T, w.k, 0.01)
        np.testing.assert_allclose(fwd.f.cpu().numpy(), f_o, rtol=1e-6, atol=1e-7)
        np.testing.assert_allclose(fwd.P.cpu().numpy(), P_o, rtol=1e-4, atol=1e-6)
        assert abs(fwd.L.item() - L_o) <= 1e-4 * abs(L_o)


def test_workspace_reuse_across_shapes():
    """One workspace sized for a large problem serves a smaller one; stale contents are ignored."""
    import mixture_experts_layer_44_amd as moe
    big = W("ws_big", T=600, d=256, E=16, k=4, d_ff=256, seed=203)
    small = W("ws_small", T=37, d=256, E=16, k=4, d_ff=256, seed=204)
    ws = torch.full((moe.workspace_bytes(moe.problem_for(big)),), 0xAB, dtype=torch.uint8,
                    device="cuda")
    for w in (big, small, big):
        inp = {k: (None if v is None else v.cuda()) for k, v in workloads.generate(w).items()}
        y = moe.forward(moe.problem_for(w), inp["x"], inp["w_gate"], inp["w1"], inp["w3"], inp["w2"],
                        ws=ws)
        y_ref = moe.forward(moe.problem_for(w), inp["x"], inp["w_gate"], inp["w1"], inp["w3"],
                            inp["w2"])
        assert torch.equal(y, y_ref)


def test_prepared_forward_and_graph_replay():
    """A prepared forward and its captured HIP graph give the eager forward's bits; the graph is
    replayed several times with new inputs and eager work in between, each replay checked."""
    import mixture_experts_layer_44_amd as moe
    w = workloads.get("decode_T8")
    inp = {k: (None if v is None else v.cuda()) for k, v in workloads.generate(w).items()}
    p = moe.problem_for(w)
    x = inp["x"].clone()
    fwd = moe.PreparedForward(p, x, inp["w_gate"], inp["w1"], inp["w3"], inp["w2"])
    y_eager = moe.forward(p, x, inp["w_gate"], inp["w1"], inp["w3"], inp["w2"])
    assert torch.equal(fwd(), y_eager)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fwd()
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda")
    for i in range(4):
        gen.manual_seed(1000 + i)
        x.copy_(torch.randn(x.shape, generator=gen, device="cuda").to(x.dtype))
        want = moe.forward(p, x, inp["w_gate"], inp["w1"], inp["w3"], inp["w2"])   # eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(fwd.y, want), f"replay {i}"


BIAS_CASES = [(6, 2, 4), (4096, 8, 256), (1, 1, 1), (0, 2, 8), (333, 3, 24), (16384, 2, 64)]


@pytest.mark.parametrize("T,k,E", BIAS_CASES, ids=[f"T{t}k{k}E{e}" for t, k, e in BIAS_CASES])
def test_bias_update_bit_exact(T, k, E):
    """moe_bias_update against the oracle's fp32 step, on counts that hit the mean, zero and
    large values; bit for bit."""
    import mixture_experts_layer_44_amd as moe
    rng = np.random.default_rng(T * 131 + E)
    p = moe.make_problem(T, 256, E, k, 256)
    mean = T * k / E
    counts = rng.integers(0, max(1, int(3 * mean) + 2), E).astype(np.int32)
    if E >= 4 and (T * k) % E == 0:
        counts[:2] = T * k // E          # exactly at the mean: unchanged
        counts[2] = 0
    bias = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    for gamma in (0.001, 0.03125, 0.0):
        want = O.bias_update(counts, bias, gamma, T, k)
        got = moe.bias_update(p, torch.from_numpy(counts).cuda(), torch.from_numpy(bias).cuda(),
                              gamma).cpu().numpy()
        np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))


def test_bias_update_loop_balances_routing():
    """Routing on the GPU with the selection bias, then moe_bias_update from the GPU's own
    pre-drop counts, repeated: every step equals the oracle's step on the same counts (bit for
    bit) and the load of a skewed router evens out."""
    import mixture_experts_layer_44_amd as moe
    w = W("bias_loop", T=1024, d=256, E=32, k=4, d_ff=256, seed=301, zipf_s=1.1, sel_bias=True)
    inp = {k_: (None if v is None else v.cuda()) for k_, v in workloads.generate(w).items()}
    p = moe.problem_for(w)
    bias = torch.zeros(w.E, dtype=torch.float32, device="cuda")
    ratios = []
    for it in range(120):          # step 0.05: the log-Zipf offset spans ~3.8 logits
        _, r = moe.forward(p, inp["x"], inp["w_gate"], inp["w1"], inp["w3"], inp["w2"],
                           logit_bias=inp["logit_bias"], sel_bias=bias, return_routing=True)
        counts = r["counts_pre"].cpu().numpy()
        ratios.append(counts.max() / (w.T * w.k / w.E))
        want = O.bias_update(counts, bias.cpu().numpy(), 0.05, w.T, w.k)
        moe.bias_update(p, r["counts_pre"], bias, 0.05)
        np.testing.assert_array_equal(bias.cpu().numpy().view(np.uint32), want.view(np.uint32))
    _say(f"[bias loop] max/mean load {ratios[0]:.2f} -> {ratios[-1]:.2f}")
    assert ratios[0] > 2.0 and ratios[-1] < 1.5, (ratios[0], ratios[-1])
