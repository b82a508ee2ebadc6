"""moe_forward_noalloc (the forward without a workspace argument, for callers that cannot
allocate) against moe_forward with its own workspace, through the C ABI: identical kernels, so
every output must be bit-identical. Two calls in a row on the same GPU, the second with a
smaller batch, so the second runs on scratch the first left dirty."""
import ctypes

import numpy as np
import pytest
import torch

import workloads

W = workloads.Workload


def _routing(p, dev):
    n = p.T * p.k
    i32 = dict(dtype=torch.int32, device=dev)
    return dict(topk_ids=torch.empty(n, **i32), topk_w=torch.empty(n, dtype=torch.float32, device=dev),
                prob_sum=torch.empty(p.E, dtype=torch.float32, device=dev),
                counts_pre=torch.empty(p.E, **i32), counts=torch.empty(p.E, **i32),
                offsets=torch.empty(p.E + 1, **i32), sorted_assign=torch.empty(n, **i32),
                assign_pos=torch.empty(n, **i32))


def test_noalloc_rejects_problems_beyond_its_scratch():
    # host-side: returns before any HIP call
    import mixture_experts_layer_44_amd as moe
    p = moe.problem_for(workloads.get("mixtral_prefill"))
    assert moe.workspace_bytes(p) > moe.NOALLOC_SCRATCH_BYTES
    status = moe.lib().moe_forward_noalloc(ctypes.byref(p), *([None] * 20))
    assert status == moe.MOE_EWORKSPACE


CASES = [
    # (first call, second call): same layer shapes, the second batch smaller
    (W("na_decode", T=128, d=2048, E=128, k=8, d_ff=768, seed=601),
     W("na_decode", T=9, d=2048, E=128, k=8, d_ff=768, seed=602)),
    (W("na_shared_cap", T=300, d=512, E=16, k=4, d_ff=256, seed=603, n_shared=1, d_ff_shared=256,
       sel_bias=True, capacity_factor=1.0, zipf_s=1.1),
     W("na_shared_cap", T=77, d=512, E=16, k=4, d_ff=256, seed=604, n_shared=1, d_ff_shared=256,
       sel_bias=True, capacity_factor=1.0, zipf_s=1.1)),
]


@pytest.mark.gpu
@pytest.mark.parametrize("pair", CASES, ids=[c[0].name for c in CASES])
def test_noalloc_matches_forward(pair):
    import mixture_experts_layer_44_amd as moe
    dev = torch.device("cuda")
    for w in pair:
        print(f"[noalloc] {w}", flush=True)
        g = {k: (None if v is None else v.to(dev)) for k, v in workloads.generate(w).items()}
        p = moe.problem_for(w)
        assert moe.workspace_bytes(p) <= moe.NOALLOC_SCRATCH_BYTES
        kw = dict(logit_bias=g["logit_bias"], sel_bias=g["sel_bias"], ws1=g["ws1"], ws3=g["ws3"],
                  ws2=g["ws2"])
        y_ref, r_ref = moe.forward(p, g["x"], g["w_gate"], g["w1"], g["w3"], g["w2"],
                                   return_routing=True, **kw)
        y = torch.full((w.T, w.d), float("nan"), dtype=torch.float32, device=dev)
        r = _routing(p, dev)
        moe.forward_noalloc(p, g["x"], g["w_gate"], g["w1"], g["w3"], g["w2"], y, routing=r, **kw)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), float((y - y_ref).abs().max())
        n_kept = int(r_ref["offsets"][-1])
        for key in ("topk_ids", "topk_w", "counts_pre", "counts", "offsets", "assign_pos"):
            a = r[key].cpu().numpy().reshape(-1)
            b = r_ref[key].cpu().numpy().reshape(-1)
            assert np.array_equal(a, b), key
        assert np.array_equal(r["sorted_assign"][:n_kept].cpu().numpy(),
                              r_ref["sorted_assign"][:n_kept].cpu().numpy())
        # prob_sum: the same per-workgroup sums added in the same order
        assert torch.equal(r["prob_sum"], r_ref["prob_sum"])
