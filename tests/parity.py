"""GPU-vs-oracle parity checking (used by the `gpu` tests and the smoke check).

Protocol, for one workload and seed:
  1. generate the inputs (seeded), run the HIP path (moe_forward with every
     routing output exported);
  2. the oracle routes every token in fp64 from the same stored values;
     top-k ids must match exactly wherever the gap between the k-th and
     (k+1)-th selection key exceeds 1e-4 (elsewhere either choice is valid, but
     the GPU's choice must still be a top-k within that gap);
  3. the oracle groups the GPU's own ids; the GPU's counts, offsets, sorted
     order and dropped set must match bit for bit (so one accepted near-tie
     flip cannot cascade into different capacity drops);
  4. the oracle's gates at the GPU's ids vs the GPU's gates (abs 1e-5);
  5. the oracle's y for the GPU's routing vs the GPU's y: every row for small
     problems, sampled rows for full-size ones. bf16 storage: max-abs <= 2e-2
     and relative Frobenius <= 1e-2; fp32 storage: both <= 1e-5.
The oracle never sees a value produced by the HIP path except the ids it is
asked to group (step 3) and the routing it is asked to evaluate (step 5)."""
from __future__ import annotations

import time
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

import oracle as O
import workloads
from util import f64

GAP = 1e-4
TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-5, 1e-5)}
GATE_TOL = 1e-5


@dataclass
class Report:
    name: str
    T: int
    id_mismatch: int = 0
    order_bad: int = 0
    near_ties: int = 0
    invalid_choice: int = 0
    align_equal: bool = True
    align_diff: str = ""
    gate_err: float = 0.0
    y_maxabs: float = 0.0
    y_relf: float = 0.0
    rows_checked: int = 0
    dropped: int = 0
    prob_sum_rel: float = 0.0
    timings: dict = field(default_factory=dict)

    def ok(self, dtype: str) -> bool:
        ma, rf = TOL[dtype]
        return (self.id_mismatch == 0 and self.order_bad == 0 and self.invalid_choice == 0
                and self.align_equal and self.gate_err <= GATE_TOL and self.y_maxabs <= ma
                and self.y_relf <= rf and self.prob_sum_rel <= 1e-4)

    def __str__(self):
        return (f"{self.name}: T={self.T} ids(mismatch={self.id_mismatch}, order={self.order_bad}, "
                f"near_ties={self.near_ties}, invalid={self.invalid_choice}) "
                f"align={'equal' if self.align_equal else 'DIFF ' + self.align_diff} "
                f"gate_err={self.gate_err:.2e} y(maxabs={self.y_maxabs:.3e}, relF={self.y_relf:.3e}, "
                f"rows={self.rows_checked}) dropped={self.dropped} psum_rel={self.prob_sum_rel:.1e}")


def check_topk(gpu_ids: np.ndarray, keys: np.ndarray, k: int, rep: Report):
    T, E = keys.shape
    if T == 0:
        return
    order = np.argsort(-keys, axis=1, kind="stable")
    srt = np.take_along_axis(keys, order, 1)
    boundary = srt[:, k - 1] - srt[:, k] if k < E else np.full(T, np.inf)
    clear = boundary > GAP
    g_sorted = np.sort(gpu_ids, 1)
    o_sorted = np.sort(order[:, :k], 1)
    rep.id_mismatch = int((clear & (g_sorted != o_sorted).any(1)).sum())
    rep.near_ties = int((~clear).sum())
    gk = np.take_along_axis(keys, gpu_ids.astype(np.int64), 1)
    rep.order_bad = int((np.diff(gk, axis=1) > GAP).any(1).sum()) if k > 1 else 0
    distinct = np.array([len(set(r)) == k for r in gpu_ids.tolist()])
    in_range = ((gpu_ids >= 0) & (gpu_ids < E)).all(1)
    # every chosen key must be within GAP of the k-th largest
    within = (gk >= srt[:, k - 1:k] - GAP).all(1)
    rep.invalid_choice = int((~(distinct & in_range & within)).sum())


def check_align(gpu: dict, want: dict, rep: Report):
    n_kept = int(np.asarray(want["offsets"])[-1])
    for key in ("counts_pre", "counts", "offsets", "sorted_assign", "assign_pos"):
        a = gpu[key].cpu().numpy().astype(np.int64)
        if key == "sorted_assign":          # only the first offsets[E] entries are defined
            a = a[:n_kept]
        b = np.asarray(want[key], dtype=np.int64)
        if a.shape != b.shape or not np.array_equal(a, b):
            rep.align_equal = False
            n = min(a.size, b.size)
            bad = np.nonzero(a[:n] != b[:n])[0]
            rep.align_diff += f"{key}(shape {a.shape} vs {b.shape}, first bad {bad[:5].tolist()}) "


def _lazy_experts(w1, w3, w2):
    def get(e):
        return f64(w1[e]), f64(w3[e]), f64(w2[e])
    return get


def run_parity(w: workloads.Workload, T: Optional[int] = None, gen_device: str = "cpu",
               sample: Optional[int] = None, seed_rows: int = 0, inputs=None) -> Report:
    """Run the HIP forward for workload `w` and compare with the oracle.

    sample=None checks every row of y; otherwise `sample` rows (a fixed
    seeded choice, always including the first and last token and, when
    something was dropped, tokens with dropped slots)."""
    import mixture_experts_layer_44_amd as moe
    T = w.T if T is None else T
    rep = Report(name=w.name, T=T)
    t0 = time.time()
    inp = inputs if inputs is not None else workloads.generate(w, device=gen_device, T=T)
    dev = torch.device("cuda")
    g = {kk: (None if v is None else v.to(dev)) for kk, v in inp.items()}
    p = moe.problem_for(w, T)
    rep.timings["generate"] = time.time() - t0
    t0 = time.time()
    y, r = moe.forward(p, g["x"], g["w_gate"], g["w1"], g["w3"], g["w2"], logit_bias=g["logit_bias"],
                       sel_bias=g["sel_bias"], ws1=g["ws1"], ws3=g["ws3"], ws2=g["ws2"],
                       return_routing=True)
    torch.cuda.synchronize()
    rep.timings["gpu"] = time.time() - t0
    assert torch.isfinite(y).all().item(), "non-finite y"

    t0 = time.time()
    x64 = f64(inp["x"])
    lb = f64(inp["logit_bias"])
    sb = f64(inp["sel_bias"])
    ids_o, _, probs, keys = O.route(x64, f64(inp["w_gate"]), w.k, lb, sb)
    gpu_ids = r["topk_ids"].cpu().numpy().astype(np.int64)
    check_topk(gpu_ids, keys, w.k, rep)
    cap = O.capacity(w.capacity_factor, T, w.k, w.E)
    al = O.align(gpu_ids, w.E, cap)
    check_align(r, al, rep)
    gates_o = O.renormalised_gates(probs, gpu_ids) if T else np.zeros((0, w.k))
    if T:
        rep.gate_err = float(np.abs(r["topk_w"].cpu().numpy().astype(np.float64) - gates_o).max())
        ps_o = probs.sum(0)
        ps_g = r["prob_sum"].cpu().numpy().astype(np.float64)
        rep.prob_sum_rel = float(np.abs(ps_g - ps_o).max() / max(np.abs(ps_o).max(), 1e-30))
    kept = (al["assign_pos"] >= 0).reshape(T, w.k)
    rep.dropped = int((~kept).sum())
    rep.timings["oracle_route_align"] = time.time() - t0

    t0 = time.time()
    if T == 0:
        rep.timings["oracle_ffn"] = 0.0
        return rep
    if sample is None or sample >= T:
        rows = np.arange(T)
    else:
        rng = np.random.default_rng(seed_rows + 7919 * T)
        pick = set(rng.choice(T, size=sample, replace=False).tolist()) | {0, T - 1}
        drop_tok = np.nonzero((~kept).any(1))[0]
        if drop_tok.size:
            pick |= set(rng.choice(drop_tok, size=min(4, drop_tok.size), replace=False).tolist())
        rows = np.array(sorted(pick))
    shared = []
    if w.n_shared:
        shared = [(f64(inp["ws1"][0]), f64(inp["ws3"][0]), f64(inp["ws2"][0]))]
    y_o = O.token_outputs(x64[rows], gpu_ids[rows], gates_o[rows], kept[rows],
                          _lazy_experts(inp["w1"], inp["w3"], inp["w2"]), shared)
    y_g = y[torch.as_tensor(rows, device=dev)].cpu().numpy().astype(np.float64)
    diff = y_g - y_o
    rep.y_maxabs = float(np.abs(diff).max())
    rep.y_relf = float(np.linalg.norm(diff) / max(np.linalg.norm(y_o), 1e-300))
    rep.rows_checked = int(rows.size)
    rep.timings["oracle_ffn"] = time.time() - t0
    return rep
