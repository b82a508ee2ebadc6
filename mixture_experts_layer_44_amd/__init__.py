"""Sparse top-k MoE layer forward on one MI355X (gfx950): thin Python binding.

Every step of the layer runs in the HIP kernels of libmoe_mi355x.so, reached
through its C ABI (include/moe_mi355x.h). This module only marshals
arguments: it checks device, dtype, shape and contiguity of torch tensors,
allocates outputs and scratch with torch (device memory and streams are
torch's), and passes raw pointers plus the current HIP stream. There is no
CPU fallback: if the library is missing, importing this package raises.

Functions mirror the ABI: route, align, expert_ffn, combine, balance, forward,
plus the host-only helpers validate, capacity and workspace_bytes.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "Problem", "MoEError", "lib", "make_problem", "validate", "capacity", "workspace_bytes",
    "route", "align", "expert_ffn", "combine", "balance", "forward", "LIB_PATH",
    "MOE_OK", "MOE_EINVAL", "MOE_EUNSUPPORTED", "MOE_EWORKSPACE", "MOE_EHIP", "forward_staged",
    "STAGES", "problem_for", "PreparedForward", "bias_update", "expert_choice_capacity",
    "expert_choice_workspace_bytes", "forward_expert_choice", "backward",
    "backward_workspace_bytes", "BWD_STAGES", "forward_noalloc", "NOALLOC_SCRATCH_BYTES",
]

# size of the per-GPU scratch array of moe_forward_noalloc (MOE_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 32 << 20

# stage names of moe_backward_staged, in event order (events 1..10 close these stages)
BWD_STAGES = ("recompute", "prep", "dgrad_down", "dgrad_x", "wgrad_down", "wgrad_up", "router",
              "router_dgrad", "router_wgrad", "dx")

# stage names of moe_forward_staged, in event order (events 1..6 close these stages)
STAGES = ("route", "align", "schedule", "gate_up", "down", "combine")

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP = range(5)
MOE_F32, MOE_BF16 = 0, 1


class Problem(ctypes.Structure):
    """Mirror of moe_problem."""
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("d_ff_shared", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("capacity_factor", ctypes.c_double)]


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {_lib.moe_status_str(status).decode()} (status {status})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libmoe_mi355x.so not found at {LIB_PATH}; build it with "
            "`python mixture_experts_layer_44_amd/build.py` (hipcc, gfx950). There is no fallback.")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(Problem)
    vp, sz, i32, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_float
    L.moe_status_str.restype = ctypes.c_char_p
    L.moe_status_str.argtypes = [ctypes.c_int]
    L.moe_validate.argtypes = [P]
    L.moe_capacity.argtypes = [P, ctypes.POINTER(i32)]
    L.moe_workspace_bytes.argtypes = [P, ctypes.POINTER(sz)]
    L.moe_route.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_align.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_expert_ffn.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_combine.argtypes = [P, vp, vp, vp, vp, vp, vp]
    L.moe_balance.argtypes = [P, vp, vp, f32, vp, vp, vp, vp]
    L.moe_bias_update.argtypes = [P, vp, f32, vp, vp]
    L.moe_expert_choice_capacity.argtypes = [P, ctypes.POINTER(i32)]
    L.moe_expert_choice_workspace_bytes.argtypes = [P, ctypes.POINTER(sz)]
    L.moe_forward_expert_choice.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                            vp, sz, vp]
    L.moe_forward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                              vp, vp, vp, vp, sz, vp]
    L.moe_forward_staged.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp]
    L.moe_forward_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                      vp, vp, vp, vp, vp]
    L.moe_backward_workspace_bytes.argtypes = [P, ctypes.POINTER(sz)]
    L.moe_backward.argtypes = [P] + [vp] * 16 + [f32, f32] + [vp] * 10 + [sz, vp]
    L.moe_backward_staged.argtypes = [P] + [vp] * 16 + [f32, f32] + [vp] * 10 + [sz, vp, vp]
    for fn in ("moe_validate", "moe_capacity", "moe_workspace_bytes", "moe_route", "moe_align",
               "moe_expert_ffn", "moe_combine", "moe_balance", "moe_forward", "moe_forward_staged",
               "moe_bias_update", "moe_expert_choice_capacity", "moe_expert_choice_workspace_bytes",
               "moe_forward_expert_choice", "moe_backward_workspace_bytes", "moe_backward",
               "moe_backward_staged", "moe_forward_noalloc"):
        getattr(L, fn).restype = ctypes.c_int
    return L


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


def _check(fn: str, status: int):
    if status != MOE_OK:
        raise MoEError(fn, status)


# ----------------------------------------------------------------------------- host helpers
def make_problem(T: int, d: int, E: int, k: int, d_ff: int, n_shared: int = 0,
                 d_ff_shared: int = 0, dtype="bf16", capacity_factor: float = 0.0) -> Problem:
    if isinstance(dtype, torch.dtype):
        dtype = {torch.bfloat16: "bf16", torch.float32: "f32"}[dtype]
    return Problem(T, d, E, k, d_ff, n_shared, d_ff_shared if n_shared else 0,
                   MOE_BF16 if dtype == "bf16" else MOE_F32, float(capacity_factor or 0.0))


def problem_for(w, T: Optional[int] = None) -> Problem:
    """Problem for a workload preset (anything with the same field names)."""
    return make_problem(w.T if T is None else T, w.d, w.E, w.k, w.d_ff, w.n_shared,
                        w.d_ff_shared, w.dtype, w.capacity_factor)


def validate(p: Problem) -> int:
    return _lib.moe_validate(ctypes.byref(p))


def capacity(p: Problem) -> Optional[int]:
    c = ctypes.c_int32()
    _check("moe_capacity", _lib.moe_capacity(ctypes.byref(p), ctypes.byref(c)))
    return None if c.value < 0 else c.value


def workspace_bytes(p: Problem) -> int:
    n = ctypes.c_size_t()
    _check("moe_workspace_bytes", _lib.moe_workspace_bytes(ctypes.byref(p), ctypes.byref(n)))
    return n.value


# ----------------------------------------------------------------------------- marshalling
def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t: Optional[torch.Tensor], name: str, shape, dtype, dev, optional=False):
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if t.device != dev:
        raise ValueError(f"{name} must be on {dev}, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _dt(p: Problem) -> torch.dtype:
    return torch.bfloat16 if p.dtype == MOE_BF16 else torch.float32


def _workspace(p: Problem, dev, ws: Optional[torch.Tensor]) -> torch.Tensor:
    need = workspace_bytes(p)
    if ws is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if ws.device != dev or ws.dtype != torch.uint8 or ws.numel() < need:
        raise ValueError(f"workspace must be a uint8 tensor of >= {need} bytes on {dev}")
    return ws


def route(p: Problem, x, w_gate, logit_bias=None, sel_bias=None, want_prob_sum=True, ws=None):
    """-> (topk_ids [T,k] int32, topk_w [T,k] fp32, prob_sum [E] fp32 or None)"""
    dev, dt = x.device, _dt(p)
    _need(x, "x", (p.T, p.d), dt, dev)
    _need(w_gate, "w_gate", (p.E, p.d), dt, dev)
    _need(logit_bias, "logit_bias", (p.E,), torch.float32, dev, optional=True)
    _need(sel_bias, "sel_bias", (p.E,), torch.float32, dev, optional=True)
    ids = torch.empty((p.T, p.k), dtype=torch.int32, device=dev)
    gates = torch.empty((p.T, p.k), dtype=torch.float32, device=dev)
    psum = torch.empty((p.E,), dtype=torch.float32, device=dev) if want_prob_sum else None
    ws = _workspace(p, dev, ws)
    _check("moe_route", _lib.moe_route(ctypes.byref(p), _ptr(x), _ptr(w_gate), _ptr(logit_bias),
                                       _ptr(sel_bias), _ptr(ids), _ptr(gates), _ptr(psum),
                                       _ptr(ws), ws.numel(), _stream(dev)))
    return ids, gates, psum


def align(p: Problem, topk_ids, ws=None):
    """-> dict(counts_pre, counts, offsets, sorted_assign, assign_pos), int32 tensors."""
    dev = topk_ids.device
    _need(topk_ids, "topk_ids", (p.T, p.k), torch.int32, dev)
    n = p.T * p.k
    out = dict(counts_pre=torch.empty(p.E, dtype=torch.int32, device=dev),
               counts=torch.empty(p.E, dtype=torch.int32, device=dev),
               offsets=torch.empty(p.E + 1, dtype=torch.int32, device=dev),
               sorted_assign=torch.empty(max(n, 1), dtype=torch.int32, device=dev),
               assign_pos=torch.empty(max(n, 1), dtype=torch.int32, device=dev))
    ws = _workspace(p, dev, ws)
    _check("moe_align", _lib.moe_align(ctypes.byref(p), _ptr(topk_ids), _ptr(out["counts_pre"]),
                                       _ptr(out["counts"]), _ptr(out["offsets"]),
                                       _ptr(out["sorted_assign"]), _ptr(out["assign_pos"]),
                                       _ptr(ws), ws.numel(), _stream(dev)))
    out["sorted_assign"] = out["sorted_assign"][:n]
    out["assign_pos"] = out["assign_pos"][:n]
    return out


def expert_ffn(p: Problem, x, w1, w3, w2, sorted_assign, offsets, ws1=None, ws3=None, ws2=None,
               ws=None):
    """-> (out_rows [T*k, d] fp32 (first offsets[E] rows valid), shared_out [T,d] or None)"""
    dev, dt = x.device, _dt(p)
    _need(x, "x", (p.T, p.d), dt, dev)
    _need(w1, "w1", (p.E, p.d_ff, p.d), dt, dev)
    _need(w3, "w3", (p.E, p.d_ff, p.d), dt, dev)
    _need(w2, "w2", (p.E, p.d, p.d_ff), dt, dev)
    if p.n_shared:
        _need(ws1, "ws1", (1, p.d_ff_shared, p.d), dt, dev)
        _need(ws3, "ws3", (1, p.d_ff_shared, p.d), dt, dev)
        _need(ws2, "ws2", (1, p.d, p.d_ff_shared), dt, dev)
    _need(offsets, "offsets", (p.E + 1,), torch.int32, dev)
    if sorted_assign.dtype != torch.int32 or sorted_assign.device != dev:
        raise ValueError("sorted_assign must be int32 on the same device")
    n = p.T * p.k
    out_rows = torch.empty((max(n, 1), p.d), dtype=torch.float32, device=dev)
    shared_out = torch.empty((p.T, p.d), dtype=torch.float32, device=dev) if p.n_shared else None
    ws = _workspace(p, dev, ws)
    _check("moe_expert_ffn", _lib.moe_expert_ffn(
        ctypes.byref(p), _ptr(x), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(ws1), _ptr(ws3), _ptr(ws2),
        _ptr(sorted_assign), _ptr(offsets), _ptr(out_rows), _ptr(shared_out), _ptr(ws), ws.numel(),
        _stream(dev)))
    return out_rows, shared_out


def combine(p: Problem, out_rows, assign_pos, topk_w, shared_out=None):
    """-> y [T,d] fp32"""
    dev = topk_w.device
    _need(topk_w, "topk_w", (p.T, p.k), torch.float32, dev)
    if assign_pos.numel() < p.T * p.k or assign_pos.dtype != torch.int32:
        raise ValueError("assign_pos must be int32 with T*k entries")
    if p.n_shared:
        _need(shared_out, "shared_out", (p.T, p.d), torch.float32, dev)
    y = torch.empty((p.T, p.d), dtype=torch.float32, device=dev)
    _check("moe_combine", _lib.moe_combine(ctypes.byref(p), _ptr(out_rows), _ptr(assign_pos),
                                           _ptr(topk_w), _ptr(shared_out), _ptr(y), _stream(dev)))
    return y


def balance(p: Problem, counts_pre, prob_sum, alpha: float = 0.01):
    """-> (f [E], P [E], L [1]) fp32"""
    dev = counts_pre.device
    _need(counts_pre, "counts_pre", (p.E,), torch.int32, dev)
    _need(prob_sum, "prob_sum", (p.E,), torch.float32, dev)
    f = torch.empty(p.E, dtype=torch.float32, device=dev)
    P = torch.empty(p.E, dtype=torch.float32, device=dev)
    L = torch.empty(1, dtype=torch.float32, device=dev)
    _check("moe_balance", _lib.moe_balance(ctypes.byref(p), _ptr(counts_pre), _ptr(prob_sum),
                                           ctypes.c_float(alpha), _ptr(f), _ptr(P), _ptr(L),
                                           _stream(dev)))
    return f, P, L


def forward(p: Problem, x, w_gate, w1, w3, w2, logit_bias=None, sel_bias=None, ws1=None, ws3=None,
            ws2=None, return_routing: bool = False, ws=None, y=None):
    """The whole layer. -> y [T,d] fp32, or (y, routing dict) with return_routing."""
    dev, dt = x.device, _dt(p)
    _need(x, "x", (p.T, p.d), dt, dev)
    _need(w_gate, "w_gate", (p.E, p.d), dt, dev)
    _need(w1, "w1", (p.E, p.d_ff, p.d), dt, dev)
    _need(w3, "w3", (p.E, p.d_ff, p.d), dt, dev)
    _need(w2, "w2", (p.E, p.d, p.d_ff), dt, dev)
    _need(logit_bias, "logit_bias", (p.E,), torch.float32, dev, optional=True)
    _need(sel_bias, "sel_bias", (p.E,), torch.float32, dev, optional=True)
    if p.n_shared:
        _need(ws1, "ws1", (1, p.d_ff_shared, p.d), dt, dev)
        _need(ws3, "ws3", (1, p.d_ff_shared, p.d), dt, dev)
        _need(ws2, "ws2", (1, p.d, p.d_ff_shared), dt, dev)
    if y is None:
        y = torch.empty((p.T, p.d), dtype=torch.float32, device=dev)
    else:
        _need(y, "y", (p.T, p.d), torch.float32, dev)
    n = p.T * p.k
    r = {}
    if return_routing:
        i32 = dict(dtype=torch.int32, device=dev)
        r = dict(topk_ids=torch.empty((p.T, p.k), **i32),
                 topk_w=torch.empty((p.T, p.k), dtype=torch.float32, device=dev),
                 prob_sum=torch.empty(p.E, dtype=torch.float32, device=dev),
                 counts_pre=torch.empty(p.E, **i32), counts=torch.empty(p.E, **i32),
                 offsets=torch.empty(p.E + 1, **i32),
                 sorted_assign=torch.empty(max(n, 1), **i32),
                 assign_pos=torch.empty(max(n, 1), **i32))
    ws = _workspace(p, dev, ws)
    g = r.get
    _check("moe_forward", _lib.moe_forward(
        ctypes.byref(p), _ptr(x), _ptr(w_gate), _ptr(logit_bias), _ptr(sel_bias), _ptr(w1),
        _ptr(w3), _ptr(w2), _ptr(ws1), _ptr(ws3), _ptr(ws2), _ptr(y), _ptr(g("topk_ids")),
        _ptr(g("topk_w")), _ptr(g("prob_sum")), _ptr(g("counts_pre")), _ptr(g("counts")),
        _ptr(g("offsets")), _ptr(g("sorted_assign")), _ptr(g("assign_pos")), _ptr(ws),
        ws.numel(), _stream(dev)))
    if not return_routing:
        return y
    r["sorted_assign"] = r["sorted_assign"][:n]
    r["assign_pos"] = r["assign_pos"][:n]
    return y, r


def forward_noalloc(p: Problem, x, w_gate, w1, w3, w2, y, routing=None, logit_bias=None,
                    sel_bias=None, ws1=None, ws3=None, ws2=None):
    """moe_forward_noalloc: the whole layer without a workspace (the library's per-GPU scratch
    array), for callers that cannot allocate. y [T,d] fp32 and every tensor in `routing`
    (topk_ids, topk_w, prob_sum, counts_pre, counts, offsets, sorted_assign, assign_pos; any
    subset) are preallocated by the caller; this function allocates nothing. Returns y."""
    dev, dt = x.device, _dt(p)
    _need(x, "x", (p.T, p.d), dt, dev)
    _need(w_gate, "w_gate", (p.E, p.d), dt, dev)
    _need(w1, "w1", (p.E, p.d_ff, p.d), dt, dev)
    _need(w3, "w3", (p.E, p.d_ff, p.d), dt, dev)
    _need(w2, "w2", (p.E, p.d, p.d_ff), dt, dev)
    _need(logit_bias, "logit_bias", (p.E,), torch.float32, dev, optional=True)
    _need(sel_bias, "sel_bias", (p.E,), torch.float32, dev, optional=True)
    _need(y, "y", (p.T, p.d), torch.float32, dev)
    if p.n_shared:
        _need(ws1, "ws1", (1, p.d_ff_shared, p.d), dt, dev)
        _need(ws3, "ws3", (1, p.d_ff_shared, p.d), dt, dev)
        _need(ws2, "ws2", (1, p.d, p.d_ff_shared), dt, dev)
    r = dict(routing or {})
    n = p.T * p.k
    shapes = dict(topk_ids=(n, torch.int32), topk_w=(n, torch.float32),
                  prob_sum=(p.E, torch.float32), counts_pre=(p.E, torch.int32),
                  counts=(p.E, torch.int32), offsets=(p.E + 1, torch.int32),
                  sorted_assign=(n, torch.int32), assign_pos=(n, torch.int32))
    for key, t in r.items():
        size, dtype = shapes[key]
        if t.device != dev or t.dtype != dtype or not t.is_contiguous() or t.numel() < size:
            raise ValueError(f"{key} must be a contiguous {dtype} tensor of >= {size} entries on {dev}")
    g = r.get
    _check("moe_forward_noalloc", _lib.moe_forward_noalloc(
        ctypes.byref(p), _ptr(x), _ptr(w_gate), _ptr(logit_bias), _ptr(sel_bias), _ptr(w1),
        _ptr(w3), _ptr(w2), _ptr(ws1), _ptr(ws3), _ptr(ws2), _ptr(y), _ptr(g("topk_ids")),
        _ptr(g("topk_w")), _ptr(g("prob_sum")), _ptr(g("counts_pre")), _ptr(g("counts")),
        _ptr(g("offsets")), _ptr(g("sorted_assign")), _ptr(g("assign_pos")), _stream(dev)))
    return y


def bias_update(p: Problem, counts_pre, sel_bias, gamma: float):
    """One auxiliary-loss-free balancing step on sel_bias (fp32 [E], updated in place) from
    the pre-drop expert counts (int32 [E]). Returns sel_bias."""
    dev = sel_bias.device
    _need(counts_pre, "counts_pre", (p.E,), torch.int32, dev)
    _need(sel_bias, "sel_bias", (p.E,), torch.float32, dev)
    _check("moe_bias_update", _lib.moe_bias_update(ctypes.byref(p), _ptr(counts_pre),
                                                   float(gamma), _ptr(sel_bias), _stream(dev)))
    return sel_bias


def expert_choice_capacity(p: Problem) -> int:
    """Bucket size C of expert-choice routing (host-only)."""
    c = ctypes.c_int32(0)
    _check("moe_expert_choice_capacity", _lib.moe_expert_choice_capacity(ctypes.byref(p),
                                                                          ctypes.byref(c)))
    return c.value


def expert_choice_workspace_bytes(p: Problem) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_expert_choice_workspace_bytes",
           _lib.moe_expert_choice_workspace_bytes(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def forward_expert_choice(p: Problem, x, w_gate, w1, w3, w2, logit_bias=None, ws1=None, ws3=None,
                          ws2=None, return_routing: bool = False, ws=None, y=None):
    """The expert-choice layer. -> y [T,d] fp32, or (y, dict(tokens [E,C], gates [E,C],
    prob_sum [E])) with return_routing."""
    dev, dt = x.device, _dt(p)
    _need(x, "x", (p.T, p.d), dt, dev)
    _need(w_gate, "w_gate", (p.E, p.d), dt, dev)
    _need(w1, "w1", (p.E, p.d_ff, p.d), dt, dev)
    _need(w3, "w3", (p.E, p.d_ff, p.d), dt, dev)
    _need(w2, "w2", (p.E, p.d, p.d_ff), dt, dev)
    _need(logit_bias, "logit_bias", (p.E,), torch.float32, dev, optional=True)
    if p.n_shared:
        _need(ws1, "ws1", (1, p.d_ff_shared, p.d), dt, dev)
        _need(ws3, "ws3", (1, p.d_ff_shared, p.d), dt, dev)
        _need(ws2, "ws2", (1, p.d, p.d_ff_shared), dt, dev)
    if y is None:
        y = torch.empty((p.T, p.d), dtype=torch.float32, device=dev)
    else:
        _need(y, "y", (p.T, p.d), torch.float32, dev)
    C = expert_choice_capacity(p)
    need = expert_choice_workspace_bytes(p)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    elif ws.device != dev or ws.dtype != torch.uint8 or ws.numel() < need:
        raise ValueError(f"workspace must be a uint8 tensor of >= {need} bytes on {dev}")
    r = {}
    if return_routing:
        r = dict(tokens=torch.empty((p.E, max(C, 0)), dtype=torch.int32, device=dev),
                 gates=torch.empty((p.E, max(C, 0)), dtype=torch.float32, device=dev),
                 prob_sum=torch.empty(p.E, dtype=torch.float32, device=dev))
    g = r.get
    _check("moe_forward_expert_choice", _lib.moe_forward_expert_choice(
        ctypes.byref(p), _ptr(x), _ptr(w_gate), _ptr(logit_bias), _ptr(w1), _ptr(w3), _ptr(w2),
        _ptr(ws1), _ptr(ws3), _ptr(ws2), _ptr(y), _ptr(g("tokens")), _ptr(g("gates")),
        _ptr(g("prob_sum")), _ptr(ws), ws.numel(), _stream(dev)))
    return (y, r) if return_routing else y


def backward_workspace_bytes(p: Problem) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_backward_workspace_bytes",
           _lib.moe_backward_workspace_bytes(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def backward(p: Problem, x, w_gate, w1, w3, w2, routing, dy, logit_bias=None, ws1=None, ws3=None,
             ws2=None, alpha: float = 0.01, dL: float = 0.0, want_dlogit_bias: bool = False,
             ws=None, out=None, events=None):
    """Layer backward (bf16 storage) for the routing a forward(..., return_routing=True) call
    returned. dy: [T,d] fp32 gradient of y; dL: gradient of the balance loss (alpha as in the
    forward's balance statistics). Returns a dict: dx [T,d] fp32, dw_gate [E,d] fp32,
    dw1/dw3 [E,d_ff,d] and dw2 [E,d,d_ff] in the weights' dtype, the shared expert's
    dws1/dws3/dws2 when it has one, and dlogit_bias [E] fp32 with want_dlogit_bias.
    `out` may hold preallocated tensors under those names. `events`: 11 raw hipEvent_t
    handles for moe_backward_staged (BWD_STAGES names the stages they close)."""
    dev, dt = x.device, _dt(p)
    _need(x, "x", (p.T, p.d), dt, dev)
    _need(w_gate, "w_gate", (p.E, p.d), dt, dev)
    _need(w1, "w1", (p.E, p.d_ff, p.d), dt, dev)
    _need(w3, "w3", (p.E, p.d_ff, p.d), dt, dev)
    _need(w2, "w2", (p.E, p.d, p.d_ff), dt, dev)
    _need(dy, "dy", (p.T, p.d), torch.float32, dev)
    _need(logit_bias, "logit_bias", (p.E,), torch.float32, dev, optional=True)
    if p.n_shared:
        _need(ws1, "ws1", (1, p.d_ff_shared, p.d), dt, dev)
        _need(ws3, "ws3", (1, p.d_ff_shared, p.d), dt, dev)
        _need(ws2, "ws2", (1, p.d, p.d_ff_shared), dt, dev)
    r = routing
    _need(r["topk_ids"], "topk_ids", (p.T, p.k), torch.int32, dev)
    _need(r["topk_w"], "topk_w", (p.T, p.k), torch.float32, dev)
    _need(r["counts_pre"], "counts_pre", (p.E,), torch.int32, dev)
    _need(r["offsets"], "offsets", (p.E + 1,), torch.int32, dev)
    for key in ("sorted_assign", "assign_pos"):
        t = r[key]
        if t.device != dev or t.dtype != torch.int32 or not t.is_contiguous() or t.numel() < p.T * p.k:
            raise ValueError(f"{key} must be a contiguous int32 tensor of >= T*k entries on {dev}")
    o = dict(out or {})
    want = dict(dx=((p.T, p.d), torch.float32), dw_gate=((p.E, p.d), torch.float32),
                dw1=((p.E, p.d_ff, p.d), dt), dw3=((p.E, p.d_ff, p.d), dt),
                dw2=((p.E, p.d, p.d_ff), dt))
    if p.n_shared:
        want.update(dws1=((1, p.d_ff_shared, p.d), dt), dws3=((1, p.d_ff_shared, p.d), dt),
                    dws2=((1, p.d, p.d_ff_shared), dt))
    if want_dlogit_bias:
        want["dlogit_bias"] = ((p.E,), torch.float32)
    for name, (shape, dtype) in want.items():
        if name in o:
            _need(o[name], name, shape, dtype, dev)
        else:
            o[name] = torch.empty(shape, dtype=dtype, device=dev)
    need = backward_workspace_bytes(p)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    elif ws.device != dev or ws.dtype != torch.uint8 or ws.numel() < need:
        raise ValueError(f"workspace must be a uint8 tensor of >= {need} bytes on {dev}")
    g = o.get
    args = (ctypes.byref(p), _ptr(x), _ptr(w_gate), _ptr(logit_bias), _ptr(w1), _ptr(w3), _ptr(w2),
            _ptr(ws1), _ptr(ws3), _ptr(ws2), _ptr(r["topk_ids"]), _ptr(r["topk_w"]),
            _ptr(r["counts_pre"]), _ptr(r["offsets"]), _ptr(r["sorted_assign"]),
            _ptr(r["assign_pos"]), _ptr(dy), float(alpha), float(dL), _ptr(g("dx")),
            _ptr(g("dw_gate")), _ptr(g("dlogit_bias")), _ptr(g("dw1")), _ptr(g("dw3")),
            _ptr(g("dw2")), _ptr(g("dws1")), _ptr(g("dws3")), _ptr(g("dws2")), _ptr(ws),
            ws.numel(), _stream(dev))
    if events is None:
        _check("moe_backward", _lib.moe_backward(*args))
    else:
        if len(events) != len(BWD_STAGES) + 1:
            raise ValueError(f"events: need {len(BWD_STAGES) + 1} handles")
        ev = (ctypes.c_void_p * len(events))(
            *[ctypes.c_void_p(int(e)) if not isinstance(e, ctypes.c_void_p) else e
              for e in events])
        _check("moe_backward_staged", _lib.moe_backward_staged(*args, ev))
    return o


class PreparedForward:
    """moe_forward with its arguments checked and marshalled once.

    Calling the object enqueues one forward on the current stream (the stream
    that is current at the call, so it can be captured into a HIP graph) and
    returns y. There are no per-call checks: the tensors passed here must stay
    alive, and every call reads their current contents. For decode-sized
    layers the per-call host work of forward() is comparable to the GPU time
    of the layer; this keeps it to one foreign call."""

    def __init__(self, p: Problem, x, w_gate, w1, w3, w2, logit_bias=None, sel_bias=None,
                 ws1=None, ws3=None, ws2=None, ws=None, y=None, balance_alpha=None):
        dev, dt = x.device, _dt(p)
        _need(x, "x", (p.T, p.d), dt, dev)
        _need(w_gate, "w_gate", (p.E, p.d), dt, dev)
        _need(w1, "w1", (p.E, p.d_ff, p.d), dt, dev)
        _need(w3, "w3", (p.E, p.d_ff, p.d), dt, dev)
        _need(w2, "w2", (p.E, p.d, p.d_ff), dt, dev)
        _need(logit_bias, "logit_bias", (p.E,), torch.float32, dev, optional=True)
        _need(sel_bias, "sel_bias", (p.E,), torch.float32, dev, optional=True)
        if p.n_shared:
            _need(ws1, "ws1", (1, p.d_ff_shared, p.d), dt, dev)
            _need(ws3, "ws3", (1, p.d_ff_shared, p.d), dt, dev)
            _need(ws2, "ws2", (1, p.d, p.d_ff_shared), dt, dev)
        if y is None:
            y = torch.empty((p.T, p.d), dtype=torch.float32, device=dev)
        else:
            _need(y, "y", (p.T, p.d), torch.float32, dev)
        ws = _workspace(p, dev, ws)
        self.p, self.y, self.ws, self.dev = p, y, ws, dev
        self._keep = (x, w_gate, w1, w3, w2, logit_bias, sel_bias, ws1, ws3, ws2)
        # balance_alpha: each call also writes the balance statistics f, P and L (moe_balance on
        # the call's counts_pre and prob_sum), kept as attributes f, P, L
        self.balance_alpha = balance_alpha
        cpre = psum = None
        if balance_alpha is not None:
            cpre = torch.empty((p.E,), dtype=torch.int32, device=dev)
            psum = torch.empty((p.E,), dtype=torch.float32, device=dev)
            self.f = torch.empty((p.E,), dtype=torch.float32, device=dev)
            self.P = torch.empty((p.E,), dtype=torch.float32, device=dev)
            self.L = torch.empty((1,), dtype=torch.float32, device=dev)
            self._bal_args = (ctypes.byref(p), _ptr(cpre), _ptr(psum), ctypes.c_float(balance_alpha),
                              _ptr(self.f), _ptr(self.P), _ptr(self.L))
        self.counts_pre, self.prob_sum = cpre, psum
        self._args = (ctypes.byref(p), _ptr(x), _ptr(w_gate), _ptr(logit_bias), _ptr(sel_bias),
                      _ptr(w1), _ptr(w3), _ptr(w2), _ptr(ws1), _ptr(ws3), _ptr(ws2), _ptr(y),
                      None, None, _ptr(psum), _ptr(cpre), None, None, None, None, _ptr(ws),
                      ws.numel())   # topk_ids, topk_w, prob_sum, counts_pre, counts, offsets,
                                    # sorted_assign, assign_pos
        self._fn = _lib.moe_forward

    def __call__(self):
        stream = torch.cuda.current_stream(self.dev).cuda_stream
        st = self._fn(*self._args, stream)
        if st != MOE_OK:
            raise MoEError("moe_forward", st)
        if self.balance_alpha is not None:
            st = _lib.moe_balance(*self._bal_args, stream)
            if st != MOE_OK:
                raise MoEError("moe_balance", st)
        return self.y


def forward_staged(p: Problem, x, w_gate, w1, w3, w2, events, logit_bias=None, sel_bias=None,
                   ws1=None, ws3=None, ws2=None, ws=None, y=None):
    """moe_forward plus stage events: `events` is a sequence of 7 raw hipEvent_t
    handles (ints or c_void_p) recorded before the router and after each of
    STAGES. Shapes are not re-checked here (call forward() once first); this is
    the measurement path and keeps per-call host work minimal."""
    dev = x.device
    ws = _workspace(p, dev, ws)
    ev = (ctypes.c_void_p * 7)(*[ctypes.c_void_p(int(e)) if not isinstance(e, ctypes.c_void_p)
                                 else e for e in events])
    _check("moe_forward_staged", _lib.moe_forward_staged(
        ctypes.byref(p), _ptr(x), _ptr(w_gate), _ptr(logit_bias), _ptr(sel_bias), _ptr(w1),
        _ptr(w3), _ptr(w2), _ptr(ws1), _ptr(ws3), _ptr(ws2), _ptr(y), _ptr(ws), ws.numel(),
        _stream(dev), ev))
    return y
