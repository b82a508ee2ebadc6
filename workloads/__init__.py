"""Seeded synthetic inputs for the sparse MoE layer forward.

This module holds the workload presets (shapes, value distributions, seeds)
and the seeded generator that both the GPU path's callers and the CPU oracle
consume. It contains none of the layer's arithmetic: no routing, no expert
math, no combine.

Value recipe (the same for every workload):
  * x ~ N(0, 1) per element;
  * router, expert and shared-expert weights ~ N(0, 0.02^2) (std 0.02);
  * selection-only bias ~ U(-0.1, 0.1) in fp32 (fine-grained workload);
  * skewed workload: a per-expert logit offset -s*ln(e+1) with s = 1.1, so the
    router prior falls off as a power of the expert's rank (Zipf-like);
  * bf16 workloads: draw in fp32, scale, round once to bf16 (round to nearest
    even, torch's conversion). The stored values are what every consumer sees.

Every tensor gets its own torch.Generator seeded from (workload seed, tensor
tag, expert index), so a single expert's weights can be regenerated on its
own, on the device that will hold it.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass
from typing import Dict, Optional

import torch

__all__ = ["Workload", "WORKLOADS", "get", "generate", "tensor_seed"]


@dataclass(frozen=True)
class Workload:
    name: str
    T: int                 # tokens
    d: int                 # hidden size
    E: int                 # routed experts
    k: int                 # experts per token
    d_ff: int              # routed-expert intermediate size
    seed: int
    dtype: str = "bf16"    # storage of x and all weights: "bf16" or "f32"
    n_shared: int = 0      # always-on shared experts (0 or 1)
    d_ff_shared: int = 0
    capacity_factor: float = 0.0   # <= 0: no capacity limit
    sel_bias: bool = False         # selection-only per-expert bias ~ U(-0.1, 0.1)
    zipf_s: float = 0.0            # per-expert logit offset -s*ln(e+1); 0 = none
    balance_alpha: float = 0.0     # > 0: the layer also outputs f, P and L_balance (this alpha)
    weight_std: float = 0.02

    def with_tokens(self, T: int, seed: Optional[int] = None) -> "Workload":
        return dataclasses.replace(self, T=T, seed=self.seed if seed is None else seed,
                                   name=f"{self.name}@T{T}")

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


def _decode(T: int) -> Workload:
    return Workload(name=f"decode_T{T}", T=T, d=2048, E=128, k=8, d_ff=768, seed=44040 + T)


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        # tiny fp32 layer: parity at 1e-5
        Workload(name="tiny_fp32", T=64, d=128, E=8, k=2, d_ff=256, seed=44001, dtype="f32"),
        # Mixtral-shaped prefill: 8 experts, top-2, wide experts
        Workload(name="mixtral_prefill", T=4096, d=4096, E=8, k=2, d_ff=14336, seed=44002),
        # DeepSeek-V3-shaped fine-grained layer: 256 routed + 1 shared, top-8, selection bias
        Workload(name="dsv3_fine", T=4096, d=7168, E=256, k=8, d_ff=2048, seed=44003,
                 n_shared=1, d_ff_shared=2048, sel_bias=True),
        # decode-sized, weight-read bound
        _decode(1), _decode(8), _decode(32), _decode(128),
        # skewed routing with a capacity limit and dropping
        Workload(name="skew_cap", T=16384, d=4096, E=64, k=2, d_ff=1408, seed=44005,
                 capacity_factor=1.25, zipf_s=1.1, balance_alpha=0.01),
        # the handbook page's naive-vs-grouped check shape (fp32, 1 shared expert)
        Workload(name="handbook_fp32", T=50, d=64, E=16, k=4, d_ff=128, seed=44006,
                 dtype="f32", n_shared=1, d_ff_shared=128),
    ]
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


_TAGS = {"x": 1, "w_gate": 2, "w1": 3, "w3": 4, "w2": 5, "ws1": 6, "ws3": 7, "ws2": 8, "sel_bias": 9}


def tensor_seed(seed: int, tag: str, index: int = 0) -> int:
    """A 63-bit generator seed for one tensor (or one expert's slice of it).

    SplitMix64-style mixing of (seed, tag, index); any fixed injective-ish mix
    would do, this one only has to be stable across runs and machines."""
    z = (seed * 0x9E3779B97F4A7C15 + _TAGS[tag] * 0xBF58476D1CE4E5B9 + index * 0x94D049BB133111EB)
    z &= (1 << 64) - 1
    z ^= z >> 30
    z = (z * 0xBF58476D1CE4E5B9) & ((1 << 64) - 1)
    z ^= z >> 27
    z = (z * 0x94D049BB133111EB) & ((1 << 64) - 1)
    z ^= z >> 31
    return z & ((1 << 63) - 1)


def _normal(shape, std: float, seed: int, dtype: torch.dtype, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def generate(w: Workload, device="cpu", T: Optional[int] = None) -> Dict[str, Optional[torch.Tensor]]:
    """All inputs of workload `w` as torch tensors on `device`.

    Returns x [T,d], w_gate [E,d], w1/w3 [E,d_ff,d], w2 [E,d,d_ff] (row-major,
    "out x in" like a linear layer's weight), the shared expert's ws1/ws3
    [n_shared,d_ff_s,d] and ws2 [n_shared,d,d_ff_s] (None without one),
    logit_bias [E] fp32 (None unless the workload is skewed) and sel_bias [E]
    fp32 (None unless the workload has one). Experts are generated one at a
    time so the peak temporary is one expert's fp32 draw."""
    T = w.T if T is None else T
    dt = w.torch_dtype
    dev = torch.device(device)
    std = w.weight_std
    out: Dict[str, Optional[torch.Tensor]] = {}
    out["x"] = _normal((T, w.d), 1.0, tensor_seed(w.seed, "x"), dt, dev)
    out["w_gate"] = _normal((w.E, w.d), std, tensor_seed(w.seed, "w_gate"), dt, dev)
    for name, shape in (("w1", (w.d_ff, w.d)), ("w3", (w.d_ff, w.d)), ("w2", (w.d, w.d_ff))):
        buf = torch.empty((w.E,) + shape, dtype=dt, device=dev)
        for e in range(w.E):
            buf[e] = _normal(shape, std, tensor_seed(w.seed, name, e), dt, dev)
        out[name] = buf
    if w.n_shared:
        for name, shape in (("ws1", (w.d_ff_shared, w.d)), ("ws3", (w.d_ff_shared, w.d)),
                            ("ws2", (w.d, w.d_ff_shared))):
            buf = torch.empty((w.n_shared,) + shape, dtype=dt, device=dev)
            for s in range(w.n_shared):
                buf[s] = _normal(shape, std, tensor_seed(w.seed, name, s), dt, dev)
            out[name] = buf
    else:
        out["ws1"] = out["ws3"] = out["ws2"] = None
    if w.zipf_s:
        out["logit_bias"] = torch.tensor([-w.zipf_s * math.log(e + 1.0) for e in range(w.E)],
                                         dtype=torch.float32, device=dev)
    else:
        out["logit_bias"] = None
    if w.sel_bias:
        g = torch.Generator(device=dev)
        g.manual_seed(tensor_seed(w.seed, "sel_bias"))
        u = torch.rand((w.E,), generator=g, device=dev, dtype=torch.float64)
        out["sel_bias"] = (u * 0.2 - 0.1).to(torch.float32)
    else:
        out["sel_bias"] = None
    return out


def capacity_inputs(w: Workload):
    """(capacity_factor, T, k, E): the numbers the capacity limit is defined on."""
    return w.capacity_factor, w.T, w.k, w.E
