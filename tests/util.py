"""Shared test helpers: golden-fixture loading and torch -> fp64 NumPy plumbing.

Nothing here computes any step of the MoE layer."""
import json
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name: str) -> dict:
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def f64(t) -> np.ndarray:
    """Exact up-cast of a stored tensor (bf16 or fp32, any device) to fp64 NumPy."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()


def oracle_inputs(inp: dict) -> dict:
    """fp64 NumPy copies of a generated input dict (small workloads only)."""
    return {k: (None if v is None else f64(v)) for k, v in inp.items()}
