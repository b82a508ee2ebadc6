"""fp64 CPU oracle for the sparse MoE layer (forward and backward) -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package; the product path never does.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import __all__  # noqa: F401
