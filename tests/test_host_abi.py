"""Host-side checks of the C ABI (no GPU needed, no compute call).

The library must load, export every entry point declared in include/*.h, and
reject invalid problems and arguments with the documented status codes
before any HIP call."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG_LIB = os.path.join(ROOT, "mixture_experts_layer_44_amd", "libmoe_mi355x.so")


@pytest.fixture(scope="module")
def moe():
    if not os.path.exists(PKG_LIB):
        from mixture_experts_layer_44_amd import build as b   # noqa: E402  (builds on CPU)
        b.build(verbose=False)
    import mixture_experts_layer_44_amd as m
    return m


def _declared():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src))
    return sorted(names)


def test_header_declares_the_entry_points():
    d = _declared()
    for n in ("moe_route", "moe_align", "moe_expert_ffn", "moe_combine", "moe_balance",
              "moe_forward", "moe_workspace_bytes", "moe_validate", "moe_capacity",
              "moe_status_str", "moe_bias_update"):
        assert n in d


def test_library_exports_every_declared_symbol(moe):
    lib = ctypes.CDLL(moe.LIB_PATH)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_problem_struct_layout(moe):
    assert ctypes.sizeof(moe.Problem) == 40
    assert moe.Problem.capacity_factor.offset == 32


def test_status_strings(moe):
    lib = moe.lib()
    assert lib.moe_status_str(0) == b"ok"
    assert lib.moe_status_str(3) == b"workspace too small"
    assert lib.moe_status_str(99) == b"unknown status"


@pytest.mark.parametrize("kw,status", [
    (dict(), 0),
    (dict(T=0), 0),
    (dict(T=-1), 1),
    (dict(d=0), 1),
    (dict(E=0), 1),
    (dict(k=0), 1),
    (dict(dtype="f32", d=100), 0),
    (dict(dtype="f32", d=102), 2),
    (dict(d=192), 2),                     # bf16: d % 128
    (dict(d_ff=200), 2),                  # bf16: d_ff % 128
    (dict(E=257, k=2), 2),
    (dict(E=4, k=5), 2),
    (dict(E=64, k=33), 2),
    (dict(n_shared=2, d_ff_shared=256), 2),
    (dict(n_shared=1, d_ff_shared=384), 2),
    (dict(n_shared=1, d_ff_shared=256), 0),
    (dict(capacity_factor=float("nan")), 1),
    (dict(capacity_factor=float("inf")), 1),
])
def test_validate(moe, kw, status):
    args = dict(T=16, d=256, E=8, k=2, d_ff=256)
    args.update(kw)
    p = moe.make_problem(**args)
    assert moe.validate(p) == status


def test_bad_dtype_enum(moe):
    p = moe.make_problem(16, 256, 8, 2, 256)
    p.dtype = 7
    assert moe.validate(p) == moe.MOE_EINVAL


def test_capacity_matches_definition(moe):
    import oracle
    import workloads
    w = workloads.get("skew_cap")
    assert moe.capacity(moe.problem_for(w)) == 640 == oracle.capacity(*workloads.capacity_inputs(w))
    for T, k, E, cf in [(10, 2, 3, 1.0), (4096, 8, 256, 1.25), (7, 1, 5, 0.1), (1000, 2, 64, 1.5)]:
        p = moe.make_problem(T, 128, E, k, 128, capacity_factor=cf)
        assert moe.capacity(p) == oracle.capacity(cf, T, k, E)
    assert moe.capacity(moe.make_problem(10, 128, 4, 2, 128)) is None


def test_workspace_bytes_positive_and_monotone(moe):
    a = moe.workspace_bytes(moe.make_problem(16, 256, 8, 2, 256))
    b = moe.workspace_bytes(moe.make_problem(1024, 256, 8, 2, 256))
    assert 0 < a < b
    assert moe.workspace_bytes(moe.make_problem(0, 256, 8, 2, 256)) > 0


def test_invalid_calls_return_before_any_launch(moe):
    """Argument errors are returned on the host; nothing reaches HIP (there is no GPU here)."""
    lib = moe.lib()
    p = moe.make_problem(16, 256, 8, 2, 256)
    fake = ctypes.c_void_p(0x1000)          # never dereferenced: validation fails first
    null = None
    # required pointer missing -> EINVAL
    assert lib.moe_forward(ctypes.byref(p), null, fake, null, null, fake, fake, fake, null, null, null,
                           fake, *([null] * 8), fake, 1 << 40, null) == moe.MOE_EINVAL
    # workspace too small -> EWORKSPACE
    assert lib.moe_forward(ctypes.byref(p), fake, fake, null, null, fake, fake, fake, null, null, null,
                           fake, *([null] * 8), fake, 16, null) == moe.MOE_EWORKSPACE
    assert lib.moe_route(ctypes.byref(p), fake, fake, null, null, fake, fake, null, fake, 16,
                         null) == moe.MOE_EWORKSPACE
    assert lib.moe_align(ctypes.byref(p), null, fake, fake, fake, fake, fake, fake, 1 << 40,
                         null) == moe.MOE_EINVAL
    # shared expert declared but its weights missing -> EINVAL
    ps = moe.make_problem(16, 256, 8, 2, 256, n_shared=1, d_ff_shared=256)
    assert lib.moe_expert_ffn(ctypes.byref(ps), fake, fake, fake, fake, null, null, null, fake, fake,
                              fake, fake, fake, 1 << 40, null) == moe.MOE_EINVAL
    assert lib.moe_combine(ctypes.byref(ps), fake, fake, fake, null, fake, null) == moe.MOE_EINVAL
    # unsupported shape -> EUNSUPPORTED, before pointers are looked at
    pu = moe.make_problem(16, 200, 8, 2, 256)
    assert lib.moe_forward(ctypes.byref(pu), *([null] * 20), 0, null) == moe.MOE_EUNSUPPORTED
    assert lib.moe_balance(ctypes.byref(p), fake, fake, ctypes.c_float(float("nan")), fake, fake,
                           fake, null) == moe.MOE_EINVAL
    # bias step: negative or non-finite step, or a missing pointer -> EINVAL
    for g in (-0.5, float("nan"), float("inf")):
        assert lib.moe_bias_update(ctypes.byref(p), fake, ctypes.c_float(g), fake, null) == moe.MOE_EINVAL
    assert lib.moe_bias_update(ctypes.byref(p), null, ctypes.c_float(0.1), fake, null) == moe.MOE_EINVAL
    # null problem
    assert lib.moe_validate(None) == moe.MOE_EINVAL


def test_package_has_no_cpu_fallback():
    """The binding holds no arithmetic of the layer: it never imports the oracle or numpy."""
    src = open(os.path.join(ROOT, "mixture_experts_layer_44_amd", "__init__.py")).read()
    assert "oracle" not in src.replace("no CPU fallback", "")
    assert "import numpy" not in src


def test_expert_choice_capacity_matches_oracle(moe):
    import oracle
    for (T, d, E, k, cf) in [(4096, 256, 8, 2, 0.0), (16384, 256, 64, 2, 1.25), (300, 256, 7, 3, 0.0),
                             (10, 256, 2, 2, 0.0), (0, 256, 8, 2, 0.0), (1, 256, 128, 8, 0.0)]:
        p = moe.make_problem(T, d, E, k, 256, capacity_factor=cf)
        assert moe.expert_choice_capacity(p) == oracle.expert_choice_capacity(cf, T, k, E)
    assert moe.expert_choice_workspace_bytes(moe.make_problem(4096, 256, 8, 2, 256)) > 0


def test_backward_validation_returns_before_any_launch(moe):
    """moe_backward's argument errors come back on the host, before anything is enqueued."""
    lib = moe.lib()
    f = ctypes.c_float
    fake = ctypes.c_void_p(0x1000)          # never dereferenced: validation fails first
    null = None
    p = moe.make_problem(16, 256, 8, 2, 256)

    def call(prob, ptrs=None, alpha=0.01, dL=1.0, ws_bytes=1 << 40, staged=None):
        ptrs = list(ptrs if ptrs is not None else [fake] * 16)
        outs = [fake, fake, null, fake, fake, fake, null, null, null]   # dx .. dws2
        args = [ctypes.byref(prob)] + ptrs + [f(alpha), f(dL)] + outs + [fake, ws_bytes, null]
        if staged is not None:
            return lib.moe_backward_staged(*args, staged)
        return lib.moe_backward(*args)

    # fp32 storage and k > 16 are not supported
    assert call(moe.make_problem(16, 256, 8, 2, 256, dtype="f32")) == moe.MOE_EUNSUPPORTED
    assert call(moe.make_problem(16, 256, 32, 17, 256)) == moe.MOE_EUNSUPPORTED
    # a missing required input (x) or a non-finite alpha / dL
    ptrs = [fake] * 16
    ptrs[0] = null
    assert call(p, ptrs) == moe.MOE_EINVAL
    assert call(p, alpha=float("nan")) == moe.MOE_EINVAL
    assert call(p, dL=float("inf")) == moe.MOE_EINVAL
    # shared expert declared but its weights (and gradient outputs) missing
    ps = moe.make_problem(16, 256, 8, 2, 256, n_shared=1, d_ff_shared=256)
    ptrs = [fake] * 16
    ptrs[6] = ptrs[7] = ptrs[8] = null
    assert call(ps, ptrs) == moe.MOE_EINVAL
    # workspace too small
    assert call(p, ws_bytes=16) == moe.MOE_EWORKSPACE
    # staged: a NULL events array
    assert lib.moe_backward_staged(ctypes.byref(p), *([fake] * 16), f(0.01), f(1.0), fake, fake,
                                   null, fake, fake, fake, null, null, null, fake, 1 << 40, null,
                                   null) == moe.MOE_EINVAL
    # workspace size: bf16 only, grows with T
    a = moe.backward_workspace_bytes(moe.make_problem(16, 256, 8, 2, 256))
    b = moe.backward_workspace_bytes(moe.make_problem(1024, 256, 8, 2, 256))
    assert 0 < a < b
    with pytest.raises(moe.MoEError):
        moe.backward_workspace_bytes(moe.make_problem(16, 256, 8, 2, 256, dtype="f32"))


def _padded_rows(T, E, k, bm):
    """Rows of the padded row table: ceil(T*k / bm) tiles plus one spare tile per expert."""
    return (-(-T * k // bm) + E) * bm


@pytest.mark.parametrize("T,status", [(140000, 0), (148000, 0), (150000, 2)])
def test_padded_rows_times_dff_must_fit_32bit_offsets(moe, T, status):
    # Mixtral-shaped layer: the down GEMM addresses h [padded rows, d_ff] with 32-bit element
    # offsets, so shapes whose table reaches 2^32 elements are refused before any launch
    rows = _padded_rows(T, 8, 2, 256)
    assert (rows * 14336 >= 2 ** 32) == (status != 0)
    assert moe.validate(moe.make_problem(T, 4096, 8, 2, 14336)) == status


@pytest.mark.parametrize("T,status", [(2 ** 19 - 1, 0), (2 ** 19, 2)])
def test_x_elements_must_fit_32bit_offsets(moe, T, status):
    # x [T, d] with d = 8192: T*d reaches 2^32 at T = 2^19
    assert moe.validate(moe.make_problem(T, 8192, 256, 1, 128)) == status


@pytest.mark.parametrize("T,status", [(70000, 0), (75000, 2)])
def test_backward_rows_times_width_must_fit_32bit_offsets(moe, T, status):
    # the backward also addresses du|dv [padded rows, 2*d_ff]
    n = ctypes.c_size_t(0)
    p = moe.make_problem(T, 4096, 8, 2, 14336)
    assert moe.validate(p) == 0
    assert moe.lib().moe_backward_workspace_bytes(ctypes.byref(p), ctypes.byref(n)) == status
    assert (_padded_rows(T, 8, 2, 256) * 2 * 14336 >= 2 ** 32) == (status != 0)
