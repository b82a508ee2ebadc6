"""Pins for the benchmark's algorithmic work model (CPU only)."""
import bench
import workloads
from util import golden


def test_expert_params_handbook_exercise():
    """Handbook exercise 1: 64 experts of 3*2048*1408, top-8, 24 layers ->
    13.29B expert parameters in total, 1.66B activated per token."""
    g = golden("param_accounting_handbook.json")
    per = bench.expert_params(g["d"], g["d_ff"])
    assert per == 3 * 2048 * 1408 == 8_650_752
    assert round(g["E"] * per * g["layers"] / 1e9, 2) == g["expected_total_billions"]
    assert round(g["k"] * per * g["layers"] / 1e9, 2) == g["expected_active_billions"]


def test_sparsity_ratio_arch():
    """MoE Architecture §1: k=2 of E=64 experts is about 3% of expert parameters per token."""
    g = golden("sparsity_ratio_arch.json")
    per = bench.expert_params(4096, 1024)
    assert round(100 * g["k"] * per / (g["E"] * per)) == g["expected_percent_rounded"]


def test_algorithmic_work_mixtral_shape():
    w = workloads.get("mixtral_prefill")
    counts = [1024] * 8                       # every assignment kept, 8 experts touched
    a = bench.algorithmic_work(w, counts)
    assert a["flops"] == 2 * 4096 * 4096 * 8 + 6 * 4096 * 14336 * 8192
    assert a["bytes"] == 4096 * 4096 * 2 + 8 * 4096 * 2 + 8 * 3 * 4096 * 14336 * 2 + 4096 * 4096 * 4
    k = bench.kernel_work(w, counts, "gate_up")
    assert k["flops"] == 4 * 4096 * 14336 * 8192
    # only touched experts' weights count
    b = bench.algorithmic_work(w, [2048, 0, 0, 0, 2048, 2048, 2048, 0])
    assert b["touched"] == 4 and b["bytes"] < a["bytes"]


def test_decode_t1_bytes():
    """Decode T=1 reads 8 experts' full weights: 8 x 3 x 2048 x 768 x 2 B = 75.5 MB."""
    w = workloads.get("decode_T1")
    a = bench.algorithmic_work(w, [1] * 8 + [0] * 120)
    assert a["touched"] == 8
    assert abs(a["bytes"] - (8 * 3 * 2048 * 768 * 2 + 2048 * 2 + 128 * 2048 * 2 + 2048 * 4)) == 0


def test_gemm_stage_names():
    """The counter post-processing finds the gate-up / down flag in each GEMM kernel family."""
    import bench
    assert bench.gemm_stage("void moe::(anonymous namespace)::gemm_bf16_st_kernel<256, 256, 4, 2, "
                            "true, false>(moe::(anonymous namespace)::GemmArgs)") == "gate_up"
    assert bench.gemm_stage("moe::gemm_bf16_st_kernel<256, 256, 4, 2, false, false>(x)") == "down"
    assert bench.gemm_stage("moe::gemm_bf16_kernel<128, 256, 2, 4, 64, 3, true>(x)") == "gate_up"
    assert bench.gemm_stage("moe::gemm_bf16_kernel<32, 128, 1, 4, 64, 4, false>(x)") == "down"
    assert bench.gemm_stage("moe::gemm_bf16_kernel<256, 256, 4, 2, 64, 2, true, true>(x)") == "gate_up"
    assert bench.gemm_stage("moe::gemm_bf16_st_kernel<192, 256, 2, 4, true, false, false>(x)") == "gate_up"
    assert bench.gemm_stage("void moe::(anonymous namespace)::gemm_bf16_w4_kernel<true>"
                            "(moe::(anonymous namespace)::GemmArgs)") == "gate_up"
    assert bench.gemm_stage("moe::gemm_bf16_w4_kernel<false>(x)") == "down"
    assert bench.gemm_stage("moe::gemm_bf16_dec_kernel<true, 8>(x)") == "gate_up"
    assert bench.gemm_stage("moe::gemm_bf16_dec_kernel<false, 3>(x)") == "down"
    assert bench.gemm_stage("moe::gemm_f32_kernel<false>(x)") == "down"
    assert bench.gemm_stage("__amd_rocclr_copyBuffer") is None
    assert bench.gemm_stage("moe::combine_kernel(float const*)") is None


def test_counter_summaries_go_void_when_a_kernel_source_changes(tmp_path, monkeypatch):
    """A profiles/traffic_*.json summary counts only while every source its stage's kernels are
    built from (the GEMM file, the tile walk, the shared definitions) is unchanged."""
    import json
    import os
    import shutil
    import bench
    csrc = os.path.join(bench.ROOT, "mixture_experts_layer_44_amd", "csrc")
    shutil.copytree(csrc, tmp_path / "mixture_experts_layer_44_amd" / "csrc")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    for stage in ("gate_up", "down"):
        for name in bench.KERNEL_SOURCES[stage]:
            assert os.path.exists(tmp_path / "mixture_experts_layer_44_amd" / "csrc" / name)
        sha = bench.source_sha(stage)
        rec = {"source_sha": sha, "traffic_bytes_per_launch": 123.0}
        (tmp_path / "profiles" / f"traffic_{stage}_w.json").write_text(json.dumps(rec))
        assert bench.traffic_from_profile(stage, "w") == 123.0
        assert bench.traffic_from_profile(stage, "other") is None
        for name in bench.KERNEL_SOURCES[stage]:     # touching any one source voids it
            path = tmp_path / "mixture_experts_layer_44_amd" / "csrc" / name
            orig = path.read_bytes()
            path.write_bytes(orig + b"\n")
            assert bench.traffic_from_profile(stage, "w") is None, name
            path.write_bytes(orig)
        assert bench.traffic_from_profile(stage, "w") == 123.0
