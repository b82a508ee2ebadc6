#!/usr/bin/env python3
"""Benchmark of the sparse top-k MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mixtral_prefill]

A step is one moe_forward call (router -> align -> grouped gate-up GEMM with
SwiGLU -> grouped down GEMM -> combine) over one batch of synthetic input
already resident in HBM. W untimed warm-up steps, then exactly K steps
between two device synchronisations. A second pass of K steps records HIP
events on the launch stream between the stages, for the per-stage times and
the dominant kernel's average launch duration (its roofline). Two cold passes
read a 1 GiB buffer before each step, outside its events, so no step finds the
last one's data in L2 or the Infinity Cache ("cold": medians): one with the
stage events (per-stage times), one timing the plain step alone. Prints ONE
JSON line on stdout: tokens/s of the whole job, that roofline, and the fp64
CPU oracle timed on a bounded sample of the same workload (1 core).

The default workload is the Mixtral-shaped prefill layer (T=4096, d=4096,
E=8, k=2, d_ff=14336, bf16). The other presets can be timed with --workload.
Only one GPU: --gpus N > 1 exits with a message.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec at 1 GPU (prefill, decode); % MFMA bf16 / HBM roofline"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)   # flop per byte
# the sources a stage's kernels are built from (the counter summaries are void once any changes)
_GEMM_SOURCES = ("gemm.hip", "mfma_tiles.h", "moe_internal.h")
KERNEL_SOURCES = {"gate_up": _GEMM_SOURCES, "down": _GEMM_SOURCES + ("down_combine.hip",),
                  "route": ("route.hip", "topk.h"), "align": ("align.hip",),
                  "schedule": ("align.hip",), "combine": ("combine.hip",)}
KERNEL_NAMES = {"gate_up": "grouped GEMM gate-up + SwiGLU (gemm_bf16_w4_kernel / gemm_bf16_st_kernel / "
                           "gemm_bf16_kernel with the gate-up flag set; kernel by row-tile class)",
                "down": "grouped GEMM down projection (gemm_bf16_w4_kernel / gemm_bf16_st_kernel / "
                        "gemm_bf16_kernel with the gate-up flag clear)"}
COPY_PATTERN = r"copyBuffer"   # the runtime's blit kernel (the calibration copy)


def gemm_stage(kernel_name: str):
    """'gate_up' / 'down' for a grouped-GEMM kernel name as rocprofv3 prints it, else None.
    The gate-up flag is the 7th template argument of gemm_bf16_kernel, the 5th of
    gemm_bf16_st_kernel and the first of gemm_bf16_w4_kernel, gemm_bf16_dec_kernel and
    gemm_f32_kernel."""
    m = re.search(r"gemm_(bf16_st|bf16_dec|bf16_w4|bf16|f32)_kernel<([^>]*)>", kernel_name)
    if not m:
        return None
    args = [a.strip() for a in m.group(2).split(",")]
    pos = {"bf16": 6, "bf16_st": 4, "bf16_w4": 0, "bf16_dec": 0, "f32": 0}[m.group(1)]
    if len(args) <= pos or args[pos] not in ("true", "false"):
        return None
    return "gate_up" if args[pos] == "true" else "down"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- accounting
def expert_params(d: int, d_ff: int) -> int:
    """Parameters of one SwiGLU expert: gate, up and down projections."""
    return 3 * d * d_ff


def algorithmic_work(w, counts, T=None):
    """Layer flops and bytes from the actual routing (kept rows per expert).

    flops: router 2*T*d*E + 6*d*d_ff per kept routed row + 6*d*d_ff_s per token for
    a shared expert. bytes: x + W_gate + the full weights of every expert with at
    least one kept row + the shared expert's weights + fp32 y. Padding rows, the
    intermediate h, per-row expert outputs and routing metadata are implementation
    traffic and are not counted."""
    T = w.T if T is None else T
    esz = 2 if w.dtype == "bf16" else 4
    kept = int(sum(counts))
    touched = int(sum(1 for c in counts if c > 0))
    flops = 2 * T * w.d * w.E + 6 * w.d * w.d_ff * kept + 6 * w.d * w.d_ff_shared * T * w.n_shared
    byts = (T * w.d * esz + w.E * w.d * esz + touched * expert_params(w.d, w.d_ff) * esz
            + w.n_shared * expert_params(w.d, w.d_ff_shared) * esz + T * w.d * 4)
    return dict(flops=flops, bytes=byts, kept=kept, touched=touched)


def kernel_work(w, counts, stage, T=None):
    """Algorithmic flops and bytes of one launch of a GEMM stage.

    gate-up: 4*d*d_ff flops per row (routed kept rows + shared rows); bytes = x
    (read once) + W1 and W3 of every touched expert (+ shared) + h written (bf16,
    one row per kept row). down: 2*d*d_ff flops per row; bytes = h read + W2 of
    every touched expert (+ shared) + fp32 output rows written."""
    T = w.T if T is None else T
    esz = 2 if w.dtype == "bf16" else 4
    hsz = 2 if w.dtype == "bf16" else 4
    kept = int(sum(counts))
    touched = int(sum(1 for c in counts if c > 0))
    rows = kept + T * w.n_shared
    wmat = w.d * w.d_ff * esz
    groups = touched + w.n_shared
    if stage == "gate_up":
        return dict(flops=4 * w.d * w.d_ff * rows,
                    bytes=T * w.d * esz + 2 * wmat * groups + rows * w.d_ff * hsz)
    if stage == "down":
        return dict(flops=2 * w.d * w.d_ff * rows,
                    bytes=rows * w.d_ff * hsz + wmat * groups + rows * w.d * 4)
    raise ValueError(stage)


def source_sha(stage: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[stage]:
        with open(os.path.join(ROOT, "mixture_experts_layer_44_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(stage: str, workload: str):
    """HBM bytes per launch from the committed counter summary, or None if there is
    none or the kernel source has changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{stage}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha") != source_sha(stage):
        return None
    return rec.get("traffic_bytes_per_launch")


def _counter_rows(csv_path: str, counter: str):
    """(kernel name, value) of every dispatch in a rocprofv3 counter_collection CSV."""
    with open(csv_path) as f:
        return [(r["Kernel_Name"], float(r["Counter_Value"])) for r in csv.DictReader(f)
                if r["Counter_Name"] == counter]


def write_traffic(fetch_csv: str, write_csv: str, workload: str, calib_mib: int, command: str):
    """Turn two rocprofv3 --pmc passes (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch) over
    `bench.py --calib-copy-mib M` into HBM bytes per launch of each grouped GEMM.

    Each counter is scaled by what it reads for the plain device-to-device copy of M MiB that
    the same run makes (M MiB read, M MiB written), so a counter that over- or under-counts
    by a constant factor is corrected. Writes profiles/traffic_<stage>_<workload>.json."""
    res = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _counter_rows(path, counter)
        copies = [v for n, v in rows if re.search(COPY_PATTERN, n)]
        if not copies:
            raise SystemExit(f"no copy-kernel dispatch in {path}: run bench.py with --calib-copy-mib")
        # the blit may be split over several dispatches: use the largest (the bulk of the copy)
        calib = calib_mib * 1024.0 / max(copies)        # true KiB / counted KiB
        for stage in ("gate_up", "down"):
            vals = [v for n, v in rows if gemm_stage(n) == stage]
            if vals:
                res.setdefault(stage, {})[counter] = dict(
                    kib_per_dispatch=sum(vals) / len(vals), dispatches=len(vals), scale=calib,
                    bytes_per_launch=sum(vals) / len(vals) * calib * 1024.0)
    if not res:
        raise SystemExit("no grouped-GEMM dispatch found in the counter files")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    for stage, c in res.items():
        if "FETCH_SIZE" not in c or "WRITE_SIZE" not in c:
            continue
        rec = {"stage": stage, "workload": workload, "kernel": KERNEL_NAMES[stage],
               "source_sha": source_sha(stage),
               "traffic_bytes_per_launch": c["FETCH_SIZE"]["bytes_per_launch"]
               + c["WRITE_SIZE"]["bytes_per_launch"],
               "fetch": c["FETCH_SIZE"], "write": c["WRITE_SIZE"],
               "calibration": f"device-to-device copy of {calib_mib} MiB in the same run",
               "command": command}
        path = os.path.join(ROOT, "profiles", f"traffic_{stage}_{workload}.json")
        with open(path, "w") as f:
            json.dump(rec, f, indent=1)
        log(f"[bench] wrote {path}: {rec['traffic_bytes_per_launch'] / 1e9:.3f} GB per launch")


def calibration_copy(mib: int, dev, reps: int = 3):
    """A plain device-to-device copy of `mib` MiB (torch issues it as the runtime's blit
    kernel), for scaling the memory counters."""
    import torch
    src = torch.empty(mib << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


# ----------------------------------------------------------------------------- CPU baseline
def cpu_model() -> str:
    """The host CPU's model name as the kernel reports it (first processor), or 'unknown'."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.lower().startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(w, inp, sample_tokens: int):
    """The fp64 oracle, as it stands, on the first `sample_tokens` tokens of the
    workload (all of its experts' weights), on one host core."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits
    import oracle as O

    S = min(sample_tokens, w.T)
    cpu = {k: (None if v is None else v[:S].cpu() if k == "x" else v.cpu()) for k, v in inp.items()}

    def f64(t):
        return None if t is None else t.to(torch.float64).numpy()

    def experts(e):
        return f64(cpu["w1"][e]), f64(cpu["w3"][e]), f64(cpu["w2"][e])

    shared = [(f64(cpu["ws1"][0]), f64(cpu["ws3"][0]), f64(cpu["ws2"][0]))] if w.n_shared else []
    torch_threads = torch.get_num_threads()
    torch.set_num_threads(1)
    try:
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            y, info = O.moe_forward(f64(cpu["x"]), f64(cpu["w_gate"]), experts, w.E, w.k,
                                    logit_bias=f64(cpu["logit_bias"]), sel_bias=f64(cpu["sel_bias"]),
                                    shared=shared, capacity_factor=w.capacity_factor)
            O.balance(info["counts_pre"], info["probs"], S, w.k)
            dt = time.perf_counter() - t0
    finally:
        torch.set_num_threads(torch_threads)
    assert np.isfinite(y).all()
    return {"value": S / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"first {S} of {w.T} tokens of {w.name}, every expert's full weights "
                      f"(fp64 up-cast included), route+align+experts+combine+balance; {dt:.1f} s",
            "seconds": dt}


# ----------------------------------------------------------------------------- expert choice
def bench_expert_choice(args, w, p, g, kw, y, torch, moe):
    """Times exactly K moe_forward_expert_choice calls; the algorithmic work counts the E*C
    bucket rows. The per-kernel times come from rocprofv3 (profiles/), not from stage events."""
    C = moe.expert_choice_capacity(p)
    ws = torch.empty(max(moe.expert_choice_workspace_bytes(p), 1), dtype=torch.uint8,
                     device=y.device)

    def step():
        moe.forward_expert_choice(p, g["x"], g["w_gate"], g["w1"], g["w3"], g["w2"],
                                  logit_bias=kw["logit_bias"], ws1=kw["ws1"], ws3=kw["ws3"],
                                  ws2=kw["ws2"], ws=ws, y=y)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    assert torch.isfinite(y).all().item()
    ms_per_step = elapsed * 1e3 / args.steps
    lw = algorithmic_work(w, [C] * w.E)
    t_layer = ms_per_step * 1e-3
    log(f"[bench] expert choice C={C}: {ms_per_step:.4f} ms/step, {w.T / (elapsed / args.steps):,.0f} tokens/s")
    cfg = {"workload": w.name, "routing": "expert_choice", "C": C, "T": w.T, "d": w.d, "E": w.E,
           "k": w.k, "d_ff": w.d_ff, "n_shared": w.n_shared, "capacity_factor": w.capacity_factor,
           "seed": w.seed}
    line = {"metric": METRIC, "value": w.T * args.steps / elapsed, "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16" if w.dtype == "bf16" else "f32", "data": "synthetic", "config": cfg,
            "roofline": None, "cpu_baseline": None,
            "layer": {"flops": lw["flops"], "bytes": lw["bytes"], "bucket_rows": w.E * C,
                      "mfma_frac": lw["flops"] / t_layer / (PEAK_BF16_TFLOPS * 1e12),
                      "hbm_frac": lw["bytes"] / t_layer / (PEAK_HBM_GBS * 1e9)},
            "launch": "eager"}
    print(json.dumps(line), flush=True)
    return 0


# ----------------------------------------------------------------------------- main
def backward_stage_work(w, counts, stage, T=None):
    """Algorithmic flops and bytes of one stage of the layer backward (bf16 storage).

    rows = kept routed rows + the shared expert's T rows; groups = touched experts (+ shared);
    every expert's weight gradient is written (zeros for an untouched one). Each distinct
    input is counted once, each output once; padding, staging copies and re-reads are not.
      recompute  4 d d_ff / row;  x, W1 and W3 of each group;  h (bf16) and u, v (fp32) rows
      dgrad_down 2 d d_ff / row;  dy (bf16, per token), W2 per group, u, v;  du|dv (bf16)
      dgrad_x    4 d d_ff / row;  du|dv, W1 and W3 per group;  fp32 output rows
      wgrad_down 2 d d_ff / row;  g dy and h rows;  dW2 of every expert (bf16)
      wgrad_up   4 d d_ff / row;  du|dv and x rows;  dW1 and dW3 of every expert (bf16)
      router_dgrad / router_wgrad  2 T E d each;  d l (bf16) + W_gate or x;  fp32 output"""
    T = w.T if T is None else T
    kept = int(sum(counts))
    touched = int(sum(1 for c in counts if c > 0))
    rows = kept + T * w.n_shared
    groups = touched + w.n_shared
    G = w.E + w.n_shared
    d, f = w.d, w.d_ff
    wmat = d * f * 2
    if stage == "recompute":
        return dict(flops=4 * d * f * rows, bytes=T * d * 2 + 2 * wmat * groups + rows * f * 10)
    if stage == "dgrad_down":
        return dict(flops=2 * d * f * rows,
                    bytes=T * d * 2 + wmat * groups + rows * f * 8 + rows * 2 * f * 2)
    if stage == "dgrad_x":
        return dict(flops=4 * d * f * rows,
                    bytes=rows * 2 * f * 2 + 2 * wmat * groups + rows * d * 4)
    if stage == "wgrad_down":
        return dict(flops=2 * d * f * rows, bytes=rows * (d + f) * 2 + wmat * G)
    if stage == "wgrad_up":
        return dict(flops=4 * d * f * rows, bytes=rows * (2 * f + d) * 2 + 2 * wmat * G)
    if stage in ("router_dgrad", "router_wgrad"):
        return dict(flops=2 * T * w.E * d, bytes=T * w.E * 2 + T * d * 2 + w.E * d * 2 + T * d * 4)
    raise ValueError(stage)


def bench_backward(args, w, p, g, kw, y, torch, moe):
    """Time moe_backward over the resident batch: K calls between two synchronisations, then
    a second pass of K staged calls for the per-stage times and the dominant kernel."""
    dev = y.device
    _, r = moe.forward(p, g["x"], g["w_gate"], g["w1"], g["w3"], g["w2"], return_routing=True, y=y,
                       **kw)
    counts = r["counts"].cpu().tolist()
    gen = torch.Generator(device=dev)
    gen.manual_seed(4401)
    dy = torch.randn((w.T, w.d), generator=gen, device=dev, dtype=torch.float32)
    bw = dict(logit_bias=kw["logit_bias"], ws1=kw["ws1"], ws3=kw["ws3"], ws2=kw["ws2"],
              alpha=0.01, dL=1.0, want_dlogit_bias=True)
    bws = torch.empty(moe.backward_workspace_bytes(p), dtype=torch.uint8, device=dev)
    out = moe.backward(p, g["x"], g["w_gate"], g["w1"], g["w3"], g["w2"], r, dy, ws=bws, **bw)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        moe.backward(p, g["x"], g["w_gate"], g["w1"], g["w3"], g["w2"], r, dy, ws=bws, out=out, **bw)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        moe.backward(p, g["x"], g["w_gate"], g["w1"], g["w3"], g["w2"], r, dy, ws=bws, out=out, **bw)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = elapsed * 1e3 / args.steps
    for name, t in out.items():
        assert torch.isfinite(t.float()).all().item(), name

    n_ev = len(moe.BWD_STAGES) + 1
    stream = torch.cuda.current_stream(dev)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    for evs in events:
        for e in evs:
            e.record(stream)
    torch.cuda.synchronize()
    for s_ in range(args.steps):
        moe.backward(p, g["x"], g["w_gate"], g["w1"], g["w3"], g["w2"], r, dy, ws=bws, out=out,
                     events=[e.cuda_event for e in events[s_]], **bw)
    torch.cuda.synchronize()
    stage_ms = {}
    for i, name in enumerate(moe.BWD_STAGES):
        vals = [events[s][i].elapsed_time(events[s][i + 1]) for s in range(args.steps)]
        stage_ms[name] = sum(vals) / len(vals)
    log("[bench] backward stage ms: " + ", ".join(f"{k}={v:.4f}" for k, v in stage_ms.items()))
    log(f"[bench] backward {ms:.4f} ms/step, {w.T / (ms * 1e-3):,.0f} tokens/s "
        f"(stage-event pass: {sum(stage_ms.values()):.4f} ms/step)")

    gemms = ("recompute", "dgrad_down", "dgrad_x", "wgrad_down", "wgrad_up")
    dom = max(gemms, key=lambda s: stage_ms[s])
    kwk = backward_stage_work(w, counts, dom)
    t_dom = stage_ms[dom] * 1e-3
    if kwk["flops"] / kwk["bytes"] >= RIDGE:
        roof = {"bound": "mfma", "achieved": kwk["flops"] / t_dom / 1e12, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": kwk["bytes"] / t_dom / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    roof["kernel"] = f"bwd_gemm_kernel ({dom})" if dom != "recompute" else "gate-up recompute"
    roof["launch_stream"] = "torch current stream (HIP events recorded around the launch)"
    roof["avg_launch_ms"] = stage_ms[dom]
    roof["algorithmic_per_launch"] = {"flops": kwk["flops"], "bytes": kwk["bytes"]}
    per_stage = {}
    for st in gemms + ("router_dgrad", "router_wgrad"):
        k_ = backward_stage_work(w, counts, st)
        t_ = stage_ms[st] * 1e-3
        per_stage[st] = {"ms": round(stage_ms[st], 5),
                         "tflops": round(k_["flops"] / t_ / 1e12, 1) if t_ > 0 else None,
                         "gbs": round(k_["bytes"] / t_ / 1e9, 1) if t_ > 0 else None}
    total_flops = sum(backward_stage_work(w, counts, st)["flops"]
                      for st in gemms + ("router_dgrad", "router_wgrad"))
    cfg = {"workload": w.name, "pass": "backward", "T": w.T, "d": w.d, "E": w.E, "k": w.k,
           "d_ff": w.d_ff, "n_shared": w.n_shared, "capacity_factor": w.capacity_factor,
           "seed": w.seed}
    line = {"metric": "MoE-layer backward tokens/sec at 1 GPU (gate-up recompute included)",
            "value": w.T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": cfg, "roofline": roof, "cpu_baseline": None,
            "layer": {"flops": total_flops,
                      "mfma_frac": total_flops / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
                      "stages": per_stage,
                      "stage_ms": {k: round(v, 5) for k, v in stage_ms.items()}},
            "launch": "eager"}
    print(json.dumps(line), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral_prefill")
    ap.add_argument("--tokens", type=int, default=0,
                    help="override the workload's token count T (same shapes and seeds otherwise)")
    ap.add_argument("--cpu-sample", type=int, default=2048,
                    help="tokens of the workload the CPU oracle baseline runs on")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--routing", choices=("token_choice", "expert_choice"), default="token_choice",
                    help="expert_choice: every expert takes its C highest-probability tokens "
                         "(moe_forward_expert_choice); reported without a per-stage roofline")
    ap.add_argument("--pass", dest="pass_", choices=("forward", "backward"), default="forward",
                    help="backward: time moe_backward (the layer's gradient, gate-up recompute "
                         "included) for the forward's routing")
    ap.add_argument("--graph", action="store_true",
                    help="replay the forward as one captured HIP graph per step (host launch "
                         "work out of the timed region)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first run a plain copy of this many MiB (counter calibration)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="post-process two rocprofv3 --pmc counter CSVs into "
                         "profiles/traffic_<stage>_<workload>.json and exit (no GPU)")
    ap.add_argument("--scrub", choices=("read", "write"), default="read",
                    help="how the cold pass evicts the caches before each step")
    ap.add_argument("--traffic-command", default="", help="command recorded with --write-traffic")
    ap.add_argument("--configs", default="all",
                    help="after the headline workload, also time these workloads (comma-separated "
                         "names, 'all', or '' for none) and report them under `configs`")
    args = ap.parse_args(argv)

    if args.write_traffic:
        write_traffic(args.write_traffic[0], args.write_traffic[1], args.workload,
                      args.calib_copy_mib, args.traffic_command)
        return 0

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer is built and measured on a single MI355X).", file=sys.stderr)
        return 2

    import torch
    import workloads
    import mixture_experts_layer_44_amd as moe

    w = workloads.get(args.workload)
    if args.tokens:
        w = w.with_tokens(args.tokens)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] workload {w}")
    t0 = time.time()
    inp = workloads.generate(w, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs generated in {time.time() - t0:.1f} s")
    if args.calib_copy_mib:
        calibration_copy(args.calib_copy_mib, dev)
    p = moe.problem_for(w)
    ws = torch.empty(moe.workspace_bytes(p), dtype=torch.uint8, device=dev)
    y = torch.empty((w.T, w.d), dtype=torch.float32, device=dev)
    g = inp
    kw = dict(logit_bias=g["logit_bias"], sel_bias=g["sel_bias"], ws1=g["ws1"], ws3=g["ws3"],
              ws2=g["ws2"], ws=ws)

    if args.routing == "expert_choice":
        return bench_expert_choice(args, w, p, g, kw, y, torch, moe)
    if args.pass_ == "backward":
        if w.dtype != "bf16":
            log("bench.py --pass backward: the backward runs on bf16 storage only")
            return 2
        return bench_backward(args, w, p, g, kw, y, torch, moe)

    del ws, y, kw
    res = measure_forward(w, args, inp, dev, torch, moe)
    torch.cuda.empty_cache()

    configs = {}
    if args.configs and not args.tokens:
        names = (ALL_CONFIGS if args.configs == "all" else
                 [n.strip() for n in args.configs.split(",") if n.strip()])
        for name in names:
            if name == w.name:
                continue
            wc = workloads.get(name)
            log(f"[bench] --- config {wc}")
            t0 = time.time()
            inp_c = workloads.generate(wc, device=dev)
            torch.cuda.synchronize()
            log(f"[bench] inputs generated in {time.time() - t0:.1f} s")
            rc = measure_forward(wc, args, inp_c, dev, torch, moe)
            configs[wc.name] = config_entry(wc, rc)
            del inp_c, rc
            torch.cuda.empty_cache()
        configs[w.name] = config_entry(w, res)

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle baseline on {args.cpu_sample} tokens ...")
        cpu = cpu_baseline(w, inp, args.cpu_sample)
        log(f"[bench] CPU oracle: {cpu['value']:.2f} tokens/s ({cpu['seconds']:.1f} s)")
        cpu.pop("seconds")

    bf16 = w.dtype == "bf16"
    cfg = {"workload": w.name, "T": w.T, "d": w.d, "E": w.E, "k": w.k, "d_ff": w.d_ff,
           "n_shared": w.n_shared, "capacity_factor": w.capacity_factor, "seed": w.seed,
           "balance_stats": w.balance_alpha > 0}
    line = {"metric": METRIC, "value": res["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["ms_per_step"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16" if bf16 else "f32", "data": "synthetic", "config": cfg,
            "roofline": res["roofline"], "cpu_baseline": cpu, "layer": res["layer"],
            "cold": res["cold"], "launch": "hip_graph" if args.graph else "eager"}
    if configs:
        line["configs"] = configs
    print(json.dumps(line), flush=True)
    return 0


# every config of the layer, timed in one default run (the headline is the first)
ALL_CONFIGS = ("mixtral_prefill", "dsv3_fine", "skew_cap", "decode_T1", "decode_T8", "decode_T32",
               "decode_T128", "tiny_fp32")


def config_entry(w, r):
    """The per-workload record of the `configs` object: warm and cold step times, tokens/s, the
    layer's binding roofline (the larger of its MFMA and HBM times at peak) and its fraction, and
    the dominant kernel with its average launch duration."""
    lay = r["layer"]
    bf16 = w.dtype == "bf16"
    if not bf16:
        bound, frac = "launch", None         # the fp32 layer is a parity case; no roofline claim
    elif lay["flops"] / (PEAK_BF16_TFLOPS * 1e12) >= lay["bytes"] / (PEAK_HBM_GBS * 1e9):
        bound, frac = "mfma", lay["mfma_frac"]
    else:
        bound, frac = "hbm", lay["hbm_frac"]
    roof = r["roofline"]
    cold_ms = r["cold"]["ms_per_step_median"]
    return {"T": w.T, "d": w.d, "E": w.E, "k": w.k, "d_ff": w.d_ff, "n_shared": w.n_shared,
            "capacity_factor": w.capacity_factor, "dtype": w.dtype, "seed": w.seed,
            "ms_per_step": round(r["ms_per_step"], 5), "tokens_per_s": r["tokens_per_s"],
            "cold_ms_per_step_median": round(cold_ms, 5),
            "cold_ms_per_step_min": round(r["cold"]["ms_per_step_min"], 5),
            "cold_tokens_per_s": w.T / (cold_ms * 1e-3) if cold_ms > 0 else None,
            "layer_bound": bound, "layer_frac": frac,
            "layer_mfma_frac": lay["mfma_frac"], "layer_hbm_frac": lay["hbm_frac"],
            "layer_flops": lay["flops"], "layer_bytes": lay["bytes"],
            "kept_rows": lay["kept_rows"], "touched_experts": lay["touched_experts"],
            "stage_ms": lay["stage_ms"], "cold_stage_ms": r["cold"]["stage_ms_median"],
            "dominant": {"stage": r["dominant"], "avg_launch_ms": round(roof["avg_launch_ms"], 5),
                         "bound": roof["bound"], "achieved": roof["achieved"],
                         "unit": roof["unit"], "frac": roof["frac"],
                         "cold_frac": r["cold"]["dominant_frac"], "traffic": roof["traffic"],
                         "algorithmic_per_launch": roof["algorithmic_per_launch"]}}


def measure_forward(w, args, g, dev, torch, moe):
    """Warm-up, then exactly K moe_forward steps between two device synchronisations (the
    throughput), a staged pass of K steps (per-stage event times, the dominant kernel's average
    launch duration), and two cold passes with the caches scrubbed before each step: K staged
    steps (per-stage times) and K plain steps, each between two events (the cold step time)."""
    p = moe.problem_for(w)
    ws = torch.empty(moe.workspace_bytes(p), dtype=torch.uint8, device=dev)
    y = torch.empty((w.T, w.d), dtype=torch.float32, device=dev)
    kw = dict(logit_bias=g["logit_bias"], sel_bias=g["sel_bias"], ws1=g["ws1"], ws3=g["ws3"],
              ws2=g["ws2"], ws=ws)
    # routing of this batch (for the algorithmic work); identical in every step
    _, r = moe.forward(p, g["x"], g["w_gate"], g["w1"], g["w3"], g["w2"], return_routing=True, y=y,
                       **kw)
    counts = r["counts"].cpu().tolist()
    del r

    n_ev = 7
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    stream = torch.cuda.current_stream(dev)
    for evs in events:                       # materialise the HIP event handles
        for e in evs:
            e.record(stream)
    torch.cuda.synchronize()
    handles = [[e.cuda_event for e in evs] for evs in events]

    # a workload that asks for the balance statistics gets them in every timed step
    bal = w.balance_alpha if w.balance_alpha > 0 else None
    fwd = moe.PreparedForward(p, g["x"], g["w_gate"], g["w1"], g["w3"], g["w2"], y=y,
                              balance_alpha=bal, **kw)
    step = fwd
    if args.graph:
        fwd()                                         # first call outside the capture
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fwd()
        torch.cuda.synchronize()
        step = graph.replay

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] {w.name}: warm-up done ({args.warmup} steps)")

    # the timed region: exactly K plain forward calls between two device synchronisations
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = w.T * args.steps / elapsed
    assert torch.isfinite(y).all().item()

    # per-stage times (and the dominant kernel's launch duration) from a second pass of K steps
    # with HIP events recorded on the launch stream between the stages; the events add a few
    # microseconds per stage, so this pass is not the one the throughput is taken from
    for s_ in range(args.steps):
        moe.forward_staged(p, g["x"], g["w_gate"], g["w1"], g["w3"], g["w2"], handles[s_], y=y, **kw)
    torch.cuda.synchronize()

    stage_ms = {}
    for i, name in enumerate(moe.STAGES):
        vals = [events[s][i].elapsed_time(events[s][i + 1]) for s in range(args.steps)]
        stage_ms[name] = sum(vals) / len(vals)
    log(f"[bench] {w.name} stage ms: " + ", ".join(f"{k}={v:.4f}" for k, v in stage_ms.items()))
    log(f"[bench] {w.name}: {ms_per_step:.4f} ms/step, {tokens_per_s:,.0f} tokens/s "
        f"(stage-event pass: {sum(stage_ms.values()):.4f} ms/step)")

    # cold pass: before each step, outside its events, read a 1 GiB buffer (more than the 256 MB
    # Infinity Cache plus the 8 x 4 MB of L2; --scrub write fills it instead), so no step finds the
    # previous step's weights or rows in a cache. Per-step and per-stage medians (the events add a
    # few microseconds each).
    scrub = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    for s_ in range(args.steps):
        if args.scrub == "write":
            scrub.fill_(s_)
        else:
            scrub.max()
        moe.forward_staged(p, g["x"], g["w_gate"], g["w1"], g["w3"], g["w2"], handles[s_], y=y, **kw)
    torch.cuda.synchronize()
    cold_stage = {name: statistics.median(events[s][i].elapsed_time(events[s][i + 1])
                                          for s in range(args.steps))
                  for i, name in enumerate(moe.STAGES)}
    staged_cold_steps = [events[s][0].elapsed_time(events[s][len(moe.STAGES)])
                         for s in range(args.steps)]
    # the cold step itself: the plain forward (the timed pass's call) between two events, the
    # caches scrubbed before each; the stage events above cost a few microseconds each, which at
    # decode sizes is a large part of a step
    for s_ in range(args.steps):
        if args.scrub == "write":
            scrub.fill_(s_)
        else:
            scrub.max()
        events[s_][0].record(stream)
        step()
        events[s_][1].record(stream)
    torch.cuda.synchronize()
    del scrub
    cold_steps = [events[s][0].elapsed_time(events[s][1]) for s in range(args.steps)]
    log(f"[bench] {w.name} cold stage ms (median): " + ", ".join(f"{k}={v:.4f}" for k, v in cold_stage.items()))
    log(f"[bench] cold step (caches scrubbed): median {statistics.median(cold_steps):.4f} ms, "
        f"min {min(cold_steps):.4f} ms (with the stage events: median "
        f"{statistics.median(staged_cold_steps):.4f} ms)")

    # dominant kernel roofline
    dom = max(("gate_up", "down"), key=lambda s: stage_ms[s])
    kwk = kernel_work(w, counts, dom)
    t_dom = stage_ms[dom] * 1e-3
    ai = kwk["flops"] / kwk["bytes"]
    bf16 = w.dtype == "bf16"
    if ai >= RIDGE and bf16:
        roof = {"bound": "mfma", "achieved": kwk["flops"] / t_dom / 1e12, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s"}
    elif not bf16:
        roof = {"bound": "alu", "achieved": kwk["flops"] / t_dom / 1e12, "peak": PEAK_F32_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": kwk["bytes"] / t_dom / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = traffic_from_profile(dom, w.name)
    roof["kernel"] = KERNEL_NAMES[dom]
    roof["launch_stream"] = "torch current stream (HIP events recorded around the launch)"
    roof["avg_launch_ms"] = stage_ms[dom]
    roof["algorithmic_per_launch"] = {"flops": kwk["flops"], "bytes": kwk["bytes"]}

    cold_dom_s = cold_stage[dom] * 1e-3
    cold = {"scrub_bytes": 1 << 30, "ms_per_step_median": statistics.median(cold_steps),
            "ms_per_step_min": min(cold_steps),
            "staged_ms_per_step_median": statistics.median(staged_cold_steps),
            "stage_ms_median": {k: round(v, 5) for k, v in cold_stage.items()},
            "dominant_achieved": (kwk["flops"] / cold_dom_s / 1e12 if roof["unit"] == "TFLOP/s"
                                  else kwk["bytes"] / cold_dom_s / 1e9),
            "dominant_unit": roof["unit"]}
    cold["dominant_frac"] = cold["dominant_achieved"] / roof["peak"]

    lw = algorithmic_work(w, counts)
    t_layer = ms_per_step * 1e-3
    layer = {"flops": lw["flops"], "bytes": lw["bytes"], "kept_rows": lw["kept"],
             "touched_experts": lw["touched"],
             "mfma_frac": lw["flops"] / t_layer / (PEAK_BF16_TFLOPS * 1e12),
             "hbm_frac": lw["bytes"] / t_layer / (PEAK_HBM_GBS * 1e9),
             "stage_ms": {k: round(v, 5) for k, v in stage_ms.items()}}

    return {"ms_per_step": ms_per_step, "tokens_per_s": tokens_per_s, "roofline": roof,
            "cold": cold, "layer": layer, "dominant": dom}


if __name__ == "__main__":
    sys.exit(main())
