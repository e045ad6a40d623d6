#!/usr/bin/env python3
"""Benchmark of the sparse MoE layer forward on one MI355X.

Prints one JSON line: tokens/s of the whole layer (moe_forward), the
grouped-FFN phase's TFLOP/s against the bf16 dense matrix-core peak (measured
live with HIP events on the stream the kernels run on), per-phase times and
HBM rates, and the CPU oracle's throughput on the machine's host cores.

A step is one forward of the whole layer (route, permute, grouped FFN,
combine) over one batch of T tokens already resident in HBM.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd tokens/sec and grouped-FFN TFLOP/s as % of bf16 MFMA peak, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def algorithmic_bytes(cfg, gather, used_experts=None):
    """Bytes each phase must move at minimum (inputs read once, outputs written once).

    With `gather` the permute phase only builds the index arrays and the FFN
    phase reads the token rows from x itself (no permuted copy). The FFN reads
    the weights of the experts that received tokens (`used_experts`, all E when
    not given)."""
    es = 2 if cfg.dtype == "bf16" else 4
    T, d, E, k, de = cfg.T, cfg.d_model, cfg.E, cfg.k, cfg.d_expert
    Eu = E if used_experts is None else used_experts
    R = T * k
    a_in = T * d * es if gather else R * d * es
    return {
        "route": T * d * es + d * E * es + R * 8,
        "permute": R * 4 + R * 8 + (0 if gather else T * d * es + R * d * es),
        "ffn": a_in + 2 * Eu * d * de * es + 2 * R * de * es + R * d * es,
        "combine": R * d * es + R * 8 + T * d * es,
    }


def gemm_source_hash():
    """sha256 (16 hex digits) of the grouped-GEMM sources with comments and
    blank space removed, so that comment edits keep a counter record valid."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in ("grouped_gemm.hip", "tiles.h", "common.h"):
        text = open(os.path.join(ROOT, "sparse_mixture_experts_route_amd", "csrc", f)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("\n".join(ln.strip() for ln in text.splitlines() if ln.strip()).encode())
    return h.hexdigest()[:16]


def measured_traffic(cfg_name):
    """HBM bytes of the grouped-FFN phase from the committed rocprofv3 counter record.

    The record stores a hash of the GEMM kernel source it was taken with; once
    the kernel changes the record no longer applies and None is returned.
    """
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(cfg_name)
    if not rec:
        return None
    if gemm_source_hash() != rec.get("gemm_source_sha256_16"):
        return None
    return rec.get("ffn_phase_hbm_bytes")


def ensure_built():
    lib = os.path.join(ROOT, "sparse_mixture_experts_route_amd", "libmoe.so")
    if not os.path.exists(lib):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_moe_build", os.path.join(ROOT, "sparse_mixture_experts_route_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()


def cpu_baseline(cfg, inp, sample_tokens, min_seconds=10.0):
    """The CPU oracle, as it stands, on the first `sample_tokens` tokens of the
    same inputs, repeated in whole passes until `min_seconds` have elapsed."""
    import numpy as np
    import oracle
    from harness import host_array
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    S = min(sample_tokens, cfg.T)
    x = host_array(inp["x"][:S])
    wr = host_array(inp["w_router"])
    b = host_array(inp["router_bias"])
    W1, W2 = host_array(inp["W1"]), host_array(inp["W2"])
    passes = 0
    t0 = time.perf_counter()
    while True:
        out = oracle.forward(x, wr, b, W1, W2, cfg.k, cfg.dtype)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    assert np.isfinite(out["y"]).all()
    return {"value": S * passes / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{passes} pass(es) over the first {S} of {cfg.T} tokens of the {cfg.name} workload, "
                      f"full expert weights; {dt:.2f} s wall (NumPy float64, BLAS threads={threads}, "
                      f"host cpus={os.cpu_count()})"}


def train_step(args, cfg, moe, inp, dev):
    """A training step (forward keeping its activations, then the backward) on
    one batch resident in HBM; HIP events around each half on the stream the
    kernels run on. FLOPs: the six expert GEMMs (2 forward, 4 backward) of
    2 T k d d_e each, plus the router's x W_r, dlogit W_r^T and x^T dlogit."""
    import torch
    from harness import make_dense
    x, wr, b, W1, W2 = inp["x"], inp["w_router"], inp["router_bias"], inp["W1"], inp["W2"]
    T, d, E, k, de = cfg.T, cfg.d_model, cfg.E, cfg.k, cfg.d_expert
    p = moe.make_problem(T, d, E, k, de, x.dtype)
    ws = torch.empty(moe.moe_workspace_size(p, moe.MOE_STAGE_TRAIN), dtype=torch.uint8, device=dev)
    bf = torch.bfloat16
    y = torch.empty((T, d), dtype=bf, device=dev)
    dy = make_dense((T, d), 1.0, seed=args.seed, tag=9, device=dev)
    dx = torch.empty((T, d), dtype=bf, device=dev)
    dwr = torch.empty((d, E), dtype=bf, device=dev)
    db = torch.empty(E, dtype=torch.float32, device=dev)
    dW1, dW2 = torch.empty_like(W1), torch.empty_like(W2)
    lf = torch.empty(E, dtype=torch.float32, device=dev)
    mp = torch.empty(E, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        moe.moe_forward_train(p, x, wr, b, W1, W2, y, ws)
        if ev:
            ev[1].record(stream)
        moe.moe_backward(p, x, wr, W1, W2, dy, dx, dwr, db, dW1, dW2, lf, mp, ws)
        if ev:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    fwd = sorted(e[0].elapsed_time(e[1]) for e in evs)[args.steps // 2]
    bwd = sorted(e[1].elapsed_time(e[2]) for e in evs)[args.steps // 2]
    tot = sum(e[0].elapsed_time(e[2]) for e in evs) / args.steps
    R = T * k
    gemm_flops = 12 * R * d * de
    router_flops = 6 * T * d * E
    tflops = (gemm_flops + router_flops) / (tot * 1e-3) / 1e12
    bwd_tflops = (8 * R * d * de + 4 * T * d * E) / (bwd * 1e-3) / 1e12
    return {
        "metric": "MoE layer training step (forward keeping activations + backward) tokens/sec, 1 GPU",
        "value": round(T / (tot * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(tot, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded normal inputs, dy and weights)",
        "config": {**cfg.describe(), "parallelism": "none (1 GPU, all experts local)", "mode": "train"},
        "forward_train_ms_median": round(fwd, 4), "backward_ms_median": round(bwd, 4),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "whole training step: 6 expert GEMMs (12 T k d d_e flops) + router GEMMs"},
        "backward_tflops": round(bwd_tflops, 2),
    }


PHASE_NAMES = ("route", "permute", "ffn", "combine")


def settle(step, seconds):
    """Untimed steps for at least `seconds` of wall time; returns the time spent."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(8):
            step()
        n += 8
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        if dt >= seconds:
            return dt


def headline(step, warmup, steps, stream):
    """`warmup` untimed steps, then exactly `steps` steps bracketed by HIP
    events on the stream the kernels run on (and synchronisations)."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    wall0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    return {"ms": ev[0].elapsed_time(ev[-1]) / steps, "median": per[len(per) // 2], "min": per[0], "wall": wall}


def phase_times(moe, cfg, layer, x, wr, b, W1, W2, warmup, steps, stream, dev):
    """Per-phase times of the stage entry points moe_forward runs (route with
    a workspace, permute of the indices, grouped FFN reading x through perm
    for bf16 layers under 2 GiB of x; else the copy path), with HIP events
    between the phases; mean over `steps` steps after `warmup` untimed ones."""
    import torch
    p = layer.problem
    bufs = layer.stages(x, wr, W1, W2, b, logits=False)  # allocates the stage outputs once
    ws_p = torch.empty(moe.moe_workspace_size(p, moe.MOE_STAGE_PERMUTE), dtype=torch.uint8, device=dev)
    ws_f = torch.empty(moe.moe_workspace_size(p, moe.MOE_STAGE_GROUPED_FFN), dtype=torch.uint8, device=dev)
    ws_r = torch.empty(moe.moe_workspace_size(p, moe.MOE_STAGE_ROUTE), dtype=torch.uint8, device=dev)
    gather = cfg.dtype == "bf16" and cfg.T * cfg.d_model * 2 < 2 ** 31 - 1

    def stage_step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        moe.moe_route_ws(p, x, wr, b, None, bufs["idx"], bufs["gate"], ws_r)
        if ev is not None:
            ev[1].record(stream)
        if gather:
            moe.moe_permute_index(p, bufs["idx"], bufs["counts"], bufs["offsets"], bufs["perm"], bufs["inv"], ws_p)
        else:
            moe.moe_permute(p, bufs["idx"], x, bufs["counts"], bufs["offsets"], bufs["perm"], bufs["inv"],
                            bufs["x_perm"], ws_p)
        if ev is not None:
            ev[2].record(stream)
        if gather:
            moe.moe_grouped_ffn_gather(p, x, bufs["perm"], bufs["offsets"], W1, W2, bufs["y_perm"], ws_f)
        else:
            moe.moe_grouped_ffn(p, bufs["x_perm"], bufs["offsets"], W1, W2, bufs["y_perm"], ws_f)
        if ev is not None:
            ev[3].record(stream)
        moe.moe_combine(p, bufs["y_perm"], bufs["inv"], bufs["gate"], bufs["y"])
        if ev is not None:
            ev[4].record(stream)

    for _ in range(warmup):
        stage_step()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    for s in range(steps):
        stage_step(events[s])
    torch.cuda.synchronize()
    ms = {n: sum(ev[i].elapsed_time(ev[i + 1]) for ev in events) / steps for i, n in enumerate(PHASE_NAMES)}
    counts = bufs["counts"].cpu()
    return {"ms": ms, "gather": gather, "y": bufs["y"], "used_experts": int((counts > 0).sum().item()),
            "counts": [int(c) for c in counts.tolist()]}


def cost_model_check(moe, cfg, counts, ms_step, phase_ms):
    """The per-phase cost model's prediction for this workload from the routed
    counts of the timed inputs, against the measured step and phases."""
    from sparse_mixture_experts_route_amd import cost_model
    if cfg.dtype != "bf16":
        return None
    pr = cost_model.calibrated().predict(cfg.T, cfg.d_model, cfg.E, cfg.k, cfg.d_expert, counts)
    return {"predicted_ms_per_step": round(pr["step"] / 1e3, 4),
            "err_vs_step": round(pr["step"] / 1e3 / ms_step - 1.0, 4),
            "predicted_phases_ms": {n: round(pr[n] / 1e3, 4) for n in PHASE_NAMES},
            "err_vs_phases": {n: round(pr[n] / 1e3 / phase_ms[n] - 1.0, 4) for n in PHASE_NAMES}}


def ffn_kernels(moe, cfg):
    """The grouped-FFN phase's launches as the library plans them."""
    plan = moe.moe_plan(moe.make_problem(cfg.T, cfg.d_model, cfg.E, cfg.k, cfg.d_expert, cfg.dtype))
    if cfg.dtype != "bf16":
        return "gemm_f32_kernel x2"
    names = {5: "256x256w8", 7: "32x256"}
    fix = sum(1 for g in plan["gemm"]
              if not g["split_in_launch"] and g["k_steps"] >= g["min_steps"] and g["max_split"] > 0)
    tiles = "/".join(names.get(g["tile"], str(g["tile"])) for g in plan["gemm"])
    return f"gemm_bf16_kernel x2 (tiles {tiles}) + gemm_fixup_kernel x{fix}"


def extra_config(moe, cfg, args, stream, dev):
    """Whole-layer tokens/s and the grouped-FFN phase's TFLOP/s of another
    workload, measured like the headline one (settle, warm-up, timed steps,
    then the per-phase region)."""
    import torch
    from harness import make_inputs
    inp = make_inputs(cfg, seed=args.seed, device=dev)
    x, wr, b, W1, W2 = inp["x"], inp["w_router"], inp["router_bias"], inp["W1"], inp["W2"]
    layer = moe.MoEForward(cfg.T, cfg.d_model, cfg.E, cfg.k, cfg.d_expert, x.dtype, device=dev)
    steps = args.steps if cfg.ffn_flops() < 2e12 else max(5, args.steps // 2)
    settle(lambda: layer(x, wr, W1, W2, b), args.settle_seconds / 2)
    head = headline(lambda: layer(x, wr, W1, W2, b), args.warmup, steps, stream)
    ph = phase_times(moe, cfg, layer, x, wr, b, W1, W2, args.warmup, steps, stream, dev)
    ffn_tflops = cfg.ffn_flops() / (ph["ms"]["ffn"] * 1e-3) / 1e12
    out = {"config": cfg.describe(), "steps": steps, "ms_per_step": round(head["ms"], 4),
           "tokens_per_s": round(cfg.T / (head["ms"] * 1e-3), 1),
           "phases_ms": {n: round(v, 4) for n, v in ph["ms"].items()},
           "ffn_tflops": round(ffn_tflops, 2),
           "ffn_frac_of_bf16_peak": round(ffn_tflops / PEAK_BF16_TFLOPS, 4) if cfg.dtype == "bf16" else None,
           "phase_sum_over_step": round(sum(ph["ms"].values()) / head["ms"], 4),
           "cost_model": cost_model_check(moe, cfg, ph["counts"], head["ms"], ph["ms"])}
    del inp, x, wr, b, W1, W2, layer, ph
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default="mixtral_coarse",
                    help="workload: tiny_fp32, mixtral_coarse, fine_grained, skewed, large_sparse")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--tokens", type=int, default=0,
                    help="batch size T instead of the workload's (e.g. 1..160 for decode-sized batches)")
    ap.add_argument("--k", type=int, default=0, help="experts per token instead of the workload's")
    ap.add_argument("--train", action="store_true",
                    help="time a training step instead: moe_forward_train + moe_backward (bf16)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=4096)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the CPU oracle pass until this much wall time has elapsed")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-seconds", type=float, default=1.5,
                    help="untimed whole-layer steps for this long before the warm-up (clocks reach steady state)")
    ap.add_argument("--extra-configs", default="fine_grained,skewed,large_sparse",
                    help="other workloads whose tokens/s and FFN TFLOP/s are added to the line ('' for none)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run one plain device-to-device copy of this many MiB (a known-size kernel "
                         "for scaling hardware byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py: this build runs the MoE layer on one GPU only; use --gpus 1 "
              "(the multi-GPU expert-parallel layout is a design note, not an implementation)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    ensure_built()
    import sparse_mixture_experts_route_amd as moe
    from harness import CONFIGS, make_inputs, scaled_config

    cfg = CONFIGS[args.config]
    if args.tokens or args.k:
        cfg = scaled_config(args.config, T=args.tokens or None, k=args.k or None, suffix=f"T{args.tokens or cfg.T}")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    inp = make_inputs(cfg, seed=args.seed, device=dev)
    x, wr, b, W1, W2 = inp["x"], inp["w_router"], inp["router_bias"], inp["W1"], inp["W2"]
    layer = moe.MoEForward(cfg.T, cfg.d_model, cfg.E, cfg.k, cfg.d_expert, x.dtype, device=dev)
    stream = torch.cuda.current_stream()

    if args.train:
        print(json.dumps(train_step(args, cfg, moe, inp, dev)), flush=True)
        return

    # ---- settle: the GPU's clocks take a second or so of matrix-core load to
    # reach their steady state; this untimed load comes before the warm-up
    # steps, so the warm-up and both timed regions below run at steady clocks
    settle_s = settle(lambda: layer(x, wr, W1, W2, b), args.settle_seconds)
    head = headline(lambda: layer(x, wr, W1, W2, b), args.warmup, args.steps, stream)
    # ---- per-phase region, after the headline: the same work through the
    # stage entry points moe_forward itself calls, with HIP events between
    # the phases on the stream the kernels run on
    ph = phase_times(moe, cfg, layer, x, wr, b, W1, W2, args.warmup, args.steps, stream, dev)
    assert torch.equal(ph["y"], layer.y), "stage path and moe_forward disagree"
    phase_ms = ph["ms"]
    gather = ph["gather"]

    flops = cfg.ffn_flops()
    used = ph["used_experts"]
    bytes_ = algorithmic_bytes(cfg, gather, used)
    ms_step = head["ms"]
    t_ffn = phase_ms["ffn"] * 1e-3
    ffn_tflops = flops / t_ffn / 1e12
    # the FFN phase is bound by the matrix cores when its flops per algorithmic
    # byte exceed the chip's balance (2.5 PFLOP/s / 8 TB/s), by HBM otherwise
    # (decode-sized batches: streaming the used experts' weights)
    mfma_bound = flops / bytes_["ffn"] > PEAK_BF16_TFLOPS / PEAK_HBM_GBS * 1e3
    if cfg.dtype == "bf16" and not mfma_bound:
        gbs = bytes_["ffn"] / t_ffn / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                    "kernel": f"grouped FFN phase: {ffn_kernels(moe, cfg)}; bytes = weights of the {used} "
                              f"experts with tokens + activations"}
    elif cfg.dtype == "bf16":
        roofline = {"bound": "mfma", "achieved": round(ffn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(ffn_tflops / PEAK_BF16_TFLOPS, 4),
                    "traffic": measured_traffic(cfg.name),
                    "kernel": f"grouped FFN phase: {ffn_kernels(moe, cfg)} (GEMM1+GELU reading x through "
                              f"perm, GEMM2)"}
    else:
        gbs = bytes_["ffn"] / t_ffn / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(gbs / PEAK_HBM_GBS, 5), "traffic": measured_traffic(cfg.name),
                    "kernel": "grouped FFN phase: gemm_f32_kernel x2"}

    phases = {n: {"ms": round(phase_ms[n], 4),
                  "GB/s": round(bytes_[n] / (phase_ms[n] * 1e-3) / 1e9, 1),
                  "hbm_frac": round(bytes_[n] / (phase_ms[n] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
              for n in PHASE_NAMES}
    phases["ffn"]["TFLOP/s"] = round(ffn_tflops, 2)
    phase_sum = sum(phase_ms.values())
    # the phases run the same kernels as a moe_forward step, with events between
    # them: their sum should not exceed the step by more than the events' cost.
    # A small float32 layer runs moe_forward as one launch instead (the same
    # bits as the stages): its phases are those of the staged launches
    one_launch = bool(moe.moe_plan(layer.problem)["forward_one_launch"])
    consistent = None if one_launch else phase_sum <= 1.05 * ms_step
    if consistent is False:
        print(f"bench.py: phase sum {phase_sum:.4f} ms exceeds 1.05 x the step ({ms_step:.4f} ms)",
              file=sys.stderr)

    result = {
        "metric": METRIC,
        "value": round(cfg.T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_median": round(head["median"], 4),
        "ms_per_step_min": round(head["min"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded normal inputs and random-init expert weights of the workload's shapes)",
        "config": {**cfg.describe(), "parallelism": "none (1 GPU, all experts local)"},
        "ffn_tflops": round(ffn_tflops, 2),
        "ffn_frac_of_bf16_peak": round(ffn_tflops / PEAK_BF16_TFLOPS, 4) if cfg.dtype == "bf16" else None,
        "phases": phases,
        "phase_sum_over_step": round(phase_sum / ms_step, 4),
        "phases_consistent": consistent,
        "forward_one_launch": one_launch,
        "roofline": roofline,
        "cost_model": cost_model_check(moe, cfg, ph["counts"], ms_step, phase_ms),
        "settle_s": round(settle_s, 2),
        "wall_s_timed_region": round(head["wall"], 4),
        "gpu": torch.cuda.get_device_name(dev),
    }
    del layer, ph
    if args.extra_configs and not (args.tokens or args.k):
        extra = {}
        for name in [c for c in args.extra_configs.split(",") if c and c != cfg.name]:
            extra[name] = extra_config(moe, CONFIGS[name], args, stream, dev)
        result["extra_configs"] = extra
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_sample_tokens, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
