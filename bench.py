#!/usr/bin/env python3
"""Benchmark of the dropless MoE layer (forward + backward) on one MI355X.

One step = one pass of the whole layer over one batch of synthetic tokens:
router scores, softmax top-k + histogram/scan/permutation, rowwise permute,
grouped SwiGLU experts, gate-weighted combine, then combine backward, routing
backward, grouped dgrad/wgrad, permute backward with the router term, and the
router weight gradient.  Inputs are resident in HBM before timing starts.

Prints ONE JSON line.  `value` is tokens/s over the timed steps.  `roofline`
describes the dominant kernel (largest total time): its algorithmic FLOPs per
launch over its average launch time, measured with HIP events recorded on the
library's stream around every launch in the timed region.  `cpu_baseline` is
the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
METRIC = "MoE-layer tokens/sec fwd+bwd at E=128 top-4; grouped-GEMM % of MFMA peak"
GEMM_KERNELS = {  # algorithmic FLOPs per launch in units of R*d*F
    "gemm_up_swiglu": 4, "gemm_down": 2, "gemm_dgrad_down_swiglu": 2, "gemm_wgrad_down": 2,
    "gemm_dgrad_up": 4, "gemm_wgrad_up": 4,
}
PROFILE_DIR = os.path.join(ROOT, "profiles")
GEMM_SOURCE = os.path.join(ROOT, "routing_grouped_expert_softmax_amd", "csrc", "gemm_bf16.hip")


def row_bytes(name, T, d, k, F, E, esz=2):
    """Algorithmic HBM bytes per launch of the row movers (read + write)."""
    R = T * k
    idx = T * k * 4
    return {
        "permute": T * d * esz + R * d * esz + idx,
        "combine": R * d * esz + T * d * esz + idx + T * k * 4,
        "combine_bwd": T * d * esz + R * d * esz + R * d * esz + idx + 2 * T * k * 4,
        "permute_bwd": R * d * esz + T * d * esz + idx * 2 + T * k * 4,
    }.get(name)


def source_hash(path):
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def read_traffic(kernel, workload):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, or None
    when absent or taken on a different version of the kernel source."""
    path = os.path.join(PROFILE_DIR, f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            kv[key.strip()] = val.strip()
    if kv.get("source_sha256_16") != source_hash(GEMM_SOURCE):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(cfg, inp, sample_tokens):
    """Time the CPU oracle (fp32 accumulation, all host cores) on the first
    `sample_tokens` tokens of the same workload: routing, token-by-token
    forward, per-row dgrad and per-expert wgrad."""
    import numpy as np

    import moe_inputs as mi
    import oracle

    S = min(sample_tokens, cfg.T)
    x = mi.f32(inp["x"][:S])
    wr = mi.f32(inp["wr"])
    wg, wu, wd = mi.f32(inp["wg"]), mi.f32(inp["wu"]), mi.f32(inp["wd"])
    dy = mi.f32(inp["dy"][:S])
    oracle.lib()
    t0 = time.perf_counter()
    logits = oracle.router_logits(x, wr, "f32")
    if "logits" in inp:
        logits = inp["logits"][:S].numpy()
    r = oracle.route(logits, cfg.k, "f32")
    oracle.layer_fwd(x, r["topk_idx"], r["gates"], wg, wu, wd, acc="f32")
    xp = oracle.permute(x, r["row_of"]).astype(np.float32)
    dyp, _ = oracle.combine_bwd(dy, np.zeros_like(xp), r["gates"], r["row_of"])
    dyp = dyp.astype(np.float32)
    oracle.expert_dgrad(xp, dyp, r["offsets"], wg, wu, wd, acc="f32")
    oracle.expert_wgrad(xp, dyp, r["offsets"], wg, wu, wd, acc="f32")
    dt = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0))
    return {"value": S / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {S} of {cfg.T} tokens of {cfg.name}, all {cfg.E} experts, full "
                      f"weights; fp32-accumulating oracle, fwd+bwd, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="uniform128",
                    choices=["uniform128", "dense8", "zipf128", "tiny"])
    ap.add_argument("--cpu-sample", type=int, default=1024,
                    help="tokens of the workload the CPU oracle baseline runs on (0 = skip)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the layer; runs on more than one GPU "
              "are not part of this build (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    import moe_inputs as mi
    import routing_grouped_expert_softmax_amd as moe

    cfg = mi.config(args.workload)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    inp = mi.layer_inputs(cfg)
    g = {k: inp[k].to(dev) for k in ("x", "wr", "wg", "wu", "wd", "dy")}
    override = inp["logits"].to(dev) if "logits" in inp else None
    dtype = torch.float32 if cfg.dtype == "fp32" else torch.bfloat16
    buf = moe.alloc_layer(cfg.T, cfg.d, cfg.E, cfg.k, cfg.F, dtype, dev)
    ctx = moe.context(0)
    ctx.ensure_workspace(cfg.T, cfg.d, cfg.E, cfg.k, moe._dt(g["x"]))

    def step():
        moe.layer_forward(g["x"], g["wr"], g["wg"], g["wu"], g["wd"], cfg.k, buf, override)
        moe.layer_backward(g["dy"], g["x"], g["wr"], g["wg"], g["wu"], g["wd"], buf)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ctx.profile(True)
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ctx.profile(False)
    gpu_ms = e0.elapsed_time(e1)
    prof = ctx.profile_results()

    ms_per_step = gpu_ms / args.steps
    tokens_per_s = cfg.T * args.steps / (gpu_ms / 1e3)
    R = cfg.T * cfg.k
    unit = R * cfg.d * cfg.F
    counts = buf.route["counts"].cpu()

    breakdown = {name: round(ms / n, 4) for name, (n, ms) in prof.items()}
    gemm_ms = sum(prof[n][1] / prof[n][0] for n in GEMM_KERNELS if n in prof)
    gemm_flops = 18.0 * unit
    dom = max((n for n in GEMM_KERNELS if n in prof), key=lambda n: prof[n][1])
    dom_launches, dom_total_ms = prof[dom]
    dom_avg_s = dom_total_ms / dom_launches / 1e3
    dom_flops = GEMM_KERNELS[dom] * unit
    achieved = dom_flops / dom_avg_s / 1e12
    rows = {}
    for name in ("permute", "combine", "combine_bwd", "permute_bwd"):
        if name in prof and cfg.dtype == "bf16":
            n, ms = prof[name]
            gbs = row_bytes(name, cfg.T, cfg.d, cfg.k, cfg.F, cfg.E) / (ms / n / 1e3) / 1e9
            rows[name] = {"GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 3)}

    result = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; inputs resident in HBM)",
        "config": {"workload": f"{cfg.name}: T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} d_ff={cfg.F} "
                               f"{cfg.dtype} SwiGLU experts, routing={cfg.routing}",
                   "tokens": cfg.T, "experts": cfg.E, "top_k": cfg.k, "d_model": cfg.d, "d_ff": cfg.F,
                   "parallelism": "single GPU (one GPU's share; no collectives)"},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": read_traffic(dom, cfg.name),
                     "flops_per_launch": dom_flops,
                     "avg_launch_ms": round(dom_avg_s * 1e3, 4)},
        "grouped_gemm": {"tflops": round(gemm_flops / (gemm_ms / 1e3) / 1e12, 1),
                         "frac_of_peak": round(gemm_flops / (gemm_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                         "ms": round(gemm_ms, 4), "flops": gemm_flops},
        "row_movers": rows,
        "kernel_ms": breakdown,
        "expert_load": {"max": int(counts.max()), "mean": float(counts.float().mean()),
                        "empty": int((counts == 0).sum())},
        "wall_s_timed": round(wall, 3),
    }
    if args.cpu_sample > 0:
        result["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_sample)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
