#!/usr/bin/env python3
"""Benchmark of the dropless MoE layer (forward + backward) on one MI355X.

One step = one pass of the whole layer over one batch of synthetic tokens:
router scores, softmax top-k + histogram/scan/permutation, rowwise permute,
grouped SwiGLU experts, gate-weighted combine, then combine backward, routing
backward, grouped dgrad/wgrad, permute backward with the router term, and the
router weight gradient.  Inputs are resident in HBM before timing starts.

Prints ONE JSON line.  `value` is tokens/s over the timed steps: W warm-up
then K replays of the whole step captured once in a HIP graph, between two
synchronisations (the replays' outputs are checked equal to the eager step's;
if capture fails the eager steps are timed instead, and `timing` says which).
`eager` is the same K steps launched kernel by kernel; `graph` adds the
median, p10 and p90 of single replays, warm and with the caches flushed by a
1 GiB write before each replay; `smi` holds rocm-smi's clocks before and
after.  `roofline`
describes the dominant kernel (largest total time): its algorithmic FLOPs per
launch over its average launch time, measured with HIP events recorded on the
library's stream around every launch in the timed region; `traffic` is its
HBM bytes per launch from the committed rocprofv3 counter summary when that
was taken on the current kernel source.  `cpu_baseline` is the CPU oracle
timed on a bounded sample of the same workload.

More legs ride on the default run: `e_scaling` times the same layer at E=8
(learned-style routing) for the expert-count scaling loss, `mxfp8` times the
MXFP8 grouped experts (quantisation included) on 65536 pre-routed rows of a
16-expert, d_model 4096, d_ff 1536 share, `mxfp8_layer` times the main
workload end to end with quantise-on-permute and MXFP8 expert GEMMs (its
tokens/s beside the bf16 layer's; for uniform128 also dense8 and zipf128,
each beside its own bf16 layer; each also with MXFP8 on the data-gradient
GEMMs only and bf16 weight gradients), `shared_expert` times the main workload
with a shared expert of the routed width added, `recompute` times it with
activation recompute (the bytes kept from forward to backward beside the
throughput), and `routing_stats` times the
routing statistics, balance loss, its logit gradient and the per-expert
weight-gradient norms on the layer's own buffers (outside the step).
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
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 MFMA (MXFP8 operands)
PEAK_FP32_TFLOPS = 157.3   # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
METRIC = "MoE-layer tokens/sec fwd+bwd at E=128 top-4; grouped-GEMM % of MFMA peak"
GEMM_KERNELS = {  # algorithmic FLOPs per launch in units of R*d*F
    "gemm_up_swiglu": 4, "gemm_down": 2, "gemm_dgrad_down_swiglu": 2, "gemm_wgrad_down": 2,
    "gemm_dgrad_up": 4, "gemm_wgrad_up": 4,
}
PROFILE_DIR = os.path.join(ROOT, "profiles")
GEMM_SOURCES = [os.path.join(ROOT, "routing_grouped_expert_softmax_amd", "csrc", f)
                for f in ("gemm_bf16.hip", "gemm_common.h")]
MX_GEMM_SOURCES = [os.path.join(ROOT, "routing_grouped_expert_softmax_amd", "csrc", f)
                   for f in ("gemm_mx.hip", "gemm_common.h")]


def row_bytes(name, T, d, k, F, E, esz=2):
    """Algorithmic HBM bytes per launch of the row movers (read + write)."""
    R = T * k
    idx = T * k * 4
    return {
        "permute": T * d * esz + R * d * esz + idx,
        "combine": R * d * esz + T * d * esz + idx + T * k * 4,
        "combine_bwd": T * d * esz + R * d * esz + R * d * esz + idx + 2 * T * k * 4,
        # bf16: the router term is folded into the gate/up dgrad, so the
        # permute backward reads only the k rows and their indices
        "permute_bwd": R * d * esz + T * d * esz + idx,
    }.get(name)


def routing_bytes(name, T, d, k, E, esz=2):
    """Algorithmic HBM bytes per launch of the routing kernels: every tensor
    the kernel needs read once and every output written once (int32 indices,
    fp32 logits and gates; the router weight gradient's minimum reads x once,
    although its expert-major walk gathers each token row k times)."""
    nblk = (T + 63) // 64          # 64-token routing blocks
    pair = T * k * 4               # one int32 or fp32 per (token, slot)
    hist = E * nblk * 4            # per-block expert counts
    return {
        "router_logits": T * d * esz + d * E * esz + T * E * 4,
        "topk_hist": T * E * 4 + 2 * pair + hist,
        "expert_scan": 2 * hist + E * 4,
        "rank": pair + hist + E * 4 + (E + 1) * 4 + 2 * pair,
        # bf16 layer: gates, dgates, row_of in; dlogits_sel and the expert-row copy out
        "route_bwd": 3 * pair + 2 * pair,
        "router_wgrad": T * d * esz + 2 * pair + (E + 1) * 4 + d * E * esz,
    }.get(name)


def _code_only(text):
    """Source text without // comments (outside string literals), trailing
    blanks and empty lines: what the kernel is built from."""
    out = []
    for line in text.splitlines():
        cut = None
        i = line.find("//")
        while i >= 0:
            if line.count('"', 0, i) % 2 == 0:
                cut = i
                break
            i = line.find("//", i + 2)
        code = (line if cut is None else line[:cut]).rstrip()
        if code:
            out.append(code)
    return "\n".join(out)


def source_hash(paths=None):
    """First 16 hex digits of the SHA-256 of the bf16 grouped-GEMM sources'
    code (comments and blank lines do not count: they cannot change the
    kernels the counters were taken on)."""
    h = hashlib.sha256()
    for path in paths or GEMM_SOURCES:
        with open(path, encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


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
    if kv.get("source_sha256_16") != source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def read_mfma_busy(workload, paths=None):
    """Per-GEMM matrix-core utilisation from the committed rocprofv3 counter
    summary profiles/mfma_gemm_<workload>.txt: {kernel: {"mfma_busy": ...,
    "clock_ghz": ..., "executed_over_algorithmic": ...}}, or None when it is
    absent or was taken on a different version of the kernel source."""
    path = os.path.join(PROFILE_DIR, f"mfma_gemm_{workload}.txt")
    if not os.path.exists(path):
        return None
    out, src = {}, None
    for line in open(path):
        if line.startswith("#") or ":" not in line:
            continue
        key, val = (s.strip() for s in line.split(":", 1))
        if key == "source_sha256_16":
            src = val
        elif key.startswith("kernel "):
            name = key.split(" ", 1)[1]
            out[name] = {k: float(v) for k, v in (kv.split("=") for kv in val.split())}
    if src != source_hash(paths) or not out:
        return None
    return out


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
    return {"value": S / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"first {S} of {cfg.T} tokens of {cfg.name}, all {cfg.E} experts, full "
                      f"weights; fp32-accumulating oracle, fwd+bwd, {dt:.1f} s"}


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None if unreadable)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def quantise_per_step(prof, steps):
    """MXFP8 quantiser launches per step and their summed time per step (the
    weight pack, H rowwise, dYp, dG, dU; kernel_ms holds the per-launch mean)."""
    if "mx_quantize" not in prof:
        return None
    n, ms = prof["mx_quantize"]
    return {"launches": round(n / steps, 2), "ms": round(ms / steps, 4)}


def time_steps(ctx, step, steps, warmup):
    """Run `warmup` untimed steps, then time exactly `steps` steps between two
    synchronisations with events on the current stream, per-kernel HIP events
    on (recorded by the library on its stream around every launch)."""
    import torch

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ctx.profile(True)
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ctx.profile(False)
    return e0.elapsed_time(e1), wall, ctx.profile_results()


def graph_timing(step, check, steps, warmup, replays=50, warm=10):
    """The step captured once in a HIP graph and replayed. First `warmup`
    replays, then exactly `steps` replays back to back between two
    synchronisations (the bench's timed steps); then each replay timed by its
    own pair of events: median, p10 and p90 per replay, "warm" (replays back
    to back) and "cold" (a 1 GiB buffer written before every replay, which
    evicts the 256 MB Infinity Cache and the L2s). `check()` compares the
    layer's outputs after all replays with the eager step's."""
    import torch

    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    out = {"steps_ms": e0.elapsed_time(e1), "steps_wall_s": time.perf_counter() - w0,
           "replays": replays, "warmup_replays": warm}
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
    for mode in ("warm", "cold"):
        for _ in range(warm):
            graph.replay()
        ev = []
        for i in range(replays):
            if mode == "cold":
                scratch.fill_(i & 0xff)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            graph.replay()
            e1.record()
            ev.append((e0, e1))
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) for a, b in ev)
        q = lambda f: ts[min(len(ts) - 1, int(round(f * (len(ts) - 1))))]  # noqa: E731
        out[mode] = {"median_ms": round(q(0.5), 4), "p10_ms": round(q(0.1), 4),
                     "p90_ms": round(q(0.9), 4)}
    out["replay_matches_eager"] = bool(check())
    del graph, scratch
    return out


def copy_peak(mib=1024, reps=10):
    """Measured HBM ceiling for the row movers: `mib` MiB copied by the
    runtime's device-to-device copy and by an elementwise fp32 kernel
    (x * 1, four floats = 16 bytes per vector access); bytes read + written
    per second of the faster, best of `reps` launches each, timed with
    events."""
    import torch

    n = mib * (1 << 20)
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    ways = {"memcpy": lambda: dst.copy_(src), "elementwise": lambda: torch.mul(src, 1.0, out=dst)}
    best = {}
    for name, f in ways.items():
        f()
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            f()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            best[name] = min(best.get(name, ms), ms)
    del src, dst
    torch.cuda.empty_cache()
    return {name: round(2 * n / (ms / 1e3) / 1e9, 1) for name, ms in best.items()}


def mfma_probe(iters=50000):
    """Sustained bf16 MFMA rate: the library's register-only probe on three
    blocks of four waves per CU (one round, no tail), timed with events;
    best of three launches."""
    import torch

    import routing_grouped_expert_softmax_amd as moe

    blocks = 3 * torch.cuda.get_device_properties(0).multi_processor_count
    sink = moe.moe_mfma_peak_probe(blocks, 1000)
    best = None
    for _ in range(3):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        moe.moe_mfma_peak_probe(blocks, iters, sink=sink)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    flops = blocks * 4 * iters * 4 * 32768
    return {"tflops": round(flops / (best / 1e3) / 1e12, 1), "ms": round(best, 3), "blocks": blocks,
            "iters": iters}


def smi_snapshot():
    """Clocks and power of the GPU from rocm-smi (a child process), or the
    reason they could not be read."""
    import subprocess

    out = {}
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--showpower", "--json"], capture_output=True,
                           text=True, timeout=30)
        data = json.loads(r.stdout)
        card = next(iter(v for k, v in sorted(data.items()) if k.startswith("card")))
        out = {k: v for k, v in card.items() if "clk" in k.lower() or "power" in k.lower()}
    except Exception as exc:  # reported, never fatal: the timing does not depend on it
        out["error"] = f"{type(exc).__name__}: {exc}"[:200]
    if not any("power" in k.lower() for k in out):
        # rocm-smi reports no package power on some systems: ask amd-smi
        try:
            r = subprocess.run(["amd-smi", "metric", "--power", "--json"], capture_output=True, text=True,
                               timeout=30)
            data = json.loads(r.stdout)
            gpu = data[0] if isinstance(data, list) else data
            if isinstance(gpu, dict) and isinstance(gpu.get("gpu_data"), list):
                gpu = gpu["gpu_data"][0]

            def flat(d, pre=""):
                for k, v in d.items():
                    if isinstance(v, dict) and set(v) >= {"value", "unit"}:
                        yield pre + k, f"{v['value']} {v['unit']}"
                    elif isinstance(v, dict):
                        yield from flat(v, pre + k + ".")
                    elif k != "gpu":
                        yield pre + k, v
            pw = {k: v for k, v in flat(gpu.get("power", gpu))}
            out.update({"amd-smi " + k: v for k, v in pw.items()} or {"power": "not reported by amd-smi"})
        except Exception as exc:
            out["power_error"] = f"{type(exc).__name__}: {exc}"[:200]
    return out


def gemm_summary(prof, unit, peak):
    """Dominant grouped-GEMM kernel (largest total time) and the six GEMMs
    together: algorithmic FLOPs over the HIP-event kernel times."""
    gemm_ms = sum(prof[n][1] / prof[n][0] for n in GEMM_KERNELS if n in prof)
    gemm_flops = 18.0 * unit
    dom = max((n for n in GEMM_KERNELS if n in prof), key=lambda n: prof[n][1])
    launches, total_ms = prof[dom]
    avg_s = total_ms / launches / 1e3
    flops = GEMM_KERNELS[dom] * unit
    achieved = flops / avg_s / 1e12
    roof = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1), "peak": peak,
            "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "flops_per_launch": flops,
            "avg_launch_ms": round(avg_s * 1e3, 4)}
    agg = {"tflops": round(gemm_flops / (gemm_ms / 1e3) / 1e12, 1),
           "frac_of_peak": round(gemm_flops / (gemm_ms / 1e3) / 1e12 / peak, 4),
           "ms": round(gemm_ms, 4), "flops": gemm_flops}
    return roof, agg


def cold_row_movers(ctx, g, buf, reps=10):
    """Each row mover of the layer launched alone on the layer's own buffers,
    with a 1 GiB buffer read before every launch, so its rows come from HBM:
    the read replaces every line of the 256 MB Infinity Cache and the L2s with
    clean ones (a write would leave dirty lines whose write-back the measured
    kernel would pay for).  Mean launch time per kernel from the library's
    HIP events."""
    import torch

    import routing_grouped_expert_softmax_amd as moe

    r = buf.route
    scratch = torch.ones(1 << 28, dtype=torch.int32, device="cuda:0")
    calls = {"permute": lambda: moe.moe_permute(g["x"], r["row_of"], buf.xp),
             "combine": lambda: moe.moe_combine(buf.ffn["yp"], r["gates"], r["row_of"], buf.y),
             "combine_bwd": lambda: moe.moe_combine_bwd(g["dy"], buf.ffn["yp"], r["gates"], r["row_of"],
                                                        buf.dyp, buf.dgates),
             "permute_bwd": lambda: moe.moe_permute_bwd(buf.bwd["dxp"], r["row_of"], dx=buf.dx)}
    torch.cuda.synchronize()
    ctx.profile(True)
    for i in range(reps):
        for f in calls.values():
            scratch.sum()
            f()
    torch.cuda.synchronize()
    ctx.profile(False)
    prof = ctx.profile_results()
    del scratch
    torch.cuda.empty_cache()
    return {n: prof[n][1] / prof[n][0] for n in calls if n in prof}


def layer_leg(cfg, steps, warmup, keep_inputs=False, with_stats=False, mxfp8=False, shared_F=0,
              recompute=False, graph=False, cold_rows=False, mx_wgrad=True):
    """Time the whole layer forward+backward on one workload (and, with
    `with_stats`, the routing statistics on its last step's buffers).
    mxfp8: quantise on the permute and run the MXFP8 expert GEMMs (with
    mx_wgrad False the weight gradients run on the bf16 operands).
    shared_F > 0: add a shared expert of that width."""
    import torch

    import moe_inputs as mi
    import routing_grouped_expert_softmax_amd as moe

    dev = "cuda:0"
    inp = mi.layer_inputs(cfg)
    g = {k: inp[k].to(dev) for k in ("x", "wr", "wg", "wu", "wd", "dy")}
    override = inp["logits"].to(dev) if "logits" in inp else None
    dtype = torch.float32 if cfg.dtype == "fp32" else torch.bfloat16
    buf = moe.alloc_layer(cfg.T, cfg.d, cfg.E, cfg.k, cfg.F, dtype, dev, mxfp8=mxfp8, shared_F=shared_F)
    ctx = moe.context(0)
    ctx.ensure_workspace(cfg.T, cfg.d, cfg.E, cfg.k, moe._dt(g["x"]))
    shared = None
    if shared_F:
        sw = mi.shared_expert_weights(cfg, shared_F)
        shared = tuple(sw[k].to(dev) for k in ("wg_s", "wu_s", "wd_s"))

    def step():
        moe.layer_forward(g["x"], g["wr"], g["wg"], g["wu"], g["wd"], cfg.k, buf, override, mxfp8=mxfp8,
                          shared=shared)
        moe.layer_backward(g["dy"], g["x"], g["wr"], g["wg"], g["wu"], g["wd"], buf, mxfp8=mxfp8,
                           shared=shared, recompute=recompute, mx_wgrad=mx_wgrad)

    gpu_ms, wall, prof = time_steps(ctx, step, steps, warmup)
    counts = buf.route["counts"].cpu()
    out = dict(cfg=cfg, gpu_ms=gpu_ms, wall=wall, prof=prof,
               tokens_per_s=cfg.T * steps / (gpu_ms / 1e3), ms_per_step=gpu_ms / steps,
               load={"max": int(counts.max()), "mean": float(counts.float().mean()),
                     "empty": int((counts == 0).sum())},
               saved_bytes=moe.saved_activation_bytes(buf, recompute=recompute))
    if graph:
        ref = {"y": buf.y.clone(), "dx": buf.dx.clone(), "dw_up": buf.bwd["dw_up"].clone(),
               "dw_router": buf.dw_router.clone()}
        for t in (buf.y, buf.dx, buf.bwd["dw_up"], buf.dw_router):
            t.zero_()
        try:
            gr = graph_timing(step, steps=steps, warmup=warmup, check=lambda: all(
                torch.equal(ref[n], t) for n, t in (("y", buf.y), ("dx", buf.dx),
                                                    ("dw_up", buf.bwd["dw_up"]),
                                                    ("dw_router", buf.dw_router))))
            gr["tokens_per_s_warm_median"] = round(cfg.T / (gr["warm"]["median_ms"] / 1e3), 1)
            gr["tokens_per_s_cold_median"] = round(cfg.T / (gr["cold"]["median_ms"] / 1e3), 1)
        except Exception as exc:  # the eager timing above still stands
            gr = {"error": f"{type(exc).__name__}: {exc}"[:300]}
        out["graph"] = gr
    if with_stats:
        out["routing_stats"] = stats_leg(ctx, cfg, override if override is not None else buf.logits,
                                         buf, counts, g)
    if cold_rows:
        out["cold_rows_ms"] = cold_row_movers(ctx, g, buf)
    if keep_inputs:
        out["inp"] = inp
    del g, buf, override
    torch.cuda.empty_cache()
    return out


AUX_ALPHA = 0.001  # balance-loss weight (a small starting value)


def stats_leg(ctx, cfg, logits, buf, counts, g, reps=20):
    """Time the routing statistics + balance loss, its logit gradient and the
    per-expert norms of the three expert weight gradients on the layer's own
    buffers; report the loss beside the real load (a balance score alone can
    hide a worsening load)."""
    import torch

    import routing_grouped_expert_softmax_amd as moe

    T, E, k = cfg.T, cfg.E, cfg.k
    r = buf.route
    dl = torch.empty(T, E, dtype=torch.float32, device=logits.device)
    norms = [torch.empty(E, dtype=torch.float32, device=logits.device) for _ in range(3)]
    st = None
    # the balance loss's share of dx and dW_r, added into copies of the
    # layer's gradients (the buffers themselves stay as the step left them)
    dx_acc, dwr_acc = buf.dx.clone(), buf.dw_router.clone()
    for it in range(reps + 2):
        if it == 2:
            torch.cuda.synchronize()
            ctx.profile(True)
        st = moe.moe_route_stats(logits, r["counts"], k, AUX_ALPHA, st)
        moe.moe_aux_loss_bwd(logits, r["counts"], k, AUX_ALPHA, 1.0, dl)
        moe.moe_router_dense_bwd(g["x"], g["wr"], dl, dx_acc, dwr_acc)
        for i, w in enumerate(("dw_gate", "dw_up", "dw_down")):
            moe.moe_expert_grad_norms(buf.bwd[w], norms[i])
    torch.cuda.synchronize()
    ctx.profile(False)
    prof = ctx.profile_results()
    ms = {n: prof[n][1] / prof[n][0] for n in ("route_stats", "aux_loss_bwd", "grad_norms",
                                                "router_dense_bwd")}
    del dx_acc, dwr_acc
    dense_flops = 4.0 * T * cfg.d * E  # dx and dW_r, one multiply-add per (t, i, e) each
    esz = buf.bwd["dw_gate"].element_size()
    nbytes = {"route_stats": T * E * 4, "aux_loss_bwd": T * E * 8, "grad_norms": E * cfg.d * cfg.F * esz}
    ms_hbm = {n: v for n, v in ms.items() if n in nbytes}
    t1 = st["top1_count"].cpu()
    gn = torch.stack(norms).cpu()
    return {
        "alpha": AUX_ALPHA, "aux_loss": float(st["aux_loss"].item()),
        "load_beside_loss": {"max": int(counts.max()), "mean": float(counts.float().mean()),
                             "max_over_mean": round(float(counts.max()) / float(counts.float().mean()), 4),
                             "top1_max": int(t1.max()),
                             "mean_top1_prob": round(float((st["top1_prob_mean"].cpu() * t1).sum() / T), 6)},
        "grad_norm_range": [round(float(gn.min()), 6), round(float(gn.max()), 6)],
        "kernel_ms": {n: round(v, 4) for n, v in ms.items()},
        "bytes_per_launch": nbytes,
        "hbm": {n: {"GB/s": round(nbytes[n] / (ms[n] / 1e3) / 1e9, 1),
                    "frac_hbm": round(nbytes[n] / (ms[n] / 1e3) / 1e9 / PEAK_HBM_GBS, 3)} for n in ms_hbm},
        # the balance loss's gradient through the router (moe_router_dense_bwd): bf16
        # with E, d multiples of 64 runs on the matrix cores (against the bf16 peak),
        # otherwise fp32 multiply-adds on the vector ALUs (against the fp32 vector peak)
        "router_dense_bwd": dense_summary(cfg, esz, dense_flops, ms["router_dense_bwd"]),
    }


def dense_summary(cfg, esz, flops, ms):
    """Roofline line of moe_router_dense_bwd on the layer's shape."""
    T, d, E = cfg.T, cfg.d, cfg.E
    mfma = esz == 2 and d % 64 == 0 and E % 64 == 0
    peak = PEAK_BF16_TFLOPS if mfma else PEAK_FP32_TFLOPS
    # dx read and written, x and dl read (W_r is L2-resident)
    nbytes = 2 * T * d * esz + T * d * esz + T * E * 4
    tf = flops / (ms / 1e3) / 1e12
    return {"alpha": AUX_ALPHA, "path": "mfma bf16" if mfma else "valu fp32", "ms": round(ms, 4),
            "gflop": round(flops / 1e9, 2), "tflops": round(tf, 2), "peak": peak,
            "frac_peak": round(tf / peak, 4), "algorithmic_bytes": nbytes,
            "GB/s": round(nbytes / (ms / 1e3) / 1e9, 1),
            "frac_hbm": round(nbytes / (ms / 1e3) / 1e9 / PEAK_HBM_GBS, 3)}


def mx_leg(steps, warmup, bf16_ref=True):
    """Time the MXFP8 grouped experts (quantisation included) forward+backward
    on the pre-routed 16-expert workload: each step quantises the weights
    once into a pack (both layouts) and runs the forward and the backward
    on it, as the layer does."""
    import torch

    import moe_inputs as mi
    import routing_grouped_expert_softmax_amd as moe

    dev = "cuda:0"
    cfg = mi.MX_CONFIG
    inp = mi.mx_inputs(cfg)
    g = {k: inp[k].to(dev) for k in ("xp", "dyp", "wg", "wu", "wd")}
    off = torch.from_numpy(inp["offsets"]).to(dev)
    R, d, F, E = cfg.rows, cfg.d, cfg.F, cfg.E
    z = lambda *s: torch.empty(*s, dtype=torch.bfloat16, device=dev)  # noqa: E731
    fo = dict(g=z(R, F), u=z(R, F), h=z(R, F), yp=z(R, d))
    bo = dict(dg=z(R, F), du=z(R, F), dxp=z(R, d), dw_gate=z(E, d, F), dw_up=z(E, d, F),
              dw_down=z(E, F, d))
    ctx = moe.context(0)
    ctx.ensure_mx_workspace(E, R, d, F)
    pack = moe.MxWeightPack(torch.empty(moe.moe_mx_weight_pack_size(E, d, F), dtype=torch.uint8, device=dev),
                            E, d, F)

    def step():
        moe.moe_mx_quantize_weights(g["wg"], g["wu"], g["wd"], pack)
        moe.moe_grouped_ffn_fwd_mxp(pack, off, xp=g["xp"], out=fo)
        moe.moe_grouped_ffn_bwd_mxp(g["xp"], pack, off, fo["g"], fo["u"], fo["h"], g["dyp"], bo)

    gpu_ms, wall, prof = time_steps(ctx, step, steps, warmup)
    roof, agg = gemm_summary(prof, R * d * F, PEAK_FP8_TFLOPS)

    # the same grouped experts in bf16 on the same rows, for the MXFP8/bf16 ratio
    def step_bf16():
        moe.moe_grouped_ffn_fwd(g["xp"], g["wg"], g["wu"], g["wd"], off, fo)
        moe.moe_grouped_ffn_bwd(g["xp"], g["wg"], g["wu"], g["wd"], off, fo["g"], fo["u"], fo["h"],
                                g["dyp"], bo)

    bf_ms = bf_prof = None
    if bf16_ref:
        bf_ms, _, bf_prof = time_steps(ctx, step_bf16, steps, warmup)
    counts = inp["counts"]
    res = {"workload": f"{cfg.name}: {R} pre-routed rows, d={d}, {E} experts, d_ff={F}, "
                       f"Zipf({cfg.zipf_s}) counts; MXFP8 E4M3 + e8m0 per 32, fp32 accumulate",
           "rows_per_s": round(R * steps / (gpu_ms / 1e3), 1), "ms_per_step": round(gpu_ms / steps, 4),
           "steps": steps, "warmup": warmup, "roofline": roof, "grouped_gemm": agg,
           "kernel_ms": {n: round(ms / c, 4) for n, (c, ms) in prof.items()},
           "expert_load": {"max": int(counts.max()), "mean": float(counts.mean()), "empty": 0}}
    busy = read_mfma_busy(cfg.name, MX_GEMM_SOURCES)
    if busy:
        agg["mfma_busy"] = {n: busy[n]["mfma_busy"] for n in GEMM_KERNELS if n in busy}
        agg["clock_ghz"] = {n: busy[n]["clock_ghz"] for n in GEMM_KERNELS if n in busy}
    if bf16_ref:
        res["bf16_same_rows"] = {"rows_per_s": round(R * steps / (bf_ms / 1e3), 1),
                                 "ms_per_step": round(bf_ms / steps, 4),
                                 "grouped_gemm": gemm_summary(bf_prof, R * d * F, PEAK_BF16_TFLOPS)[1]}
        res["mxfp8_vs_bf16"] = round(bf_ms / gpu_ms, 4)
    del g, fo, bo, off
    torch.cuda.empty_cache()
    return res


def copy_calibration(mib, reps):
    """A plain device copy of `mib` MiB, `reps` times: the known-size kernel
    that scales rocprofv3's FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch

    n = mib * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "launches": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="uniform128",
                    choices=["uniform128", "dense8", "zipf128", "tiny"])
    ap.add_argument("--cpu-sample", type=int, default=8192,
                    help="tokens of the workload the CPU oracle baseline runs on (0 = skip)")
    ap.add_argument("--no-escaling", action="store_true",
                    help="skip the E=8 leg that gives the expert-count scaling loss")
    ap.add_argument("--no-mx", action="store_true", help="skip the MXFP8 grouped-expert leg")
    ap.add_argument("--no-mx-layer", action="store_true",
                    help="skip the end-to-end MXFP8 layer leg (keeps the MXFP8 grouped-expert leg)")
    ap.add_argument("--no-mx-bf16-ref", action="store_true",
                    help="skip timing the bf16 grouped experts on the MXFP8 leg's rows")
    ap.add_argument("--no-shared", action="store_true", help="skip the shared-expert leg")
    ap.add_argument("--no-recompute", action="store_true", help="skip the activation-recompute leg")
    ap.add_argument("--no-stats", action="store_true",
                    help="skip the routing-statistics / balance-loss / gradient-norm leg")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay timing (median / p10 / p90, warm and cold)")
    ap.add_argument("--no-smi", action="store_true", help="skip reading clocks and power with rocm-smi")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured MFMA-rate and device-copy ceilings")
    ap.add_argument("--mx-steps", type=int, default=10)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the layer; runs on more than one GPU "
              "are not supported (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    import moe_inputs as mi

    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, 4)
        return

    cfg = mi.config(args.workload)
    smi_before = smi_snapshot() if not args.no_smi else None
    main_leg = layer_leg(cfg, args.steps, args.warmup, keep_inputs=args.cpu_sample > 0,
                         with_stats=not args.no_stats, graph=not args.no_graph,
                         cold_rows=cfg.dtype == "bf16" and not args.no_ceilings)
    smi_after = smi_snapshot() if not args.no_smi else None
    prof = main_leg["prof"]
    R = cfg.T * cfg.k
    unit = R * cfg.d * cfg.F
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_FP32_TFLOPS
    roof, agg = gemm_summary(prof, unit, peak)
    roof["traffic"] = read_traffic(roof["kernel"], cfg.name)
    roof["traffic_source"] = ("rocprofv3 FETCH_SIZE + WRITE_SIZE per launch, calibrated on a plain copy: "
                              "bytes between the L2s and the memory fabric, Infinity Cache hits "
                              "included, so an upper bound of the HBM bytes")
    busy = read_mfma_busy(cfg.name)
    if busy:
        agg["mfma_busy"] = {n: busy[n]["mfma_busy"] for n in GEMM_KERNELS if n in busy}
        agg["clock_ghz"] = {n: busy[n]["clock_ghz"] for n in GEMM_KERNELS if n in busy}
        if roof["kernel"] in busy:
            roof["mfma_busy"] = busy[roof["kernel"]]["mfma_busy"]
    agg["mfma_busy_source"] = (f"profiles/mfma_gemm_{cfg.name}.txt (rocprofv3 SQ_VALU_MFMA_BUSY_CYCLES over "
                               "1024 SIMDs x GRBM_GUI_ACTIVE / 8 XCDs)" if busy else
                               "absent or taken on another version of the GEMM source")
    probe = None
    if cfg.dtype == "bf16" and not args.no_ceilings:
        probe = mfma_probe()
        probe["frac_of_published_peak"] = round(probe["tflops"] / PEAK_BF16_TFLOPS, 4)
        agg["frac_of_measured_peak"] = round(agg["tflops"] / probe["tflops"], 4)
    rows = {}
    copies = copy_peak() if not args.no_ceilings else None
    copy_gbs = max(copies.values()) if copies else None
    cold = main_leg.get("cold_rows_ms") or {}
    for name in ("permute", "combine", "combine_bwd", "permute_bwd"):
        if name in prof and cfg.dtype == "bf16":
            n, ms = prof[name]
            nbytes = row_bytes(name, cfg.T, cfg.d, cfg.k, cfg.F, cfg.E)
            warm = nbytes / (ms / n / 1e3) / 1e9
            # "in_layer": inside the step, where a row mover may find its rows in the
            # 256 MB Infinity Cache (the kernel before it just touched them);
            # "GB/s" / "frac_hbm": the same launch with the caches flushed first
            rows[name] = {"in_layer_GB/s": round(warm, 1)}
            if name in cold:
                gbs = nbytes / (cold[name] / 1e3) / 1e9
                rows[name].update({"GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 3),
                                   "cold_ms": round(cold[name], 4)})
                if copy_gbs:
                    rows[name]["frac_copy"] = round(gbs / copy_gbs, 3)
    if copies:
        rows["copy_peak_GB/s"] = copies
    # routing kernels (scores, top-k + histogram, scan, ranks; the routing
    # backward and the router weight gradient) against HBM, from the same run
    routing = {}
    if cfg.dtype == "bf16":
        for name in ("router_logits", "topk_hist", "expert_scan", "rank", "route_bwd", "router_wgrad"):
            if name in prof:
                n, ms = prof[name]
                nbytes = routing_bytes(name, cfg.T, cfg.d, cfg.k, cfg.E)
                gbs = nbytes / (ms / n / 1e3) / 1e9
                routing[name] = {"ms": round(ms / n, 4), "algorithmic_bytes": nbytes, "GB/s": round(gbs, 1),
                                 "frac_hbm": round(gbs / PEAK_HBM_GBS, 3)}
        if "router_logits" in routing:
            tf = 2.0 * cfg.T * cfg.d * cfg.E / (routing["router_logits"]["ms"] / 1e3) / 1e12
            routing["router_logits"].update({"TFLOP/s": round(tf, 1), "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)})

    # The timed steps: K replays of the whole step captured in one HIP graph
    # (outputs checked against the eager step), else K eager steps.
    gr = main_leg.get("graph") or {}
    if gr.get("replay_matches_eager"):
        timed_ms, wall, timing = gr["steps_ms"], gr["steps_wall_s"], "hip_graph_replay"
    else:
        timed_ms, wall, timing = main_leg["gpu_ms"], main_leg["wall"], "eager"
    result = {
        "metric": METRIC,
        "value": round(cfg.T * args.steps / (timed_ms / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(timed_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; inputs resident in HBM)",
        "config": {"workload": f"{cfg.name}: T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} d_ff={cfg.F} "
                               f"{cfg.dtype} SwiGLU experts, routing={cfg.routing}",
                   "tokens": cfg.T, "experts": cfg.E, "top_k": cfg.k, "d_model": cfg.d, "d_ff": cfg.F,
                   "parallelism": "single GPU (one GPU's share; no collectives)"},
        "roofline": roof,
        "grouped_gemm": agg,
        "mfma_probe": probe,
        "row_movers": rows,
        "routing_kernels": routing,
        "kernel_ms": {name: round(ms / n, 4) for name, (n, ms) in prof.items()},
        "expert_load": main_leg["load"],
        "timing": timing,
        "wall_s_timed": round(wall, 3),
        "eager": {"tokens_per_s": round(main_leg["tokens_per_s"], 1),
                  "ms_per_step": round(main_leg["ms_per_step"], 4),
                  "note": "K steps launched one kernel at a time; kernel_ms and roofline come from this run"},
    }
    if "graph" in main_leg:
        result["graph"] = main_leg["graph"]
    if smi_before is not None:
        result["smi"] = {"before": smi_before, "after": smi_after}
    if "routing_stats" in main_leg:
        result["routing_stats"] = main_leg["routing_stats"]
    base = None
    if not args.no_escaling and cfg.name == "uniform128":
        base = layer_leg(mi.config("dense8"), args.steps, args.warmup, graph=not args.no_graph)

        def timed_tps(leg):  # the same timing as `value`: graph replays when they ran and matched
            g = leg.get("graph") or {}
            if g.get("replay_matches_eager"):
                return leg["cfg"].T * args.steps / (g["steps_ms"] / 1e3), "hip_graph_replay"
            return leg["tokens_per_s"], "eager"

        (t8, m8), (t128, m128) = timed_tps(base), timed_tps(main_leg)
        if m8 != m128:  # compare like with like
            t8, t128, m8 = base["tokens_per_s"], main_leg["tokens_per_s"], "eager"
        result["e_scaling"] = {
            "dense8_tokens_per_s": round(t8, 1),
            "uniform128_tokens_per_s": round(t128, 1),
            "loss": round(1.0 - t128 / t8, 4),
            "timing": m8,
            "loss_eager": round(1.0 - main_leg["tokens_per_s"] / base["tokens_per_s"], 4),
            "dense8_grouped_gemm_tflops": gemm_summary(base["prof"], 16384 * 4 * 2048 * 1024,
                                                       PEAK_BF16_TFLOPS)[1]["tflops"]}
    if not args.no_shared and cfg.dtype == "bf16":
        sl = layer_leg(cfg, args.mx_steps, 3, shared_F=cfg.F)
        extra_ms = sl["ms_per_step"] - main_leg["ms_per_step"]
        sflops = 18.0 * cfg.T * cfg.d * cfg.F
        result["shared_expert"] = {
            "workload": f"{cfg.name} + one shared SwiGLU expert of d_ff {cfg.F} over every token",
            "tokens_per_s": round(sl["tokens_per_s"], 1), "ms_per_step": round(sl["ms_per_step"], 4),
            "added_ms_per_step": round(extra_ms, 4), "shared_gflop_per_step": round(sflops / 1e9, 1),
            "shared_tflops_from_added_time": round(sflops / (extra_ms / 1e3) / 1e12, 1) if extra_ms > 0 else None}
    if not args.no_recompute:
        rl = layer_leg(cfg, args.mx_steps, 3, recompute=True)
        result["recompute"] = {
            "workload": f"{cfg.name}; backward re-permutes x and recomputes g, u, h (gate/up GEMM)",
            "tokens_per_s": round(rl["tokens_per_s"], 1), "ms_per_step": round(rl["ms_per_step"], 4),
            "throughput_vs_saved": round(rl["tokens_per_s"] / main_leg["tokens_per_s"], 4),
            "saved_activation_bytes": main_leg["saved_bytes"],
            "recompute_activation_bytes": rl["saved_bytes"],
            "activation_fraction": round(rl["saved_bytes"] / main_leg["saved_bytes"], 4)}
    if not args.no_mx:
        result["mxfp8"] = mx_leg(args.mx_steps, 3, bf16_ref=not args.no_mx_bf16_ref)
        if cfg.dtype == "bf16" and not args.no_mx_layer:
            ml = layer_leg(cfg, args.mx_steps, 3, mxfp8=True)
            mroof, magg = gemm_summary(ml["prof"], unit, PEAK_FP8_TFLOPS)
            result["mxfp8_layer"] = {
                "workload": f"{cfg.name} end to end with MXFP8 experts (quantise-on-permute)",
                "tokens_per_s": round(ml["tokens_per_s"], 1), "ms_per_step": round(ml["ms_per_step"], 4),
                "vs_bf16_layer": round(ml["tokens_per_s"] / main_leg["tokens_per_s"], 4),
                "grouped_gemm": magg, "roofline": mroof,
                "kernel_ms": {n: round(ms / c, 4) for n, (c, ms) in ml["prof"].items()},
                "quantise_per_step": quantise_per_step(ml["prof"], args.mx_steps)}
            # MXFP8 on the data-gradient GEMMs only, weight gradients in bf16
            mw = layer_leg(cfg, args.mx_steps, 3, mxfp8=True, mx_wgrad=False)
            result["mxfp8_layer"]["bf16_weight_gradients"] = {
                "tokens_per_s": round(mw["tokens_per_s"], 1), "ms_per_step": round(mw["ms_per_step"], 4),
                "vs_bf16_layer": round(mw["tokens_per_s"] / main_leg["tokens_per_s"], 4),
                "kernel_ms": {n: round(ms / c, 4) for n, (c, ms) in mw["prof"].items()},
                "quantise_per_step": quantise_per_step(mw["prof"], args.mx_steps)}
            if cfg.name == "uniform128":
                # the other two routed workloads end to end in MXFP8 beside bf16
                others = {}
                for name in ("dense8", "zipf128"):
                    oc = mi.config(name)
                    ob = base if (name == "dense8" and base is not None) else layer_leg(oc, args.mx_steps, 3)
                    om = layer_leg(oc, args.mx_steps, 3, mxfp8=True)
                    ow = layer_leg(oc, args.mx_steps, 3, mxfp8=True, mx_wgrad=False)
                    others[name] = {"bf16_tokens_per_s": round(ob["tokens_per_s"], 1),
                                    "mxfp8_tokens_per_s": round(om["tokens_per_s"], 1),
                                    "mxfp8_vs_bf16": round(om["tokens_per_s"] / ob["tokens_per_s"], 4),
                                    "mxfp8_bf16_wgrad_tokens_per_s": round(ow["tokens_per_s"], 1),
                                    "mxfp8_bf16_wgrad_vs_bf16": round(ow["tokens_per_s"] / ob["tokens_per_s"], 4),
                                    "mxfp8_expert_load": om["load"]}
                result["mxfp8_layer"]["other_workloads"] = others
    if args.cpu_sample > 0:
        result["cpu_baseline"] = cpu_baseline(cfg, main_leg["inp"], args.cpu_sample)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
