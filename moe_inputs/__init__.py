"""Seeded synthetic inputs for the dropless MoE layer.

This module only draws inputs: it holds none of the layer's arithmetic, and
both the HIP library's tests/benchmark and the CPU oracle consume the tensors
it returns.  Every draw comes from numpy's PCG64 seeded through SeedSequence,
with child streams spawned in a fixed order (x, W_r, Wg, Wu, Wd, dy, routing
noise, expert order); normals are drawn in float32 (values exact), scaled,
then rounded to bf16 with round-to-nearest-even where the workload is bf16.

Workloads (shapes from the benchmark definitions; no public dataset is
involved, these synthetic tensors stand in for training activations):
  tiny     fp32  T=256   d=128  E=8   k=2 F=256   routing from x.W_r
  dense8   bf16  T=16384 d=2048 E=8   k=4 F=1024  routing from x.W_r
  uniform128 bf16 T=16384 d=2048 E=128 k=4 F=1024 logits iid N(0,1)
  zipf128  bf16  T=32768 d=2048 E=128 k=4 F=1024  logits = ln Zipf(1.1) + Gumbel
  mx16     MXFP8 65536 pre-routed rows, d=4096, 16 experts, F=1536,
           Zipf(0.8) per-expert counts
A shared expert's weights (shared_expert_weights) come from streams of
their own, so adding one leaves every other draw unchanged.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np
import torch


@dataclass(frozen=True)
class LayerConfig:
    name: str
    dtype: str  # "fp32" or "bf16"
    T: int
    d: int
    E: int
    k: int
    F: int
    routing: str  # "router" (logits = x.W_r), "uniform" (iid N(0,1) logits), "zipf"
    seed: int
    x_std: float = 1.0
    w_std: float = 0.02
    wr_std: float = 0.02
    zipf_s: float = 1.1
    n_dead: int = 4


CONFIGS = {
    "tiny": LayerConfig("tiny", "fp32", 256, 128, 8, 2, 256, "router", 0, x_std=0.02),
    "dense8": LayerConfig("dense8", "bf16", 16384, 2048, 8, 4, 1024, "router", 1),
    "uniform128": LayerConfig("uniform128", "bf16", 16384, 2048, 128, 4, 1024, "uniform", 2),
    "zipf128": LayerConfig("zipf128", "bf16", 32768, 2048, 128, 4, 1024, "zipf", 3),
}


@dataclass(frozen=True)
class MxConfig:
    name: str
    rows: int
    d: int
    E: int
    F: int
    zipf_s: float
    seed: int


MX_CONFIG = MxConfig("mx16", 65536, 4096, 16, 1536, 0.8, 4)


def config(name: str, **overrides) -> LayerConfig:
    c = CONFIGS[name]
    return replace(c, **overrides) if overrides else c


def _streams(seed: int, n: int = 8):
    ss = np.random.SeedSequence(seed)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(n)]


def _normal(rng, shape, std):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def to_dtype(a: np.ndarray, dtype: str) -> torch.Tensor:
    """float32 numpy -> torch CPU tensor of the workload dtype (bf16 by RNE)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def zipf_probs(n: int, s: float) -> np.ndarray:
    p = 1.0 / np.arange(1, n + 1, dtype=np.float64) ** s
    return p / p.sum()


def layer_inputs(cfg: LayerConfig, with_weights: bool = True) -> dict:
    """Host tensors for one layer workload.  Returns torch CPU tensors in the
    workload dtype: x [T,d], wr [d,E], wg/wu [E,d,F], wd [E,F,d], dy [T,d],
    plus `logits` [T,E] fp32 when routing is not taken from x.W_r, and
    `order` (the seeded expert order used by skewed routing)."""
    rx, rwr, rwg, rwu, rwd, rdy, rnoise, rorder = _streams(cfg.seed)
    T, d, E, F = cfg.T, cfg.d, cfg.E, cfg.F
    out = dict(cfg=cfg)
    out["x"] = to_dtype(_normal(rx, (T, d), cfg.x_std), cfg.dtype)
    out["wr"] = to_dtype(_normal(rwr, (d, E), cfg.wr_std), cfg.dtype)
    if with_weights:
        out["wg"] = to_dtype(_normal(rwg, (E, d, F), cfg.w_std), cfg.dtype)
        out["wu"] = to_dtype(_normal(rwu, (E, d, F), cfg.w_std), cfg.dtype)
        out["wd"] = to_dtype(_normal(rwd, (E, F, d), cfg.w_std), cfg.dtype)
    out["dy"] = to_dtype(_normal(rdy, (T, d), 1.0), cfg.dtype)
    order = rorder.permutation(E)
    out["order"] = order
    if cfg.routing == "uniform":
        out["logits"] = torch.from_numpy(_normal(rnoise, (T, E), 1.0))
    elif cfg.routing == "zipf":
        live = E - cfg.n_dead
        bias = np.full(E, -1.0e4, dtype=np.float64)
        bias[order[:live]] = np.log(zipf_probs(live, cfg.zipf_s))
        u = rnoise.random(size=(T, E))
        u = np.clip(u, np.finfo(np.float64).tiny, None)
        gumbel = -np.log(-np.log(u))
        out["logits"] = torch.from_numpy((bias[None, :] + gumbel).astype(np.float32))
    elif cfg.routing != "router":
        raise ValueError(cfg.routing)
    return out


def shared_expert_weights(cfg: LayerConfig, Fs: int | None = None) -> dict:
    """Weights of a shared expert of width Fs (default cfg.F): wg_s, wu_s
    [1,d,Fs] and wd_s [1,Fs,d], N(0, w_std^2) in the workload dtype, drawn
    from their own seeded streams (the layer's streams are unchanged)."""
    Fs = cfg.F if Fs is None else Fs
    rg, ru, rd = _streams(cfg.seed + 1_000_003, 3)
    return dict(wg_s=to_dtype(_normal(rg, (1, cfg.d, Fs), cfg.w_std), cfg.dtype),
                wu_s=to_dtype(_normal(ru, (1, cfg.d, Fs), cfg.w_std), cfg.dtype),
                wd_s=to_dtype(_normal(rd, (1, Fs, cfg.d), cfg.w_std), cfg.dtype))


def largest_remainder(total: int, p: np.ndarray) -> np.ndarray:
    """Integer counts summing to `total`, proportional to p (largest remainder)."""
    raw = total * p
    base = np.floor(raw).astype(np.int64)
    short = total - int(base.sum())
    rem_order = np.argsort(-(raw - base), kind="stable")
    base[rem_order[:short]] += 1
    return base


def mx_counts(cfg: MxConfig = MX_CONFIG) -> np.ndarray:
    """Per-expert row counts of the pre-routed MXFP8 workload: Zipf(s) over
    the experts by rank, largest-remainder rounded, mapped through the seeded
    expert order."""
    streams = _streams(cfg.seed)
    order = streams[7].permutation(cfg.E)
    by_rank = largest_remainder(cfg.rows, zipf_probs(cfg.E, cfg.zipf_s))
    counts = np.zeros(cfg.E, dtype=np.int64)
    counts[order] = by_rank
    return counts.astype(np.int32)


def mx_inputs(cfg: MxConfig = MX_CONFIG, with_weights: bool = True) -> dict:
    """Pre-routed rows for the MXFP8 grouped GEMM: xp [rows,d] and dyp [rows,d]
    bf16 ~ N(0,1), expert weights bf16 ~ N(0, 0.02^2), counts/offsets int32."""
    rx, _, rwg, rwu, rwd, rdy, _, _ = _streams(cfg.seed)
    counts = mx_counts(cfg)
    offsets = np.zeros(cfg.E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    out = dict(cfg=cfg, counts=counts, offsets=offsets)
    out["xp"] = to_dtype(_normal(rx, (cfg.rows, cfg.d), 1.0), "bf16")
    if with_weights:
        out["wg"] = to_dtype(_normal(rwg, (cfg.E, cfg.d, cfg.F), 0.02), "bf16")
        out["wu"] = to_dtype(_normal(rwu, (cfg.E, cfg.d, cfg.F), 0.02), "bf16")
        out["wd"] = to_dtype(_normal(rwd, (cfg.E, cfg.F, cfg.d), 0.02), "bf16")
    out["dyp"] = to_dtype(_normal(rdy, (cfg.rows, cfg.d), 1.0), "bf16")
    return out


def rows_inputs(R: int, d: int, E: int, F: int, counts: np.ndarray, seed: int, dtype: str = "bf16",
                x_std: float = 1.0, w_std: float = 0.02) -> dict:
    """Expert-major rows with given per-expert counts (for testing the grouped
    FFN on its own): xp [R,d], dyp [R,d], weights, offsets."""
    assert int(np.sum(counts)) == R
    rx, _, rwg, rwu, rwd, rdy, _, _ = _streams(seed)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return dict(
        counts=np.asarray(counts, dtype=np.int32), offsets=offsets,
        xp=to_dtype(_normal(rx, (R, d), x_std), dtype),
        dyp=to_dtype(_normal(rdy, (R, d), 1.0), dtype),
        wg=to_dtype(_normal(rwg, (E, d, F), w_std), dtype),
        wu=to_dtype(_normal(rwu, (E, d, F), w_std), dtype),
        wd=to_dtype(_normal(rwd, (E, F, d), w_std), dtype),
    )


def f32(t: torch.Tensor) -> np.ndarray:
    """Exact float32 values of a CPU tensor (bf16 widens exactly)."""
    return t.detach().to(torch.float32).cpu().numpy()
