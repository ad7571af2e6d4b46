"""Activation recompute (the pages trade activation memory for throughput by
recomputing in the backward; [P1] 四): the backward that re-permutes x and
recomputes g, u, h with the gate/up GEMM alone must give bit-identical
gradients to the backward that reads the forward's saved tensors — the
saved ones are overwritten with NaN first, so nothing stale can leak in."""
import numpy as np
import pytest
import torch

import moe_inputs as mi

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def moe():
    import routing_grouped_expert_softmax_amd as m
    m.context(0)
    return m


def _grads(buf):
    out = {"dx": buf.dx, "dw_router": buf.dw_router, "dgates": buf.dgates, "dlogits": buf.dlogits_sel}
    out.update({k: buf.bwd[k] for k in ("dw_gate", "dw_up", "dw_down", "dxp")})
    if buf.shared is not None:
        out.update({"s_" + k: buf.shared["bwd"][k] for k in ("dw_gate", "dw_up", "dw_down", "dxp")})
    return {k: v.clone() for k, v in out.items()}


@pytest.mark.parametrize("name,over,Fs,mx", [
    ("tiny", {}, 0, False),
    ("tiny", dict(dtype="bf16", T=700, E=16, k=4, x_std=1.0, routing="uniform"), 0, False),
    ("tiny", dict(dtype="bf16", T=1000, d=256, E=8, k=2, F=384, x_std=1.0, routing="zipf", n_dead=2), 256, False),
    ("tiny", dict(dtype="bf16", T=512, d=256, E=8, k=2, F=256, x_std=1.0), 256, True)])
def test_recompute_backward_is_bit_identical(moe, name, over, Fs, mx):
    cfg = mi.config(name, **over)
    inp = mi.layer_inputs(cfg)
    g = {k: inp[k].to(DEV) for k in ("x", "wr", "wg", "wu", "wd", "dy")}
    override = inp["logits"].to(DEV) if "logits" in inp else None
    shared = None
    if Fs:
        sw = mi.shared_expert_weights(cfg, Fs)
        shared = tuple(sw[k].to(DEV) for k in ("wg_s", "wu_s", "wd_s"))
    dt = torch.float32 if cfg.dtype == "fp32" else torch.bfloat16
    buf = moe.alloc_layer(cfg.T, cfg.d, cfg.E, cfg.k, cfg.F, dt, DEV, mxfp8=mx, shared_F=Fs)
    fwd = lambda: moe.layer_forward(g["x"], g["wr"], g["wg"], g["wu"], g["wd"], cfg.k, buf, override,  # noqa: E731
                                    mxfp8=mx, shared=shared)
    fwd()
    moe.layer_backward(g["dy"], g["x"], g["wr"], g["wg"], g["wu"], g["wd"], buf, mxfp8=mx, shared=shared)
    torch.cuda.synchronize()
    ref = _grads(buf)
    saved = {k: buf.ffn[k].clone() for k in ("g", "u", "h")}
    fwd()
    torch.cuda.synchronize()
    clobber = [buf.xp, buf.ffn["g"], buf.ffn["u"], buf.ffn["h"]]
    if Fs:
        clobber += [buf.shared["ffn"][k] for k in ("g", "u", "h")]
    for t in clobber:
        t.fill_(float("nan"))
    moe.layer_backward(g["dy"], g["x"], g["wr"], g["wg"], g["wu"], g["wd"], buf, mxfp8=mx, shared=shared,
                       recompute=True)
    torch.cuda.synchronize()
    got = _grads(buf)
    for k in ref:
        assert torch.equal(got[k], ref[k]), k
    for k in saved:  # the recomputed g, u, h equal the forward's
        assert torch.equal(buf.ffn[k], saved[k]), k
    assert moe.saved_activation_bytes(buf, recompute=True) < moe.saved_activation_bytes(buf)
