"""GPU parity of the MXFP8 backward with bf16 weight gradients (MXFP8 on the
data-gradient GEMMs only; the bigchange.ai page's overview names MXFP8 for
selected operations, the first page section 三 the MXFP8 expert GEMMs).

* dg, du and dxp are the all-MXFP8 backward's bytes (the same kernels on the
  same operands), checked bit for bit against moe_grouped_ffn_bwd_mxp.
* The weight gradients compare with the oracle's chain with wgrad="bf16"
  (fp64 products of the bf16 operands, pinned by brute-force loops) within
  the bf16 bound; experts without rows give exact zeros.  One group of 2048
  rows takes the split-K form of the weight gradients.
* The layer with mx_wgrad=False compares end to end with the oracle chain
  route -> permute -> MX experts (bf16 weight gradients) -> combine and back.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from tolerance import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL_MX = 6e-2   # MXFP8 products
TOL_BF = 2e-2   # bf16 operands and outputs


@pytest.fixture(scope="module")
def moe():
    import routing_grouped_expert_softmax_amd as m
    m.context(0)
    return m


def _f(t):
    return t.detach().float().cpu().numpy()


CASES = [(256, 384, [300, 0, 129, 517]), (128, 128, [31, 1, 128, 256, 0]), (256, 256, [2048]),
         (128, 256, [0, 0, 0])]


@pytest.mark.parametrize("d,F,counts", CASES)
def test_bf16w_backward(moe, d, F, counts):
    counts = np.array(counts)
    E, R = len(counts), int(counts.sum())
    print(f"bf16w backward d={d} F={F} counts={counts.tolist()}", flush=True)
    inp = mi.rows_inputs(R, d, E, F, counts, seed=R + 5)
    g = {k: inp[k].to(DEV) for k in ("xp", "dyp", "wg", "wu", "wd")}
    off = torch.from_numpy(inp["offsets"]).to(DEV)
    pack = moe.moe_mx_quantize_weights(g["wg"], g["wu"], g["wd"])
    fw = moe.moe_grouped_ffn_fwd_mxp(pack, off, xp=g["xp"])
    mx = moe.moe_grouped_ffn_bwd_mxp(g["xp"], pack, off, fw["g"], fw["u"], fw["h"], g["dyp"])
    bw = moe.moe_grouped_ffn_bwd_mxp_bf16w(g["xp"], pack, off, fw["g"], fw["u"], fw["h"], g["dyp"])
    torch.cuda.synchronize()
    for name in ("dg", "du", "dxp"):
        assert torch.equal(bw[name], mx[name]), name
    xp, dyp = mi.f32(inp["xp"]), mi.f32(inp["dyp"])
    wg, wu, wd = mi.f32(inp["wg"]), mi.f32(inp["wu"]), mi.f32(inp["wd"])
    ofw = oracle.mx_expert_fwd(xp, inp["offsets"], wg, wu, wd)
    ref = oracle.mx_expert_bwd(xp, dyp, inp["offsets"], wg, wu, wd, ofw["g"], ofw["u"], ofw["h"], wgrad="bf16")
    if R:
        assert_close(_f(bw["dxp"]), ref["dxp"], TOL_MX, "dxp")
    for name, key in (("dw_gate", "dwg"), ("dw_up", "dwu"), ("dw_down", "dwd")):
        got = _f(bw[name])
        for e in range(E):
            assert_close(got[e], ref[key][e], TOL_BF, f"{name}[{e}] (count {counts[e]})")


def test_bf16w_rejects_bad_arguments(moe):
    E, d, F = 2, 128, 128
    w = torch.zeros(E, d, F, dtype=torch.bfloat16, device=DEV)
    wd = torch.zeros(E, F, d, dtype=torch.bfloat16, device=DEV)
    pack = moe.moe_mx_quantize_weights(w, w, wd)
    xp = torch.zeros(64, d, dtype=torch.bfloat16, device=DEV)
    off = torch.tensor([0, 32, 64], dtype=torch.int32, device=DEV)
    t = torch.zeros(64, F, dtype=torch.bfloat16, device=DEV)
    other = moe.MxWeightPack(pack.data, E, d, 2 * F)  # a pack for another shape
    with pytest.raises(moe.MoeError):
        moe.moe_grouped_ffn_bwd_mxp_bf16w(xp, other, off, t, t, t, xp)
    out = dict(dg=t, du=t, dxp=xp, dw_gate=w, dw_up=w, dw_down=wd)  # dg and du overlap
    with pytest.raises(moe.MoeError):
        moe.moe_grouped_ffn_bwd_mxp_bf16w(xp, pack, off, t, t, t, xp, out=out)
    torch.cuda.synchronize()


@pytest.mark.parametrize("over", [dict(T=512, d=256, E=8, k=2, F=256),
                                  dict(T=1000, d=256, E=8, k=2, F=384, routing="zipf", n_dead=2)])
def test_mx_layer_bf16_wgrad_end_to_end(moe, over):
    cfg = mi.config("tiny", dtype="bf16", x_std=1.0, **over)
    print(f"MX layer, bf16 weight gradients: {over}", flush=True)
    inp = mi.layer_inputs(cfg)
    g = {k: inp[k].to(DEV) for k in ("x", "wr", "wg", "wu", "wd", "dy")}
    override = inp["logits"].to(DEV) if "logits" in inp else None
    buf = moe.alloc_layer(cfg.T, cfg.d, cfg.E, cfg.k, cfg.F, torch.bfloat16, DEV, mxfp8=True)
    moe.layer_forward(g["x"], g["wr"], g["wg"], g["wu"], g["wd"], cfg.k, buf, override, mxfp8=True)
    moe.layer_backward(g["dy"], g["x"], g["wr"], g["wg"], g["wu"], g["wd"], buf, mxfp8=True, mx_wgrad=False)
    torch.cuda.synchronize()
    src = inp["logits"].numpy() if "logits" in inp else buf.logits.cpu().numpy()
    r = oracle.route(src, cfg.k)
    assert np.array_equal(buf.route["row_of"].cpu().numpy(), r["row_of"])
    x, wr, dy = mi.f32(inp["x"]), mi.f32(inp["wr"]), mi.f32(inp["dy"])
    wg, wu, wd = mi.f32(inp["wg"]), mi.f32(inp["wu"]), mi.f32(inp["wd"])
    xp = oracle.permute(x, r["row_of"])
    fw = oracle.mx_expert_fwd(xp, r["offsets"], wg, wu, wd)
    dyp, dgates = oracle.combine_bwd(dy, fw["yp"], r["gates"], r["row_of"])
    dls = oracle.route_bwd(r["gates"], dgates)
    bw = oracle.mx_expert_bwd(xp, oracle._bf16_round(dyp), r["offsets"], wg, wu, wd, fw["g"], fw["u"], fw["h"],
                              wgrad="bf16")
    dx = oracle.permute_bwd(bw["dxp"], r["row_of"], r["topk_idx"], dls, wr)
    assert_close(_f(buf.dx), dx, TOL_MX, "dx")
    assert_close(_f(buf.dw_router), oracle.router_wgrad(x, dls, r["topk_idx"], cfg.E), TOL_MX, "dW_r")
    for name, key in (("dw_gate", "dwg"), ("dw_up", "dwu"), ("dw_down", "dwd")):
        got = _f(buf.bwd[name])
        for e in range(cfg.E):
            # the forward's h and the combine backward's dyp carry MXFP8 error
            assert_close(got[e], bw[key][e], TOL_MX, f"{name}[{e}] (count {r['counts'][e]})")
