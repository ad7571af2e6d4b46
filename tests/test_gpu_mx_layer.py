"""GPU parity of the end-to-end MXFP8 layer with quantise-on-permute ([P1] 三:
MXFP8 routed experts; [P1] 二: rows written straight into the experts'
buffers) against the oracle.

The permute's codes and scale bytes are integer work: bit-exact against the
oracle's MX codec applied to the permuted rows.  The pre-quantised forward is
bit-identical to the forward that quantises its rows itself.  The layer
compares with the oracle chain route -> permute -> MX experts -> combine and
back, on the same routing, within the MXFP8 bound 6e-2."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from tolerance import assert_close

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 6e-2


@pytest.fixture(scope="module")
def moe():
    import routing_grouped_expert_softmax_amd as m
    m.context(0)
    return m


def _special_rows(T, d, seed):
    """bf16 rows reaching every branch of the codec: normals, tiny and huge
    blocks, zero blocks with signed zeros, exact E4M3 ties."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((T, d)).astype(np.float32)
    kinds = rng.integers(0, 6, size=(T, d // 32))
    for t in range(T):
        for b in range(d // 32):
            blk = a[t, 32 * b:32 * b + 32]
            if kinds[t, b] == 1:
                blk *= np.float32(2.0 ** -128)
            elif kinds[t, b] == 2:
                blk *= np.float32(2.0 ** 100)
            elif kinds[t, b] == 3:
                blk[:] = 0.0
                blk[::3] = -0.0
            elif kinds[t, b] == 4:
                blk[:] = rng.integers(-64, 65, size=32) / 64.0
                blk[0] = 1.0
    return torch.from_numpy(a).to(torch.bfloat16)


def _routing(moe, T, E, k, seed):
    lg = torch.from_numpy(np.random.default_rng(seed).standard_normal((T, E)).astype(np.float32)).to(DEV)
    return moe.moe_route(lg, k)


@pytest.mark.parametrize("T,d,E,k", [(1, 32, 4, 1), (300, 96, 8, 3), (1000, 2048, 128, 4), (77, 4096, 16, 8)])
def test_permute_mx_bitexact(moe, T, d, E, k):
    x = _special_rows(T, d, T + d)
    r = _routing(moe, T, E, k, T)
    xp, codes, scales = moe.moe_permute_mx(x.to(DEV), r["row_of"])
    _, codes2, scales2 = moe.moe_permute_mx(x.to(DEV), r["row_of"], with_bf16=False)
    torch.cuda.synchronize()
    row_of = r["row_of"].cpu().numpy()
    xp_ref = oracle.permute(mi.f32(x), row_of)
    assert np.array_equal(mi.f32(xp.cpu()), xp_ref)
    rc, rs = oracle.mx_quantize(xp_ref, axis=0)
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert torch.equal(codes, codes2) and torch.equal(scales, scales2)


def test_permute_mx_rejects_bad_arguments(moe):
    x = torch.zeros(4, 48, dtype=torch.bfloat16, device=DEV)  # d not a multiple of 32
    row_of = torch.zeros(4, 1, dtype=torch.int32, device=DEV)
    with pytest.raises(moe.MoeError):
        moe.moe_permute_mx(x, row_of)


@pytest.mark.parametrize("counts,d,F", [([300, 0, 129, 517], 256, 384), ([1000], 512, 256)])
def test_ffn_fwd_mxq_matches_internal_quantisation(moe, counts, d, F):
    counts = np.array(counts)
    E, R = len(counts), int(counts.sum())
    inp = mi.rows_inputs(R, d, E, F, counts, seed=R)
    g = {k: inp[k].to(DEV) for k in ("xp", "wg", "wu", "wd")}
    off = torch.from_numpy(inp["offsets"]).to(DEV)
    ref = moe.moe_grouped_ffn_fwd(g["xp"], g["wg"], g["wu"], g["wd"], off, mxfp8=True)
    codes, scales = moe.moe_mx_quantize(g["xp"], 0)
    got = moe.moe_grouped_ffn_fwd_mxq(codes, scales, g["wg"], g["wu"], g["wd"], off)
    torch.cuda.synchronize()
    for key in ref:
        assert torch.equal(got[key], ref[key]), key


def run_mx_layer(moe, cfg, inp):
    g = {k: inp[k].to(DEV) for k in ("x", "wr", "wg", "wu", "wd", "dy")}
    override = inp["logits"].to(DEV) if "logits" in inp else None
    buf = moe.alloc_layer(cfg.T, cfg.d, cfg.E, cfg.k, cfg.F, torch.bfloat16, DEV, mxfp8=True)
    moe.layer_forward(g["x"], g["wr"], g["wg"], g["wu"], g["wd"], cfg.k, buf, override, mxfp8=True)
    moe.layer_backward(g["dy"], g["x"], g["wr"], g["wg"], g["wu"], g["wd"], buf, mxfp8=True)
    torch.cuda.synchronize()
    return buf


def _f(t):
    return t.detach().float().cpu().numpy()


@pytest.mark.parametrize("over", [dict(T=512, d=256, E=8, k=2, F=256),
                                  dict(T=700, d=384, E=16, k=4, F=128, routing="uniform"),
                                  dict(T=1000, d=256, E=8, k=2, F=384, routing="zipf", n_dead=2)])
def test_mx_layer_end_to_end(moe, over):
    cfg = mi.config("tiny", dtype="bf16", x_std=1.0, **over)
    inp = mi.layer_inputs(cfg)
    buf = run_mx_layer(moe, cfg, inp)
    # the oracle routes the GPU's own scores (same selection, same rows)
    src = inp["logits"].numpy() if "logits" in inp else buf.logits.cpu().numpy()
    r = oracle.route(src, cfg.k)
    for key in ("topk_idx", "counts", "offsets", "row_of"):
        assert np.array_equal(buf.route[key].cpu().numpy(), r[key]), key
    x, wr, dy = mi.f32(inp["x"]), mi.f32(inp["wr"]), mi.f32(inp["dy"])
    wg, wu, wd = mi.f32(inp["wg"]), mi.f32(inp["wu"]), mi.f32(inp["wd"])
    xp = oracle.permute(x, r["row_of"])
    fw = oracle.mx_expert_fwd(xp, r["offsets"], wg, wu, wd)
    y = oracle.combine(fw["yp"], r["gates"], r["row_of"])
    dyp, dgates = oracle.combine_bwd(dy, fw["yp"], r["gates"], r["row_of"])
    dls = oracle.route_bwd(r["gates"], dgates)
    bw = oracle.mx_expert_bwd(xp, oracle._bf16_round(dyp), r["offsets"], wg, wu, wd, fw["g"], fw["u"], fw["h"])
    dx = oracle.permute_bwd(bw["dxp"], r["row_of"], r["topk_idx"], dls, wr)
    dwr = oracle.router_wgrad(x, dls, r["topk_idx"], cfg.E)
    assert np.array_equal(_f(buf.xp), xp)
    assert_close(_f(buf.ffn["h"]), fw["h"], TOL, "h")
    assert_close(_f(buf.y), y, TOL, "y")
    assert_close(_f(buf.dgates), dgates, TOL, "dgates")
    assert_close(_f(buf.dx), dx, TOL, "dx")
    assert_close(_f(buf.dw_router), dwr, TOL, "dW_r")
    counts = r["counts"]
    for name, key in (("dw_gate", "dwg"), ("dw_up", "dwu"), ("dw_down", "dwd")):
        got = _f(buf.bwd[name])
        for e in range(cfg.E):
            assert_close(got[e], bw[key][e], TOL, f"{name}[{e}] (count {counts[e]})")


@pytest.mark.slow
def test_mx_layer_full_size_sampled(moe):
    """uniform128 end to end in MXFP8: y and dx of sampled tokens against the
    oracle chain evaluated for those tokens' rows only."""
    cfg = mi.config("uniform128")
    inp = mi.layer_inputs(cfg)
    buf = run_mx_layer(moe, cfg, inp)
    r = {k: v.cpu().numpy() for k, v in buf.route.items()}
    assert np.array_equal(r["topk_idx"], oracle.route(inp["logits"].numpy(), cfg.k)["topk_idx"])
    x, wr, dy = mi.f32(inp["x"]), mi.f32(inp["wr"]), mi.f32(inp["dy"])
    wg, wu, wd = mi.f32(inp["wg"]), mi.f32(inp["wu"]), mi.f32(inp["wd"])
    rng = np.random.default_rng(7)
    tok = np.unique(np.concatenate([[0, cfg.T - 1], rng.integers(0, cfg.T, 10)]))
    rows = r["row_of"][tok].reshape(-1)
    R = cfg.T * cfg.k
    xp = np.zeros((R, cfg.d), dtype=np.float32)
    xp[rows] = x[np.repeat(tok, cfg.k)]
    # upstream rows (they do not depend on yp), stored bf16 on the GPU
    dyp, _ = oracle.combine_bwd(dy, np.zeros((R, cfg.d), dtype=np.float32), r["gates"], r["row_of"])
    ref = oracle.mx_expert_rows(xp, oracle._bf16_round(dyp), r["offsets"], wg, wu, wd, rows)
    del dyp
    yp = np.zeros((R, cfg.d))
    yp[rows] = ref["yp"]
    y = oracle.combine(yp, r["gates"], r["row_of"])[tok]
    assert_close(_f(buf.y)[tok], y, TOL, "y")
    dgates = oracle.combine_bwd(dy, yp, r["gates"], r["row_of"])[1][tok]
    dls = oracle.route_bwd(r["gates"][tok], dgates)
    dxp = np.zeros((R, cfg.d))
    dxp[rows] = ref["dxp"]
    dx = oracle.permute_bwd(dxp, r["row_of"][tok], r["topk_idx"][tok], dls, wr)
    assert_close(_f(buf.dgates)[tok], dgates, TOL, "dgates")
    assert_close(_f(buf.dx)[tok], dx, TOL, "dx")
