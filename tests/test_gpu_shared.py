"""GPU parity of the layer with a shared expert ([P1] 四: shared experts) —
one SwiGLU FFN over every token, ungated, added in the combine; its input
gradient added in the permute backward — against the oracle (the routed
layer plus the oracle's shared expert)."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from tolerance import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def moe():
    import routing_grouped_expert_softmax_amd as m
    m.context(0)
    return m


def run_shared(moe, cfg, inp, sw, Fs):
    g = {k: inp[k].to(DEV) for k in ("x", "wr", "wg", "wu", "wd", "dy")}
    shared = tuple(sw[k].to(DEV) for k in ("wg_s", "wu_s", "wd_s"))
    override = inp["logits"].to(DEV) if "logits" in inp else None
    dt = torch.float32 if cfg.dtype == "fp32" else torch.bfloat16
    buf = moe.alloc_layer(cfg.T, cfg.d, cfg.E, cfg.k, cfg.F, dt, DEV, shared_F=Fs)
    moe.layer_forward(g["x"], g["wr"], g["wg"], g["wu"], g["wd"], cfg.k, buf, override, shared=shared)
    moe.layer_backward(g["dy"], g["x"], g["wr"], g["wg"], g["wu"], g["wd"], buf, shared=shared)
    torch.cuda.synchronize()
    return buf


def _f(t):
    return t.detach().float().cpu().numpy()


@pytest.mark.parametrize("name,over,Fs", [("tiny", {}, 256),
                                          ("tiny", dict(dtype="bf16", T=700, E=16, k=4, x_std=1.0,
                                                        routing="uniform"), 192),
                                          ("tiny", dict(dtype="bf16", T=1000, d=256, E=8, k=2, F=320,
                                                        x_std=1.0, routing="zipf", n_dead=2), 320)])
def test_shared_layer_end_to_end(moe, name, over, Fs):
    cfg = mi.config(name, **over)
    inp = mi.layer_inputs(cfg)
    sw = mi.shared_expert_weights(cfg, Fs)
    buf = run_shared(moe, cfg, inp, sw, Fs)
    src = inp["logits"].numpy() if "logits" in inp else buf.logits.cpu().numpy()
    r = oracle.route(src, cfg.k)
    assert np.array_equal(buf.route["topk_idx"].cpu().numpy(), r["topk_idx"])
    tol = 1e-4 if cfg.dtype == "fp32" else 2e-2
    x, wr, dy = mi.f32(inp["x"]), mi.f32(inp["wr"]), mi.f32(inp["dy"])
    wg, wu, wd = mi.f32(inp["wg"]), mi.f32(inp["wu"]), mi.f32(inp["wd"])
    ws = [mi.f32(sw[k]) for k in ("wg_s", "wu_s", "wd_s")]
    sf = oracle.shared_expert_fwd(x, *ws)
    sb = oracle.shared_expert_bwd(x, dy, *ws)
    y = oracle.layer_fwd(x, r["topk_idx"], r["gates"], wg, wu, wd) + sf["yp"]
    b = oracle.layer_bwd(x, wr, r["topk_idx"], r["gates"], dy, wg, wu, wd)
    assert_close(_f(buf.shared["ffn"]["yp"]), sf["yp"], tol, "y_shared")
    assert_close(_f(buf.y), y, tol, "y")
    assert_close(_f(buf.dgates), b["dgates"], tol, "dgates")
    assert_close(_f(buf.dx), b["dx"] + sb["dx"], tol, "dx")
    assert_close(_f(buf.dw_router), b["dwr"], tol, "dW_r")
    for name_, key in (("dw_gate", "dwg"), ("dw_up", "dwu"), ("dw_down", "dwd")):
        assert_close(_f(buf.shared["bwd"][name_])[0], sb[key][0], tol, f"shared {name_}")
        got = _f(buf.bwd[name_])
        for e in range(cfg.E):
            assert_close(got[e], b[key][e], tol, f"{name_}[{e}]")


def test_combine_and_permute_bwd_addends(moe):
    """The addend paths alone: y = combine + y_shared and dx = permute_bwd +
    dx_shared (fp32 data, so the only difference is fp32 summation)."""
    rng = np.random.default_rng(31)
    T, d, E, k = 300, 64, 8, 3
    lg = torch.from_numpy(rng.standard_normal((T, E)).astype(np.float32)).to(DEV)
    r = moe.moe_route(lg, k)
    yp = torch.from_numpy(rng.standard_normal((T * k, d)).astype(np.float32)).to(DEV)
    add = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).to(DEV)
    y = moe.moe_combine(yp, r["gates"], r["row_of"], y_shared=add)
    dx = moe.moe_permute_bwd(yp, r["row_of"], dx_shared=add)
    torch.cuda.synchronize()
    row_of, gates = r["row_of"].cpu().numpy(), r["gates"].cpu().numpy()
    ypn, addn = yp.cpu().numpy(), add.cpu().numpy()
    assert_close(y.cpu().numpy(), oracle.combine(ypn, gates, row_of) + addn, 1e-6, "y")
    assert_close(dx.cpu().numpy(), oracle.permute_bwd(ypn, row_of) + addn, 1e-6, "dx")


@pytest.mark.slow
def test_shared_layer_full_size_sampled(moe):
    """uniform128 with a shared expert of the routed width, launched as
    bench.py does: sampled tokens of y and dx, sampled elements of the shared
    weight gradients."""
    cfg = mi.config("uniform128")
    inp = mi.layer_inputs(cfg)
    sw = mi.shared_expert_weights(cfg)
    buf = run_shared(moe, cfg, inp, sw, cfg.F)
    r = oracle.route(inp["logits"].numpy(), cfg.k, "f32")
    assert np.array_equal(buf.route["topk_idx"].cpu().numpy(), r["topk_idx"])
    x, wr, dy = mi.f32(inp["x"]), mi.f32(inp["wr"]), mi.f32(inp["dy"])
    wg, wu, wd = mi.f32(inp["wg"]), mi.f32(inp["wu"]), mi.f32(inp["wd"])
    ws = [mi.f32(sw[k]) for k in ("wg_s", "wu_s", "wd_s")]
    rng = np.random.default_rng(5)
    tok = np.unique(np.concatenate([[0, cfg.T - 1], rng.choice(cfg.T, 24, replace=False)]))
    y = oracle.layer_fwd(x[tok], r["topk_idx"][tok], r["gates"][tok], wg, wu, wd) + \
        oracle.shared_expert_fwd(x[tok], *ws)["yp"]
    assert_close(_f(buf.y)[tok], y, 2e-2, "y (sampled tokens)")
    b = oracle.layer_bwd(x[tok], wr, r["topk_idx"][tok], r["gates"][tok], dy[tok], wg, wu, wd)
    dxs = oracle.shared_expert_bwd(x[tok], dy[tok], *ws)["dx"]
    assert_close(_f(buf.dx)[tok], b["dx"] + dxs, 2e-2, "dx (sampled tokens)")
    off = np.array([0, cfg.T], dtype=np.int32)
    for which, name_, shp in [(0, "dw_gate", (cfg.d, cfg.F)), (1, "dw_up", (cfg.d, cfg.F)),
                              (2, "dw_down", (cfg.F, cfg.d))]:
        el = np.stack([np.zeros(8, dtype=np.int64), rng.integers(0, shp[0], 8), rng.integers(0, shp[1], 8)], 1)
        ref = oracle.expert_wgrad_elems(x, dy, off, *ws, which, el)
        got = _f(buf.shared["bwd"][name_])[el[:, 0], el[:, 1], el[:, 2]]
        assert_close(got, ref, 2e-2, f"shared {name_} (sampled elements)")
