"""The balance loss's gradient carried into the router ([P1] 四: the router
balances load; [P2] 2.2, 4.3): moe_router_dense_bwd adds dl W_r^T to dx and
x^T dl to dW_r in place (bf16 with E, d multiples of 64 on the matrix cores,
the rest on the vector ALUs).  Checked against the oracle's router_dense_bwd on
its own (zero and nonzero starting gradients, ragged E and d, the benchmark's
full shape) and inside the layer (layer_backward with aux_alpha) against the
oracle's layer gradients plus the balance loss's share."""
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


def _f(t):
    return t.detach().float().cpu().numpy()


@pytest.mark.parametrize("dtype,T,d,E,start", [("fp32", 300, 128, 8, "zero"), ("fp32", 77, 64, 1000, "zero"),
                                               ("bf16", 1000, 264, 100, "zero"), ("bf16", 513, 2048, 128, "rand"),
                                               ("fp32", 1030, 40, 33, "rand"), ("bf16", 16384, 2048, 128, "zero")])
def test_router_dense_bwd_matches_oracle(moe, dtype, T, d, E, start):
    rng = np.random.default_rng(T + d + E)
    dt = torch.float32 if dtype == "fp32" else torch.bfloat16
    x = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).to(dt)
    wr = torch.from_numpy((0.02 * rng.standard_normal((d, E))).astype(np.float32)).to(dt)
    dl = (1e-3 * rng.standard_normal((T, E))).astype(np.float32)
    ref = oracle.router_dense_bwd(mi.f32(x), mi.f32(wr), dl)
    if start == "zero":
        dx0, dw0 = torch.zeros(T, d, dtype=dt), torch.zeros(d, E, dtype=dt)
    else:  # same scale as the added terms, so the sum is checked, not hidden
        dx0 = torch.from_numpy((np.abs(ref["dx"]).mean() * rng.standard_normal((T, d))).astype(np.float32)).to(dt)
        dw0 = torch.from_numpy((np.abs(ref["dwr"]).mean() * rng.standard_normal((d, E))).astype(np.float32)).to(dt)
    gx, gw = dx0.to(DEV), dw0.to(DEV)
    moe.moe_router_dense_bwd(x.to(DEV), wr.to(DEV), torch.from_numpy(dl).to(DEV), gx, gw)
    torch.cuda.synchronize()
    tol = 1e-4 if dtype == "fp32" else 2e-2
    if T <= 2048:
        assert_close(_f(gx), mi.f32(dx0) + ref["dx"], tol, "dx")
    else:  # full size: every row checked against the product, sampled rows in fp64 above
        rows = rng.choice(T, 64, replace=False)
        assert_close(_f(gx)[rows], mi.f32(dx0)[rows] + ref["dx"][rows], tol, "dx (sampled rows)")
    assert_close(_f(gw), mi.f32(dw0) + ref["dwr"], tol, "dW_r")
    # deterministic: a second call from the same start gives the same bits
    gx2, gw2 = dx0.to(DEV), dw0.to(DEV)
    moe.moe_router_dense_bwd(x.to(DEV), wr.to(DEV), torch.from_numpy(dl).to(DEV), gx2, gw2)
    torch.cuda.synchronize()
    assert torch.equal(gx, gx2) and torch.equal(gw, gw2)


def test_router_dense_bwd_empty_batch(moe):
    wr = torch.randn(64, 16, device=DEV, dtype=torch.bfloat16)
    dw = torch.full((64, 16), 0.5, device=DEV, dtype=torch.bfloat16)
    e = torch.empty(0, 64, device=DEV, dtype=torch.bfloat16)
    moe.moe_router_dense_bwd(e, wr, torch.empty(0, 16, device=DEV), e.clone(), dw)
    torch.cuda.synchronize()
    assert torch.all(dw == 0.5)


ALPHA = 1000.0  # large, so the balance loss's share is a visible part of dx and dW_r


@pytest.mark.parametrize("name,over", [("tiny", {}),
                                       ("tiny", dict(dtype="bf16", T=700, E=16, k=4, x_std=1.0)),
                                       ("tiny", dict(dtype="bf16", T=1000, d=256, E=8, k=2, F=320, x_std=1.0)),
                                       # E and d multiples of 64: the matrix-core path
                                       ("tiny", dict(dtype="bf16", T=600, d=256, E=64, k=4, F=256, x_std=1.0))])
def test_layer_with_balance_loss(moe, name, over):
    cfg = mi.config(name, **over)
    inp = mi.layer_inputs(cfg)
    assert "logits" not in inp  # learned routing: the loss is a function of x W_r
    g = {k: inp[k].to(DEV) for k in ("x", "wr", "wg", "wu", "wd", "dy")}
    dt = torch.float32 if cfg.dtype == "fp32" else torch.bfloat16
    buf = moe.alloc_layer(cfg.T, cfg.d, cfg.E, cfg.k, cfg.F, dt, DEV)
    moe.layer_forward(g["x"], g["wr"], g["wg"], g["wu"], g["wd"], cfg.k, buf)
    moe.layer_backward(g["dy"], g["x"], g["wr"], g["wg"], g["wu"], g["wd"], buf, aux_alpha=ALPHA)
    torch.cuda.synchronize()
    logits = buf.logits.cpu().numpy()
    r = oracle.route(logits, cfg.k)
    assert np.array_equal(buf.route["topk_idx"].cpu().numpy(), r["topk_idx"])
    x, wr, dy = mi.f32(inp["x"]), mi.f32(inp["wr"]), mi.f32(inp["dy"])
    wg, wu, wd = mi.f32(inp["wg"]), mi.f32(inp["wu"]), mi.f32(inp["wd"])
    b = oracle.layer_bwd(x, wr, r["topk_idx"], r["gates"], dy, wg, wu, wd)
    aux = oracle.router_dense_bwd(x, wr, oracle.aux_loss_bwd(logits, r["counts"], cfg.k, ALPHA))
    # the balance loss's share is not negligible at this weight
    assert np.linalg.norm(aux["dwr"]) > 0.05 * np.linalg.norm(b["dwr"])
    tol = 1e-4 if cfg.dtype == "fp32" else 2e-2
    assert_close(_f(buf.aux_dl), oracle.aux_loss_bwd(logits, r["counts"], cfg.k, ALPHA), 1e-4, "aux dl")
    assert_close(_f(buf.dx), b["dx"] + aux["dx"], tol, "dx")
    assert_close(_f(buf.dw_router), b["dwr"] + aux["dwr"], tol, "dW_r")
