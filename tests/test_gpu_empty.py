"""An empty batch (T = 0 tokens) through the whole layer, forward and
backward, in bf16, fp32 and MXFP8, with and without a shared expert.

A dropless layer must take any token count, zero included: every expert then
receives no rows ([P1] 二, the grouped GEMM over a count list that may hold
zeros), so each expert's weight gradient is a sum over no rows and must be
exactly zero, as must the router's.  Every output is pre-filled with NaN so
that one left unwritten fails the check."""
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


def _nan_fill(t):
    if t.is_floating_point():
        t.fill_(float("nan"))
    else:
        t.fill_(-7)


@pytest.mark.parametrize("dtype,mxfp8,shared", [("bf16", False, False), ("bf16", False, True),
                                                ("fp32", False, False), ("bf16", True, False),
                                                ("bf16", True, True)])
@pytest.mark.parametrize("recompute", [False, True])
def test_empty_batch_layer(moe, dtype, mxfp8, shared, recompute):
    cfg = mi.config("tiny", dtype=dtype, T=16, d=256, E=8, k=2, F=256)
    inp = mi.layer_inputs(cfg)
    g = {k: inp[k].to(DEV) for k in ("wr", "wg", "wu", "wd")}
    tdt = inp["x"].dtype
    x = torch.empty(0, cfg.d, dtype=tdt, device=DEV)
    dy = torch.empty(0, cfg.d, dtype=tdt, device=DEV)
    sw = None
    Fs = 0
    if shared:
        w = mi.shared_expert_weights(cfg, 128)
        sw = tuple(w[k].to(DEV) for k in ("wg_s", "wu_s", "wd_s"))
        Fs = 128
    buf = moe.alloc_layer(0, cfg.d, cfg.E, cfg.k, cfg.F, tdt, DEV, mxfp8=mxfp8, shared_F=Fs)
    outs = [buf.route["counts"], buf.route["offsets"], buf.dw_router, *buf.bwd.values()]
    if shared:
        outs += list(buf.shared["bwd"].values())
    for t in outs:
        _nan_fill(t)
    moe.layer_forward(x, g["wr"], g["wg"], g["wu"], g["wd"], cfg.k, buf, mxfp8=mxfp8, shared=sw)
    moe.layer_backward(dy, x, g["wr"], g["wg"], g["wu"], g["wd"], buf, mxfp8=mxfp8, shared=sw,
                       recompute=recompute)
    torch.cuda.synchronize()
    assert buf.y.shape == (0, cfg.d) and buf.dx.shape == (0, cfg.d)
    assert not buf.route["counts"].any() and not buf.route["offsets"].any()
    assert buf.dw_router.shape == (cfg.d, cfg.E)
    grads = [buf.dw_router] + [buf.bwd[n] for n in ("dw_gate", "dw_up", "dw_down")]
    if shared:
        grads += [buf.shared["bwd"][n] for n in ("dw_gate", "dw_up", "dw_down")]
    for t in grads:
        assert torch.equal(t, torch.zeros_like(t)), tuple(t.shape)


def test_empty_batch_statistics(moe):
    """Statistics and the balance-loss gradient of an empty batch: zero
    counts, zero means, zero loss, an empty gradient."""
    E, k = 8, 2
    lg = torch.empty(0, E, device=DEV)
    r = moe.moe_route(lg, k)
    s = moe.moe_route_stats(lg, r["counts"], k, 0.01)
    d = moe.moe_aux_loss_bwd(lg, r["counts"], k, 0.01)
    torch.cuda.synchronize()
    assert not r["counts"].any() and not r["offsets"].any()
    assert s["aux_loss"].item() == 0.0 and not s["prob_mean"].any()
    assert d.shape == (0, E)
