"""GPU parity of the gate/up dgrad with the router's input-gradient term
folded in (moe_grouped_ffn_bwd_router) against the oracle.

The router scores are x W_r, so the layer's input gradient has the term
sum_j dl[t,j] W_r[:, S_tj] ([P2] 2.2, the router's share of the backward).
The folded call adds dl[t,j] W_r[:, e] to the dgrad row of token t's slot j
before rounding; summing each token's k rows (the oracle's permute backward
without its router term) must then match the oracle's permute backward with
the router term over the oracle's own dgrad rows, within the bf16 bound
2e-2.  Every other output is bit-identical to the call without the term.
The route backward's expert-row copy of the logit gradients is integer
placement: bit-exact."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from tolerance import assert_close

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 2e-2


@pytest.fixture(scope="module")
def moe():
    import routing_grouped_expert_softmax_amd as m
    m.context(0)
    return m


def _case(T, k, E, d, F, seed, dead=()):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    for e in dead:
        lg[:, e] = -1e4
    r = oracle.route(lg, k)
    inp = mi.rows_inputs(T * k, d, E, F, r["counts"], seed=seed)
    dls = rng.standard_normal((T, k)).astype(np.float32)
    wr = torch.from_numpy((rng.standard_normal((d, E)) * 0.02).astype(np.float32)).to(torch.bfloat16)
    return r, inp, dls, wr


@pytest.mark.parametrize("T,k,E,d,F,dead", [(700, 2, 8, 256, 384, ()), (300, 4, 16, 384, 256, (3, 11)),
                                            (1, 1, 4, 256, 128, ()), (2000, 4, 64, 512, 256, ())])
def test_router_term_folded_into_dgrad(moe, T, k, E, d, F, dead):
    r, inp, dls, wr = _case(T, k, E, d, F, T + E, dead)
    g = {n: inp[n].to(DEV) for n in ("xp", "dyp", "wg", "wu", "wd")}
    off = torch.from_numpy(inp["offsets"]).to(DEV)
    f = moe.moe_grouped_ffn_fwd(g["xp"], g["wg"], g["wu"], g["wd"], off)
    plain = moe.moe_grouped_ffn_bwd(g["xp"], g["wg"], g["wu"], g["wd"], off, f["g"], f["u"], f["h"], g["dyp"])
    dl_rows = dls.reshape(-1)[r["src_tk"]]  # row r holds its (token, slot)'s value
    router = (torch.from_numpy(dl_rows).to(DEV), wr.to(DEV))
    folded = moe.moe_grouped_ffn_bwd(g["xp"], g["wg"], g["wu"], g["wd"], off, f["g"], f["u"], f["h"],
                                     g["dyp"], router=router)
    torch.cuda.synchronize()
    for name in ("dg", "du", "dw_gate", "dw_up", "dw_down"):
        assert torch.equal(plain[name], folded[name]), name
    rd = oracle.expert_dgrad(mi.f32(inp["xp"]), mi.f32(inp["dyp"]), inp["offsets"], mi.f32(inp["wg"]),
                             mi.f32(inp["wu"]), mi.f32(inp["wd"]))
    want = oracle.permute_bwd(rd["dxp"], r["row_of"], r["topk_idx"], dls, mi.f32(wr))
    got = oracle.permute_bwd(mi.f32(folded["dxp"].cpu()), r["row_of"])
    assert_close(got, want, TOL, "sum_j dxp rows (router term folded)")


def test_router_fold_rejects_bad_arguments(moe):
    r, inp, dls, wr = _case(64, 2, 4, 256, 128, 5)
    g = {n: inp[n].to(DEV) for n in ("xp", "dyp", "wg", "wu", "wd")}
    off = torch.from_numpy(inp["offsets"]).to(DEV)
    f = moe.moe_grouped_ffn_fwd(g["xp"], g["wg"], g["wu"], g["wd"], off)
    args = (g["xp"], g["wg"], g["wu"], g["wd"], off, f["g"], f["u"], f["h"], g["dyp"])
    dl = torch.from_numpy(dls.reshape(-1)[r["src_tk"]]).to(DEV)
    with pytest.raises(moe.MoeError):  # W_r transposed
        moe.moe_grouped_ffn_bwd(*args, router=(dl, wr.t().contiguous().to(DEV)))
    with pytest.raises(moe.MoeError):  # too few row gradients
        moe.moe_grouped_ffn_bwd(*args, router=(dl[:-1], wr.to(DEV)))
    with pytest.raises(moe.MoeError):  # fp32 is not supported by the folded call
        a32 = [t.float() if t.dtype == torch.bfloat16 else t for t in args]
        moe.moe_grouped_ffn_bwd(*a32, router=(dl, wr.float().to(DEV)))


@pytest.mark.parametrize("T,E,k", [(1, 4, 1), (1000, 128, 4), (777, 16, 8)])
def test_route_bwd_rows(moe, T, E, k):
    rng = np.random.default_rng(T)
    lg = torch.from_numpy(rng.standard_normal((T, E)).astype(np.float32)).to(DEV)
    r = moe.moe_route(lg, k)
    dgates = torch.from_numpy(rng.standard_normal((T, k)).astype(np.float32)).to(DEV)
    plain = moe.moe_route_bwd(r["gates"], dgates)
    dls, dl_rows = moe.moe_route_bwd(r["gates"], dgates, row_of=r["row_of"])
    torch.cuda.synchronize()
    assert torch.equal(plain, dls)
    row_of = r["row_of"].cpu().numpy()
    got = dl_rows.cpu().numpy()
    assert np.array_equal(got[row_of.reshape(-1)], dls.cpu().numpy().reshape(-1))
    ref = oracle.route_bwd(r["gates"].cpu().numpy(), dgates.cpu().numpy())
    assert_close(dls.cpu().numpy(), ref, 1e-5, "dlogits_sel")
