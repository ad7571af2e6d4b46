"""GPU parity of each C-ABI call against the CPU oracle, on seeded inputs at
sizes the oracle finishes in seconds (several tiles plus ragged tails, empty
experts, adversarial routing).  Integer outputs bit-exact; floating outputs
within the stated tolerances (fp32 data: 1e-4; bf16 data: 2e-2)."""
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


def tol_for(dtype):
    return 1e-4 if dtype == "fp32" else 2e-2


def tdt(dtype):
    return torch.float32 if dtype == "fp32" else torch.bfloat16


# ------------------------------------------------------------------ routing
def route_case(moe, logits_np, k):
    lg = torch.from_numpy(np.ascontiguousarray(logits_np, dtype=np.float32)).to(DEV)
    out = moe.moe_route(lg, k)
    torch.cuda.synchronize()
    got = {key: v.cpu().numpy() for key, v in out.items()}
    ref = oracle.route(logits_np, k)
    T, E = logits_np.shape
    for key in ("topk_idx", "counts", "offsets", "row_of"):
        assert np.array_equal(got[key], ref[key]), key
    assert np.array_equal(got["src_tk"][:T * k], ref["src_tk"])
    np.testing.assert_allclose(got["gates"], ref["gates"], rtol=0, atol=1e-5)


@pytest.mark.parametrize("T,E,k,seed", [(256, 8, 2, 0), (1000, 128, 4, 1), (333, 5, 5, 2), (1, 16, 4, 3),
                                        (4097, 64, 8, 4), (700, 1024, 32, 5), (257, 1, 1, 6)])
def test_route_random(moe, T, E, k, seed):
    rng = np.random.default_rng(seed)
    route_case(moe, rng.standard_normal((T, E)).astype(np.float32), k)


def test_route_adversarial(moe):
    rng = np.random.default_rng(9)
    # all-equal rows, integer ties with signed zeros, one expert takes all
    route_case(moe, np.full((300, 8), 0.5, dtype=np.float32), 4)
    lg = rng.integers(-2, 3, size=(777, 16)).astype(np.float32)
    lg[(lg == 0) & (rng.random(lg.shape) < 0.5)] = -0.0
    route_case(moe, lg, 4)
    hot = np.zeros((513, 32), dtype=np.float32)
    hot[:, 31] = 3.0
    route_case(moe, hot, 1)
    route_case(moe, rng.standard_normal((100, 6)).astype(np.float32), 6)  # k == E


@pytest.mark.parametrize("dtype,T,d,E", [("fp32", 256, 128, 8), ("bf16", 300, 256, 8),
                                         ("bf16", 520, 512, 128), ("bf16", 64, 2048, 16),
                                         # E > 64 on the VALU kernel in 64-expert passes:
                                         # fp32, bf16 with E % 8 != 0 or d % 64 != 0
                                         ("fp32", 300, 128, 128), ("fp32", 70, 64, 1000),
                                         ("fp32", 33, 2048, 77), ("bf16", 130, 128, 100),
                                         ("bf16", 200, 96, 128)])
def test_router_logits(moe, dtype, T, d, E):
    c = mi.layer_inputs(mi.config("tiny", T=T, d=d, E=E, dtype=dtype, x_std=1.0), with_weights=False)
    got = moe.moe_router_logits(c["x"].to(DEV), c["wr"].to(DEV)).cpu().numpy()
    ref = oracle.router_logits(mi.f32(c["x"]), mi.f32(c["wr"]))
    assert_close(got, ref, 1e-5, "logits")


# ------------------------------------------------------------------ rows
# The row kernels have a guard-free form for k equal to the dispatch width
# (2, 4, 8, 32) with rows of whole lane passes: bf16 top-4 d=2048, fp32 top-2
# d=2048 (also the permute's), bf16 top-8 d=1024 and top-32 d=512 take it;
# the ragged widths (d=264, fp32 d=128) take the guarded form.
@pytest.mark.parametrize("dtype,T,d,E,k", [("fp32", 256, 128, 8, 2), ("bf16", 333, 264, 16, 4),
                                           ("bf16", 1000, 2048, 8, 4), ("fp32", 300, 2048, 8, 2),
                                           ("bf16", 200, 1024, 16, 8), ("bf16", 100, 512, 32, 32)])
def test_permute_combine_and_backward(moe, dtype, T, d, E, k):
    rng = np.random.default_rng(T)
    c = mi.layer_inputs(mi.config("tiny", T=T, d=d, E=E, k=k, dtype=dtype, x_std=1.0), with_weights=False)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    r = moe.moe_route(torch.from_numpy(logits).to(DEV), k)
    x = c["x"].to(DEV)
    xp = moe.moe_permute(x, r["row_of"])
    ro = r["row_of"].cpu().numpy()
    xf = mi.f32(c["x"])
    # permute is a copy: bit-exact
    assert np.array_equal(mi.f32(xp.cpu()), oracle.permute(xf, ro).astype(np.float32))
    # combine(permute(x)) with unit gates is exactly k*x (bf16 sums exact for k=2,4)
    ones = torch.ones(T, k, dtype=torch.float32, device=DEV)
    y1 = moe.moe_combine(xp, ones, r["row_of"])
    assert np.array_equal(mi.f32(y1.cpu()), (k * xf).astype(np.float32))
    # gate-weighted combine vs the oracle
    gates = r["gates"]
    yp = torch.from_numpy(rng.standard_normal((T * k, d)).astype(np.float32)).to(tdt(dtype)).to(DEV)
    y = moe.moe_combine(yp, gates, r["row_of"])
    ypf = mi.f32(yp.cpu())
    g = gates.cpu().numpy()
    assert_close(mi.f32(y.cpu()), oracle.combine(ypf, g, ro), tol_for(dtype), "combine")
    # combine backward
    dy = c["dy"].to(DEV)
    dyp, dgates = moe.moe_combine_bwd(dy, yp, gates, r["row_of"])
    ref_dyp, ref_dg = oracle.combine_bwd(mi.f32(c["dy"]), ypf, g, ro)
    assert_close(mi.f32(dyp.cpu()), ref_dyp, tol_for(dtype), "dyp")
    assert_close(dgates.cpu().numpy(), ref_dg, 1e-4, "dgates")
    # route backward
    dls = moe.moe_route_bwd(gates, dgates)
    assert_close(dls.cpu().numpy(), oracle.route_bwd(g, dgates.cpu().numpy()), 1e-4, "dlogits")
    # permute backward with and without the router term
    dxp = yp
    dx0 = moe.moe_permute_bwd(dxp, r["row_of"])
    assert_close(mi.f32(dx0.cpu()), oracle.permute_bwd(ypf, ro), tol_for(dtype), "dx (rows)")
    wr = c["wr"].to(DEV)
    dx1 = moe.moe_permute_bwd(dxp, r["row_of"], r["topk_idx"], dls, wr)
    ref = oracle.permute_bwd(ypf, ro, r["topk_idx"].cpu().numpy(), dls.cpu().numpy(), mi.f32(c["wr"]))
    assert_close(mi.f32(dx1.cpu()), ref, tol_for(dtype), "dx (rows + router)")
    # router weight gradient
    dwr = moe.moe_router_wgrad(x, dls, r["src_tk"], r["offsets"], E)
    ref = oracle.router_wgrad(xf, dls.cpu().numpy(), r["topk_idx"].cpu().numpy(), E)
    assert_close(mi.f32(dwr.cpu()), ref, tol_for(dtype), "dW_r")


@pytest.mark.parametrize("dtype,T,d,E,k", [("bf16", 3000, 512, 16, 2), ("fp32", 1500, 256, 8, 4)])
def test_router_wgrad_skewed(moe, dtype, T, d, E, k):
    """One hot expert whose rows span many 256-row chunks, two empty experts,
    ragged chunk tails: against the oracle, and bit-identical on a repeat."""
    rng = np.random.default_rng(T + d)
    c = mi.layer_inputs(mi.config("tiny", T=T, d=d, E=E, k=k, dtype=dtype, x_std=1.0), with_weights=False)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:, 3] += 6.0  # nearly every token picks expert 3
    logits[:, [1, E - 1]] = -1e4  # never picked
    r = moe.moe_route(torch.from_numpy(logits).to(DEV), k)
    counts = r["counts"].cpu().numpy()
    assert counts[3] > 4 * 256 and counts[1] == 0 and counts[E - 1] == 0
    x = c["x"].to(DEV)
    dls = torch.from_numpy(rng.standard_normal((T, k)).astype(np.float32)).to(DEV)
    dwr = moe.moe_router_wgrad(x, dls, r["src_tk"], r["offsets"], E)
    again = moe.moe_router_wgrad(x, dls, r["src_tk"], r["offsets"], E)
    torch.cuda.synchronize()
    assert torch.equal(dwr, again)
    ref = oracle.router_wgrad(mi.f32(c["x"]), dls.cpu().numpy(), r["topk_idx"].cpu().numpy(), E)
    got = mi.f32(dwr.cpu())
    assert not got[:, 1].any() and not got[:, E - 1].any()
    assert_close(got, ref, tol_for(dtype), "dW_r (skewed)")


# ------------------------------------------------------------------ grouped FFN
FFN_CASES = [
    # dtype, d, F, counts
    ("fp32", 128, 256, [70, 0, 129, 33, 0, 64, 200, 16]),
    ("bf16", 128, 256, [70, 0, 129, 33, 0, 64, 200, 16]),
    ("bf16", 256, 384, [300, 1, 0, 257, 511, 40]),
    ("bf16", 512, 192, [0, 0, 1000, 3]),
    ("bf16", 192, 128, [5] * 40 + [0] * 8 + [300]),
    # few long groups: the weight gradients split K (fp32 partials, fixed-order sum)
    ("bf16", 256, 256, [4096]),
    ("bf16", 256, 384, [3000, 5, 0, 2500]),
    ("bf16", 128, 256, [2049]),
    # around the dgrads' 288-row tiles (256 rows plus a 32-row strip): strips
    # full, partly filled (257..287 rows) and absent, in first and second tiles
    ("bf16", 256, 256, [288, 289, 575, 576, 577, 270, 256, 32, 0, 544]),
    # many small experts: the tile schedulers' threads hold 2 and 4 experts each
    ("bf16", 128, 128, [(i * 37) % 23 for i in range(300)]),
    ("bf16", 128, 128, [(i * 13) % 7 for i in range(1000)]),
]


@pytest.mark.parametrize("dtype,d,F,counts", FFN_CASES)
def test_grouped_ffn(moe, dtype, d, F, counts):
    counts = np.array(counts)
    E, R = len(counts), int(counts.sum())
    inp = mi.rows_inputs(R, d, E, F, counts, seed=R, dtype=dtype)
    g = {k: inp[k].to(DEV) for k in ("xp", "dyp", "wg", "wu", "wd")}
    off = torch.from_numpy(inp["offsets"]).to(DEV)
    f = moe.moe_grouped_ffn_fwd(g["xp"], g["wg"], g["wu"], g["wd"], off)
    b = moe.moe_grouped_ffn_bwd(g["xp"], g["wg"], g["wu"], g["wd"], off, f["g"], f["u"], f["h"], g["dyp"])
    torch.cuda.synchronize()
    xp, dyp = mi.f32(inp["xp"]), mi.f32(inp["dyp"])
    wg, wu, wd = mi.f32(inp["wg"]), mi.f32(inp["wu"]), mi.f32(inp["wd"])
    rf = oracle.expert_fwd(xp, inp["offsets"], wg, wu, wd)
    rd = oracle.expert_dgrad(xp, dyp, inp["offsets"], wg, wu, wd)
    rw = oracle.expert_wgrad(xp, dyp, inp["offsets"], wg, wu, wd)
    tol = tol_for(dtype)
    for name, ref in [("g", rf["g"]), ("u", rf["u"]), ("h", rf["h"]), ("yp", rf["yp"])]:
        assert_close(mi.f32(f[name].cpu()), ref, tol, name)
    for name, ref in [("dg", rd["dg"]), ("du", rd["du"]), ("dxp", rd["dxp"])]:
        assert_close(mi.f32(b[name].cpu()), ref, tol, name)
    for name, ref in [("dw_gate", rw["dwg"]), ("dw_up", rw["dwu"]), ("dw_down", rw["dwd"])]:
        got = mi.f32(b[name].cpu())
        for e in range(E):
            assert_close(got[e], ref[e], tol, f"{name}[{e}] (count {counts[e]})")


def test_grouped_ffn_deterministic(moe):
    counts = np.array([300, 0, 77, 500, 123])
    E, R, d, F = 5, int(counts.sum()), 256, 256
    inp = mi.rows_inputs(R, d, E, F, counts, seed=1)
    g = {k: inp[k].to(DEV) for k in ("xp", "dyp", "wg", "wu", "wd")}
    off = torch.from_numpy(inp["offsets"]).to(DEV)
    outs = []
    for _ in range(2):
        f = moe.moe_grouped_ffn_fwd(g["xp"], g["wg"], g["wu"], g["wd"], off)
        b = moe.moe_grouped_ffn_bwd(g["xp"], g["wg"], g["wu"], g["wd"], off, f["g"], f["u"], f["h"], g["dyp"])
        outs.append({**{k: v.clone() for k, v in f.items()}, **{k: v.clone() for k, v in b.items()}})
    for k in outs[0]:
        assert torch.equal(outs[0][k], outs[1][k]), k
