"""Activation recompute (the pages trade activation memory for throughput by
recomputing in the backward; [P1] 四): the backward that re-permutes x and
recomputes g, u, h with the gate/up GEMM alone is checked two ways.

* Against the CPU oracle: every gradient of the recomputing backward (and the
  shared expert's) within the dtype's bound — fp32 1e-4, bf16 2e-2, MXFP8
  6e-2 — on the oracle's own chain for the same routing (MXFP8 both with
  MXFP8 and with bf16 weight gradients).
* Against the saving backward: bit-identical gradients, after the saved
  tensors are overwritten with NaN, so nothing stale can leak in.

The full-size uniform128 case is the one the benchmark's recompute leg times:
sampled tokens and weight-gradient elements against the oracle, and the
whole gradient set bit-identical to the saving backward."""
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


def _grads(buf):
    out = {"dx": buf.dx, "dw_router": buf.dw_router, "dgates": buf.dgates, "dlogits": buf.dlogits_sel}
    out.update({k: buf.bwd[k] for k in ("dw_gate", "dw_up", "dw_down", "dxp")})
    if buf.shared is not None:
        out.update({"s_" + k: buf.shared["bwd"][k] for k in ("dw_gate", "dw_up", "dw_down", "dxp")})
    return {k: v.clone() for k, v in out.items()}


def _setup(moe, cfg, inp, Fs, mx):
    """mx: False (bf16/fp32), True (MXFP8, every GEMM) or "bf16w" (MXFP8
    forward and data gradients, bf16 weight gradients)."""
    g = {k: inp[k].to(DEV) for k in ("x", "wr", "wg", "wu", "wd", "dy")}
    override = inp["logits"].to(DEV) if "logits" in inp else None
    shared, sw = None, None
    if Fs:
        sw = mi.shared_expert_weights(cfg, Fs)
        shared = tuple(sw[k].to(DEV) for k in ("wg_s", "wu_s", "wd_s"))
    dt = torch.float32 if cfg.dtype == "fp32" else torch.bfloat16
    mxf = bool(mx)
    buf = moe.alloc_layer(cfg.T, cfg.d, cfg.E, cfg.k, cfg.F, dt, DEV, mxfp8=mxf, shared_F=Fs)

    def fwd():
        moe.layer_forward(g["x"], g["wr"], g["wg"], g["wu"], g["wd"], cfg.k, buf, override,
                          mxfp8=mxf, shared=shared)

    def bwd(recompute):
        moe.layer_backward(g["dy"], g["x"], g["wr"], g["wg"], g["wu"], g["wd"], buf, mxfp8=mxf,
                           shared=shared, recompute=recompute, mx_wgrad=mx != "bf16w")
    return buf, fwd, bwd, sw


def _clobber(buf):
    """Overwrite every tensor the forward saves for a non-recomputing backward."""
    ts = [buf.xp, buf.ffn["g"], buf.ffn["u"], buf.ffn["h"]]
    if buf.shared is not None:
        ts += [buf.shared["ffn"][k] for k in ("g", "u", "h")]
    for t in ts:
        t.fill_(float("nan"))


def _oracle_grads(cfg, inp, r, sw, mx):
    """The oracle's gradients of the layer (+ shared expert) for routing r:
    dx, dgates, dlogits, dW_r, the expert weight gradients and the shared
    expert's.  bf16/fp32: the plain fp64 definition; MXFP8: the oracle's MX
    chain (each GEMM operand quantised where the GPU quantises it; with
    mx == "bf16w" the weight gradients from the bf16 operands)."""
    x, wr, dy = mi.f32(inp["x"]), mi.f32(inp["wr"]), mi.f32(inp["dy"])
    wg, wu, wd = mi.f32(inp["wg"]), mi.f32(inp["wu"]), mi.f32(inp["wd"])
    ws = [mi.f32(sw[k]) for k in ("wg_s", "wu_s", "wd_s")] if sw is not None else None
    out = {}
    if not mx:
        b = oracle.layer_bwd(x, wr, r["topk_idx"], r["gates"], dy, wg, wu, wd)
        out.update(dx=b["dx"], dgates=b["dgates"], dlogits=b["dlogits_sel"], dw_router=b["dwr"],
                   dw_gate=b["dwg"], dw_up=b["dwu"], dw_down=b["dwd"])
        if ws is not None:
            sb = oracle.shared_expert_bwd(x, dy, *ws)
            out["dx"] = out["dx"] + sb["dx"]
            out.update(s_dw_gate=sb["dwg"], s_dw_up=sb["dwu"], s_dw_down=sb["dwd"])
        return out
    xp = oracle.permute(x, r["row_of"])
    fw = oracle.mx_expert_fwd(xp, r["offsets"], wg, wu, wd)
    dyp, dgates = oracle.combine_bwd(dy, fw["yp"], r["gates"], r["row_of"])
    dls = oracle.route_bwd(r["gates"], dgates)
    wgrad = "bf16" if mx == "bf16w" else "mx"
    bw = oracle.mx_expert_bwd(xp, oracle._bf16_round(dyp), r["offsets"], wg, wu, wd, fw["g"], fw["u"], fw["h"],
                              wgrad=wgrad)
    dx = oracle.permute_bwd(bw["dxp"], r["row_of"], r["topk_idx"], dls, wr)
    out.update(dgates=dgates, dlogits=dls, dw_router=oracle.router_wgrad(x, dls, r["topk_idx"], cfg.E),
               dw_gate=bw["dwg"], dw_up=bw["dwu"], dw_down=bw["dwd"])
    if ws is not None:
        one = np.array([0, cfg.T], dtype=np.int32)
        sf = oracle.mx_expert_fwd(x, one, *ws)
        sb = oracle.mx_expert_bwd(x, dy, one, *ws, sf["g"], sf["u"], sf["h"], wgrad=wgrad)
        dx = dx + sb["dxp"]
        out.update(s_dw_gate=sb["dwg"], s_dw_up=sb["dwu"], s_dw_down=sb["dwd"])
    out["dx"] = dx
    return out


CASES = [
    ("tiny", {}, 0, False),
    ("tiny", dict(dtype="bf16", T=700, E=16, k=4, x_std=1.0, routing="uniform"), 0, False),
    ("tiny", dict(dtype="bf16", T=1000, d=256, E=8, k=2, F=384, x_std=1.0, routing="zipf", n_dead=2), 256, False),
    ("tiny", dict(dtype="bf16", T=512, d=256, E=8, k=2, F=256, x_std=1.0), 256, True),
    ("tiny", dict(dtype="bf16", T=640, d=256, E=8, k=2, F=256, x_std=1.0, routing="zipf", n_dead=1), 256,
     "bf16w")]


@pytest.mark.parametrize("name,over,Fs,mx", CASES)
def test_recompute_backward_matches_oracle(moe, name, over, Fs, mx):
    cfg = mi.config(name, **over)
    inp = mi.layer_inputs(cfg)
    buf, fwd, bwd, sw = _setup(moe, cfg, inp, Fs, mx)
    fwd()
    torch.cuda.synchronize()
    _clobber(buf)
    bwd(True)
    torch.cuda.synchronize()
    # the oracle routes the same fp32 scores the GPU routed
    src = inp["logits"].numpy() if "logits" in inp else buf.logits.cpu().numpy()
    r = oracle.route(src, cfg.k)
    for key in ("topk_idx", "counts", "offsets", "row_of"):
        assert np.array_equal(buf.route[key].cpu().numpy(), r[key]), key
    ref = _oracle_grads(cfg, inp, r, sw, mx)
    tol = 6e-2 if mx else (1e-4 if cfg.dtype == "fp32" else 2e-2)
    got = _grads(buf)
    for key in ("dx", "dgates", "dlogits", "dw_router"):
        assert_close(_f(got[key]), ref[key], tol, key)
    for key in ("dw_gate", "dw_up", "dw_down"):
        a = _f(got[key])
        for e in range(cfg.E):
            assert_close(a[e], ref[key][e], tol, f"{key}[{e}] (count {r['counts'][e]})")
        if Fs:
            assert_close(_f(got["s_" + key])[0], ref["s_" + key][0], tol, "shared " + key)


@pytest.mark.parametrize("name,over,Fs,mx", CASES)
def test_recompute_backward_is_bit_identical(moe, name, over, Fs, mx):
    cfg = mi.config(name, **over)
    inp = mi.layer_inputs(cfg)
    buf, fwd, bwd, _ = _setup(moe, cfg, inp, Fs, mx)
    fwd()
    bwd(False)
    torch.cuda.synchronize()
    ref = _grads(buf)
    saved = {k: buf.ffn[k].clone() for k in ("g", "u", "h")}
    fwd()
    torch.cuda.synchronize()
    _clobber(buf)
    bwd(True)
    torch.cuda.synchronize()
    got = _grads(buf)
    for k in ref:
        assert torch.equal(got[k], ref[k]), k
    for k in saved:  # the recomputed g, u, h equal the forward's
        assert torch.equal(buf.ffn[k], saved[k]), k
    assert moe.saved_activation_bytes(buf, recompute=True) < moe.saved_activation_bytes(buf)


@pytest.mark.slow
def test_recompute_full_size_sampled(moe):
    """uniform128 (T=16384, d=2048, E=128, top-4, d_ff=1024, bf16) with
    recompute, launched as the benchmark's recompute leg: every gradient
    bit-identical to the saving backward; dx and dgates of sampled tokens and
    sampled weight-gradient elements against the oracle."""
    cfg = mi.config("uniform128")
    inp = mi.layer_inputs(cfg)
    buf, fwd, bwd, _ = _setup(moe, cfg, inp, 0, False)
    fwd()
    bwd(False)
    torch.cuda.synchronize()
    ref_gpu = _grads(buf)
    fwd()
    torch.cuda.synchronize()
    _clobber(buf)
    bwd(True)
    torch.cuda.synchronize()
    got = _grads(buf)
    for k in ref_gpu:
        assert torch.equal(got[k], ref_gpu[k]), k
    del ref_gpu
    r = oracle.route(inp["logits"].numpy(), cfg.k, "f32")
    for key in ("topk_idx", "counts", "offsets", "row_of", "src_tk"):
        assert np.array_equal(buf.route[key].cpu().numpy(), r[key]), key
    x, wr, dy = mi.f32(inp["x"]), mi.f32(inp["wr"]), mi.f32(inp["dy"])
    wg, wu, wd = mi.f32(inp["wg"]), mi.f32(inp["wu"]), mi.f32(inp["wd"])
    rng = np.random.default_rng(77)
    tok = np.unique(np.concatenate([[0, cfg.T - 1], rng.choice(cfg.T, 32, replace=False)]))
    b = oracle.layer_bwd(x[tok], wr, r["topk_idx"][tok], r["gates"][tok], dy[tok], wg, wu, wd)
    assert_close(_f(got["dx"])[tok], b["dx"], 2e-2, "dx (sampled tokens)")
    assert_close(_f(got["dgates"])[tok], b["dgates"], 2e-2, "dgates (sampled tokens)")
    src = r["src_tk"]
    xp = x[src // cfg.k]
    dyp = (r["gates"].reshape(-1)[src][:, None] * dy[src // cfg.k]).astype(np.float32)
    experts = np.unique(rng.choice(cfg.E, 4, replace=False))
    for which, name_, shp in [(0, "dw_gate", (cfg.d, cfg.F)), (1, "dw_up", (cfg.d, cfg.F)),
                              (2, "dw_down", (cfg.F, cfg.d))]:
        el = np.stack([np.repeat(experts, 6), rng.integers(0, shp[0], 6 * len(experts)),
                       rng.integers(0, shp[1], 6 * len(experts))], 1)
        ref = oracle.expert_wgrad_elems(xp, dyp, r["offsets"], wg, wu, wd, which, el)
        a = _f(got[name_])[el[:, 0], el[:, 1], el[:, 2]]
        assert_close(a, ref, 2e-2, f"{name_} (sampled elements)")
