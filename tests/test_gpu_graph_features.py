"""The extended layer — MXFP8 experts with quantise-on-permute, a shared
expert (whose weight gradients split K) and activation recompute — issues
no host synchronisation and no allocation inside a step: it is captured in
one HIP graph, and every replay reproduces the eager result bit for bit."""
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


@pytest.mark.parametrize("mx,T", [(True, 512), (False, 4096)])
def test_extended_layer_graph_replay(moe, mx, T):
    cfg = mi.config("tiny", dtype="bf16", T=T, d=256, E=16, k=4, F=256, x_std=1.0)
    inp = mi.layer_inputs(cfg)
    sw = mi.shared_expert_weights(cfg, 256)
    g = {k: inp[k].to(DEV) for k in ("x", "wr", "wg", "wu", "wd", "dy")}
    shared = tuple(sw[k].to(DEV) for k in ("wg_s", "wu_s", "wd_s"))
    buf = moe.alloc_layer(cfg.T, cfg.d, cfg.E, cfg.k, cfg.F, torch.bfloat16, DEV, mxfp8=mx, shared_F=256)

    def step():
        moe.layer_forward(g["x"], g["wr"], g["wg"], g["wu"], g["wd"], cfg.k, buf, mxfp8=mx, shared=shared)
        moe.layer_backward(g["dy"], g["x"], g["wr"], g["wg"], g["wu"], g["wd"], buf, mxfp8=mx, shared=shared,
                           recompute=True)

    step()  # eager: sizes every workspace before capture
    torch.cuda.synchronize()
    outs = lambda: {"y": buf.y, "dx": buf.dx, "dwr": buf.dw_router, "dwg": buf.bwd["dw_gate"],  # noqa: E731
                    "dwd": buf.bwd["dw_down"], "s_dwg": buf.shared["bwd"]["dw_gate"],
                    "s_dwd": buf.shared["bwd"]["dw_down"]}
    eager = {k: v.clone() for k, v in outs().items()}
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs().values():
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in outs().items():
            assert torch.equal(v, eager[k]), (rep, k)
