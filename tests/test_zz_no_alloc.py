"""moe_route_noalloc (the routing call for callers that cannot allocate: its
block counts live in a static device array instead of the registered
workspace) against moe_route through the C ABI: bit-identical outputs on two
calls in a row, the second smaller, in a context with no workspace of its
own; shapes past the array's size are rejected on the host."""
import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def moe():
    import routing_grouped_expert_softmax_amd as m
    return m


def _outs(T, E, k):
    i32 = dict(dtype=torch.int32, device=DEV)
    # poisoned, so an unwritten entry cannot pass
    return dict(topk_idx=torch.full((T, k), -7, **i32),
                gates=torch.full((T, k), float("nan"), device=DEV),
                counts=torch.full((E,), -7, **i32), offsets=torch.full((E + 1,), -7, **i32),
                row_of=torch.full((T, k), -7, **i32), src_tk=torch.full((max(T * k, 1),), -7, **i32))


def _noalloc(moe, h, logits, k, out):
    T, E = logits.shape
    v = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    return moe.lib().moe_route_noalloc(h, v(logits), T, E, k, v(out["topk_idx"]), v(out["gates"]),
                                       v(out["counts"]), v(out["offsets"]), v(out["row_of"]),
                                       v(out["src_tk"]))


def test_noalloc_route_matches_route(moe):
    L = moe.lib()
    h = ctypes.c_void_p()
    assert L.moe_create(0, None, ctypes.byref(h)) == 0  # a context with no workspace
    s = torch.cuda.current_stream()
    assert L.moe_set_stream(h, ctypes.c_void_p(s.cuda_stream)) == 0
    try:
        rng = np.random.default_rng(41)
        for T, E, k in [(16384, 128, 4), (3001, 96, 8)]:  # the second call is smaller
            logits = torch.from_numpy(rng.standard_normal((T, E)).astype(np.float32)).to(DEV)
            got = _outs(T, E, k)
            assert _noalloc(moe, h, logits, k, got) == 0, L.moe_last_error(h)
            torch.cuda.synchronize()
            ref = moe.moe_route(logits, k)
            torch.cuda.synchronize()
            for key in ref:
                assert torch.equal(got[key], ref[key]), (T, key)
        # E * ceil(T / 64) past the 2^20-entry array: rejected before any launch
        big = torch.empty(65600, 1024, device=DEV)
        out = _outs(65600, 1024, 1)
        assert _noalloc(moe, h, big, 1, out) == 2 and b"scratch" in L.moe_last_error(h)
        assert int(out["counts"][0]) == -7  # nothing ran
    finally:
        L.moe_destroy(h)
