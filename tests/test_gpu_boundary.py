"""Host-side validation of the C ABI on a GPU context: a call whose output
arrays overlap is rejected with MOE_ERR_INVALID_ARGUMENT before anything is
enqueued, and outputs that only touch (one ends where the next begins) are
accepted.  Calls go straight through ctypes with raw device addresses, the
way a C caller would make them."""
import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
INVALID = 1


@pytest.fixture(scope="module")
def moe():
    import routing_grouped_expert_softmax_amd as m
    m.context(0)
    return m


class Arena:
    """One device buffer; p(off) is the device address at byte offset off."""

    def __init__(self, nbytes):
        self.t = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
        self.base = self.t.data_ptr()

    def p(self, off):
        return ctypes.c_void_p(self.base + off)


def _vp(t):
    return ctypes.c_void_p(t.data_ptr())


def _err(moe):
    return moe.lib().moe_last_error(moe.context(0).handle).decode()


def test_route_outputs(moe):
    L, c = moe.lib(), moe.context(0)
    T, E, k = 64, 8, 2
    c.ensure_workspace(T, 64, E, k, moe.MOE_BF16)
    c.bind_stream()
    logits = torch.randn(T, E, device=DEV)
    a = Arena(1 << 16)
    tk = T * k * 4  # 512 bytes
    # gates overlaps topk_idx
    st = L.moe_route(c.handle, _vp(logits), T, E, k, a.p(0), a.p(tk - 16), a.p(4096), a.p(8192),
                     a.p(12288), a.p(16384))
    assert st == INVALID and "overlap" in _err(moe)
    # offsets overlaps counts' last entry
    st = L.moe_route(c.handle, _vp(logits), T, E, k, a.p(0), a.p(1024), a.p(4096), a.p(4096 + 16),
                     a.p(12288), a.p(16384))
    assert st == INVALID and "counts" in _err(moe) and "offsets" in _err(moe)
    # touching outputs are fine, and the result equals the binding's routing
    st = L.moe_route(c.handle, _vp(logits), T, E, k, a.p(0), a.p(tk), a.p(2 * tk), a.p(2 * tk + 32),
                     a.p(2 * tk + 80), a.p(3 * tk + 80))
    assert st == 0, _err(moe)
    ref = moe.moe_route(logits, k)
    torch.cuda.synchronize()
    got = a.t[:tk].view(torch.int32).reshape(T, k)
    assert torch.equal(got, ref["topk_idx"])


def test_other_calls_reject_overlapping_outputs(moe):
    L, c = moe.lib(), moe.context(0)
    c.bind_stream()
    h = c.handle
    T, d, E, k, F = 64, 128, 4, 2, 128
    R = T * k
    bf = dict(dtype=torch.bfloat16, device=DEV)
    x = torch.zeros(T, d, **bf)
    xp = torch.zeros(R, d, **bf)
    wg = torch.zeros(E, d, F, **bf)
    wd = torch.zeros(E, F, d, **bf)
    rf = torch.zeros(R, F, **bf)
    gates = torch.zeros(T, k, device=DEV)
    row_of = torch.arange(R, dtype=torch.int32, device=DEV).reshape(T, k)
    offsets = torch.tensor([0, R, R, R, R], dtype=torch.int32, device=DEV)
    counts = torch.zeros(E, dtype=torch.int32, device=DEV)
    a = Arena(8 << 20)
    BF16 = moe.MOE_BF16
    cases = {
        "moe_combine_bwd": lambda: L.moe_combine_bwd(
            h, _vp(x), _vp(xp), _vp(gates), _vp(row_of), T, d, k, BF16, a.p(0), a.p(1024)),
        "moe_route_bwd_rows": lambda: L.moe_route_bwd_rows(
            h, _vp(gates), _vp(gates), _vp(row_of), T, k, a.p(0), a.p(256)),
        "moe_grouped_ffn_fwd": lambda: L.moe_grouped_ffn_fwd(
            h, _vp(xp), _vp(wg), _vp(wg), _vp(wd), _vp(offsets), E, R, d, F, BF16,
            a.p(0), a.p(1 << 20), a.p(1 << 20), a.p(2 << 20)),
        "moe_grouped_ffn_bwd": lambda: L.moe_grouped_ffn_bwd(
            h, _vp(xp), _vp(wg), _vp(wg), _vp(wd), _vp(offsets), _vp(rf), _vp(rf), _vp(rf), _vp(xp),
            E, R, d, F, BF16, a.p(0), a.p(1 << 20), a.p(2 << 20), a.p(3 << 20), a.p(3 << 20),
            a.p(5 << 20)),
        "moe_permute_mx": lambda: L.moe_permute_mx(
            h, _vp(x), _vp(row_of), T, d, k, a.p(0), a.p(1 << 20), a.p((1 << 20) + 64)),
        "moe_mx_quantize": lambda: L.moe_mx_quantize(
            h, _vp(xp), R, d, 0, None, 1, a.p(0), a.p(R * d - 32), 0),
        "moe_route_stats": lambda: L.moe_route_stats(
            h, _vp(gates), _vp(counts), T, E, k, ctypes.c_float(0.01), a.p(0), a.p(16), a.p(32),
            a.p(44)),
    }
    for name, call in cases.items():
        st = call()
        assert st == INVALID, (name, st)
        assert "overlap" in _err(moe), (name, _err(moe))
    torch.cuda.synchronize()
    assert not a.t.any()  # nothing was enqueued
