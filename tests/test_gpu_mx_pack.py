"""GPU parity of the one-read MXFP8 quantisation (an operand that a
data-gradient GEMM and a weight-gradient GEMM both read, quantised along each
one's K from a single read; MXFP8 is named on the first page, section 三) and
of the weight pack (the expert weights quantised once per step, in both
layouts, for the forward and the backward).

* moe_mx_quantize_both: codes and scale bytes bit-exact against the oracle's
  MX codec along both axes, on the codec's special values (subnormal and
  huge blocks, zero blocks, rounding ties, saturation, NaN) and ragged
  groups (empty ones included), and equal to the single-axis calls.
* The weight pack: the MXFP8 forward and backward that read it give the same
  outputs, bit for bit, as the calls that quantise the bf16 weights
  themselves, which tests/test_gpu_mx.py compares with the oracle's MX chain;
  the layer tests (tests/test_gpu_mx_layer.py, the MXFP8 recompute case)
  run the pack path against the oracle end to end."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from test_gpu_mx import _bf16_tensor, _cols_layout_check, _special_matrix

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def moe():
    import routing_grouped_expert_softmax_amd as m
    m.context(0)
    return m


BOTH_CASES = [([300], 64, 0, "rows"), ([40, 0, 129, 1, 256, 77], 96, 1, "cols"),
              ([0, 0, 5], 32, 2, "rows"), ([1000, 3000, 17], 256, 3, "cols"), ([128, 128], 4096, 4, "rows")]


@pytest.mark.parametrize("counts,cols,seed,special", BOTH_CASES)
def test_mx_quantize_both_bitexact(moe, counts, cols, seed, special):
    counts = np.array(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = int(offsets[-1])
    if special == "rows":  # special 32-blocks along the rows
        a = _special_matrix(rows, cols, seed)
    else:  # along the columns: built on the transpose
        a = np.ascontiguousarray(_special_matrix(cols, (rows + 31) // 32 * 32, seed)[:, :rows].T)
    src = _bf16_tensor(a).to(DEV)
    off = torch.from_numpy(offsets).to(DEV)
    cc, cs, rc, rs = moe.moe_mx_quantize_both(src, off, len(counts))
    torch.cuda.synchronize()
    orc, ors = oracle.mx_quantize(a, axis=0)
    assert np.array_equal(rs.cpu().numpy(), ors), "row scales"
    assert np.array_equal(rc.cpu().numpy(), orc), "row codes"
    _cols_layout_check(a, offsets, cc, cs)
    # and the same bytes as the two single-axis calls (column layout: the
    # written K positions; the buffer's slack past the last group is not)
    c1, s1 = moe.moe_mx_quantize(src, 1, off, len(counts))
    c0, s0 = moe.moe_mx_quantize(src, 0)
    torch.cuda.synchronize()
    kt = int(sum((n + 127) // 128 * 128 for n in counts))
    assert torch.equal(cc[:, :kt], c1[:, :kt]) and torch.equal(cs[:, :kt // 32], s1[:, :kt // 32])
    assert torch.equal(rc, c0) and torch.equal(rs, s0)


def test_mx_quantize_both_one_group_without_offsets(moe):
    a = _special_matrix(200, 128, 9)
    src = _bf16_tensor(a).to(DEV)
    cc, cs, rc, rs = moe.moe_mx_quantize_both(src)
    torch.cuda.synchronize()
    orc, ors = oracle.mx_quantize(a, axis=0)
    assert np.array_equal(rc.cpu().numpy(), orc) and np.array_equal(rs.cpu().numpy(), ors)
    _cols_layout_check(a, np.array([0, 200], dtype=np.int32), cc, cs)


PACK_CASES = [(256, 384, [300, 0, 129, 517]), (128, 128, [31, 1, 128, 256, 0]), (512, 256, [1000])]


@pytest.mark.parametrize("d,F,counts", PACK_CASES)
def test_weight_pack_ffn_is_bit_identical(moe, d, F, counts):
    counts = np.array(counts)
    E, R = len(counts), int(counts.sum())
    inp = mi.rows_inputs(R, d, E, F, counts, seed=R + 11)
    g = {k: inp[k].to(DEV) for k in ("xp", "dyp", "wg", "wu", "wd")}
    off = torch.from_numpy(inp["offsets"]).to(DEV)
    ref_f = moe.moe_grouped_ffn_fwd(g["xp"], g["wg"], g["wu"], g["wd"], off, mxfp8=True)
    ref_b = moe.moe_grouped_ffn_bwd(g["xp"], g["wg"], g["wu"], g["wd"], off, ref_f["g"], ref_f["u"], ref_f["h"],
                                    g["dyp"], mxfp8=True)
    pack = moe.moe_mx_quantize_weights(g["wg"], g["wu"], g["wd"])
    f_bf = moe.moe_grouped_ffn_fwd_mxp(pack, off, xp=g["xp"])
    xq, xs = moe.moe_mx_quantize(g["xp"], 0)
    f_q = moe.moe_grouped_ffn_fwd_mxp(pack, off, xp_codes=xq, xp_scales=xs)
    f_up = moe.moe_grouped_ffn_fwd_mxp(pack, off, xp=g["xp"], up_only=True)
    b = moe.moe_grouped_ffn_bwd_mxp(g["xp"], pack, off, ref_f["g"], ref_f["u"], ref_f["h"], g["dyp"])
    torch.cuda.synchronize()
    for name in ("g", "u", "h", "yp"):
        assert torch.equal(f_bf[name], ref_f[name]), name
        assert torch.equal(f_q[name], ref_f[name]), name + " (pre-quantised rows)"
    assert "yp" not in f_up
    for name in ("g", "u", "h"):
        assert torch.equal(f_up[name], ref_f[name]), name + " (gate/up alone)"
    for name in ref_b:
        assert torch.equal(b[name], ref_b[name]), name


def test_weight_pack_is_reused_and_requantised(moe):
    """A pack holds the weights it was made from: after the weights change,
    the forward reads the old codes until the pack is quantised again."""
    counts = np.array([200, 56])
    inp = mi.rows_inputs(256, 128, 2, 128, counts, seed=3)
    g = {k: inp[k].to(DEV) for k in ("xp", "wg", "wu", "wd")}
    off = torch.from_numpy(inp["offsets"]).to(DEV)
    pack = moe.moe_mx_quantize_weights(g["wg"], g["wu"], g["wd"])
    before = moe.moe_grouped_ffn_fwd_mxp(pack, off, xp=g["xp"])
    wg2 = (g["wg"].float() * 2).to(torch.bfloat16)
    stale = moe.moe_grouped_ffn_fwd_mxp(pack, off, xp=g["xp"])
    moe.moe_mx_quantize_weights(wg2, g["wu"], g["wd"], pack)
    fresh = moe.moe_grouped_ffn_fwd_mxp(pack, off, xp=g["xp"])
    ref = moe.moe_grouped_ffn_fwd(g["xp"], wg2, g["wu"], g["wd"], off, mxfp8=True)
    torch.cuda.synchronize()
    assert torch.equal(stale["yp"], before["yp"])
    for name in ("g", "u", "h", "yp"):
        assert torch.equal(fresh[name], ref[name]), name
    # doubling Wg doubles g exactly (power-of-two scale, same codes)
    assert torch.equal(fresh["g"].float(), before["g"].float() * 2)


def test_weight_pack_rejects_bad_arguments(moe):
    E, d, F = 2, 128, 128
    w = torch.zeros(E, d, F, dtype=torch.bfloat16, device=DEV)
    wd = torch.zeros(E, F, d, dtype=torch.bfloat16, device=DEV)
    n = moe.moe_mx_weight_pack_size(E, d, F)
    assert n >= 2 * 3 * E * d * F * (1 + 1 / 32)
    with pytest.raises(moe.MoeError):  # shape not a multiple of 128
        moe.moe_mx_weight_pack_size(E, 96, F)
    small = moe.MxWeightPack(torch.empty(n - 256, dtype=torch.uint8, device=DEV), E, d, F)
    with pytest.raises(moe.MoeError):  # too small
        moe.moe_mx_quantize_weights(w, w, wd, small)
    big = torch.empty(n + 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(moe.MoeError):  # not 256-byte aligned
        moe.moe_mx_quantize_weights(w, w, wd, moe.MxWeightPack(big[16:16 + n], E, d, F))
    with pytest.raises(moe.MoeError):  # pack made for another shape
        moe.moe_mx_quantize_weights(w, w, wd, moe.MxWeightPack(big[:n], E, d, 2 * F))
    pack = moe.moe_mx_quantize_weights(w, w, wd)
    xp = torch.zeros(64, d, dtype=torch.bfloat16, device=DEV)
    off = torch.tensor([0, 32, 64], dtype=torch.int32, device=DEV)
    xq, xs = moe.moe_mx_quantize(xp, 0)
    with pytest.raises(moe.MoeError):  # both bf16 rows and codes
        moe.moe_grouped_ffn_fwd_mxp(pack, off, xp=xp, xp_codes=xq, xp_scales=xs)
    torch.cuda.synchronize()
