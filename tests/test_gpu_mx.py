"""GPU parity of the MXFP8 path (E4M3 elements, 32-element blocks with e8m0
scales; MXFP8 grouped GEMMs are named on the first page, section 三) against
the oracle's MX codec and MX expert chain.

Quantisation is integer/byte work: codes and scale bytes bit-exact.  The MX
GEMMs compare with the oracle's chain on the same quantised operands within
6e-2 (the two differ only by fp32 accumulation order, which can move a bf16
rounding of g, u, dg or du by one unit and, rarely, the E4M3 code of the
re-quantised h, dg or du)."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from tolerance import assert_close

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 6e-2


@pytest.fixture(scope="module")
def moe():
    import routing_grouped_expert_softmax_amd as m
    m.context(0)
    return m


def _bf16_tensor(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def _special_matrix(rows, cols, seed):
    """bf16 values that reach every branch of the codec: ordinary normals,
    blocks scaled to tiny (subnormal bf16) and huge magnitudes, all-zero
    blocks, signed zeros, exact E4M3 rounding ties, saturating values and NaN
    elements (code 0x7f; the block scale comes from the other elements)."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((rows, cols)).astype(np.float32)
    nblk = cols // 32
    kinds = rng.integers(0, 8, size=(rows, nblk))
    for r in range(rows):
        for b in range(nblk):
            blk = a[r, 32 * b:32 * b + 32]
            k = kinds[r, b]
            if k == 1:
                blk *= np.float32(2.0 ** -128)
            elif k == 2:
                blk *= np.float32(2.0 ** 100)
            elif k == 3:
                blk[:] = 0.0
                blk[::3] = -0.0
            elif k == 4:
                # amax 1 (scale 2^-8): values on and halfway between E4M3 steps
                blk[:] = rng.integers(-64, 65, size=32) / 64.0
                blk[0] = 1.0
            elif k == 5:
                blk[:] = rng.integers(-1000, 1001, size=32) * np.float32(2.0 ** -20)
            elif k == 6:
                blk[rng.integers(0, 32, size=2)] = np.nan
                blk[rng.integers(0, 32)] = np.copysign(np.float32(np.nan), np.float32(-1.0))
    return mi.f32(_bf16_tensor(a))


@pytest.mark.parametrize("rows,cols,seed", [(1, 32, 0), (257, 96, 1), (1000, 4096, 2)])
def test_mx_quantize_rows_bitexact(moe, rows, cols, seed):
    a = _special_matrix(rows, cols, seed)
    codes, scales = moe.moe_mx_quantize(_bf16_tensor(a).to(DEV), 0)
    torch.cuda.synchronize()
    rc, rs = oracle.mx_quantize(a, axis=0)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def _cols_layout_check(a, offsets, codes, scales):
    """Map the oracle's group-major column blocks onto the library's
    transposed, 128-padded layout and compare byte for byte."""
    rc, rs = oracle.mx_quantize(a, axis=1, offsets=offsets)
    rows, cols = a.shape
    codes, scales = codes.cpu().numpy(), scales.cpu().numpy()
    kbase, blk = 0, 0
    for gi in range(len(offsets) - 1):
        lo, hi = int(offsets[gi]), int(offsets[gi + 1])
        n = hi - lo
        padded = (n + 127) // 128 * 128
        assert np.array_equal(codes[:, kbase:kbase + n], rc[lo:hi].T), f"group {gi} codes"
        assert not np.any(codes[:, kbase + n:kbase + padded]), f"group {gi} padding"
        nb = (n + 31) // 32
        assert np.array_equal(scales[:, kbase // 32:kbase // 32 + nb], rs[blk:blk + nb].T), f"group {gi} scales"
        assert not np.any(scales[:, kbase // 32 + nb:(kbase + padded) // 32]), f"group {gi} pad scales"
        kbase += padded
        blk += nb


@pytest.mark.parametrize("counts,cols,seed", [([300], 64, 0), ([40, 0, 129, 1, 256, 77], 96, 1),
                                             ([0, 0, 5], 32, 2), ([1000, 3000, 17], 256, 3)])
def test_mx_quantize_cols_groups_bitexact(moe, counts, cols, seed):
    counts = np.array(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = int(offsets[-1])
    # column blocks: build row-block specials on the transpose
    a = np.ascontiguousarray(_special_matrix(cols, (rows + 31) // 32 * 32, seed)[:, :rows].T)
    off = torch.from_numpy(offsets).to(DEV)
    codes, scales = moe.moe_mx_quantize(_bf16_tensor(a).to(DEV), 1, off, len(counts))
    torch.cuda.synchronize()
    _cols_layout_check(a, offsets, codes, scales)


def test_mx_quantize_rejects_bad_arguments(moe):
    src = torch.zeros(64, 48, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(moe.MoeError):
        moe.moe_mx_quantize(src, 0)  # cols not a multiple of 32
    src = torch.zeros(64, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(moe.MoeError):
        moe.moe_mx_quantize(src, 2)


def _ffn_mx(moe, inp):
    g = {k: inp[k].to(DEV) for k in ("xp", "dyp", "wg", "wu", "wd")}
    off = torch.from_numpy(inp["offsets"]).to(DEV)
    f = moe.moe_grouped_ffn_fwd(g["xp"], g["wg"], g["wu"], g["wd"], off, mxfp8=True)
    b = moe.moe_grouped_ffn_bwd(g["xp"], g["wg"], g["wu"], g["wd"], off, f["g"], f["u"], f["h"], g["dyp"],
                                mxfp8=True)
    torch.cuda.synchronize()
    return f, b


@pytest.mark.parametrize("d,F,counts", [(256, 384, [300, 0, 129, 517]), (128, 128, [31, 1, 128, 256, 0]),
                                        (512, 256, [1000]),
                                        (128, 128, [(i * 37) % 23 for i in range(300)])])
def test_mx_grouped_ffn(moe, d, F, counts):
    counts = np.array(counts)
    E, R = len(counts), int(counts.sum())
    inp = mi.rows_inputs(R, d, E, F, counts, seed=R + 7)
    f, b = _ffn_mx(moe, inp)
    xp, dyp = mi.f32(inp["xp"]), mi.f32(inp["dyp"])
    wg, wu, wd = mi.f32(inp["wg"]), mi.f32(inp["wu"]), mi.f32(inp["wd"])
    off = inp["offsets"]
    rf = oracle.mx_expert_fwd(xp, off, wg, wu, wd)
    rb = oracle.mx_expert_bwd(xp, dyp, off, wg, wu, wd, rf["g"], rf["u"], rf["h"])
    for name in ("g", "u", "h", "yp"):
        assert_close(mi.f32(f[name].cpu()), rf[name], TOL, name)
    for name in ("dg", "du", "dxp"):
        assert_close(mi.f32(b[name].cpu()), rb[name], TOL, name)
    for name, key in (("dw_gate", "dwg"), ("dw_up", "dwu"), ("dw_down", "dwd")):
        got = mi.f32(b[name].cpu())
        for e in range(E):
            assert_close(got[e], rb[key][e], TOL, f"{name}[{e}] (count {counts[e]})")


def test_mx_grouped_ffn_deterministic(moe):
    counts = np.array([300, 0, 77, 500])
    inp = mi.rows_inputs(int(counts.sum()), 256, 4, 256, counts, seed=5)
    o1 = _ffn_mx(moe, inp)
    o2 = _ffn_mx(moe, inp)
    for a, b in zip(o1, o2):
        for k in a:
            assert torch.equal(a[k], b[k]), k


@pytest.mark.slow
def test_mx_full_size_sampled(moe):
    """The pre-routed MXFP8 workload at full size (65536 rows, d 4096, 16
    experts of F 1536, Zipf-skewed counts): sampled rows of every per-row
    output and sampled weight-gradient elements against the oracle."""
    inp = mi.mx_inputs()
    cfg = mi.MX_CONFIG
    off = inp["offsets"]
    counts = np.diff(off)
    f, b = _ffn_mx(moe, inp)
    xp, dyp = mi.f32(inp["xp"]), mi.f32(inp["dyp"])
    wg, wu, wd = mi.f32(inp["wg"]), mi.f32(inp["wu"]), mi.f32(inp["wd"])
    rng = np.random.default_rng(123)
    # first and last row of every non-empty expert plus random rows
    rows = sorted({int(r) for e in range(cfg.E) if counts[e]
                   for r in (off[e], off[e + 1] - 1)} | set(rng.integers(0, cfg.rows, 16).tolist()))
    rows = np.array(rows)
    ref = oracle.mx_expert_rows(xp, dyp, off, wg, wu, wd, rows)
    for name, t in (("g", f["g"]), ("u", f["u"]), ("h", f["h"]), ("yp", f["yp"]),
                    ("dg", b["dg"]), ("du", b["du"]), ("dxp", b["dxp"])):
        assert_close(mi.f32(t[torch.from_numpy(rows).to(DEV)].cpu()), ref[name], TOL, name)
    # weight gradients: the two smallest experts and one mid-sized one
    order = np.argsort(counts)
    experts = [int(order[0]), int(order[1]), int(order[len(order) // 2])]
    for which, name, shp in ((0, "dw_gate", (cfg.d, cfg.F)), (1, "dw_up", (cfg.d, cfg.F)),
                             (2, "dw_down", (cfg.F, cfg.d))):
        el = np.array([[e, rng.integers(0, shp[0]), rng.integers(0, shp[1])] for e in experts for _ in range(4)])
        want = oracle.mx_expert_wgrad_elems(xp, dyp, off, wg, wu, wd, which, el)
        got = mi.f32(b[name][el[:, 0], el[:, 1], el[:, 2]].cpu())
        assert_close(got, want, TOL, name)
