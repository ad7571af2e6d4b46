"""Pins of the oracle's MXFP8 expert chain (MXFP8 grouped GEMMs named on the
first page, section 三; the expert is the SwiGLU FFN of the second page,
section 2.1).

The chain is a composition of the pinned MX codec and fp64 products, so its
pins check the composition: operands that MX represents exactly must give the
fp64 oracle's values (up to the stated bf16 rounding), and random operands
must stay within MXFP8's rounding bound of the fp64 oracle, which a dropped
term, a wrong expert, a transposed operand or a mis-placed scale would break
by far.
"""
import numpy as np

import oracle
from tolerance import rel_errors


def _bf16(a):
    return oracle._bf16_round(a)


def _ragged(seed, E, counts, d, F, grid=False):
    rng = np.random.default_rng(seed)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    if grid:
        # every block quantises exactly: values in {0, +-0.5, +-1, +-1.5, +-2}
        pick = lambda *s: rng.integers(-4, 5, size=s) * 0.5  # noqa: E731
        xp, wg, wu, wd = pick(R, d), pick(E, d, F), pick(E, d, F), pick(E, F, d)
        dyp = pick(R, d)
    else:
        xp = rng.standard_normal((R, d))
        wg = rng.standard_normal((E, d, F)) / np.sqrt(d)
        wu = rng.standard_normal((E, d, F)) / np.sqrt(d)
        wd = rng.standard_normal((E, F, d)) / np.sqrt(F)
        dyp = rng.standard_normal((R, d))
    f = lambda a: _bf16(a).astype(np.float32)  # noqa: E731 — bf16 inputs
    return offsets, f(xp), f(wg), f(wu), f(wd), f(dyp)


def test_grid_operands_are_lossless():
    for a in (np.arange(-4, 5) * 0.5,):
        m = np.tile(a, (2, 4))[:, :32]
        assert np.array_equal(oracle.mx_rows(m), m)
        assert np.array_equal(oracle.mx_cols(m.T.copy(), None), m.T)


def test_mx_fwd_exact_on_grid_operands():
    counts = [40, 0, 33, 64]
    offsets, xp, wg, wu, wd, _ = _ragged(11, 4, counts, 64, 96, grid=True)
    ref = oracle.expert_fwd(xp, offsets, wg, wu, wd)
    mx = oracle.mx_expert_fwd(xp, offsets, wg, wu, wd)
    assert np.array_equal(mx["g"], _bf16(ref["g"]))
    assert np.array_equal(mx["u"], _bf16(ref["u"]))
    assert np.array_equal(mx["h"], _bf16(mx["g"] / (1 + np.exp(-mx["g"])) * mx["u"]))


def test_mx_dgrad_exact_first_product_on_grid_operands():
    # with lossless dyp and Wd, dh is exact, so dg and du are the bf16
    # rounding of the fp64 SwiGLU backward evaluated at the chain's g, u
    counts = [40, 0, 33, 64]
    offsets, xp, wg, wu, wd, dyp = _ragged(12, 4, counts, 64, 96, grid=True)
    f = oracle.mx_expert_fwd(xp, offsets, wg, wu, wd)
    b = oracle.mx_expert_bwd(xp, dyp, offsets, wg, wu, wd, f["g"], f["u"], f["h"])
    dh = np.zeros_like(f["g"])
    for e in range(4):
        lo, hi = offsets[e], offsets[e + 1]
        dh[lo:hi] = dyp[lo:hi].astype(np.float64) @ wd[e].astype(np.float64).T
    s = 1 / (1 + np.exp(-f["g"]))
    assert np.array_equal(b["dg"], _bf16(dh * f["u"] * s * (1 + f["g"] * (1 - s))))
    assert np.array_equal(b["du"], _bf16(dh * f["g"] * s))


def test_mx_chain_within_rounding_bound_of_fp64():
    counts = [200, 0, 37, 129, 96]
    offsets, xp, wg, wu, wd, dyp = _ragged(13, 5, counts, 128, 256)
    ref = oracle.expert_fwd(xp, offsets, wg, wu, wd)
    mx = oracle.mx_expert_fwd(xp, offsets, wg, wu, wd)
    # E4M3 keeps 3 mantissa bits: each operand carries relative error <= 2^-4
    # (RMS about 2^-4/sqrt(3)); a product of two such operands stays near 4%
    # in L2 and every stage here is one or two products deep.
    for name, tol in (("g", 0.06), ("u", 0.06), ("yp", 0.09)):
        l2, _ = rel_errors(mx[name], ref[name])
        assert l2 < tol, (name, l2)
        assert l2 > 1e-3, (name, l2)  # the chain really quantises
    rd = oracle.expert_dgrad(xp, dyp, offsets, wg, wu, wd)
    rw = oracle.expert_wgrad(xp, dyp, offsets, wg, wu, wd)
    b = oracle.mx_expert_bwd(xp, dyp, offsets, wg, wu, wd, mx["g"], mx["u"], mx["h"])
    for name, r, tol in (("dg", rd["dg"], 0.12), ("du", rd["du"], 0.12), ("dxp", rd["dxp"], 0.14),
                         ("dwg", rw["dwg"], 0.14), ("dwu", rw["dwu"], 0.14), ("dwd", rw["dwd"], 0.12)):
        l2, _ = rel_errors(b[name], r)
        assert l2 < tol, (name, l2)
    # an expert with no rows has zero weight gradients
    assert not np.any(b["dwg"][1]) and not np.any(b["dwd"][1])


def test_mx_chain_detects_planted_transpose():
    # the bound above is tight enough to see a transposed weight
    counts = [64, 64]
    offsets, xp, wg, wu, wd, _ = _ragged(14, 2, counts, 64, 64)
    ref = oracle.expert_fwd(xp, offsets, wg, wu, wd)
    wg_t = np.ascontiguousarray(np.transpose(wg, (0, 2, 1)))
    bad = oracle.mx_expert_fwd(xp, offsets, wg_t, wu, wd)
    assert rel_errors(bad["g"], ref["g"])[0] > 0.5


def test_sampled_rows_and_elements_match_full_chain():
    counts = [70, 0, 33, 129]
    offsets, xp, wg, wu, wd, dyp = _ragged(15, 4, counts, 64, 128)
    f = oracle.mx_expert_fwd(xp, offsets, wg, wu, wd)
    b = oracle.mx_expert_bwd(xp, dyp, offsets, wg, wu, wd, f["g"], f["u"], f["h"])
    rows = np.array([0, 69, 70, 102, 103, 231])
    s = oracle.mx_expert_rows(xp, dyp, offsets, wg, wu, wd, rows)
    for k in ("g", "u", "h", "yp"):
        np.testing.assert_allclose(s[k], f[k][rows], rtol=1e-12, atol=1e-12)
    for k in ("dg", "du", "dxp"):
        np.testing.assert_allclose(s[k], b[k][rows], rtol=1e-12, atol=1e-12)
    el = np.array([[0, 3, 5], [2, 63, 127], [3, 10, 0], [1, 4, 4]])
    for which, name in ((0, "dwg"), (1, "dwu")):
        got = oracle.mx_expert_wgrad_elems(xp, dyp, offsets, wg, wu, wd, which, el)
        want = b[name][el[:, 0], el[:, 1], el[:, 2]]
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    el2 = np.array([[0, 3, 5], [2, 127, 63], [3, 10, 0], [1, 4, 4]])
    got = oracle.mx_expert_wgrad_elems(xp, dyp, offsets, wg, wu, wd, 2, el2)
    np.testing.assert_allclose(got, b["dwd"][el2[:, 0], el2[:, 1], el2[:, 2]], rtol=1e-12, atol=1e-12)
