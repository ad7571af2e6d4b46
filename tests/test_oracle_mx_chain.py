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


# ------------------------------------------------------------------ exact backward pins
# Operands for which every backward product of the chain is lossless along the
# axis the chain must quantise it on, and lossy along any other: powers of two
# (closed under products, so dh, dg, du stay on E4M3's grid) with scale
# structure the MX block axis must respect.
#   * Wg, Wu: row i of an expert's [d, F] matrix carries 2^(18 (i mod 3)), so
#     blocks along F (the dgrad's reduction axis) share one binade range,
#     while blocks along d would span 2^36 and flush their small entries.
#   * xp, h: expert e's rows carry 2^(18 e) and column j another
#     2^(18 (j mod 3)): blocks down a column that restart at each expert are
#     lossless; blocks that straddle two experts, or run along the row, flush.
#   * g = 64 everywhere: sigmoid(64) is exactly 1 in fp64, so dg = dh u and
#     du = 64 dh exactly (the SwiGLU backward's own formula is pinned above).
#   * dyp has one nonzero per row, so dh = dyp Wd^T is a single product.
_AXIS_D, _AXIS_F = 64, 96
_AXIS_COUNTS = [40, 0, 64, 37]


def _axis_operands(seed=21):
    rng = np.random.default_rng(seed)
    d, F, counts = _AXIS_D, _AXIS_F, _AXIS_COUNTS
    E = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    pw = lambda *s: rng.choice([-2.0, -1.0, -0.5, 0.5, 1.0, 2.0], size=s)  # noqa: E731
    expert = np.repeat(np.arange(E), counts)
    rowscale = np.ldexp(1.0, 18 * expert)[:, None]
    xp = pw(R, d) * rowscale * np.ldexp(1.0, 18 * (np.arange(d) % 3))[None, :]
    h = pw(R, F) * rowscale * np.ldexp(1.0, 18 * (np.arange(F) % 3))[None, :]
    wscale = np.ldexp(1.0, 18 * (np.arange(d) % 3))[None, :, None]
    wg, wu = pw(E, d, F) * wscale, pw(E, d, F) * wscale
    wd = pw(E, F, d) * (rng.random((E, F, d)) < 0.8)
    dyp = np.zeros((R, d))
    dyp[np.arange(R), rng.integers(0, d, R)] = pw(R)
    g = np.full((R, F), 64.0)
    u = pw(R, F)
    f32 = lambda a: a.astype(np.float32)  # noqa: E731 — exact: every value is a float32
    return offsets, f32(xp), f32(dyp), f32(wg), f32(wu), f32(wd), g, u, f32(h)


def _exact_bwd(offsets, xp, dyp, wg, wu, wd, u):
    """fp64 products of the unquantised operands (exact here: every sum is of
    powers of two within a few dozen binades)."""
    E = wg.shape[0]
    R, F = u.shape
    dh = np.zeros((R, F))
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        dh[lo:hi] = dyp[lo:hi].astype(np.float64) @ wd[e].astype(np.float64).T
    dg, du = dh * u, 64.0 * dh
    dxp = np.zeros((R, xp.shape[1]))
    dwg, dwu = np.zeros(wg.shape), np.zeros(wu.shape)
    dwd = np.zeros(wd.shape)
    return dh, dg, du, dxp, dwg, dwu, dwd


def _axis_pin(b, offsets, xp, dyp, wg, wu, wd, u, h):
    """Which outputs of the chain's backward equal the exact products."""
    _, dg, du, dxp, dwg, dwu, dwd = _exact_bwd(offsets, xp, dyp, wg, wu, wd, u)
    x64, h64, y64 = xp.astype(np.float64), h.astype(np.float64), dyp.astype(np.float64)
    for e in range(wg.shape[0]):
        lo, hi = offsets[e], offsets[e + 1]
        dxp[lo:hi] = dg[lo:hi] @ wg[e].astype(np.float64).T + du[lo:hi] @ wu[e].astype(np.float64).T
        dwg[e] = x64[lo:hi].T @ dg[lo:hi]
        dwu[e] = x64[lo:hi].T @ du[lo:hi]
        dwd[e] = h64[lo:hi].T @ y64[lo:hi]
    want = dict(dg=dg, du=du, dxp=dxp, dwg=dwg, dwu=dwu, dwd=dwd)
    return {k: bool(np.array_equal(b[k], want[k])) for k in want}


def test_axis_operands_are_lossless_only_on_the_chain_axes():
    offsets, xp, dyp, wg, wu, wd, g, u, h = _axis_operands()
    for w in (wg[0], wu[2]):
        assert np.array_equal(oracle.mx_rows(w), w)              # blocks along F
        assert not np.array_equal(oracle.mx_cols(w, None), w)    # blocks along d
    for a in (xp, h):
        assert np.array_equal(oracle.mx_cols(a, offsets), a)     # restart per expert
        assert not np.array_equal(oracle.mx_cols(a, None), a)    # straddling experts
        assert not np.array_equal(oracle.mx_rows(a), a)          # along the row


def test_mx_bwd_exact_on_axis_structured_operands():
    offsets, xp, dyp, wg, wu, wd, g, u, h = _axis_operands()
    b = oracle.mx_expert_bwd(xp, dyp, offsets, wg, wu, wd, g, u, h)
    ok = _axis_pin(b, offsets, xp, dyp, wg, wu, wd, u, h)
    assert all(ok.values()), ok
    assert np.any(b["dxp"]) and np.any(b["dwg"]) and np.any(b["dwd"])
    assert not np.any(b["dwg"][1]) and not np.any(b["dwd"][1])  # the empty expert


def test_mx_bwd_pin_detects_planted_wrong_axes(monkeypatch):
    """Each planted mistake in the chain's quantisation axes breaks the exact
    pin on the outputs it feeds."""
    offsets, xp, dyp, wg, wu, wd, g, u, h = _axis_operands()
    rows, cols = oracle.mx_rows, oracle.mx_cols
    d, F = _AXIS_D, _AXIS_F

    def run():
        b = oracle.mx_expert_bwd(xp, dyp, offsets, wg, wu, wd, g, u, h)
        return _axis_pin(b, offsets, xp, dyp, wg, wu, wd, u, h)

    # Wg^T / Wu^T of the dgrad quantised along d instead of F
    monkeypatch.setattr(oracle, "mx_rows", lambda a: cols(a, None) if a.shape == (d, F) else rows(a))
    ok = run()
    assert not ok["dxp"] and ok["dwg"] and ok["dwd"], ok
    monkeypatch.setattr(oracle, "mx_rows", rows)
    # weight-gradient column blocks that do not restart at expert boundaries
    monkeypatch.setattr(oracle, "mx_cols", lambda a, off: cols(a, None))
    ok = run()
    assert not ok["dwg"] and not ok["dwu"] and not ok["dwd"] and ok["dxp"], ok
    # weight-gradient operands blocked along their rows instead of down columns
    monkeypatch.setattr(oracle, "mx_cols", lambda a, off: rows(a) if off is not None else cols(a, off))
    ok = run()
    assert not ok["dwg"] and not ok["dwu"] and not ok["dwd"] and ok["dxp"], ok


def _brute_wgrads(offsets, xp, dyp, dg, du, h):
    """Weight gradients by triple loops over the bf16 operands (fp64 sums)."""
    E = len(offsets) - 1
    R, d = xp.shape
    F = dg.shape[1]
    dwg = np.zeros((E, d, F))
    dwu = np.zeros((E, d, F))
    dwd = np.zeros((E, F, d))
    for e in range(E):
        for r in range(int(offsets[e]), int(offsets[e + 1])):
            for a in range(d):
                for b in range(F):
                    dwg[e, a, b] += float(xp[r, a]) * float(dg[r, b])
                    dwu[e, a, b] += float(xp[r, a]) * float(du[r, b])
            for a in range(F):
                for b in range(d):
                    dwd[e, a, b] += float(h[r, a]) * float(dyp[r, b])
    return dwg, dwu, dwd


def _bf16_wgrad_case():
    counts = [5, 0, 9, 3]
    offsets, xp, wg, wu, wd, dyp = _ragged(23, 4, counts, 32, 32)
    fw = oracle.mx_expert_fwd(xp, offsets, wg, wu, wd)
    return offsets, xp, dyp, wg, wu, wd, fw


def test_mx_bwd_bf16_wgrad_brute_force():
    """wgrad='bf16': the data gradients are the all-MXFP8 chain's, bit for
    bit; the weight gradients are the exact products of the bf16 operands
    (checked by loops), and differ from the MX weight gradients."""
    offsets, xp, dyp, wg, wu, wd, fw = _bf16_wgrad_case()
    mx = oracle.mx_expert_bwd(xp, dyp, offsets, wg, wu, wd, fw["g"], fw["u"], fw["h"])
    bb = oracle.mx_expert_bwd(xp, dyp, offsets, wg, wu, wd, fw["g"], fw["u"], fw["h"], wgrad="bf16")
    for k in ("dg", "du", "dxp"):
        assert np.array_equal(bb[k], mx[k]), k
    dwg, dwu, dwd = _brute_wgrads(offsets, xp, dyp, bb["dg"], bb["du"], fw["h"])
    for k, want in (("dwg", dwg), ("dwu", dwu), ("dwd", dwd)):
        np.testing.assert_allclose(bb[k], want, rtol=1e-12, atol=1e-12, err_msg=k)
        assert not np.array_equal(bb[k], mx[k]), k
    assert not np.any(bb["dwg"][1]) and not np.any(bb["dwd"][1])  # the empty expert


def test_mx_bwd_bf16_wgrad_pin_detects_planted_swap(monkeypatch):
    """A planted mistake (dg and du swapped in the gate/up weight gradients)
    fails the brute-force pin."""
    offsets, xp, dyp, wg, wu, wd, fw = _bf16_wgrad_case()
    ref = oracle.mx_expert_bwd(xp, dyp, offsets, wg, wu, wd, fw["g"], fw["u"], fw["h"])
    real = oracle.mx_expert_bwd

    def planted(*a, **kw):
        out = real(*a, **kw)
        out["dwg"], out["dwu"] = out["dwu"], out["dwg"]
        return out

    monkeypatch.setattr(oracle, "mx_expert_bwd", planted)
    bb = oracle.mx_expert_bwd(xp, dyp, offsets, wg, wu, wd, fw["g"], fw["u"], fw["h"], wgrad="bf16")
    dwg, _, _ = _brute_wgrads(offsets, xp, dyp, ref["dg"], ref["du"], fw["h"])
    assert not np.allclose(bb["dwg"], dwg, rtol=1e-12, atol=1e-12)


def test_mx_bwd_rejects_unknown_wgrad():
    offsets, xp, dyp, wg, wu, wd, fw = _bf16_wgrad_case()
    try:
        oracle.mx_expert_bwd(xp, dyp, offsets, wg, wu, wd, fw["g"], fw["u"], fw["h"], wgrad="fp8")
    except ValueError:
        return
    raise AssertionError("unknown wgrad accepted")
