"""CPU oracle of the dropless MoE feed-forward layer — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never imports it
and the two share no code.

``liboracle.so`` (``oracle.cpp``) holds the arithmetic; this module marshals
numpy arrays and adds the trivial row-movement definitions (permute, combine
and their backward, routing backward, router weight gradient) in numpy fp64.
Page keys ([P1], [P2], [P3]) are those listed in ``oracle.h``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SOURCES = [os.path.join(_HERE, "oracle.cpp")]
CXXFLAGS = ["-O3", "-march=x86-64-v3", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
            "-std=c++17", "-Wall"]


def build(force: bool = True) -> str:
    """Compile liboracle.so with g++ (plain C++17 + OpenMP, no fast-math)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.run(["g++", *CXXFLAGS, *SOURCES, "-o", tmp], check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None

_f = ctypes.POINTER(ctypes.c_float)
_d = ctypes.POINTER(ctypes.c_double)
_i = ctypes.POINTER(ctypes.c_int32)
_u8 = ctypes.POINTER(ctypes.c_uint8)
_int = ctypes.c_int


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(LIB_PATH)
        for acc in ("f64", "f32"):
            getattr(L, f"oracle_router_logits_{acc}").argtypes = [_f, _f, _int, _int, _int, _f]
            getattr(L, f"oracle_route_{acc}").argtypes = [_f, _int, _int, _int, _i, _d, _i, _i, _i, _i]
            getattr(L, f"oracle_expert_fwd_{acc}").argtypes = [
                _f, _i, _int, _int, _int, _int, _f, _f, _f, _i, _int, _d, _d, _d, _d]
            getattr(L, f"oracle_expert_dgrad_{acc}").argtypes = [
                _f, _f, _i, _int, _int, _int, _int, _f, _f, _f, _i, _int, _d, _d, _d]
            getattr(L, f"oracle_expert_wgrad_{acc}").argtypes = [
                _f, _f, _i, _int, _int, _int, _int, _f, _f, _f, _d, _d, _d]
            getattr(L, f"oracle_layer_fwd_{acc}").argtypes = [
                _f, _i, _d, _int, _int, _int, _int, _int, _f, _f, _f, _d, _d]
        L.oracle_expert_wgrad_elems_f64.argtypes = [
            _f, _f, _i, _int, _int, _int, _int, _f, _f, _f, _int, _i, _int, _d]
        L.oracle_layer_bwd_f64.argtypes = [
            _f, _f, _i, _d, _f, _int, _int, _int, _int, _int, _f, _f, _f, _d, _d, _d, _d, _d, _d, _d]
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_decode.restype = ctypes.c_float
        L.oracle_mx_scale_code.argtypes = [ctypes.c_float]
        L.oracle_mx_scale_code.restype = ctypes.c_uint8
        L.oracle_mx_quantize.argtypes = [_f, _int, _int, _int, _i, _int, _u8, _u8]
        _lib = L
    return _lib


def _fp(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a, a.ctypes.data_as(_f)


def _ip(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(_i)


def _dp(a):
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a, a.ctypes.data_as(_d)


def _out(shape, dtype=np.float64):
    a = np.zeros(shape, dtype=dtype)
    return a, a.ctypes.data_as({np.float64: _d, np.float32: _f, np.int32: _i, np.uint8: _u8}[dtype])


# ------------------------------------------------------------------ routing
def router_logits(x, wr, acc="f64"):
    """logits = x . W_r rounded once to fp32 ([P2] 2.1)."""
    T, d = x.shape
    E = wr.shape[1]
    x, px = _fp(x)
    wr, pw = _fp(wr)
    lg, pl = _out((T, E), np.float32)
    getattr(lib(), f"oracle_router_logits_{acc}")(px, pw, T, d, E, pl)
    return lg


def route(logits, k, acc="f64"):
    """Softmax, top-k (lower index first on equal logits), renormalised gates,
    counts, offsets, row_of, src_tk ([P2] 1.1, 2.1; [P1] 二)."""
    T, E = logits.shape
    lg, pl = _fp(logits)
    topk, p1 = _out((T, k), np.int32)
    gates, p2 = _out((T, k))
    counts, p3 = _out((E,), np.int32)
    offsets, p4 = _out((E + 1,), np.int32)
    row_of, p5 = _out((T, k), np.int32)
    src_tk, p6 = _out((T * k,), np.int32)
    getattr(lib(), f"oracle_route_{acc}")(pl, T, E, k, p1, p2, p3, p4, p5, p6)
    return dict(topk_idx=topk, gates=gates, counts=counts, offsets=offsets, row_of=row_of,
                src_tk=src_tk)


# ------------------------------------------------------------------ experts
def expert_fwd(xp, offsets, wg, wu, wd, rows=None, acc="f64"):
    """Per-row SwiGLU expert over expert-major rows; returns g, u, h, yp for
    the requested rows (all rows when rows is None)."""
    R, d = xp.shape
    E, _, F = wg.shape
    xp, pxp = _fp(xp)
    off, poff = _ip(offsets)
    wg, pg = _fp(wg)
    wu, pu = _fp(wu)
    wd, pd = _fp(wd)
    if rows is None:
        rw, prw, n = None, None, R
    else:
        rw, prw = _ip(rows)
        n = len(rw)
    g, p1 = _out((n, F))
    u, p2 = _out((n, F))
    h, p3 = _out((n, F))
    yp, p4 = _out((n, d))
    getattr(lib(), f"oracle_expert_fwd_{acc}")(pxp, poff, E, R, d, F, pg, pu, pd, prw, n, p1, p2, p3, p4)
    return dict(g=g, u=u, h=h, yp=yp)


def expert_dgrad(xp, dyp, offsets, wg, wu, wd, rows=None, acc="f64"):
    R, d = xp.shape
    E, _, F = wg.shape
    xp, pxp = _fp(xp)
    dyp, pdy = _fp(dyp)
    off, poff = _ip(offsets)
    wg, pg = _fp(wg)
    wu, pu = _fp(wu)
    wd, pd = _fp(wd)
    if rows is None:
        rw, prw, n = None, None, R
    else:
        rw, prw = _ip(rows)
        n = len(rw)
    dg, p1 = _out((n, F))
    du, p2 = _out((n, F))
    dxp, p3 = _out((n, d))
    getattr(lib(), f"oracle_expert_dgrad_{acc}")(pxp, pdy, poff, E, R, d, F, pg, pu, pd, prw, n, p1, p2, p3)
    return dict(dg=dg, du=du, dxp=dxp)


def expert_wgrad(xp, dyp, offsets, wg, wu, wd, acc="f64"):
    R, d = xp.shape
    E, _, F = wg.shape
    xp, pxp = _fp(xp)
    dyp, pdy = _fp(dyp)
    off, poff = _ip(offsets)
    wg, pg = _fp(wg)
    wu, pu = _fp(wu)
    wd, pd = _fp(wd)
    dwg, p1 = _out((E, d, F))
    dwu, p2 = _out((E, d, F))
    dwd, p3 = _out((E, F, d))
    getattr(lib(), f"oracle_expert_wgrad_{acc}")(pxp, pdy, poff, E, R, d, F, pg, pu, pd, p1, p2, p3)
    return dict(dwg=dwg, dwu=dwu, dwd=dwd)


def expert_wgrad_elems(xp, dyp, offsets, wg, wu, wd, which, elems):
    """Selected weight-gradient elements; which 0=dWg, 1=dWu, 2=dWd;
    elems is an (n,3) int array of (e, a, b) indices into dW[e][a][b]."""
    R, d = xp.shape
    E, _, F = wg.shape
    xp, pxp = _fp(xp)
    dyp, pdy = _fp(dyp)
    off, poff = _ip(offsets)
    wg, pg = _fp(wg)
    wu, pu = _fp(wu)
    wd, pd = _fp(wd)
    el, pel = _ip(np.asarray(elems).reshape(-1, 3))
    out, po = _out((len(el),))
    lib().oracle_expert_wgrad_elems_f64(pxp, pdy, poff, E, R, d, F, pg, pu, pd, which, pel, len(el), po)
    return out


# ------------------------------------------------------------------ shared expert
# [P1] 四 lists shared experts among the router options: an expert every
# token uses besides its k routed ones.  Read as one SwiGLU FFN over all T
# tokens, ungated, added to the routed output.
def shared_expert_fwd(x, wg_s, wu_s, wd_s):
    """The shared expert on every token: the grouped expert with one group
    holding all T rows (weights [1,d,Fs], [1,d,Fs], [1,Fs,d])."""
    off = np.array([0, x.shape[0]], dtype=np.int32)
    return expert_fwd(x, off, wg_s, wu_s, wd_s)


def shared_expert_bwd(x, dy, wg_s, wu_s, wd_s):
    """Its backward for upstream dy (ungated, so dy reaches it unchanged):
    dx_shared plus the three weight gradients."""
    off = np.array([0, x.shape[0]], dtype=np.int32)
    dg = expert_dgrad(x, dy, off, wg_s, wu_s, wd_s)
    wgr = expert_wgrad(x, dy, off, wg_s, wu_s, wd_s)
    return dict(dx=dg["dxp"], dg=dg["dg"], du=dg["du"], dwg=wgr["dwg"], dwu=wgr["dwu"], dwd=wgr["dwd"])


# ------------------------------------------------------------------ whole layer
def layer_fwd(x, topk_idx, gates, wg, wu, wd, acc="f64", want_ytj=False):
    """Token-by-token layer forward: y_t = sum_j g_tj * expert_{S_tj}(x_t)
    ([P2] 2.1).  Returns y and optionally Y_tj [T,k,d]."""
    T, d = x.shape
    E, _, F = wg.shape
    k = topk_idx.shape[1]
    x, px = _fp(x)
    ti, pti = _ip(topk_idx)
    ga, pga = _dp(gates)
    wg, pg = _fp(wg)
    wu, pu = _fp(wu)
    wd, pd = _fp(wd)
    y, py = _out((T, d))
    if want_ytj:
        ytj, pyt = _out((T, k, d))
    else:
        ytj, pyt = None, None
    getattr(lib(), f"oracle_layer_fwd_{acc}")(px, pti, pga, T, d, E, k, F, pg, pu, pd, py, pyt)
    return (y, ytj) if want_ytj else y


def layer_bwd(x, wr, topk_idx, gates, dy, wg, wu, wd):
    """fp64 whole-layer backward ([P2] 1.2): dgates, dlogits_sel, dx, dWg,
    dWu, dWd, dWr."""
    T, d = x.shape
    E, _, F = wg.shape
    k = topk_idx.shape[1]
    x, px = _fp(x)
    wr, pwr = _fp(wr)
    ti, pti = _ip(topk_idx)
    ga, pga = _dp(gates)
    dy, pdy = _fp(dy)
    wg, pg = _fp(wg)
    wu, pu = _fp(wu)
    wd, pd = _fp(wd)
    dgates, p1 = _out((T, k))
    dls, p2 = _out((T, k))
    dx, p3 = _out((T, d))
    dwg, p4 = _out((E, d, F))
    dwu, p5 = _out((E, d, F))
    dwd, p6 = _out((E, F, d))
    dwr, p7 = _out((d, E))
    lib().oracle_layer_bwd_f64(px, pwr, pti, pga, pdy, T, d, E, k, F, pg, pu, pd, p1, p2, p3, p4, p5,
                               p6, p7)
    return dict(dgates=dgates, dlogits_sel=dls, dx=dx, dwg=dwg, dwu=dwu, dwd=dwd, dwr=dwr)


# ------------------------------------------------------------------ row movement (definitions)
def permute(x, row_of):
    """Xp[row_of[t,j]] = x_t: each token written into its k expert rows
    ([P1] 二, rowwise writes into the experts' input buffers)."""
    T, k = row_of.shape
    xp = np.zeros((T * k, x.shape[1]), dtype=np.float64)
    for j in range(k):
        xp[row_of[:, j]] = x
    return xp


def combine(yp, gates, row_of):
    """y_t = sum_j gates[t,j] * Yp[row_of[t,j]] in slot order, fp64
    ([P2] 2.1: results return along the original path and are restored)."""
    T, k = row_of.shape
    y = np.zeros((T, yp.shape[1]), dtype=np.float64)
    for j in range(k):
        y += gates[:, j:j + 1].astype(np.float64) * yp[row_of[:, j]].astype(np.float64)
    return y


def combine_bwd(dy, yp, gates, row_of):
    """dYp[row_of[t,j]] = gates[t,j]*dy_t and dgates[t,j] = <dy_t, Yp[row_of[t,j]]>."""
    T, k = row_of.shape
    dyp = np.zeros((T * k, dy.shape[1]), dtype=np.float64)
    dgates = np.zeros((T, k), dtype=np.float64)
    dy = dy.astype(np.float64)
    for j in range(k):
        dyp[row_of[:, j]] = gates[:, j:j + 1].astype(np.float64) * dy
        dgates[:, j] = np.einsum("td,td->t", dy, yp[row_of[:, j]].astype(np.float64))
    return dyp, dgates


def route_bwd(gates, dgates):
    """Selected-slot logit gradient of the renormalised softmax gates:
    dl_tj = g_tj * (dg_tj - sum_i g_ti dg_ti); unselected logits get 0."""
    g = gates.astype(np.float64)
    dg = dgates.astype(np.float64)
    return g * (dg - (g * dg).sum(axis=1, keepdims=True))


def permute_bwd(dxp, row_of, topk_idx=None, dlogits_sel=None, wr=None):
    """dx_t = sum_j dXp[row_of[t,j]] (+ sum_j dl_tj * W_r[:, S_tj] when the
    router terms are given)."""
    T, k = row_of.shape
    dx = np.zeros((T, dxp.shape[1]), dtype=np.float64)
    for j in range(k):
        dx += dxp[row_of[:, j]].astype(np.float64)
    if dlogits_sel is not None:
        wr = wr.astype(np.float64)
        for j in range(k):
            dx += dlogits_sel[:, j:j + 1].astype(np.float64) * wr[:, topk_idx[:, j]].T
    return dx


def router_wgrad(x, dlogits_sel, topk_idx, E):
    """dW_r[:, e] = sum over (t,j) with S_tj = e of dl_tj * x_t."""
    T, d = x.shape
    dwr = np.zeros((d, E), dtype=np.float64)
    x = x.astype(np.float64)
    for j in range(topk_idx.shape[1]):
        for e in range(E):
            m = topk_idx[:, j] == e
            if m.any():
                dwr[:, e] += (dlogits_sel[m, j].astype(np.float64)[:, None] * x[m]).sum(axis=0)
    return dwr


# ------------------------------------------------------------------ routing statistics
# [P2] 2.2 (imbalance grows with the expert pool, so frameworks add a
# load-balancing auxiliary loss), 4.2 (tokens per expert; twice the mean
# flags imbalance), 4.3 (aux-loss weight, e.g. 0.001), 5.2 (tokens per
# expert, mean top-1 probability, expert-gradient L2 norms); [P1] 四 (the
# router supports load balancing) and the negative-results section (a
# balance score can improve while the real load worsens, so the real counts
# are always reported beside it).
def router_probs(logits):
    """p_t = softmax of token t's logits over all E experts, in fp64."""
    lg = logits.astype(np.float64)
    z = np.exp(lg - lg.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def top1_expert(logits):
    """Each token's expert with the largest logit, the lower index among
    equal logits (the first slot of the top-k order)."""
    lg = logits.astype(np.float32)
    T = lg.shape[0]
    out = np.empty(T, dtype=np.int32)
    for t in range(T):
        out[t] = int(np.flatnonzero(lg[t] == lg[t].max())[0])
    return out


def route_stats(logits, counts, k, alpha):
    """Per-expert routing statistics and the switch-style balance loss.

    prob_mean[e] = (1/T) sum_t p_te (the mean router probability);
    top1_count[e] = tokens whose top-1 expert is e; top1_prob_mean[e] = their
    mean top-1 probability (0 when there are none); with the load fraction
    f_e = counts[e] / (T k), aux_loss = alpha * E * sum_e f_e * prob_mean[e]
    (alpha exactly when load and probability are both uniform)."""
    T, E = logits.shape
    p = router_probs(logits)
    t1 = top1_expert(logits)
    prob_mean = p.sum(axis=0) / max(T, 1)
    top1_count = np.bincount(t1, minlength=E).astype(np.int64)
    top1_sum = np.zeros(E)
    for t in range(T):
        top1_sum[t1[t]] += p[t, t1[t]]
    top1_prob_mean = np.where(top1_count > 0, top1_sum / np.maximum(top1_count, 1), 0.0)
    f = counts.astype(np.float64) / max(T * k, 1)
    aux = alpha * E * float((f * prob_mean).sum())
    return dict(prob_mean=prob_mean, top1_count=top1_count, top1_prob_mean=top1_prob_mean,
                aux_loss=aux)


def aux_loss_bwd(logits, counts, k, alpha, dloss=1.0):
    """Gradient of dloss * aux_loss with respect to every logit.  The load
    fractions are counts (piecewise constant in the logits), so only the mean
    probabilities carry gradient: with a_e = alpha * E * f_e / T,
    dl[t, e] = dloss * p_te * (a_e - sum_i p_ti a_i)."""
    T, E = logits.shape
    p = router_probs(logits)
    a = alpha * E * (counts.astype(np.float64) / max(T * k, 1)) / max(T, 1)
    return dloss * p * (a[None, :] - (p * a[None, :]).sum(axis=1, keepdims=True))


def router_dense_bwd(x, wr, dlogits):
    """The router's share of a gradient that reaches every logit (the balance
    loss's dense dl from aux_loss_bwd; [P1] 四: the router balances load, so
    that loss trains the router): with logits = x W_r,
    dx[t, i] = sum_e dl[t, e] * W_r[i, e] and dW_r[i, e] = sum_t x[t, i] * dl[t, e],
    both as fp64 products.  The result adds to the layer's own dx and dW_r."""
    dl = np.asarray(dlogits, dtype=np.float64)
    return dict(dx=dl @ np.asarray(wr, dtype=np.float64).T,
                dwr=np.asarray(x, dtype=np.float64).T @ dl)


def expert_grad_norms(dw):
    """L2 (Frobenius) norm of each expert's weight-gradient matrix dw[e],
    from the stored values, accumulated in fp64."""
    E = dw.shape[0]
    v = dw.reshape(E, -1).astype(np.float64)
    return np.sqrt((v * v).sum(axis=1))


# ------------------------------------------------------------------ MXFP8
def e4m3_encode(v):
    return lib().oracle_e4m3_encode(float(v))


def e4m3_decode(c):
    return lib().oracle_e4m3_decode(int(c))


def mx_scale_code(amax):
    return lib().oracle_mx_scale_code(float(amax))


def e4m3_values():
    """Value of each of the 256 codes (NaN codes are NaN)."""
    return np.array([lib().oracle_e4m3_decode(c) for c in range(256)], dtype=np.float32)


def mx_quantize(src, axis, offsets=None):
    """MX quantisation of a [rows, cols] matrix; returns (codes, scales).  See
    oracle.h for the block layouts."""
    rows, cols = src.shape
    s, ps = _fp(src)
    codes, pc = _out((rows, cols), np.uint8)
    if axis == 0:
        assert cols % 32 == 0
        scales, psc = _out((rows, cols // 32), np.uint8)
        lib().oracle_mx_quantize(ps, rows, cols, 0, None, 0, pc, psc)
    else:
        if offsets is None:
            offsets = np.array([0, rows], dtype=np.int32)
        off, poff = _ip(offsets)
        nblk = int(sum((int(off[g + 1]) - int(off[g]) + 31) // 32 for g in range(len(off) - 1)))
        scales, psc = _out((nblk, cols), np.uint8)
        lib().oracle_mx_quantize(ps, rows, cols, 1, poff, len(off) - 1, pc, psc)
    return codes, scales


def mx_dequantize_rows(codes, scales):
    """Exact values of axis-0 quantised data: code value * 2^(scale-127)."""
    vals = e4m3_values().astype(np.float64)[codes]
    sc = np.ldexp(1.0, scales.astype(np.int32) - 127)
    return vals * np.repeat(sc, 32, axis=1)


def mx_dequantize_cols(codes, scales, offsets):
    """Exact values of axis-1 quantised data (group-major blocks)."""
    vals = e4m3_values().astype(np.float64)[codes]
    out = np.empty_like(vals)
    blk = 0
    for g in range(len(offsets) - 1):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        for b in range((hi - lo + 31) // 32):
            r0, r1 = lo + 32 * b, min(lo + 32 * b + 32, hi)
            out[r0:r1] = vals[r0:r1] * np.ldexp(1.0, scales[blk].astype(np.int32) - 127)[None, :]
            blk += 1
    return out


# ------------------------------------------------------------------ MXFP8 expert chain
def _bf16_round(a):
    """Round float64 values to bf16 (nearest even) and return them as float64."""
    a32 = np.ascontiguousarray(a, dtype=np.float32)
    u = a32.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def mx_rows(a):
    """Exact values of `a` after MX quantisation along its rows (axis 0)."""
    c, s = mx_quantize(np.ascontiguousarray(a, dtype=np.float32), axis=0)
    return mx_dequantize_rows(c, s)


def mx_cols(a, offsets):
    """Exact values of `a` after MX quantisation down its columns in blocks
    restarting at each group of rows."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if offsets is None:
        offsets = np.array([0, a.shape[0]], dtype=np.int32)
    c, s = mx_quantize(a, axis=1, offsets=offsets)
    return mx_dequantize_cols(c, s, offsets)


def mx_expert_fwd(xp, offsets, wg, wu, wd):
    """MXFP8 forward of the grouped SwiGLU experts ([P1] 三).  Each GEMM takes
    its operands quantised along its reduction axis (activations rowwise,
    weights down their columns, one block set per expert), dequantised
    exactly, summed in fp64; g and u are rounded to bf16, h = silu(g)*u is
    formed in fp64 from those values, rounded to bf16 and quantised again
    for the down projection.  Returns g, u, h (bf16 values) and yp."""
    R, d = xp.shape
    E, _, F = wg.shape
    xq = mx_rows(xp)
    g = np.zeros((R, F))
    u = np.zeros((R, F))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        g[lo:hi] = xq[lo:hi] @ mx_cols(wg[e], None)
        u[lo:hi] = xq[lo:hi] @ mx_cols(wu[e], None)
    g = _bf16_round(g)
    u = _bf16_round(u)
    h = _bf16_round(g / (1.0 + np.exp(-g)) * u)
    hq = mx_rows(h)
    yp = np.zeros((R, d))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            yp[lo:hi] = hq[lo:hi] @ mx_cols(wd[e], None)
    return dict(g=g, u=u, h=h, yp=yp)


def mx_expert_bwd(xp, dyp, offsets, wg, wu, wd, g, u, h, wgrad="mx"):
    """MXFP8 backward for upstream rows dyp, given the forward's bf16 g, u and
    h: dh = Q(dyp) Q(Wd^T) (blocks along d), dg/du from bf16 g, u in fp64
    then rounded to bf16, dxp = Q(dg) Q(Wg^T) + Q(du) Q(Wu^T) (blocks along F),
    and per expert dWd = Qc(h)^T Qc(dyp), dWg = Qc(xp)^T Qc(dg),
    dWu = Qc(xp)^T Qc(du) with blocks along that expert's rows.

    wgrad="bf16": MXFP8 on the data-gradient products only (the bigchange.ai
    page's overview names MXFP8 for selected operations); the weight
    gradients are the fp64 products of the unquantised bf16 operands,
    dWd = h^T dyp, dWg = xp^T dg, dWu = xp^T du per expert, the data
    gradients unchanged."""
    if wgrad not in ("mx", "bf16"):
        raise ValueError("wgrad must be 'mx' or 'bf16'")
    R, d = xp.shape
    E, _, F = wg.shape
    dyq = mx_rows(dyp)
    dh = np.zeros((R, F))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            dh[lo:hi] = dyq[lo:hi] @ mx_rows(wd[e]).T
    s = 1.0 / (1.0 + np.exp(-g))
    dg = _bf16_round(dh * u * s * (1.0 + g * (1.0 - s)))
    du = _bf16_round(dh * g * s)
    dgq, duq = mx_rows(dg), mx_rows(du)
    dxp = np.zeros((R, d))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            dxp[lo:hi] = dgq[lo:hi] @ mx_rows(wg[e]).T + duq[lo:hi] @ mx_rows(wu[e]).T
    off = np.asarray(offsets, dtype=np.int32)
    if wgrad == "mx":
        xc, hc, yc = mx_cols(xp, off), mx_cols(h, off), mx_cols(dyp, off)
        gc, uc = mx_cols(dg, off), mx_cols(du, off)
    else:
        f64 = lambda a: np.asarray(a, dtype=np.float64)  # noqa: E731
        xc, hc, yc, gc, uc = f64(xp), f64(h), f64(dyp), dg, du
    dwg = np.zeros((E, d, F))
    dwu = np.zeros((E, d, F))
    dwd = np.zeros((E, F, d))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            dwg[e] = xc[lo:hi].T @ gc[lo:hi]
            dwu[e] = xc[lo:hi].T @ uc[lo:hi]
            dwd[e] = hc[lo:hi].T @ yc[lo:hi]
    return dict(dg=dg, du=du, dxp=dxp, dwg=dwg, dwu=dwu, dwd=dwd)


def _expert_of(offsets, r):
    return int(np.searchsorted(np.asarray(offsets), r, side="right") - 1)


def mx_expert_rows(xp, dyp, offsets, wg, wu, wd, rows):
    """The MX chain's per-row outputs (g, u, h, yp, dg, du, dxp) for the
    selected rows only: every one of them depends on its own row and its
    expert's weights, since rowwise blocks never span rows."""
    E, d, F = wg.shape
    rows = np.asarray(rows)
    out = {k: np.zeros((len(rows), F)) for k in ("g", "u", "h", "dg", "du")}
    out["yp"] = np.zeros((len(rows), d))
    out["dxp"] = np.zeros((len(rows), d))
    ex = np.array([_expert_of(offsets, r) for r in rows])
    for e in np.unique(ex):
        sel = np.nonzero(ex == e)[0]
        r = rows[sel]
        xq = mx_rows(xp[r])
        g = _bf16_round(xq @ mx_cols(wg[e], None))
        u = _bf16_round(xq @ mx_cols(wu[e], None))
        h = _bf16_round(g / (1.0 + np.exp(-g)) * u)
        yp = mx_rows(h) @ mx_cols(wd[e], None)
        dh = mx_rows(dyp[r]) @ mx_rows(wd[e]).T
        s = 1.0 / (1.0 + np.exp(-g))
        dg = _bf16_round(dh * u * s * (1.0 + g * (1.0 - s)))
        du = _bf16_round(dh * g * s)
        dxp = mx_rows(dg) @ mx_rows(wg[e]).T + mx_rows(du) @ mx_rows(wu[e]).T
        for k, v in (("g", g), ("u", u), ("h", h), ("yp", yp), ("dg", dg), ("du", du), ("dxp", dxp)):
            out[k][sel] = v
    return out


def mx_expert_wgrad_elems(xp, dyp, offsets, wg, wu, wd, which, elems):
    """Selected elements of the MX chain's weight gradients; which 0=dWg,
    1=dWu, 2=dWd, elems (n,3) of (e, a, b) into dW[e][a][b].  Needs only the
    columns a and b of the two operands over expert e's rows; column blocks
    restart at the expert's first row."""
    E, d, F = wg.shape
    elems = np.asarray(elems).reshape(-1, 3)
    out = np.zeros(len(elems))
    for e in np.unique(elems[:, 0]):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        sel = np.nonzero(elems[:, 0] == e)[0]
        one = np.array([0, hi - lo], dtype=np.int32)
        xq = mx_rows(xp[lo:hi])
        dyq = mx_rows(dyp[lo:hi])
        wgc, wuc, wdc = mx_cols(wg[e], None), mx_cols(wu[e], None), mx_cols(wd[e], None)
        wdr = mx_rows(wd[e])

        def gu(c):
            g = _bf16_round(xq @ wgc[:, c])
            u = _bf16_round(xq @ wuc[:, c])
            return g, u

        def col(v):  # column quantisation of one column over the expert's rows
            return mx_cols(v.reshape(-1, 1), one)[:, 0]

        for i in sel:
            _, a, b = (int(t) for t in elems[i])
            if which == 2:  # dWd[a][b] = sum_r Qc(h)[r,a] Qc(dyp)[r,b]
                g, u = gu(a)
                h = _bf16_round(g / (1.0 + np.exp(-g)) * u)
                out[i] = col(h) @ col(dyp[lo:hi, b].astype(np.float64))
            else:  # dWg/dWu[a][b] = sum_r Qc(xp)[r,a] Qc(dg or du)[r,b]
                g, u = gu(b)
                dh = dyq @ wdr[b, :]
                s = 1.0 / (1.0 + np.exp(-g))
                v = dh * u * s * (1.0 + g * (1.0 - s)) if which == 0 else dh * g * s
                out[i] = col(xp[lo:hi, a].astype(np.float64)) @ col(_bf16_round(v))
        del xq, dyq, wgc, wuc, wdc, wdr
    return out
