"""Python binding of the MI355X dropless MoE layer library (libmoe.so).

Argument marshalling only: every step of the layer runs in the HIP kernels of
``libmoe.so``.  PyTorch provides device memory and the current HIP stream.
The functions carry the C ABI's names (``include/moe.h``) and take torch
tensors; each raises ``MoeError`` on a non-OK status.  There is no CPU
fallback: importing works without the library, but any call raises when
``libmoe.so`` is missing or no GPU is present.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_F32, MOE_BF16, MOE_MXFP8 = 0, 1, 2
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace", 4: "HIP error"}


class MoeError(RuntimeError):
    pass


_lib = None
_vp = ctypes.c_void_p
_int = ctypes.c_int
_flt = ctypes.c_float

# name -> argument types after the context pointer
_SIGS = {
    "moe_router_logits": [_vp, _vp, _int, _int, _int, _int, _vp],
    "moe_route": [_vp, _int, _int, _int, _vp, _vp, _vp, _vp, _vp, _vp],
    "moe_route_noalloc": [_vp, _int, _int, _int, _vp, _vp, _vp, _vp, _vp, _vp],
    "moe_permute": [_vp, _vp, _int, _int, _int, _int, _vp],
    "moe_grouped_ffn_fwd": [_vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _int, _vp, _vp, _vp, _vp],
    "moe_combine": [_vp, _vp, _vp, _int, _int, _int, _int, _vp],
    "moe_combine_bwd": [_vp, _vp, _vp, _vp, _int, _int, _int, _int, _vp, _vp],
    "moe_route_bwd": [_vp, _vp, _int, _int, _vp],
    "moe_grouped_ffn_bwd": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _int,
                            _vp, _vp, _vp, _vp, _vp, _vp],
    "moe_grouped_ffn_bwd_router": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _int,
                                   _int, _int, _int, _vp, _vp, _vp, _vp, _vp, _vp],
    "moe_route_bwd_rows": [_vp, _vp, _vp, _int, _int, _vp, _vp],
    "moe_permute_bwd": [_vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _int, _vp],
    "moe_router_wgrad": [_vp, _vp, _vp, _vp, _int, _int, _int, _int, _int, _vp],
    "moe_mx_quantize": [_vp, _int, _int, _int, _vp, _int, _vp, _vp, _int],
    "moe_permute_mx": [_vp, _vp, _int, _int, _int, _vp, _vp, _vp],
    "moe_grouped_ffn_fwd_mxq": [_vp, _vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _vp, _vp, _vp, _vp],
    "moe_combine_shared": [_vp, _vp, _vp, _vp, _int, _int, _int, _int, _vp],
    "moe_permute_bwd_shared": [_vp, _vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _int, _vp],
    "moe_route_stats": [_vp, _vp, _int, _int, _int, _flt, _vp, _vp, _vp, _vp],
    "moe_aux_loss_bwd": [_vp, _vp, _int, _int, _int, _flt, _flt, _vp],
    "moe_expert_grad_norms": [_vp, _int, _int, _int, _int, _vp],
    "moe_router_dense_bwd": [_vp, _vp, _vp, _int, _int, _int, _int, _vp, _vp],
    "moe_mfma_peak_probe": [_int, _int, _flt, _flt, _vp],
    "moe_mx_quantize_both": [_vp, _int, _int, _vp, _int, _vp, _vp, _int, _vp, _vp],
    "moe_mx_quantize_weights": [_vp, _vp, _vp, _int, _int, _int, _vp, ctypes.c_size_t],
    "moe_grouped_ffn_fwd_mxp": [_vp, _vp, _vp, _vp, ctypes.c_size_t, _vp, _int, _int, _int, _int, _vp, _vp,
                                _vp, _vp],
    "moe_grouped_ffn_bwd_mxp": [_vp, _vp, ctypes.c_size_t, _vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int,
                                _vp, _vp, _vp, _vp, _vp, _vp],
    "moe_grouped_ffn_bwd_mxp_bf16w": [_vp, _vp, ctypes.c_size_t, _vp, _vp, _vp, _vp, _vp, _int, _int, _int,
                                      _int, _vp, _vp, _vp, _vp, _vp, _vp],
}
EXPORTS = ["moe_create", "moe_destroy", "moe_set_stream", "moe_status_string", "moe_last_error",
           "moe_workspace_size", "moe_set_workspace", *_SIGS.keys(), "moe_profile_enable",
           "moe_profile_query", "moe_kernel_name", "moe_mx_workspace_size", "moe_ffn_bwd_workspace_size",
           "moe_mx_weight_pack_size"]

# kernel ids of the profiling hook (moe_kernel_id in include/moe.h)
KERNELS = ["router_logits", "topk_hist", "expert_scan", "rank", "permute", "gemm_up_swiglu",
           "gemm_down", "combine", "combine_bwd", "route_bwd", "gemm_dgrad_down_swiglu",
           "gemm_wgrad_down", "gemm_dgrad_up", "gemm_wgrad_up", "permute_bwd", "router_wgrad",
           "mx_quantize", "route_stats", "aux_loss_bwd", "grad_norms", "router_dense_bwd"]


def lib():
    """Load libmoe.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MoeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m routing_grouped_expert_softmax_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.moe_create.argtypes = [_int, _vp, ctypes.POINTER(_vp)]
        L.moe_destroy.argtypes = [_vp]
        L.moe_set_stream.argtypes = [_vp, _vp]
        L.moe_status_string.argtypes = [_int]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = [_vp]
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_workspace_size.argtypes = [_vp, _int, _int, _int, _int, _int, ctypes.POINTER(ctypes.c_size_t)]
        L.moe_set_workspace.argtypes = [_vp, _vp, ctypes.c_size_t]
        L.moe_mx_workspace_size.argtypes = [_vp, _int, _int, _int, _int, ctypes.POINTER(ctypes.c_size_t)]
        L.moe_ffn_bwd_workspace_size.argtypes = [_vp, _int, _int, _int, _int, _int,
                                                 ctypes.POINTER(ctypes.c_size_t)]
        L.moe_mx_weight_pack_size.argtypes = [_vp, _int, _int, _int, ctypes.POINTER(ctypes.c_size_t)]
        for name, sig in _SIGS.items():
            getattr(L, name).argtypes = [_vp, *sig]
        L.moe_profile_enable.argtypes = [_vp, _int]
        L.moe_profile_query.argtypes = [_vp, _int, ctypes.POINTER(_int), ctypes.POINTER(ctypes.c_double)]
        L.moe_kernel_name.argtypes = [_int]
        L.moe_kernel_name.restype = ctypes.c_char_p
        _lib = L
    return _lib


class Context:
    """One library context per (device, stream); owns a torch workspace."""

    def __init__(self, device: int = 0):
        if not torch.cuda.is_available():
            raise MoeError("no GPU: the MoE library runs only on the GPU")
        self.device = device
        h = _vp()
        self._check(lib().moe_create(device, None, ctypes.byref(h)), None)
        self.handle = h
        self._ws = None
        self._ws_bytes = 0

    def _check(self, st, handle="self"):
        if st != 0:
            msg = ""
            if handle is not None and getattr(self, "handle", None) is not None:
                msg = lib().moe_last_error(self.handle).decode()
            raise MoeError(f"{_STATUS.get(st, st)}: {msg}")

    def bind_stream(self):
        s = torch.cuda.current_stream(self.device)
        self._check(lib().moe_set_stream(self.handle, _vp(s.cuda_stream)))

    def ensure_workspace(self, T, d, E, k, dtype):
        n = ctypes.c_size_t()
        self._check(lib().moe_workspace_size(self.handle, T, d, E, k, dtype, ctypes.byref(n)))
        self._grow(n.value)

    def ensure_mx_workspace(self, E, R, d, F):
        n = ctypes.c_size_t()
        self._check(lib().moe_mx_workspace_size(self.handle, E, R, d, F, ctypes.byref(n)))
        self._grow(n.value)

    def ensure_ffn_bwd_workspace(self, E, R, d, F, dtype):
        n = ctypes.c_size_t()
        self._check(lib().moe_ffn_bwd_workspace_size(self.handle, E, R, d, F, dtype, ctypes.byref(n)))
        self._grow(n.value)

    def _grow(self, nbytes):
        n = ctypes.c_size_t(nbytes)
        if n.value > self._ws_bytes:
            self._ws = torch.empty(max(n.value, 256), dtype=torch.uint8, device=f"cuda:{self.device}")
            self._ws_bytes = n.value
            self._check(lib().moe_set_workspace(self.handle, _vp(self._ws.data_ptr()), n.value))

    def call(self, name, *args):
        self.bind_stream()
        self._check(getattr(lib(), name)(self.handle, *args))

    def profile(self, on: bool):
        """Turn per-kernel HIP-event timing on (clearing old records) or off."""
        self._check(lib().moe_profile_enable(self.handle, 1 if on else 0))

    def profile_results(self):
        """{kernel name: (launches, total ms)} since profiling was enabled."""
        out = {}
        for i, name in enumerate(KERNELS):
            n, ms = _int(), ctypes.c_double()
            self._check(lib().moe_profile_query(self.handle, i, ctypes.byref(n), ctypes.byref(ms)))
            if n.value:
                out[name] = (n.value, ms.value)
        return out

    def close(self):
        if getattr(self, "handle", None) is not None:
            lib().moe_destroy(self.handle)
            self.handle = None


_ctx = {}


def context(device: int | None = None) -> Context:
    dev = torch.cuda.current_device() if device is None else device
    if dev not in _ctx:
        _ctx[dev] = Context(dev)
    return _ctx[dev]


def _p(t):
    return None if t is None else _vp(t.data_ptr())


def _dt(t):
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise MoeError(f"unsupported dtype {t.dtype}")


def _need_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise MoeError("tensors must be contiguous GPU tensors")


# ------------------------------------------------------------------ ABI calls
def moe_router_logits(x, w_router, logits=None):
    _need_cuda(x, w_router)
    T, d = x.shape
    E = w_router.shape[1]
    if logits is None:
        logits = torch.empty(T, E, dtype=torch.float32, device=x.device)
    context(x.device.index).call("moe_router_logits", _p(x), _p(w_router), T, d, E, _dt(x), _p(logits))
    return logits


def moe_route(logits, k, out=None):
    """Returns dict(topk_idx, gates, counts, offsets, row_of, src_tk)."""
    _need_cuda(logits)
    T, E = logits.shape
    dev = logits.device
    if out is None:
        out = dict(topk_idx=torch.empty(T, k, dtype=torch.int32, device=dev),
                   gates=torch.empty(T, k, dtype=torch.float32, device=dev),
                   counts=torch.empty(E, dtype=torch.int32, device=dev),
                   offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
                   row_of=torch.empty(T, k, dtype=torch.int32, device=dev),
                   src_tk=torch.empty(max(T * k, 1), dtype=torch.int32, device=dev))
    ctx = context(dev.index)
    ctx.ensure_workspace(T, 8, E, k, MOE_F32)
    ctx.call("moe_route", _p(logits), T, E, k, _p(out["topk_idx"]), _p(out["gates"]), _p(out["counts"]),
             _p(out["offsets"]), _p(out["row_of"]), _p(out["src_tk"]))
    return out


def moe_route_noalloc(out, logits, k):
    """moe_route into caller-provided outputs (the dict moe_route returns),
    without the library workspace: the call allocates nothing."""
    _need_cuda(logits)
    T, E = logits.shape
    context(logits.device.index).call(
        "moe_route_noalloc", _p(logits), T, E, k, _p(out["topk_idx"]), _p(out["gates"]),
        _p(out["counts"]), _p(out["offsets"]), _p(out["row_of"]), _p(out["src_tk"]))
    return out


def moe_permute(x, row_of, xp=None):
    _need_cuda(x, row_of)
    T, d = x.shape
    k = row_of.shape[1]
    if xp is None:
        xp = torch.empty(T * k, d, dtype=x.dtype, device=x.device)
    context(x.device.index).call("moe_permute", _p(x), _p(row_of), T, d, k, _dt(x), _p(xp))
    return xp


@dataclass
class MxWeightPack:
    """The expert weights quantised once in both MXFP8 layouts
    (moe_mx_quantize_weights): a uint8 device buffer and its shape."""
    data: torch.Tensor
    E: int
    d: int
    F: int


def moe_mx_weight_pack_size(E, d, F, device=0):
    n = ctypes.c_size_t()
    ctx = context(device)
    ctx._check(lib().moe_mx_weight_pack_size(ctx.handle, E, d, F, ctypes.byref(n)))
    return n.value


def moe_mx_quantize_weights(w_gate, w_up, w_down, pack: MxWeightPack | None = None):
    """Quantise the bf16 expert weights (w_gate, w_up [E,d,F], w_down
    [E,F,d]) into a pack read by moe_grouped_ffn_fwd_mxp/bwd_mxp; returns it."""
    _need_cuda(w_gate, w_up, w_down)
    E, d, F = w_gate.shape
    dev = w_gate.device
    if pack is None:
        n = moe_mx_weight_pack_size(E, d, F, dev.index)
        pack = MxWeightPack(torch.empty(n, dtype=torch.uint8, device=dev), E, d, F)
    if (pack.E, pack.d, pack.F) != (E, d, F):
        raise MoeError(f"pack is for E={pack.E} d={pack.d} F={pack.F}, weights are {E}x{d}x{F}")
    context(dev.index).call("moe_mx_quantize_weights", _p(w_gate), _p(w_up), _p(w_down), E, d, F,
                            _p(pack.data), pack.data.numel())
    return pack


def moe_mx_quantize_both(src, group_offsets=None, groups=1):
    """Both MX layouts of a bf16 [rows, cols] tensor from one read: returns
    (codes_cols [cols, kpad], scales_cols [cols, kpad/32], codes_rows
    [rows, cols], scales_rows [rows, cols/32]) as moe_mx_quantize axis 1 and
    axis 0 give them."""
    _need_cuda(src, group_offsets)
    rows, cols = src.shape
    dev = src.device
    kp = mx_kpad(rows, groups)
    cc = torch.empty(cols, kp, dtype=torch.uint8, device=dev)
    cs = torch.empty(cols, kp // 32, dtype=torch.uint8, device=dev)
    rc = torch.empty(rows, cols, dtype=torch.uint8, device=dev)
    rs = torch.empty(rows, cols // 32, dtype=torch.uint8, device=dev)
    context(dev.index).call("moe_mx_quantize_both", _p(src), rows, cols, _p(group_offsets), groups, _p(cc),
                            _p(cs), kp, _p(rc), _p(rs))
    return cc, cs, rc, rs


def moe_grouped_ffn_fwd_mxp(pack: MxWeightPack, offsets, xp=None, xp_codes=None, xp_scales=None, out=None,
                            up_only=False):
    """MXFP8 grouped FFN forward with the weights from a pack, on bf16 rows xp
    or on rows already quantised (xp_codes, xp_scales); returns dict(g, u, h,
    yp), without yp when up_only (the gate/up GEMM alone)."""
    rows = xp if xp is not None else xp_codes
    _need_cuda(rows, xp_scales, offsets, pack.data)
    R = rows.shape[0]
    E, d, F = pack.E, pack.d, pack.F
    dev = rows.device
    context(dev.index).ensure_mx_workspace(E, R, d, F)
    if out is None:
        out = dict(g=torch.empty(R, F, dtype=torch.bfloat16, device=dev),
                   u=torch.empty(R, F, dtype=torch.bfloat16, device=dev),
                   h=torch.empty(R, F, dtype=torch.bfloat16, device=dev))
        if not up_only:
            out["yp"] = torch.empty(R, d, dtype=torch.bfloat16, device=dev)
    context(dev.index).call("moe_grouped_ffn_fwd_mxp", _p(xp), _p(xp_codes), _p(xp_scales), _p(pack.data),
                            pack.data.numel(), _p(offsets), E, R, d, F, _p(out["g"]), _p(out["u"]),
                            _p(out["h"]), None if up_only else _p(out["yp"]))
    return out


def moe_grouped_ffn_bwd_mxp(xp, pack: MxWeightPack, offsets, g, u, h, dyp, out=None):
    """MXFP8 grouped FFN backward with the weights from a pack; returns
    dict(dg, du, dxp, dw_gate, dw_up, dw_down)."""
    return _ffn_bwd_pack("moe_grouped_ffn_bwd_mxp", xp, pack, offsets, g, u, h, dyp, out)


def moe_grouped_ffn_bwd_mxp_bf16w(xp, pack: MxWeightPack, offsets, g, u, h, dyp, out=None):
    """moe_grouped_ffn_bwd_mxp with MXFP8 on the data gradients only: dg, du
    and dxp as there, the weight gradients from the bf16 operands."""
    return _ffn_bwd_pack("moe_grouped_ffn_bwd_mxp_bf16w", xp, pack, offsets, g, u, h, dyp, out)


def _ffn_bwd_pack(name, xp, pack, offsets, g, u, h, dyp, out):
    _need_cuda(xp, offsets, g, u, h, dyp, pack.data)
    R = xp.shape[0]
    E, d, F = pack.E, pack.d, pack.F
    dev = xp.device
    context(dev.index).ensure_mx_workspace(E, R, d, F)
    if out is None:
        bf = torch.bfloat16
        out = dict(dg=torch.empty(R, F, dtype=bf, device=dev), du=torch.empty(R, F, dtype=bf, device=dev),
                   dxp=torch.empty(R, d, dtype=bf, device=dev), dw_gate=torch.empty(E, d, F, dtype=bf, device=dev),
                   dw_up=torch.empty(E, d, F, dtype=bf, device=dev),
                   dw_down=torch.empty(E, F, d, dtype=bf, device=dev))
    context(dev.index).call(name, _p(xp), _p(pack.data), pack.data.numel(), _p(offsets),
                            _p(g), _p(u), _p(h), _p(dyp), E, R, d, F, _p(out["dg"]), _p(out["du"]),
                            _p(out["dxp"]), _p(out["dw_gate"]), _p(out["dw_up"]), _p(out["dw_down"]))
    return out


def moe_permute_mx(x, row_of, xp=None, codes=None, scales=None, with_bf16=True):
    """Quantise-on-permute: returns (xp bf16 [T*k,d] or None, codes [T*k,d]
    uint8, scales [T*k,d/32] uint8)."""
    _need_cuda(x, row_of)
    T, d = x.shape
    k = row_of.shape[1]
    dev = x.device
    if with_bf16 and xp is None:
        xp = torch.empty(T * k, d, dtype=x.dtype, device=dev)
    if codes is None:
        codes = torch.empty(T * k, d, dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty(T * k, d // 32, dtype=torch.uint8, device=dev)
    context(dev.index).call("moe_permute_mx", _p(x), _p(row_of), T, d, k, _p(xp if with_bf16 else None),
                            _p(codes), _p(scales))
    return xp if with_bf16 else None, codes, scales


def moe_grouped_ffn_fwd_mxq(xp_codes, xp_scales, w_gate, w_up, w_down, offsets, out=None):
    """MXFP8 grouped FFN forward on pre-quantised rows; returns dict(g, u, h, yp)."""
    _need_cuda(xp_codes, xp_scales, w_gate, w_up, w_down, offsets)
    R, d = xp_codes.shape
    E, _, F = w_gate.shape
    dev = xp_codes.device
    context(dev.index).ensure_mx_workspace(E, R, d, F)
    if out is None:
        out = dict(g=torch.empty(R, F, dtype=w_gate.dtype, device=dev),
                   u=torch.empty(R, F, dtype=w_gate.dtype, device=dev),
                   h=torch.empty(R, F, dtype=w_gate.dtype, device=dev),
                   yp=torch.empty(R, d, dtype=w_gate.dtype, device=dev))
    context(dev.index).call("moe_grouped_ffn_fwd_mxq", _p(xp_codes), _p(xp_scales), _p(w_gate), _p(w_up),
                            _p(w_down), _p(offsets), E, R, d, F, _p(out["g"]), _p(out["u"]), _p(out["h"]),
                            _p(out["yp"]))
    return out


def moe_grouped_ffn_fwd(xp, w_gate, w_up, w_down, offsets, out=None, mxfp8=False):
    """Returns dict(g, u, h, yp).  mxfp8=True runs the MXFP8 GEMMs on the bf16
    tensors (quantised inside the call)."""
    _need_cuda(xp, w_gate, w_up, w_down, offsets)
    R, d = xp.shape
    E, _, F = w_gate.shape
    dt = MOE_MXFP8 if mxfp8 else _dt(xp)
    if mxfp8:
        context(xp.device.index).ensure_mx_workspace(E, R, d, F)
    if out is None:
        out = dict(g=torch.empty(R, F, dtype=xp.dtype, device=xp.device),
                   u=torch.empty(R, F, dtype=xp.dtype, device=xp.device),
                   h=torch.empty(R, F, dtype=xp.dtype, device=xp.device),
                   yp=torch.empty(R, d, dtype=xp.dtype, device=xp.device))
    context(xp.device.index).call("moe_grouped_ffn_fwd", _p(xp), _p(w_gate), _p(w_up), _p(w_down),
                                  _p(offsets), E, R, d, F, dt, _p(out["g"]), _p(out["u"]),
                                  _p(out["h"]), _p(out["yp"]))
    return out


def moe_grouped_ffn_up(xp, w_gate, w_up, offsets, out=None, mxfp8=False):
    """The gate/up GEMM + SwiGLU alone (moe_grouped_ffn_fwd with w_down and
    yp NULL): recomputes g, u, h; returns dict(g, u, h)."""
    _need_cuda(xp, w_gate, w_up, offsets)
    R, d = xp.shape
    E, _, F = w_gate.shape
    dt = MOE_MXFP8 if mxfp8 else _dt(xp)
    if mxfp8:
        context(xp.device.index).ensure_mx_workspace(E, R, d, F)
    if out is None:
        out = dict(g=torch.empty(R, F, dtype=xp.dtype, device=xp.device),
                   u=torch.empty(R, F, dtype=xp.dtype, device=xp.device),
                   h=torch.empty(R, F, dtype=xp.dtype, device=xp.device))
    context(xp.device.index).call("moe_grouped_ffn_fwd", _p(xp), _p(w_gate), _p(w_up), None, _p(offsets),
                                  E, R, d, F, dt, _p(out["g"]), _p(out["u"]), _p(out["h"]), None)
    return out


def moe_combine(yp, gates, row_of, y=None, y_shared=None):
    """y = sum_j gates * yp[row_of] (+ y_shared, the shared expert's rows)."""
    _need_cuda(yp, gates, row_of, y_shared)
    T, k = row_of.shape
    d = yp.shape[1]
    if y is None:
        y = torch.empty(T, d, dtype=yp.dtype, device=yp.device)
    ctx = context(yp.device.index)
    if y_shared is None:
        ctx.call("moe_combine", _p(yp), _p(gates), _p(row_of), T, d, k, _dt(yp), _p(y))
    else:
        ctx.call("moe_combine_shared", _p(yp), _p(gates), _p(row_of), _p(y_shared), T, d, k, _dt(yp), _p(y))
    return y


def moe_combine_bwd(dy, yp, gates, row_of, dyp=None, dgates=None):
    _need_cuda(dy, yp, gates, row_of)
    T, k = row_of.shape
    d = yp.shape[1]
    if dyp is None:
        dyp = torch.empty(T * k, d, dtype=yp.dtype, device=yp.device)
    if dgates is None:
        dgates = torch.empty(T, k, dtype=torch.float32, device=yp.device)
    context(yp.device.index).call("moe_combine_bwd", _p(dy), _p(yp), _p(gates), _p(row_of), T, d, k,
                                  _dt(yp), _p(dyp), _p(dgates))
    return dyp, dgates


def moe_route_bwd(gates, dgates, dlogits_sel=None, row_of=None, dl_rows=None):
    """Logit gradient at the selected slots [T,k]; with row_of also returns
    dl_rows [T*k], the same values in expert-row order."""
    _need_cuda(gates, dgates, row_of, dl_rows)
    T, k = gates.shape
    if dlogits_sel is None:
        dlogits_sel = torch.empty(T, k, dtype=torch.float32, device=gates.device)
    ctx = context(gates.device.index)
    if row_of is None:
        ctx.call("moe_route_bwd", _p(gates), _p(dgates), T, k, _p(dlogits_sel))
        return dlogits_sel
    if dl_rows is None:
        dl_rows = torch.empty(T * k, dtype=torch.float32, device=gates.device)
    ctx.call("moe_route_bwd_rows", _p(gates), _p(dgates), _p(row_of), T, k, _p(dlogits_sel), _p(dl_rows))
    return dlogits_sel, dl_rows


def moe_grouped_ffn_bwd(xp, w_gate, w_up, w_down, offsets, g, u, h, dyp, out=None, mxfp8=False, router=None):
    """Returns dict(dg, du, dxp, dw_gate, dw_up, dw_down).  router =
    (dl_rows [R] fp32, w_router [d,E]) folds the router's input-gradient
    term into dxp (bf16 only): row r of expert e then also holds
    dl_rows[r] * w_router[:, e] (dl_rows from moe_route_bwd(..., row_of))."""
    _need_cuda(xp, w_gate, w_up, w_down, offsets, g, u, h, dyp)
    R, d = xp.shape
    E, _, F = w_gate.shape
    dt = MOE_MXFP8 if mxfp8 else _dt(xp)
    context(xp.device.index).ensure_ffn_bwd_workspace(E, R, d, F, dt)
    if out is None:
        dev, tdt = xp.device, xp.dtype
        out = dict(dg=torch.empty(R, F, dtype=tdt, device=dev), du=torch.empty(R, F, dtype=tdt, device=dev),
                   dxp=torch.empty(R, d, dtype=tdt, device=dev),
                   dw_gate=torch.empty_like(w_gate), dw_up=torch.empty_like(w_up),
                   dw_down=torch.empty_like(w_down))
    outs = (_p(out["dg"]), _p(out["du"]), _p(out["dxp"]), _p(out["dw_gate"]), _p(out["dw_up"]),
            _p(out["dw_down"]))
    if router is None:
        context(xp.device.index).call("moe_grouped_ffn_bwd", _p(xp), _p(w_gate), _p(w_up), _p(w_down),
                                      _p(offsets), _p(g), _p(u), _p(h), _p(dyp), E, R, d, F, dt, *outs)
    else:
        dl_rows, w_router = router
        _need_cuda(dl_rows, w_router)
        if w_router.shape != (d, E):
            raise MoeError(f"w_router must be [{d}, {E}], got {tuple(w_router.shape)}")
        if dl_rows.numel() < R or dl_rows.dtype != torch.float32:
            raise MoeError("dl_rows must be fp32 with R entries")
        context(xp.device.index).call("moe_grouped_ffn_bwd_router", _p(xp), _p(w_gate), _p(w_up), _p(w_down),
                                      _p(offsets), _p(g), _p(u), _p(h), _p(dyp), _p(dl_rows),
                                      _p(w_router), E, R, d, F, dt, *outs)
    return out


def moe_permute_bwd(dxp, row_of, topk_idx=None, dlogits_sel=None, w_router=None, dx=None, dx_shared=None):
    """dx = sum_j dxp[row_of] (+ dx_shared) (+ the router term)."""
    _need_cuda(dxp, row_of, topk_idx, dlogits_sel, w_router, dx_shared)
    T, k = row_of.shape
    d = dxp.shape[1]
    E = w_router.shape[1] if w_router is not None else 1
    if dx is None:
        dx = torch.empty(T, d, dtype=dxp.dtype, device=dxp.device)
    ctx = context(dxp.device.index)
    if w_router is not None:
        ctx.ensure_workspace(T, d, E, min(k, E), _dt(dxp))
    if dx_shared is None:
        ctx.call("moe_permute_bwd", _p(dxp), _p(row_of), _p(topk_idx), _p(dlogits_sel), _p(w_router),
                 T, d, E, k, _dt(dxp), _p(dx))
    else:
        ctx.call("moe_permute_bwd_shared", _p(dxp), _p(row_of), _p(topk_idx), _p(dlogits_sel),
                 _p(w_router), _p(dx_shared), T, d, E, k, _dt(dxp), _p(dx))
    return dx


def moe_router_wgrad(x, dlogits_sel, src_tk, offsets, E, dw_router=None):
    _need_cuda(x, dlogits_sel, src_tk, offsets)
    T, d = x.shape
    k = dlogits_sel.shape[1]
    if dw_router is None:
        dw_router = torch.empty(d, E, dtype=x.dtype, device=x.device)
    context(x.device.index).ensure_workspace(T, d, E, min(k, E), _dt(x))
    context(x.device.index).call("moe_router_wgrad", _p(x), _p(dlogits_sel), _p(src_tk), _p(offsets),
                                 T, d, E, k, _dt(x), _p(dw_router))
    return dw_router


def mx_kpad(rows, groups):
    """Leading dimension of a column-quantised MXFP8 operand."""
    return (rows + 127 * groups + 127 + 127) // 128 * 128


def moe_mx_quantize(src, axis, group_offsets=None, groups=1):
    """MXFP8 quantisation of a bf16 [rows, cols] tensor.  axis 0 -> (codes
    [rows, cols], scales [rows, cols/32]); axis 1 -> (codes [cols, kpad],
    scales [cols, kpad/32]) with per-group 128-padded K positions."""
    _need_cuda(src, group_offsets)
    rows, cols = src.shape
    dev = src.device
    if axis == 0:
        kp = 0
        codes = torch.empty(rows, cols, dtype=torch.uint8, device=dev)
        scales = torch.empty(rows, cols // 32, dtype=torch.uint8, device=dev)
    else:
        kp = mx_kpad(rows, groups)
        codes = torch.empty(cols, kp, dtype=torch.uint8, device=dev)
        scales = torch.empty(cols, kp // 32, dtype=torch.uint8, device=dev)
    context(dev.index).call("moe_mx_quantize", _p(src), rows, cols, axis, _p(group_offsets), groups,
                            _p(codes), _p(scales), kp)
    return codes, scales


def moe_route_stats(logits, counts, k, alpha, out=None):
    """Returns dict(prob_mean [E] fp32, top1_count [E] int32, top1_prob_mean
    [E] fp32, aux_loss [1] fp32), all on the GPU."""
    _need_cuda(logits, counts)
    T, E = logits.shape
    dev = logits.device
    if out is None:
        out = dict(prob_mean=torch.empty(E, dtype=torch.float32, device=dev),
                   top1_count=torch.empty(E, dtype=torch.int32, device=dev),
                   top1_prob_mean=torch.empty(E, dtype=torch.float32, device=dev),
                   aux_loss=torch.empty(1, dtype=torch.float32, device=dev))
    ctx = context(dev.index)
    ctx.ensure_workspace(T, 8, E, min(k, E), MOE_F32)
    ctx.call("moe_route_stats", _p(logits), _p(counts), T, E, k, float(alpha), _p(out["prob_mean"]),
             _p(out["top1_count"]), _p(out["top1_prob_mean"]), _p(out["aux_loss"]))
    return out


def moe_aux_loss_bwd(logits, counts, k, alpha, dloss=1.0, dlogits=None):
    """Dense [T,E] fp32 logit gradient of dloss * aux_loss."""
    _need_cuda(logits, counts)
    T, E = logits.shape
    if dlogits is None:
        dlogits = torch.empty(T, E, dtype=torch.float32, device=logits.device)
    context(logits.device.index).call("moe_aux_loss_bwd", _p(logits), _p(counts), T, E, k, float(alpha),
                                      float(dloss), _p(dlogits))
    return dlogits


def moe_router_dense_bwd(x, w_router, dlogits, dx, dw_router):
    """Add the router's share of a dense [T,E] logit gradient in place:
    dx += dlogits @ w_router^T, dw_router += x^T @ dlogits."""
    _need_cuda(x, w_router, dlogits, dx, dw_router)
    T, d = x.shape
    E = w_router.shape[1]
    ctx = context(x.device.index)
    ctx.ensure_workspace(T, d, E, 1, _dt(x))
    ctx.call("moe_router_dense_bwd", _p(x), _p(w_router), _p(dlogits), T, d, E, _dt(x), _p(dx),
             _p(dw_router))
    return dx, dw_router


def moe_expert_grad_norms(dw, norms=None):
    """Per-expert L2 norms [E] fp32 of a [E, rows, cols] weight gradient."""
    _need_cuda(dw)
    E, rows, cols = dw.shape
    if norms is None:
        norms = torch.empty(E, dtype=torch.float32, device=dw.device)
    ctx = context(dw.device.index)
    ctx.ensure_workspace(1, 8, E, 1, MOE_F32)
    ctx.call("moe_expert_grad_norms", _p(dw), E, rows, cols, _dt(dw), _p(norms))
    return norms


# ------------------------------------------------------------------ the layer
@dataclass
class LayerBuffers:
    """Every device buffer of one forward+backward, allocated once."""
    logits: torch.Tensor
    route: dict
    xp: torch.Tensor
    ffn: dict
    y: torch.Tensor
    dyp: torch.Tensor
    dgates: torch.Tensor
    dlogits_sel: torch.Tensor
    bwd: dict
    dx: torch.Tensor
    dw_router: torch.Tensor
    xq: torch.Tensor | None = None  # MXFP8 codes of xp (quantise-on-permute)
    xs: torch.Tensor | None = None  # their scale bytes
    shared: dict | None = None      # shared expert: offsets {0,T}, its forward and backward buffers
    dl_rows: torch.Tensor | None = None  # logit gradients in expert-row order (bf16 router fold)
    aux_dl: torch.Tensor | None = None   # dense [T,E] balance-loss logit gradient (aux_alpha)
    wpack: MxWeightPack | None = None    # MXFP8: the expert weights quantised once per step


def alloc_layer(T, d, E, k, F, dtype, device, mxfp8=False, shared_F=0):
    """Every buffer of one forward+backward; shared_F > 0 adds a shared
    expert of width shared_F (weights [1,d,shared_F] and [1,shared_F,d])."""
    dev = torch.device(device)
    R = T * k
    z = lambda *s, dt=dtype: torch.empty(*s, dtype=dt, device=dev)  # noqa: E731
    route = dict(topk_idx=z(T, k, dt=torch.int32), gates=z(T, k, dt=torch.float32),
                 counts=z(E, dt=torch.int32), offsets=z(E + 1, dt=torch.int32),
                 row_of=z(T, k, dt=torch.int32), src_tk=z(max(R, 1), dt=torch.int32))
    ffn = dict(g=z(R, F), u=z(R, F), h=z(R, F), yp=z(R, d))
    bwd = dict(dg=z(R, F), du=z(R, F), dxp=z(R, d), dw_gate=z(E, d, F), dw_up=z(E, d, F),
               dw_down=z(E, F, d))
    buf = LayerBuffers(logits=z(T, E, dt=torch.float32), route=route, xp=z(R, d), ffn=ffn, y=z(T, d),
                       dyp=z(R, d), dgates=z(T, k, dt=torch.float32),
                       dlogits_sel=z(T, k, dt=torch.float32), bwd=bwd, dx=z(T, d), dw_router=z(d, E),
                       dl_rows=z(R, dt=torch.float32))
    if shared_F:
        Fs = shared_F
        buf.shared = dict(offsets=torch.tensor([0, T], dtype=torch.int32, device=dev),
                          ffn=dict(g=z(T, Fs), u=z(T, Fs), h=z(T, Fs), yp=z(T, d)),
                          bwd=dict(dg=z(T, Fs), du=z(T, Fs), dxp=z(T, d), dw_gate=z(1, d, Fs),
                                   dw_up=z(1, d, Fs), dw_down=z(1, Fs, d)))
    if mxfp8:
        buf.xq = z(R, d, dt=torch.uint8)
        buf.xs = z(R, d // 32, dt=torch.uint8)
        buf.wpack = MxWeightPack(z(moe_mx_weight_pack_size(E, d, F, dev.index), dt=torch.uint8), E, d, F)
        context(dev.index).ensure_mx_workspace(E, R, d, F)
        if shared_F:
            n = moe_mx_weight_pack_size(1, d, shared_F, dev.index)
            buf.shared["wpack"] = MxWeightPack(z(n, dt=torch.uint8), 1, d, shared_F)
            context(dev.index).ensure_mx_workspace(1, T, d, shared_F)
    return buf


def saved_activation_bytes(buf: LayerBuffers, recompute=False):
    """Bytes the forward keeps for the backward (besides x and the weights):
    routing metadata, gates, the routed yp (for the gate gradient) and,
    without recompute, xp and g, u, h (and the shared expert's g, u, h)."""
    r = buf.route
    keep = [r["topk_idx"], r["gates"], r["counts"], r["offsets"], r["row_of"], r["src_tk"], buf.ffn["yp"]]
    if not recompute:
        keep += [buf.xp, buf.ffn["g"], buf.ffn["u"], buf.ffn["h"]]
        if buf.shared is not None:
            keep += [buf.shared["ffn"][k] for k in ("g", "u", "h")]
    return sum(t.numel() * t.element_size() for t in keep)


def layer_forward(x, w_router, w_gate, w_up, w_down, k, buf: LayerBuffers, logits_override=None,
                  mxfp8=False, shared=None):
    """Router scores -> route -> permute -> grouped SwiGLU experts -> combine.
    `logits_override` (optional [T,E] fp32 on the GPU) replaces the router
    scores as the routing input after the router GEMM has run.  mxfp8=True
    (buffers from alloc_layer(..., mxfp8=True)) quantises the expert weights
    once into buf.wpack (both layouts, for this forward and the backward of
    the step), quantises on the permute and runs the MXFP8 expert GEMMs.  shared = (w_gate, w_up, w_down) of a shared
    expert (buffers from alloc_layer(..., shared_F=F_s)) runs it over every
    token as one group and adds its rows in the combine."""
    moe_router_logits(x, w_router, buf.logits)
    moe_route(buf.logits if logits_override is None else logits_override, k, buf.route)
    if mxfp8:
        # the weights are quantised once here, in both layouts; the backward
        # of this step reads the same pack
        moe_mx_quantize_weights(w_gate, w_up, w_down, buf.wpack)
        moe_permute_mx(x, buf.route["row_of"], buf.xp, buf.xq, buf.xs)
        moe_grouped_ffn_fwd_mxp(buf.wpack, buf.route["offsets"], xp_codes=buf.xq, xp_scales=buf.xs, out=buf.ffn)
    else:
        moe_permute(x, buf.route["row_of"], buf.xp)
        moe_grouped_ffn_fwd(buf.xp, w_gate, w_up, w_down, buf.route["offsets"], buf.ffn)
    ys = None
    if shared is not None:
        if mxfp8:
            moe_mx_quantize_weights(*shared, buf.shared["wpack"])
            moe_grouped_ffn_fwd_mxp(buf.shared["wpack"], buf.shared["offsets"], xp=x, out=buf.shared["ffn"])
        else:
            moe_grouped_ffn_fwd(x, *shared, buf.shared["offsets"], buf.shared["ffn"])
        ys = buf.shared["ffn"]["yp"]
    moe_combine(buf.ffn["yp"], buf.route["gates"], buf.route["row_of"], buf.y, y_shared=ys)
    return buf.y


def layer_backward(dy, x, w_router, w_gate, w_up, w_down, buf: LayerBuffers, mxfp8=False, shared=None,
                   recompute=False, aux_alpha=None, mx_wgrad=True):
    """combine_bwd -> route_bwd -> grouped FFN bwd -> permute_bwd (+router
    dgrad) -> router wgrad.  In bf16 the router's input-gradient term is
    folded into the gate/up dgrad (moe_grouped_ffn_bwd_router) and the
    permute backward only sums rows; fp32 and MXFP8 add it in the permute
    backward.  Returns dx; weight grads are in buf.bwd and
    buf.dw_router.  mxfp8: the weights are read from buf.wpack, which
    layer_forward of this step filled (run it after every weight change).  recompute=True reads from the forward only yp, the gates
    and the routing: xp is permuted again from x and g, u, h (the shared
    expert's too) are recomputed by the gate/up GEMM before they are used,
    so the forward need not keep them.  aux_alpha (the balance-loss weight)
    adds the gradient of that loss, taken at the router's scores with this
    step's counts, to dx and dW_r (moe_aux_loss_bwd, moe_router_dense_bwd).
    mx_wgrad=False (with mxfp8): MXFP8 on the data gradients only, the weight
    gradients from the bf16 operands (moe_grouped_ffn_bwd_mxp_bf16w)."""
    r = buf.route
    ffn_bwd_pack = moe_grouped_ffn_bwd_mxp if mx_wgrad else moe_grouped_ffn_bwd_mxp_bf16w
    if recompute:
        moe_permute(x, r["row_of"], buf.xp)
        if mxfp8:
            moe_grouped_ffn_fwd_mxp(buf.wpack, r["offsets"], xp=buf.xp, out=buf.ffn, up_only=True)
        else:
            moe_grouped_ffn_up(buf.xp, w_gate, w_up, r["offsets"], buf.ffn)
        if shared is not None:
            if mxfp8:
                moe_grouped_ffn_fwd_mxp(buf.shared["wpack"], buf.shared["offsets"], xp=x, out=buf.shared["ffn"],
                                        up_only=True)
            else:
                moe_grouped_ffn_up(x, shared[0], shared[1], buf.shared["offsets"], buf.shared["ffn"])
    moe_combine_bwd(dy, buf.ffn["yp"], r["gates"], r["row_of"], buf.dyp, buf.dgates)
    fold = not mxfp8 and buf.xp.dtype == torch.bfloat16
    if fold:
        moe_route_bwd(r["gates"], buf.dgates, buf.dlogits_sel, row_of=r["row_of"], dl_rows=buf.dl_rows)
    else:
        moe_route_bwd(r["gates"], buf.dgates, buf.dlogits_sel)
    if mxfp8:
        ffn_bwd_pack(buf.xp, buf.wpack, r["offsets"], buf.ffn["g"], buf.ffn["u"], buf.ffn["h"], buf.dyp, buf.bwd)
    else:
        moe_grouped_ffn_bwd(buf.xp, w_gate, w_up, w_down, r["offsets"], buf.ffn["g"], buf.ffn["u"],
                            buf.ffn["h"], buf.dyp, buf.bwd, router=(buf.dl_rows, w_router) if fold else None)
    dxs = None
    if shared is not None:
        sh = buf.shared
        if mxfp8:
            ffn_bwd_pack(x, sh["wpack"], sh["offsets"], sh["ffn"]["g"], sh["ffn"]["u"], sh["ffn"]["h"], dy,
                         sh["bwd"])
        else:
            moe_grouped_ffn_bwd(x, *shared, sh["offsets"], sh["ffn"]["g"], sh["ffn"]["u"], sh["ffn"]["h"], dy,
                                sh["bwd"])
        dxs = sh["bwd"]["dxp"]
    if fold:
        moe_permute_bwd(buf.bwd["dxp"], r["row_of"], dx=buf.dx, dx_shared=dxs)
    else:
        moe_permute_bwd(buf.bwd["dxp"], r["row_of"], r["topk_idx"], buf.dlogits_sel, w_router, buf.dx,
                        dx_shared=dxs)
    moe_router_wgrad(x, buf.dlogits_sel, r["src_tk"], r["offsets"], w_router.shape[1], buf.dw_router)
    if aux_alpha is not None:
        T, E = buf.logits.shape
        if buf.aux_dl is None:
            buf.aux_dl = torch.empty(T, E, dtype=torch.float32, device=buf.logits.device)
        moe_aux_loss_bwd(buf.logits, r["counts"], r["topk_idx"].shape[1], aux_alpha, 1.0, buf.aux_dl)
        moe_router_dense_bwd(x, w_router, buf.aux_dl, buf.dx, buf.dw_router)
    return buf.dx


def moe_mfma_peak_probe(blocks, iters, a=1.0, b=1.0, sink=None):
    """Launch the matrix-core rate probe: `blocks` blocks of four waves, each
    wave `iters` rounds of four v_mfma_f32_32x32x16_bf16 on register operands
    (32768 FLOPs each).  Returns the sink, one float per thread, equal to
    1024·a·b·iters (a and b as bf16) while that is exact in fp32."""
    if sink is None:
        sink = torch.empty(blocks * 256, dtype=torch.float32, device=f"cuda:{torch.cuda.current_device()}")
    _need_cuda(sink)
    if sink.dtype != torch.float32 or sink.numel() < blocks * 256:
        raise MoeError("sink must be float32 with at least blocks*256 elements")
    context().call("moe_mfma_peak_probe", blocks, iters, a, b, _p(sink))
    return sink
