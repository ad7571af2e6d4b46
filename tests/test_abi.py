"""The C-ABI library loads and exports every entry point include/moe.h
declares; status strings and host-side rejection without a GPU."""
import ctypes
import os
import re

import pytest

import routing_grouped_expert_softmax_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_symbols()
    for n in ["moe_route", "moe_permute", "moe_grouped_ffn_fwd", "moe_grouped_ffn_bwd", "moe_combine",
              "moe_combine_bwd", "moe_route_bwd", "moe_permute_bwd", "moe_router_logits",
              "moe_router_wgrad"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    L = moe.lib()
    missing = [n for n in declared_symbols() if not hasattr(L, n)]
    assert not missing, missing
    assert set(declared_symbols()) == set(moe.EXPORTS)
    names = [L.moe_kernel_name(i).decode() for i in range(len(moe.KERNELS))]
    assert names == moe.KERNELS
    assert L.moe_kernel_name(len(moe.KERNELS)) == b"unknown"


def test_status_strings_and_null_context():
    L = moe.lib()
    assert L.moe_status_string(0) == b"ok"
    assert L.moe_status_string(1) == b"invalid argument"
    assert L.moe_status_string(3).startswith(b"workspace")
    assert L.moe_last_error(None) == b"null context"
    # every call rejects a null context on the host, without touching a GPU
    v = ctypes.c_void_p
    assert L.moe_route(None, None, 1, 1, 1, None, None, None, None, None, None) == 1
    assert L.moe_permute(None, None, None, 1, 8, 1, 1, None) == 1
    assert L.moe_destroy(None) == 1
    out = v()
    assert L.moe_create(-1, None, ctypes.byref(out)) == 1 and out.value is None


def test_no_cpu_fallback_without_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(moe.MoeError):
        moe.context(0)


def test_library_has_no_unresolved_kernels():
    """Every kernel launched from host code is defined in the library (a
    kernel whose stub the host pass failed to emit would be an undefined
    symbol that only fails at load time)."""
    import subprocess
    import routing_grouped_expert_softmax_amd as m
    ctypes.CDLL(m.LIB_PATH, mode=os.RTLD_NOW)
    out = subprocess.run(["nm", "-C", "--undefined-only", m.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    bad = [ln for ln in out.splitlines() if "anonymous namespace" in ln or "moe" in ln]
    assert not bad, bad
