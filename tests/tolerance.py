"""Parity measures shared by the tests.

Floating point: per tensor, in fp64, the relative L2 error
||a-b|| / ||b|| must be <= tol AND max|a-b| <= tol * max|b|; where the
reference is exactly zero the result must be exactly zero.
"""
import numpy as np


def rel_errors(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    diff = a - b
    nb = np.linalg.norm(b)
    mb = np.abs(b).max() if b.size else 0.0
    l2 = np.linalg.norm(diff) / nb if nb > 0 else np.linalg.norm(diff)
    mx = np.abs(diff).max() / mb if mb > 0 else (np.abs(diff).max() if diff.size else 0.0)
    return float(l2), float(mx)


def assert_close(a, b, tol, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    if not np.any(b):
        assert not np.any(a), f"{what}: reference is exactly zero, result is not"
        return
    l2, mx = rel_errors(a, b)
    assert l2 <= tol and mx <= tol, f"{what}: rel L2 {l2:.3e}, rel max {mx:.3e} > {tol}"
    return l2, mx
