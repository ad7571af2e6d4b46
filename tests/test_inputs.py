"""The seeded workload generators: determinism and the stated structure."""
import numpy as np
import torch

import moe_inputs as mi


def test_deterministic_and_dtypes():
    a = mi.layer_inputs(mi.config("tiny"))
    b = mi.layer_inputs(mi.config("tiny"))
    for key in ("x", "wr", "wg", "wu", "wd", "dy"):
        assert torch.equal(a[key], b[key])
        assert a[key].dtype == torch.float32
    c = mi.layer_inputs(mi.config("tiny", T=64, d=64, dtype="bf16"))
    assert c["x"].dtype == torch.bfloat16 and c["x"].shape == (64, 64)
    # stated distributions (tiny: every input N(0, 0.02^2), dy N(0, 1))
    assert abs(a["x"].std().item() - 0.02) < 0.002
    assert abs(a["dy"].std().item() - 1.0) < 0.02


def test_mx_counts():
    c = mi.mx_counts()
    assert c.sum() == 65536
    assert sorted(c.tolist(), reverse=True)[:5] == [15164, 8709, 6297, 5002, 4184]
    assert (c % 32 != 0).sum() >= 15
    assert abs(c.max() / c.mean() - 3.70) < 0.01


def test_largest_remainder():
    p = np.array([0.5, 0.3, 0.2])
    assert mi.largest_remainder(10, p).tolist() == [5, 3, 2]
    assert mi.largest_remainder(7, p).sum() == 7
