"""Pins of the oracle's shared expert ([P1] 四: shared experts): it must
equal the oracle's token-by-token layer with a single expert that every
token selects with gate 1 (an independent code path of the oracle), and the
sum routed + shared must be linear in the two parts."""
import numpy as np

import oracle


def _weights(rng, E, d, F):
    s = 1 / np.sqrt(d)
    return (rng.standard_normal((E, d, F)) * s, rng.standard_normal((E, d, F)) * s,
            rng.standard_normal((E, F, d)) / np.sqrt(F))


def test_shared_expert_equals_single_expert_layer():
    rng = np.random.default_rng(21)
    T, d, F = 37, 16, 24
    x = rng.standard_normal((T, d)).astype(np.float32)
    dy = rng.standard_normal((T, d)).astype(np.float32)
    wg, wu, wd = (w.astype(np.float32) for w in _weights(rng, 1, d, F))
    wr = rng.standard_normal((d, 1)).astype(np.float32)
    topk = np.zeros((T, 1), dtype=np.int32)
    gates = np.ones((T, 1))
    f = oracle.shared_expert_fwd(x, wg, wu, wd)
    np.testing.assert_allclose(f["yp"], oracle.layer_fwd(x, topk, gates, wg, wu, wd), rtol=1e-12, atol=1e-12)
    b = oracle.shared_expert_bwd(x, dy, wg, wu, wd)
    ref = oracle.layer_bwd(x, wr, topk, gates, dy, wg, wu, wd)
    # one expert with gate 1: the router gradient vanishes, so the layer's
    # dx is the expert's own input gradient
    assert np.abs(ref["dlogits_sel"]).max() < 1e-12
    np.testing.assert_allclose(b["dx"], ref["dx"], rtol=1e-10, atol=1e-12)
    for k in ("dwg", "dwu", "dwd"):
        np.testing.assert_allclose(b[k], ref[k], rtol=1e-10, atol=1e-12)


def test_shared_expert_row_independence():
    # each token's shared output depends on its own row only: permuting the
    # tokens permutes the outputs
    rng = np.random.default_rng(22)
    T, d, F = 20, 8, 16
    x = rng.standard_normal((T, d)).astype(np.float32)
    wg, wu, wd = (w.astype(np.float32) for w in _weights(rng, 1, d, F))
    perm = rng.permutation(T)
    a = oracle.shared_expert_fwd(x, wg, wu, wd)["yp"]
    b = oracle.shared_expert_fwd(x[perm], wg, wu, wd)["yp"]
    np.testing.assert_allclose(b, a[perm], rtol=1e-13, atol=1e-13)
