"""Pins of the oracle's routing: softmax, top-k, gates, histogram, offsets and
the stable permutation, checked against independent formulations and the
invariants the method fixes (each token appears exactly k times, counts sum
to T*k, uniform routing gives uniform expected load)."""
import numpy as np
import pytest
from scipy import stats

import moe_inputs as mi
import oracle


def topk_by_argsort(logits, k):
    # Independent selection: stable sort of the negated logits keeps the
    # lower index first among equal logits (+0 and -0 compare equal).
    order = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def gates_selected_softmax(logits, topk):
    sel = np.take_along_axis(logits.astype(np.float64), topk, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def check_invariants(r, T, E, k):
    topk, counts, offsets = r["topk_idx"], r["counts"], r["offsets"]
    row_of, src_tk = r["row_of"], r["src_tk"]
    # counts sum to T*k and match a histogram of the selection
    assert counts.sum() == T * k
    assert np.array_equal(counts, np.bincount(topk.ravel(), minlength=E))
    # offsets are the exclusive scan of counts
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    # distinct experts per token
    assert all(len(set(row)) == k for row in topk.tolist())
    # row_of and src_tk are inverse permutations of [0, T*k)
    flat = row_of.ravel()
    assert np.array_equal(np.sort(flat), np.arange(T * k))
    assert np.array_equal(src_tk[flat], np.arange(T * k))
    # each token appears exactly k times in the expert buffers
    assert np.array_equal(np.bincount(src_tk // k, minlength=T), np.full(T, k))
    # rows of expert e hold exactly its (t,j) in ascending flat order
    for e in range(E):
        seg = src_tk[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(topk.ravel()[seg] == e)


@pytest.mark.parametrize("acc", ["f64", "f32"])
@pytest.mark.parametrize("T,E,k,seed", [(256, 8, 2, 0), (300, 16, 4, 1), (97, 5, 5, 2),
                                        (64, 1, 1, 3), (1, 128, 4, 4), (500, 128, 4, 5)])
def test_route_random(acc, T, E, k, seed):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    r = oracle.route(logits, k, acc)
    assert np.array_equal(r["topk_idx"], topk_by_argsort(logits, k))
    np.testing.assert_allclose(r["gates"], gates_selected_softmax(logits, r["topk_idx"]),
                               rtol=0, atol=1e-6 if acc == "f32" else 1e-14)
    np.testing.assert_allclose(r["gates"].sum(axis=1), 1.0, atol=1e-6)
    assert np.all(np.diff(r["gates"], axis=1) <= 1e-7)
    check_invariants(r, T, E, k)


def test_route_full_softmax_then_renormalise():
    # The gates equal the full softmax over E restricted to the selection and
    # renormalised (scipy softmax as the independent formulation).
    rng = np.random.default_rng(7)
    logits = (3 * rng.standard_normal((200, 32))).astype(np.float32)
    r = oracle.route(logits, 4)
    from scipy.special import softmax
    p = softmax(logits.astype(np.float64), axis=1)
    sel = np.take_along_axis(p, r["topk_idx"], axis=1)
    np.testing.assert_allclose(r["gates"], sel / sel.sum(axis=1, keepdims=True), atol=1e-14)


def test_route_all_equal_rows():
    # Every logit equal: experts 0..k-1 in order, gates exactly 1/k.
    T, E, k = 50, 8, 4
    r = oracle.route(np.full((T, E), 0.25, dtype=np.float32), k)
    assert np.array_equal(r["topk_idx"], np.tile(np.arange(k, dtype=np.int32), (T, 1)))
    assert np.all(r["gates"] == 1.0 / k)
    assert np.array_equal(r["counts"], np.array([T] * k + [0] * (E - k)))


def test_route_integer_ties_and_signed_zero():
    rng = np.random.default_rng(11)
    T, E, k = 400, 16, 4
    logits = rng.integers(-2, 3, size=(T, E)).astype(np.float32)
    # sprinkle -0.0 where the value is 0 so +0/-0 ties occur
    z = (logits == 0) & (rng.random((T, E)) < 0.5)
    logits[z] = -0.0
    assert np.signbit(logits).any()
    r = oracle.route(logits, k)
    assert np.array_equal(r["topk_idx"], topk_by_argsort(logits, k))
    check_invariants(r, T, E, k)
    # hand case: [0, -0, 1, 1] top-3 -> 2, 3, 0
    r2 = oracle.route(np.array([[0.0, -0.0, 1.0, 1.0]], dtype=np.float32), 3)
    assert r2["topk_idx"].tolist() == [[2, 3, 0]]


def test_route_one_expert_takes_everything():
    T, E = 300, 8
    logits = np.zeros((T, E), dtype=np.float32)
    logits[:, 5] = 10.0
    r = oracle.route(logits, 1)
    assert np.all(r["topk_idx"] == 5) and r["counts"][5] == T
    assert np.all(r["gates"] == 1.0)
    assert np.array_equal(r["src_tk"], np.arange(T))


def test_route_k_equals_E_is_full_softmax():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((40, 6)).astype(np.float32)
    r = oracle.route(logits, 6)
    from scipy.special import softmax
    p = softmax(logits.astype(np.float64), axis=1)
    np.testing.assert_allclose(np.take_along_axis(p, r["topk_idx"], axis=1), r["gates"], atol=1e-14)
    assert np.all(r["counts"] == 40)


def test_uniform_routing_gives_uniform_load():
    # i.i.d. logits: by exchangeability each expert is selected with
    # probability exactly k/E; counts ~ Binomial(T, k/E) per expert.
    cfg = mi.config("uniform128")
    inp = mi.layer_inputs(cfg, with_weights=False)
    r = oracle.route(inp["logits"].numpy(), cfg.k, "f32")
    c = r["counts"]
    mean = cfg.T * cfg.k / cfg.E
    sd = np.sqrt(cfg.T * (cfg.k / cfg.E) * (1 - cfg.k / cfg.E))
    assert np.all(np.abs(c - mean) < 6 * sd)
    chi2 = ((c - mean) ** 2 / mean).sum()
    assert stats.chi2.sf(chi2, cfg.E - 1) > 1e-4
    check_invariants(r, cfg.T, cfg.E, cfg.k)


def test_zipf_routing_skew_and_empty_groups():
    cfg = mi.config("zipf128")
    inp = mi.layer_inputs(cfg, with_weights=False)
    r = oracle.route(inp["logits"].numpy(), cfg.k, "f32")
    c = r["counts"]
    mean = cfg.T * cfg.k / cfg.E
    assert (c == 0).sum() == cfg.n_dead
    assert (c > 5 * mean).sum() >= 3
    assert c.max() > 15 * mean
    check_invariants(r, cfg.T, cfg.E, cfg.k)


def test_router_logits_against_matmul():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((33, 40)).astype(np.float32)
    wr = rng.standard_normal((40, 7)).astype(np.float32)
    ref = (x.astype(np.float64) @ wr.astype(np.float64)).astype(np.float32)
    assert np.array_equal(oracle.router_logits(x, wr, "f64"), ref)
    np.testing.assert_allclose(oracle.router_logits(x, wr, "f32"), ref, rtol=1e-5, atol=1e-5)
