"""Pins of the oracle's routing statistics and balance loss ([P2] 2.2, 4.2,
4.3, 5.2; [P1] 四 and the negative-results section).

The pins come from outside the functions under test: a small example worked
by hand, the closed form at uniform load and probability, central finite
differences of the loss, the invariants of a softmax gradient, the C++
oracle's own routing (top-1 = first selected slot), and numpy's norm."""
import numpy as np
import pytest

import oracle


def test_hand_worked_example():
    # T=2, E=3, k=1.  Token 0: logits (0, ln 2, 0) -> p = (1/4, 1/2, 1/4),
    # top-1 expert 1.  Token 1: (ln 3, 0, 0) -> p = (3/5, 1/5, 1/5), top-1
    # expert 0.  counts (1, 1, 0), so f = (1/2, 1/2, 0);
    # prob_mean = (0.425, 0.35, 0.225); loss = alpha * 3 * 0.3875.
    lg = np.array([[0.0, np.log(2.0), 0.0], [np.log(3.0), 0.0, 0.0]])
    counts = np.array([1, 1, 0])
    s = oracle.route_stats(lg, counts, 1, 0.01)
    np.testing.assert_allclose(s["prob_mean"], [0.425, 0.35, 0.225], rtol=1e-12)
    assert list(s["top1_count"]) == [1, 1, 0]
    np.testing.assert_allclose(s["top1_prob_mean"], [0.6, 0.5, 0.0], rtol=1e-12)
    assert s["aux_loss"] == pytest.approx(0.01 * 1.1625, rel=1e-12)
    # a = alpha*E*f/T = alpha*(0.75, 0.75, 0); token 0: <p,a> = 0.5625 alpha,
    # token 1: <p,a> = 0.6 alpha
    d = oracle.aux_loss_bwd(lg, counts, 1, 0.01)
    np.testing.assert_allclose(d, 0.01 * np.array([[0.046875, 0.09375, -0.140625],
                                                   [0.09, 0.03, -0.12]]), rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("E,k", [(8, 2), (128, 4), (5, 5)])
def test_uniform_closed_form(E, k):
    # equal logits: p = 1/E everywhere, every token's top-1 is expert 0 (lower
    # index first); with equal counts the loss is alpha exactly and its
    # gradient vanishes
    T = 16 * E
    lg = np.zeros((T, E), dtype=np.float32)
    counts = np.full(E, T * k // E)
    s = oracle.route_stats(lg, counts, k, 0.02)
    np.testing.assert_allclose(s["prob_mean"], 1.0 / E, rtol=1e-14)
    assert s["top1_count"][0] == T and not s["top1_count"][1:].any()
    assert s["top1_prob_mean"][0] == pytest.approx(1.0 / E, rel=1e-14)
    assert s["aux_loss"] == pytest.approx(0.02, rel=1e-14)
    assert np.abs(oracle.aux_loss_bwd(lg, counts, k, 0.02)).max() < 1e-18


def test_gradient_matches_finite_differences():
    rng = np.random.default_rng(3)
    T, E, k, alpha = 6, 7, 2, 0.05
    lg = rng.standard_normal((T, E))
    counts = oracle.route(lg.astype(np.float32), k)["counts"]
    d = oracle.aux_loss_bwd(lg, counts, k, alpha, dloss=1.7)
    h = 1e-5
    for t in range(T):
        for e in range(E):
            up, dn = lg.copy(), lg.copy()
            up[t, e] += h
            dn[t, e] -= h
            fd = (oracle.route_stats(up, counts, k, alpha)["aux_loss"]
                  - oracle.route_stats(dn, counts, k, alpha)["aux_loss"]) / (2 * h)
            assert 1.7 * fd == pytest.approx(d[t, e], rel=1e-6, abs=1e-11), (t, e)


def test_invariants_and_top1_against_routing():
    rng = np.random.default_rng(4)
    T, E, k = 300, 16, 3
    lg = rng.standard_normal((T, E)).astype(np.float32)
    # every 7th token: experts 2 and 5 share the largest logit (lower index first)
    lg[::7, 2] = lg[::7].max(axis=1) + 1
    lg[::7, 5] = lg[::7, 2]
    r = oracle.route(lg, k)
    s = oracle.route_stats(lg, r["counts"], k, 0.01)
    assert np.array_equal(oracle.top1_expert(lg), r["topk_idx"][:, 0])
    assert s["prob_mean"].sum() == pytest.approx(1.0, rel=1e-13)
    assert s["top1_count"].sum() == T
    # the largest of E probabilities is at least 1/E
    assert np.all(s["top1_prob_mean"][s["top1_count"] > 0] >= 1.0 / E - 1e-12)
    d = oracle.aux_loss_bwd(lg, r["counts"], k, 0.01)
    np.testing.assert_allclose(d.sum(axis=1), 0.0, atol=1e-18)


def test_expert_grad_norms():
    rng = np.random.default_rng(5)
    dw = rng.standard_normal((4, 33, 40)).astype(np.float32)
    dw[2] = -0.5
    dw[3] = 0.0
    n = oracle.expert_grad_norms(dw)
    assert n[2] == pytest.approx(0.5 * np.sqrt(33 * 40), rel=1e-14)
    assert n[3] == 0.0
    for e in range(4):
        assert n[e] == pytest.approx(np.linalg.norm(dw[e].astype(np.float64)), rel=1e-13)


# ---------------------------------------------------------------- balance loss -> router
def _aux_of(x, wr, counts, k, alpha):
    return oracle.route_stats(x @ wr, counts, k, alpha)["aux_loss"]


def test_router_dense_bwd_matches_finite_differences():
    # The balance loss as a function of the router's inputs, loss(x W_r) with
    # the counts held at their routed values (piecewise constant): central
    # differences in x and in W_r against router_dense_bwd of the loss's
    # dense logit gradient.
    rng = np.random.default_rng(11)
    T, d, E, k, alpha, dloss = 9, 5, 6, 2, 0.07, 1.3
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((d, E)) * 0.5
    counts = oracle.route((x @ wr).astype(np.float32), k)["counts"]
    g = oracle.router_dense_bwd(x, wr, oracle.aux_loss_bwd(x @ wr, counts, k, alpha, dloss))
    assert g["dx"].shape == (T, d) and g["dwr"].shape == (d, E)
    h = 1e-6
    for (t, i) in [(0, 0), (3, 4), (8, 2), (5, 1)]:
        up, dn = x.copy(), x.copy()
        up[t, i] += h
        dn[t, i] -= h
        fd = (_aux_of(up, wr, counts, k, alpha) - _aux_of(dn, wr, counts, k, alpha)) / (2 * h)
        assert dloss * fd == pytest.approx(g["dx"][t, i], rel=1e-6, abs=1e-12), (t, i)
    for i in range(d):
        for e in range(E):
            up, dn = wr.copy(), wr.copy()
            up[i, e] += h
            dn[i, e] -= h
            fd = (_aux_of(x, up, counts, k, alpha) - _aux_of(x, dn, counts, k, alpha)) / (2 * h)
            assert dloss * fd == pytest.approx(g["dwr"][i, e], rel=1e-6, abs=1e-12), (i, e)


def test_router_dense_bwd_pin_sees_planted_mistakes():
    # the finite-difference reference differs clearly from plausible slips:
    # a dropped transpose in dx (square case) or dl summed without x
    rng = np.random.default_rng(12)
    T, d, E, k, alpha = 7, 6, 6, 2, 0.05
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((d, E))
    counts = oracle.route((x @ wr).astype(np.float32), k)["counts"]
    dl = oracle.aux_loss_bwd(x @ wr, counts, k, alpha)
    h = 1e-6
    fd_dx = np.zeros((T, d))
    for t in range(T):
        for i in range(d):
            up, dn = x.copy(), x.copy()
            up[t, i] += h
            dn[t, i] -= h
            fd_dx[t, i] = (_aux_of(up, wr, counts, k, alpha) - _aux_of(dn, wr, counts, k, alpha)) / (2 * h)
    good = oracle.router_dense_bwd(x, wr, dl)["dx"]
    assert np.abs(good - fd_dx).max() < 1e-8 * np.abs(fd_dx).max() + 1e-14
    assert np.abs(dl @ wr - fd_dx).max() > 0.1 * np.abs(fd_dx).max()   # W_r not transposed
