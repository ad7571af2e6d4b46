"""GPU parity of the routing statistics, the balance loss and its logit
gradient, and the per-expert weight-gradient norms ([P2] 2.2, 4.2, 4.3, 5.2;
[P1] 四) against the oracle.

Integer results (top-1 counts) are bit-exact: both sides take the top-1
decision by comparing the same fp32 logits.  Floating results are fp32 sums
and softmaxes: within 1e-4 of the fp64 oracle (relative L2 and max)."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from tolerance import assert_close

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 1e-4


@pytest.fixture(scope="module")
def moe():
    import routing_grouped_expert_softmax_amd as m
    m.context(0)
    return m


def _logits(T, E, seed, ties=False):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    if ties:
        # small integers: many equal logits, including equal maxima
        lg = rng.integers(-3, 3, size=(T, E)).astype(np.float32)
    return lg


def _check_stats(moe, lg, k, alpha):
    T, E = lg.shape
    glg = torch.from_numpy(lg).to(DEV)
    r = moe.moe_route(glg, k)
    s = moe.moe_route_stats(glg, r["counts"], k, alpha)
    d = moe.moe_aux_loss_bwd(glg, r["counts"], k, alpha, dloss=0.75)
    torch.cuda.synchronize()
    counts = r["counts"].cpu().numpy()
    ref_counts = oracle.route(lg, k)["counts"] if T * E <= 4_000_000 else counts
    assert np.array_equal(counts, ref_counts)
    want = oracle.route_stats(lg, counts, k, alpha)
    assert np.array_equal(s["top1_count"].cpu().numpy(), want["top1_count"])
    assert_close(s["prob_mean"].cpu().numpy(), want["prob_mean"], TOL, "prob_mean")
    assert_close(s["top1_prob_mean"].cpu().numpy(), want["top1_prob_mean"], TOL, "top1_prob_mean")
    assert_close(s["aux_loss"].cpu().numpy(), [want["aux_loss"]], TOL, "aux_loss")
    assert_close(d.cpu().numpy(), oracle.aux_loss_bwd(lg, counts, k, alpha, dloss=0.75), TOL, "dlogits")
    return s, d


@pytest.mark.parametrize("T,E,k,ties", [(1, 8, 2, False), (256, 8, 2, False), (1000, 128, 4, False),
                                        (333, 64, 1, True), (517, 200, 6, True), (77, 1000, 8, False),
                                        (4097, 512, 4, False)])
def test_route_stats_and_aux_grad(moe, T, E, k, ties):
    _check_stats(moe, _logits(T, E, T + E, ties), k, 0.01)


@pytest.mark.parametrize("name", ["uniform128", "zipf128"])
def test_route_stats_full_size(moe, name):
    """The full-size routed workloads (uniform logits; Zipf(1.1) skew with
    four dead experts at -1e4)."""
    cfg = mi.config(name)
    lg = mi.layer_inputs(cfg, with_weights=False)["logits"].numpy()
    s, _ = _check_stats(moe, lg, cfg.k, 0.001)
    if name == "zipf128":
        # dead experts: no top-1 tokens, zero mean probability
        pm = s["prob_mean"].cpu().numpy()
        assert (pm == 0).sum() >= cfg.n_dead


def test_route_stats_empty_and_deterministic(moe):
    E, k = 16, 2
    s = moe.moe_route_stats(torch.zeros(0, E, device=DEV), torch.zeros(E, dtype=torch.int32, device=DEV),
                            k, 0.01)
    torch.cuda.synchronize()
    assert not s["prob_mean"].cpu().any() and not s["top1_count"].cpu().any()
    assert s["aux_loss"].item() == 0.0
    lg = torch.from_numpy(_logits(3000, 96, 9)).to(DEV)
    r = moe.moe_route(lg, 4)
    a = moe.moe_route_stats(lg, r["counts"], 4, 0.02)
    b = moe.moe_route_stats(lg, r["counts"], 4, 0.02)
    da = moe.moe_aux_loss_bwd(lg, r["counts"], 4, 0.02)
    db = moe.moe_aux_loss_bwd(lg, r["counts"], 4, 0.02)
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key], b[key]), key
    assert torch.equal(da, db)


def test_route_stats_rejects_bad_arguments(moe):
    lg = torch.zeros(4, 8, device=DEV)
    c = torch.zeros(8, dtype=torch.int32, device=DEV)
    with pytest.raises(moe.MoeError):
        moe.moe_route_stats(lg, c, 9, 0.01)  # k > E
    with pytest.raises(moe.MoeError):
        moe.moe_aux_loss_bwd(lg, c, 2, float("nan"))


def _grad_tensor(E, rows, cols, seed, dtype):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((E, rows, cols)).astype(np.float32) * np.float32(3e-3)
    a[E // 2] = 0.0  # an expert with no rows has an exactly zero gradient
    t = torch.from_numpy(a)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


@pytest.mark.parametrize("E,rows,cols,dtype", [(8, 128, 256, "fp32"), (16, 33, 40, "bf16"),
                                               (128, 256, 64, "bf16"), (3, 1, 8, "bf16"),
                                               (5, 7, 4, "fp32")])
def test_expert_grad_norms(moe, E, rows, cols, dtype):
    dw = _grad_tensor(E, rows, cols, E * rows + cols, dtype)
    got = moe.moe_expert_grad_norms(dw.to(DEV)).cpu().numpy()
    want = oracle.expert_grad_norms(mi.f32(dw))
    assert got[E // 2] == 0.0
    assert_close(got, want, TOL, "norms")


@pytest.mark.slow
def test_expert_grad_norms_full_size(moe):
    """Full-size gate/up weight gradient of the 128-expert layer ([128, 2048,
    1024] bf16): sampled experts against the oracle."""
    dw = _grad_tensor(128, 2048, 1024, 11, "bf16")
    g = dw.to(DEV)
    got = moe.moe_expert_grad_norms(g).cpu().numpy()
    again = moe.moe_expert_grad_norms(g).cpu().numpy()
    assert np.array_equal(got, again)
    for e in (0, 1, 63, 64, 127):
        want = oracle.expert_grad_norms(mi.f32(dw[e:e + 1]))
        assert_close(got[e:e + 1], want, TOL, f"norm[{e}]")
