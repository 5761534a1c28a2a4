"""Pins of the oracle's auxiliary load-balancing loss.

PARITY UNPINNED as to the formula: the lesson "专家组合 (MoE)" (Load balancing
item 1, Key terms) and the explainer pages name a penalty on uneven expert
usage but print no formula.  The oracle takes the Switch/GShard form
L = alpha * E/(T*k) * sum_e counts_e * mean_t p[t,e]; these tests pin that
definition's closed forms and its gradients (finite differences, autograd)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from workloads import CONFIGS, make_inputs, scaled


def test_balanced_usage_costs_alpha_and_collapse_costs_alpha_times_E():
    T, E, k, alpha = 64, 8, 2, 0.01
    counts = np.full(E, T * k // E)
    uniform = np.zeros((T, E))                       # every expert equally likely
    assert oracle.aux_loss(uniform, counts, k, "softmax", alpha) == pytest.approx(alpha, rel=1e-14)
    collapsed = np.full((T, E), -60.0)
    collapsed[:, 0] = 60.0                           # probability ~1 on expert 0, which takes every token
    c1 = np.zeros(E)
    c1[0] = T
    assert oracle.aux_loss(collapsed, c1, 1, "softmax", alpha) == pytest.approx(alpha * E, rel=1e-12)


@pytest.mark.parametrize("fn", oracle.SCORE_FNS)
def test_aux_gradient_matches_finite_differences(fn):
    rng = np.random.default_rng(1)
    T, E, k, alpha = 20, 7, 3, 0.3
    l = rng.standard_normal((T, E))
    counts = rng.integers(0, 12, E)
    g = oracle.aux_grad_logits(l, counts, k, fn, alpha)
    h = 1e-6
    for _ in range(25):
        i = (int(rng.integers(0, T)), int(rng.integers(0, E)))
        lp, lm = l.copy(), l.copy()
        lp[i] += h
        lm[i] -= h
        fd = (oracle.aux_loss(lp, counts, k, fn, alpha) - oracle.aux_loss(lm, counts, k, fn, alpha)) / (2 * h)
        assert abs(fd - g[i]) <= 1e-9 + 1e-6 * abs(fd)


@pytest.mark.parametrize("fn", oracle.SCORE_FNS)
def test_aux_loss_and_gradient_match_torch(fn):
    rng = np.random.default_rng(2)
    T, E, k, alpha = 33, 9, 2, 0.05
    l = rng.standard_normal((T, E))
    counts = rng.integers(0, 10, E)
    lt = torch.tensor(l, requires_grad=True)
    if fn == "softmax":
        p = torch.softmax(lt, dim=1)
    else:
        s = torch.sigmoid(lt) if fn == "sigmoid" else torch.sqrt(F.softplus(lt, threshold=1000.0))
        p = s / s.sum(dim=1, keepdim=True)
    loss = alpha * E / (T * k) * (torch.tensor(counts, dtype=torch.float64) * p.mean(dim=0)).sum()
    loss.backward()
    assert oracle.aux_loss(l, counts, k, fn, alpha) == pytest.approx(float(loss.detach()), rel=1e-13)
    np.testing.assert_allclose(oracle.aux_grad_logits(l, counts, k, fn, alpha), lt.grad.numpy(), rtol=1e-11, atol=1e-15)


@pytest.mark.parametrize("fn", oracle.SCORE_FNS)
def test_layer_backward_with_aux_loss_matches_finite_differences(fn):
    cfg = scaled(CONFIGS["tiny"], T=24)
    inp = make_inputs(cfg)
    dy = np.random.default_rng(11).standard_normal((cfg.T, cfg.d))
    p = {k: np.asarray(inp[k], np.float64) for k in ("x", "w_router", "w_gate_up", "w_down")}
    alpha = 0.7

    def run():
        return oracle.forward(p["x"], p["w_router"], p["w_gate_up"], p["w_down"], cfg.k, fn, False,
                              sel_bias=inp["bias"])

    f0 = run()
    assert f0["margin"].min() > 1e-5
    g = oracle.backward(f0, dy, p["x"], p["w_router"], p["w_gate_up"], p["w_down"], fn, False, aux_alpha=alpha)

    def total():
        o = run()
        assert np.array_equal(o["idx"], f0["idx"])
        return float(np.sum(o["out"] * dy)) + oracle.aux_loss(o["logits"], f0["counts"], cfg.k, fn, alpha)

    rng = np.random.default_rng(8)
    h = 1e-6
    for name, gname in (("x", "dx"), ("w_router", "dw_router")):
        arr, grad = p[name], g[gname]
        for _ in range(12):
            i = tuple(int(rng.integers(0, s)) for s in arr.shape)
            old = arr[i]
            arr[i] = old + h
            lp = total()
            arr[i] = old - h
            lm = total()
            arr[i] = old
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grad[i]) <= 1e-7 + 1e-6 * abs(fd), (name, i, fd, grad[i])
