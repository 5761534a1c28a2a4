"""Pins of the oracle's backward: fp64 central finite differences of
L = sum(out * dY) with the routing held fixed (steps far below every routing
margin), and torch.autograd on an independently written forward."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from workloads import CONFIGS, make_inputs, scaled


def _setup(fn, shared=False, seed=0):
    cfg = CONFIGS["tiny"]
    if shared:
        cfg = scaled(cfg, shared=1, f_shared=40)
    cfg = scaled(cfg, T=24, seed=seed)
    inp = make_inputs(cfg)
    dy = np.random.default_rng(11).standard_normal((cfg.T, cfg.d))
    p = {k: np.asarray(inp[k], np.float64) for k in ("x", "w_router", "w_gate_up", "w_down")}
    if shared:
        p["w_gate_up_shared"] = np.asarray(inp["w_gate_up_shared"], np.float64)
        p["w_down_shared"] = np.asarray(inp["w_down_shared"], np.float64)
    return cfg, inp, p, dy


def _loss(p, cfg, fn, bias, dy, idx):
    o = oracle.forward(p["x"], p["w_router"], p["w_gate_up"], p["w_down"], cfg.k, fn, False,
                       sel_bias=bias, w_gate_up_shared=p.get("w_gate_up_shared"),
                       w_down_shared=p.get("w_down_shared"))
    assert np.array_equal(o["idx"], idx), "routing moved under the finite-difference step"
    return float(np.sum(o["out"] * dy))


@pytest.mark.parametrize("fn", oracle.SCORE_FNS)
@pytest.mark.parametrize("shared", [False, True])
def test_backward_matches_finite_differences(fn, shared):
    cfg, inp, p, dy = _setup(fn, shared)
    fwd = oracle.forward(p["x"], p["w_router"], p["w_gate_up"], p["w_down"], cfg.k, fn, False,
                         sel_bias=inp["bias"], w_gate_up_shared=p.get("w_gate_up_shared"),
                         w_down_shared=p.get("w_down_shared"))
    assert fwd["margin"].min() > 1e-5
    g = oracle.backward(fwd, dy, p["x"], p["w_router"], p["w_gate_up"], p["w_down"], fn, False,
                        w_gate_up_shared=p.get("w_gate_up_shared"), w_down_shared=p.get("w_down_shared"))
    names = {"x": "dx", "w_router": "dw_router", "w_gate_up": "dw_gate_up", "w_down": "dw_down"}
    if shared:
        names["w_gate_up_shared"] = "dw_gate_up_shared"
        names["w_down_shared"] = "dw_down_shared"
    rng = np.random.default_rng(5)
    h = 1e-6
    for name, gname in names.items():
        grad = np.asarray(g[gname], np.float64)
        arr = p[name]
        for _ in range(12):
            i = tuple(int(rng.integers(0, s)) for s in arr.shape)
            old = arr[i]
            arr[i] = old + h
            lp = _loss(p, cfg, fn, inp["bias"], dy, fwd["idx"])
            arr[i] = old - h
            lm = _loss(p, cfg, fn, inp["bias"], dy, fwd["idx"])
            arr[i] = old
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grad[i]) <= 1e-7 + 1e-6 * abs(fd), (name, i, fd, grad[i])


def _torch_forward(x, wr, wgu, wd, idx, fn, bias):
    """An independent torch formulation with the expert choice given."""
    l = x @ wr.T
    if fn == "softmax":
        g = torch.softmax(torch.gather(l, 1, idx), dim=1)
    else:
        s = torch.sigmoid(l) if fn == "sigmoid" else torch.sqrt(F.softplus(l, threshold=1000.0))
        sc = torch.gather(s, 1, idx)
        g = sc / sc.sum(dim=1, keepdim=True)
    f = wd.shape[2]
    out = torch.zeros_like(x)
    for j in range(idx.shape[1]):
        e = idx[:, j]
        gt = torch.einsum("td,tfd->tf", x, wgu[e, :f])
        up = torch.einsum("td,tfd->tf", x, wgu[e, f:])
        y = torch.einsum("tf,tdf->td", F.silu(gt) * up, wd[e])
        out = out + g[:, j:j + 1] * y
    return out


@pytest.mark.parametrize("fn", oracle.SCORE_FNS)
def test_backward_matches_torch_autograd(fn):
    cfg, inp, p, dy = _setup(fn)
    fwd = oracle.forward(p["x"], p["w_router"], p["w_gate_up"], p["w_down"], cfg.k, fn, False,
                         sel_bias=inp["bias"])
    g = oracle.backward(fwd, dy, p["x"], p["w_router"], p["w_gate_up"], p["w_down"], fn, False)
    t = {k: torch.tensor(v, requires_grad=True) for k, v in p.items()}
    out = _torch_forward(t["x"], t["w_router"], t["w_gate_up"], t["w_down"],
                         torch.from_numpy(fwd["idx"]), fn, inp["bias"])
    np.testing.assert_allclose(out.detach().numpy(), fwd["out"], rtol=1e-12, atol=1e-13)
    (out * torch.from_numpy(dy)).sum().backward()
    for k, gk in (("x", "dx"), ("w_router", "dw_router"), ("w_gate_up", "dw_gate_up"), ("w_down", "dw_down")):
        np.testing.assert_allclose(g[gk], t[k].grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=k)


def test_bias_gets_no_gradient():
    """Selection bias and logit offset sit outside the loss's gradient: the
    gradients with and without them agree whenever the choice is unchanged."""
    cfg, inp, p, dy = _setup("sigmoid")
    fwd0 = oracle.forward(p["x"], p["w_router"], p["w_gate_up"], p["w_down"], cfg.k, "sigmoid", False)
    fwd1 = oracle.forward(p["x"], p["w_router"], p["w_gate_up"], p["w_down"], cfg.k, "sigmoid", False,
                          idx=fwd0["idx"], sel_bias=inp["bias"])
    g0 = oracle.backward(fwd0, dy, p["x"], p["w_router"], p["w_gate_up"], p["w_down"], "sigmoid", False)
    g1 = oracle.backward(fwd1, dy, p["x"], p["w_router"], p["w_gate_up"], p["w_down"], "sigmoid", False)
    for k in ("dx", "dw_router", "dw_gate_up", "dw_down"):
        np.testing.assert_array_equal(g0[k], g1[k])


def test_bf16_points_in_backward():
    cfg, inp, p, dy = _setup("softmax")
    fwd = oracle.forward(p["x"], p["w_router"], p["w_gate_up"], p["w_down"], cfg.k, "softmax", True)
    g = oracle.backward(fwd, dy, p["x"], p["w_router"], p["w_gate_up"], p["w_down"], "softmax", True)
    assert np.array_equal(g["dy_perm"], oracle.bf16_round(g["dy_perm"]))
    assert np.array_equal(g["dgu"], oracle.bf16_round(g["dgu"]))
    g0 = oracle.backward(fwd, dy, p["x"], p["w_router"], p["w_gate_up"], p["w_down"], "softmax", False)
    # rounding points move the gradients by bf16-sized amounts only
    np.testing.assert_allclose(g["dx"], g0["dx"], atol=3e-2 * np.abs(g0["dx"]).max())
