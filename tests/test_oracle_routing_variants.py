"""Pins of the routing variants of the lesson "专家组合 (MoE)":

* Exercises item 2, a hash router (deterministic, nothing learned): the
  SplitMix64 key against the published output sequence, the defining
  k-smallest property, balance, and the 1/k gates;
* Exercises item 3, routing replay: forcing a recorded choice reproduces the
  gates of that choice;
* the announcement's question whether a model can be served with fewer
  experts per token than it was trained with: the smaller choice is a prefix
  of the larger and its gates are the renormalised prefix of the larger
  gates (a closed form of both gate rules).
The hash router's layer backward (constant gates) is pinned by finite
differences and torch.autograd."""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from workloads import CONFIGS, make_inputs, scaled

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "splitmix64.json")


def test_splitmix_key_is_the_published_generator():
    g = json.load(open(GOLDEN))
    seed = int(g["seed"])
    got = [int(oracle.splitmix_key(seed >> 32, seed & 0xFFFFFFFF, salt)) for salt in range(5)]
    assert got == [int(v) for v in g["outputs"]]


def test_hash_route_takes_the_k_smallest_keys():
    ids = np.random.default_rng(0).integers(0, 50000, 300)
    E, k = 37, 5
    r = oracle.hash_route(ids, E, k, salt=3)
    keys = oracle.splitmix_key(ids[:, None], np.arange(E)[None, :], 3)
    for t in range(len(ids)):
        chosen = r["idx"][t]
        assert len(set(chosen.tolist())) == k
        kc = keys[t, chosen]
        assert np.all(np.diff(kc.astype(object)) > 0)                  # ascending keys
        rest = np.setdiff1d(np.arange(E), chosen)
        assert kc.max() < keys[t, rest].min()                          # every chosen key below every other
    np.testing.assert_array_equal(r["gates"], np.full((len(ids), k), 1.0 / k))


def test_hash_route_is_deterministic_balanced_and_salted():
    ids = np.arange(20000)
    E, k = 16, 2
    a = oracle.hash_route(ids, E, k)
    b = oracle.hash_route(ids, E, k)
    np.testing.assert_array_equal(a["idx"], b["idx"])
    load = np.bincount(a["idx"].ravel(), minlength=E)
    target = len(ids) * k / E
    assert np.all(np.abs(load - target) < 0.06 * target)               # binomial spread is ~2%
    c = oracle.hash_route(ids, E, k, salt=1)
    assert np.mean(np.any(c["idx"] != a["idx"], axis=1)) > 0.8


@pytest.mark.parametrize("fn", oracle.SCORE_FNS)
def test_serving_with_fewer_experts_is_a_renormalised_prefix(fn):
    cfg = scaled(CONFIGS["fine"], T=200, d=64, E=32, k=8, f=64, bias="uniform")
    inp = make_inputs(cfg, experts=False)
    big = oracle.route(inp["x"], inp["w_router"], 8, fn, inp["bias"], inp["logit_offset"])
    for k in (1, 3, 6):
        small = oracle.route(inp["x"], inp["w_router"], k, fn, inp["bias"], inp["logit_offset"])
        np.testing.assert_array_equal(small["idx"], big["idx"][:, :k])
        pre = big["gates"][:, :k]
        np.testing.assert_allclose(small["gates"], pre / pre.sum(axis=1, keepdims=True), rtol=1e-13, atol=0)


@pytest.mark.parametrize("fn", oracle.SCORE_FNS)
def test_replaying_a_choice_reproduces_its_gates(fn):
    cfg = scaled(CONFIGS["tiny"], score=fn)
    inp = make_inputs(cfg)
    a = (inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"], cfg.k, fn, False)
    free = oracle.forward(*a, sel_bias=inp["bias"])
    rep = oracle.forward(*a, idx=free["idx"])                          # no bias needed to replay
    np.testing.assert_allclose(rep["gates"], free["gates"], rtol=1e-15, atol=0)
    np.testing.assert_allclose(rep["out"], free["out"], rtol=1e-13, atol=1e-15)


def test_hash_layer_backward_matches_finite_differences_and_autograd():
    cfg = scaled(CONFIGS["tiny"], T=24)
    inp = make_inputs(cfg)
    ids = np.random.default_rng(2).integers(0, 1000, cfg.T)
    idx = oracle.hash_route(ids, cfg.E, cfg.k)["idx"]
    dy = np.random.default_rng(3).standard_normal((cfg.T, cfg.d))
    p = {k: np.asarray(inp[k], np.float64) for k in ("x", "w_gate_up", "w_down")}

    def fwd():
        return oracle.forward(p["x"], None, p["w_gate_up"], p["w_down"], cfg.k, "uniform", False, idx=idx)

    f0 = fwd()
    g = oracle.backward(f0, dy, p["x"], None, p["w_gate_up"], p["w_down"], "uniform", False)
    assert np.all(g["dl"] == 0) and np.all(g["dw_router"] == 0)
    rng = np.random.default_rng(4)
    h = 1e-6
    for name, gname in (("x", "dx"), ("w_gate_up", "dw_gate_up"), ("w_down", "dw_down")):
        arr, grad = p[name], g[gname]
        for _ in range(10):
            i = tuple(int(rng.integers(0, s)) for s in arr.shape)
            old = arr[i]
            arr[i] = old + h
            lp = float(np.sum(fwd()["out"] * dy))
            arr[i] = old - h
            lm = float(np.sum(fwd()["out"] * dy))
            arr[i] = old
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grad[i]) <= 1e-7 + 1e-6 * abs(fd), (name, i, fd, grad[i])
    t = {k: torch.tensor(v, requires_grad=True) for k, v in p.items()}
    f = t["w_down"].shape[2]
    out = torch.zeros_like(t["x"])
    for j in range(cfg.k):
        e = torch.from_numpy(idx[:, j])
        gt = torch.einsum("td,tfd->tf", t["x"], t["w_gate_up"][e, :f])
        up = torch.einsum("td,tfd->tf", t["x"], t["w_gate_up"][e, f:])
        out = out + torch.einsum("tf,tdf->td", F.silu(gt) * up, t["w_down"][e]) / cfg.k
    np.testing.assert_allclose(out.detach().numpy(), f0["out"], rtol=1e-12, atol=1e-14)
    (out * torch.from_numpy(dy)).sum().backward()
    for k, gk in (("x", "dx"), ("w_gate_up", "dw_gate_up"), ("w_down", "dw_down")):
        np.testing.assert_allclose(g[gk], t[k].grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=k)


# ---------------------------------------------------------------------------- a replayed choice must be a choice

@pytest.mark.parametrize("bad", [-1, 8, 1 << 20])
def test_replay_rejects_ids_outside_the_experts(bad):
    """Routing replay (lesson, Exercises item 3) forces experts that fired, so
    each id names one of the E experts; an id outside [0, E) is not a routing
    choice and the oracle gives it no meaning."""
    cfg = scaled(CONFIGS["tiny"], T=6)
    inp = make_inputs(cfg)
    idx = np.stack([np.arange(cfg.k) + t % 3 for t in range(cfg.T)]).astype(np.int64)
    idx[2, 1] = bad
    with pytest.raises(ValueError):
        oracle.forward(inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"], cfg.k, "softmax", False, idx=idx)


def test_replay_rejects_a_repeated_expert():
    """A token picks k distinct experts (the lesson's top-k): a replayed row
    naming one expert twice is not a choice."""
    cfg = scaled(CONFIGS["tiny"], T=4)
    inp = make_inputs(cfg)
    idx = np.tile(np.arange(cfg.k, dtype=np.int64), (cfg.T, 1))
    idx[1] = 3
    with pytest.raises(ValueError):
        oracle.forward(inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"], cfg.k, "sigmoid", False, idx=idx)
