"""Pins of the oracle's router, top-k and gates against things other than the
oracle: library routines, brute force over subsets, closed forms and the
properties the MoE lesson and the handbook article state."""
import itertools

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from workloads import CONFIGS, make_inputs, scaled


def _rand(seed, T, d, E, scale=0.3):
    r = np.random.default_rng(seed)
    return r.standard_normal((T, d)), r.standard_normal((E, d)) * scale


def test_logits_equal_torch_linear():
    x, w = _rand(1, 17, 24, 9)
    o = np.random.default_rng(2).standard_normal(9)
    r = oracle.route(x, w, 3, "softmax", logit_offset=o)
    ref = torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(w), torch.from_numpy(o))
    np.testing.assert_allclose(r["logits"], ref.numpy(), rtol=0, atol=1e-13)


def test_score_functions_against_libraries():
    l = np.linspace(-30, 30, 2001)
    np.testing.assert_allclose(oracle.score(l, "sigmoid"), scipy.special.expit(l), rtol=1e-15, atol=0)
    sp = torch.nn.functional.softplus(torch.from_numpy(l), threshold=1000.0).numpy()
    np.testing.assert_allclose(oracle.score(l, "sqrt_softplus"), np.sqrt(sp), rtol=1e-14)
    assert oracle.score(np.array([0.0]), "sqrt_softplus")[0] == pytest.approx(np.sqrt(np.log(2.0)), rel=1e-15)
    assert np.array_equal(oracle.score(l, "softmax"), l)


def _first_k_by_rule(keys, k):
    """Brute force: the unique k-subset S such that every member beats every
    non-member under (higher key, then lower index)."""
    E = len(keys)
    hits = []
    for S in itertools.combinations(range(E), k):
        rest = [j for j in range(E) if j not in S]
        if all(keys[i] > keys[j] or (keys[i] == keys[j] and i < j) for i in S for j in rest):
            hits.append(set(S))
    assert len(hits) == 1
    return hits[0]


@pytest.mark.parametrize("fn", oracle.SCORE_FNS)
def test_topk_bruteforce_with_ties(fn):
    rng = np.random.default_rng(7)
    for trial in range(60):
        E = int(rng.integers(2, 9))
        k = int(rng.integers(1, min(3, E) + 1))
        d = 4
        x = rng.standard_normal((3, d))
        w = rng.standard_normal((E, d))
        if trial % 3 == 0:            # force exact ties: duplicated router rows
            w[E - 1] = w[0]
        b = np.round(rng.uniform(-0.3, 0.3, E), 1) if trial % 2 else None
        r = oracle.route(x, w, k, fn, sel_bias=b)
        for t in range(3):
            keys = r["keys"][t]
            assert set(r["idx"][t].tolist()) == _first_k_by_rule(keys, k)
            sl = r["idx"][t]
            for a, c in zip(sl[:-1], sl[1:]):   # slot order: key desc, index asc
                assert keys[a] > keys[c] or (keys[a] == keys[c] and a < c)


def test_equal_logits_go_to_lower_index():
    x = np.ones((1, 4))
    w = np.zeros((6, 4))
    w[2] = w[5] = 0.25
    w[4] = 0.1
    r = oracle.route(x, w, 1, "softmax")
    assert r["idx"][0, 0] == 2
    r = oracle.route(x, w, 2, "sigmoid")
    assert r["idx"][0].tolist() == [2, 5]
    assert r["margin"][0] > 0


def test_bf16_router_counterexample():
    """Two logits that differ in fp32 but round to the same bf16 value: the
    exact router picks the true winner, a bf16 router would hand the win to the
    lower index (the handbook article's router-precision paragraph)."""
    x = np.array([[1.0]])
    w = np.array([[1.0], [1.0 + 2.0 ** -9]])       # fp32-distinct, bf16-equal
    assert np.float32(w[1, 0]) != np.float32(w[0, 0])
    assert oracle.bf16_round(w[1, 0]) == oracle.bf16_round(w[0, 0])
    r = oracle.route(x, w, 1, "softmax")
    assert r["idx"][0, 0] == 1
    lb = oracle.bf16_round(x @ w.T)
    assert np.argsort(-lb[0], kind="stable")[0] == 0   # the bf16 router's (wrong) pick


@pytest.mark.parametrize("fn", oracle.SCORE_FNS)
def test_gates_sum_to_one_and_k1_is_one(fn):
    cfg = CONFIGS["tiny"]
    inp = make_inputs(cfg)
    for k in (1, 2, 5, 8):
        r = oracle.route(inp["x"], inp["w_router"], k, fn, sel_bias=inp["bias"])
        np.testing.assert_allclose(r["gates"].sum(axis=1), 1.0, rtol=0, atol=1e-15)
        assert np.all(r["gates"] > 0)
        if k == 1:
            assert np.all(r["gates"] == 1.0)


def test_softmax_over_chosen_is_renormalised_full_softmax():
    x, w = _rand(3, 40, 16, 8)
    b = np.random.default_rng(4).uniform(-0.5, 0.5, 8)
    r = oracle.route(x, w, 3, "softmax", sel_bias=b)
    full = scipy.special.softmax(x @ w.T, axis=1)
    for t in range(40):
        p = full[t, r["idx"][t]]
        np.testing.assert_allclose(r["gates"][t], p / p.sum(), rtol=1e-13)


@pytest.mark.parametrize("fn", ["sigmoid", "sqrt_softplus"])
def test_normalised_gates_are_score_ratios(fn):
    x, w = _rand(5, 30, 16, 8)
    r = oracle.route(x, w, 4, fn)
    s = oracle.score(x @ w.T, fn)
    for t in range(30):
        sc = s[t, r["idx"][t]]
        np.testing.assert_allclose(r["gates"][t], sc / sc.sum(), rtol=1e-14)


@pytest.mark.parametrize("fn", oracle.SCORE_FNS)
def test_bias_moves_selection_not_gates(fn):
    cfg = CONFIGS["tiny"]
    inp = make_inputs(cfg)
    x, w = inp["x"], inp["w_router"]
    r0 = oracle.route(x, w, 2, fn)
    r1 = oracle.route(x, w, 2, fn, sel_bias=inp["bias"])
    same = [t for t in range(cfg.T) if set(r0["idx"][t]) == set(r1["idx"][t])]
    assert len(same) > 10
    for t in same:   # same chosen set => same gate per expert, bias or not
        g0 = dict(zip(r0["idx"][t].tolist(), r0["gates"][t]))
        g1 = dict(zip(r1["idx"][t].tolist(), r1["gates"][t]))
        for e in g0:
            assert g0[e] == g1[e]
    # a huge bias forces expert 5 into every token's choice, its gate still
    # comes from the raw scores
    big = np.zeros(cfg.E)
    big[5] = 1e6
    r2 = oracle.route(x, w, 2, fn, sel_bias=big)
    assert np.all(r2["idx"][:, 0] == 5)
    s = oracle.score(r2["logits"], fn)
    for t in range(cfg.T):
        ch = r2["idx"][t]
        if fn == "softmax":
            p = scipy.special.softmax(r2["logits"][t, ch])
        else:
            p = s[t, ch] / s[t, ch].sum()
        np.testing.assert_allclose(r2["gates"][t], p, rtol=1e-13)


def test_margin_definition():
    x = np.array([[1.0, 0.0]])
    w = np.array([[3.0, 0], [2.0, 0], [1.0, 0], [2.0 + 1e-7, 0]])
    r = oracle.route(x, w, 2, "softmax")
    assert r["idx"][0].tolist() == [0, 3]
    assert r["margin"][0] == pytest.approx((1e-7) / (2.0 + 1e-7), rel=1e-6)
    r = oracle.route(x, w, 4, "softmax")
    assert r["margin"][0] == np.inf


def test_router_runs_on_bf16_bits():
    cfg = scaled(CONFIGS["fine"], T=32, d=64, E=16, k=4, f=64)
    inp = make_inputs(cfg, experts=False)
    assert inp["x"].dtype == np.uint16
    r = oracle.route(inp["x"], inp["w_router"], 4, "sigmoid", logit_offset=inp["logit_offset"])
    xf = (inp["x"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    np.testing.assert_allclose(r["logits"], xf @ inp["w_router"].astype(np.float64).T
                               + inp["logit_offset"].astype(np.float64), atol=1e-12)
