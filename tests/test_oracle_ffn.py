"""Pins of the oracle's experts, permutation and combine: torch's own linear
and silu, the dense-FFN special cases the lesson and the handbook article give
(one expert with k=1, identical upcycled experts), the stable-argsort library
routine and the permute/combine round trip."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from workloads import CONFIGS, make_inputs, scaled


def _torch_swiglu(x, wgu, wd):
    x, wgu, wd = (torch.from_numpy(np.asarray(a, np.float64)) for a in (x, wgu, wd))
    f = wd.shape[1]
    return F.linear(F.silu(F.linear(x, wgu[:f])) * F.linear(x, wgu[f:]), wd).numpy()


def test_expert_ffn_equals_torch_swiglu():
    r = np.random.default_rng(0)
    x = r.standard_normal((9, 16))
    wgu = r.standard_normal((2 * 24, 16)) * 0.3
    wd = r.standard_normal((16, 24)) * 0.3
    o = oracle.expert_ffn(x, wgu, wd, bf16_points=False)
    np.testing.assert_allclose(o["Y"], _torch_swiglu(x, wgu, wd), rtol=1e-12, atol=1e-13)


def test_bf16_round_equals_torch_bfloat16():
    r = np.random.default_rng(1)
    v = np.concatenate([r.standard_normal(20000).astype(np.float32) * 10.0 ** r.integers(-20, 20, 20000),
                        np.float32([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, 1.5, 65504.0])])
    v = v.astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.bf16_round(v.astype(np.float64)), ref)
    bits = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_from_bits(bits), ref)


def test_bf16_points_round_h_and_saved_gu_only():
    r = np.random.default_rng(2)
    x = r.standard_normal((5, 16))
    wgu = r.standard_normal((32, 16)) * 0.3
    wd = r.standard_normal((16, 16)) * 0.3
    a = oracle.expert_ffn(x, wgu, wd, bf16_points=False)
    b = oracle.expert_ffn(x, wgu, wd, bf16_points=True)
    assert np.array_equal(b["H"], oracle.bf16_round(a["H"]))     # H from unrounded G, U
    assert np.array_equal(b["G"], oracle.bf16_round(a["G"]))
    np.testing.assert_allclose(b["Y"], b["H"] @ wd.T, rtol=1e-14)


@pytest.mark.parametrize("fn", oracle.SCORE_FNS)
def test_one_expert_top1_equals_dense_ffn(fn):
    """A 1-expert, k=1 MoE is the dense FFN (the handbook's upcycling check)."""
    cfg = CONFIGS["tiny_dense"]
    inp = make_inputs(cfg)
    o = oracle.forward(inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"], 1, fn, False,
                       sel_bias=inp["bias"])
    assert np.all(o["gates"] == 1.0)
    dense = _torch_swiglu(inp["x"], inp["w_gate_up"][0], inp["w_down"][0])
    np.testing.assert_allclose(o["out"], dense, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("fn", oracle.SCORE_FNS)
def test_identical_experts_equal_dense_for_any_routing(fn):
    """E copies of one FFN (an upcycled dense layer): gates sum to one, so the
    MoE output is the dense output whatever the router picks."""
    cfg = CONFIGS["tiny"]
    inp = make_inputs(cfg)
    wgu = np.repeat(inp["w_gate_up"][:1], cfg.E, axis=0)
    wd = np.repeat(inp["w_down"][:1], cfg.E, axis=0)
    for k in (1, 2, 3):
        o = oracle.forward(inp["x"], inp["w_router"], wgu, wd, k, fn, False, sel_bias=inp["bias"])
        dense = _torch_swiglu(inp["x"], wgu[0], wd[0])
        np.testing.assert_allclose(o["out"], dense, rtol=1e-12, atol=1e-13)


def test_shared_expert_adds_dense_ffn_output():
    cfg = scaled(CONFIGS["tiny"], shared=1, f_shared=48)
    inp = make_inputs(cfg)
    o = oracle.forward(inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"], 2, "sigmoid", False,
                       sel_bias=inp["bias"], w_gate_up_shared=inp["w_gate_up_shared"],
                       w_down_shared=inp["w_down_shared"])
    o0 = oracle.forward(inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"], 2, "sigmoid", False,
                        sel_bias=inp["bias"])
    sh = _torch_swiglu(inp["x"], inp["w_gate_up_shared"][0], inp["w_down_shared"][0])
    np.testing.assert_allclose(o["out"] - o0["out"], sh, rtol=1e-11, atol=1e-13)


def _random_idx(rng, T, E, k):
    return np.stack([rng.permutation(E)[:k] for _ in range(T)])


@pytest.mark.parametrize("T,E,k", [(50, 8, 2), (37, 5, 5), (64, 16, 1), (1, 3, 2)])
def test_permute_is_stable_argsort(T, E, k):
    rng = np.random.default_rng(T * E + k)
    idx = _random_idx(rng, T, E, k)
    counts, offsets, row_of, token_of = oracle.permute(idx, E)
    flat = idx.reshape(-1)
    order = np.argsort(flat, kind="stable")      # library stable sort of (t, j) by expert
    assert np.array_equal(token_of, order // k)
    inv = np.empty_like(order)
    inv[order] = np.arange(T * k)
    assert np.array_equal(row_of.reshape(-1), inv)
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and offsets[-1] == T * k
    for t in range(T):
        for j in range(k):
            r = row_of[t, j]
            assert token_of[r] == t and offsets[idx[t, j]] <= r < offsets[idx[t, j] + 1]


def test_permute_skew_extremes():
    T, E = 40, 6
    idx = np.zeros((T, 1), np.int64)          # every token to expert 0
    counts, offsets, row_of, token_of = oracle.permute(idx, E)
    assert counts.tolist() == [T, 0, 0, 0, 0, 0]
    assert offsets.tolist() == [0] + [T] * E
    assert np.array_equal(token_of, np.arange(T))
    idx = np.tile(np.array([[5, 2]]), (T, 1))  # two experts, the rest empty
    counts, offsets, row_of, token_of = oracle.permute(idx, E)
    assert counts.tolist() == [0, 0, T, 0, 0, T]
    assert np.array_equal(row_of[:, 1], np.arange(T)) and np.array_equal(row_of[:, 0], T + np.arange(T))


@pytest.mark.parametrize("fn", oracle.SCORE_FNS)
def test_permute_combine_round_trip(fn):
    """Expert outputs equal to the expert inputs and gates summing to one give
    the layer input back."""
    cfg = CONFIGS["tiny"]
    inp = make_inputs(cfg)
    r = oracle.route(inp["x"], inp["w_router"], 3, fn, sel_bias=inp["bias"])
    counts, offsets, row_of, token_of = oracle.permute(r["idx"], cfg.E)
    x_perm = np.asarray(inp["x"], np.float64)[token_of]
    back = oracle.combine(x_perm, row_of, r["gates"])
    np.testing.assert_allclose(back, inp["x"], rtol=1e-14, atol=1e-15)


def test_grouped_ffn_skips_empty_experts():
    cfg = CONFIGS["tiny"]
    inp = make_inputs(cfg)
    offsets = np.array([0, 0, 10, 10, 30, 30, 30, 30, 40])
    x = np.asarray(inp["x"][:40], np.float64)
    o = oracle.grouped_ffn(x, offsets, inp["w_gate_up"], inp["w_down"], False)
    for e in range(cfg.E):
        a, b = offsets[e], offsets[e + 1]
        if b > a:
            np.testing.assert_allclose(o["Y"][a:b], _torch_swiglu(x[a:b], inp["w_gate_up"][e], inp["w_down"][e]),
                                       rtol=1e-12, atol=1e-14)
