"""Pins of the bias controller (its stated rule, case by case, and the
balancing behaviour the lesson describes) and of the parameter arithmetic
(numbers the handbook article and the lesson print; tests/golden)."""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bias_update_rule_case_by_case():
    """Over-used experts move down by gamma, under-used up, on-target stay
    (lesson, Load balancing and Build it step 2); float32 storage."""
    E, T, k, gamma = 4, 6, 2, 1e-3          # uniform target T*k/E = 3
    b0 = np.float32([0.1, -0.2, 0.0, 0.05])
    counts = np.array([5, 3, 1, 3])
    b1 = oracle.bias_update(b0, counts, T, k, gamma)
    g = np.float32(gamma)
    assert b1.dtype == np.float32
    assert b1[0] == np.float32(b0[0] - g)    # over-used
    assert b1[1] == b0[1]                    # on target
    assert b1[2] == np.float32(b0[2] + g)    # under-used
    assert b1[3] == b0[3]
    assert b1[0] < b0[0] and b1[2] > b0[2]


def test_bias_update_integer_target():
    """T*k/E not an integer: the comparison is exact, never rounded."""
    E, T, k = 3, 5, 2                         # target 10/3
    b = oracle.bias_update(np.zeros(3, np.float32), np.array([4, 3, 3]), T, k, 0.5)
    assert b.tolist() == [-0.5, 0.5, 0.5]


def test_bias_controller_balances_usage():
    """100 tokens, routing skewed towards one expert; running the controller
    step after step (the lesson's exercise runs it for 50 steps) brings the
    busiest expert's load toward the mean."""
    rng = np.random.default_rng(0)
    E, d, k, T = 8, 16, 2, 100
    w = rng.standard_normal((E, d)) * 0.3
    off = np.zeros(E)
    off[3] = 1.5                              # expert 3 takes most tokens
    bias = np.zeros(E, np.float32)
    loads = []
    for step in range(50):
        x = rng.standard_normal((T, d))
        r = oracle.route(x, w, k, "softmax", sel_bias=bias, logit_offset=off)
        counts = np.bincount(r["idx"].reshape(-1), minlength=E)
        loads.append(counts.max() / counts.mean())
        bias = oracle.bias_update(bias, counts, T, k, 0.05)
    assert loads[0] > 2.5
    assert np.mean(loads[-10:]) < 0.6 * loads[0]
    assert bias[3] < 0 and bias.argmin() == 3


def test_parameter_counts_match_the_printed_teaching_model():
    g = json.load(open(os.path.join(GOLDEN, "param_counts.json")))
    m = g["teaching_model"]
    L, d, F, E, k = m["layers"], m["d_model"], m["dense_ffn"], m["experts"], m["top_k"]
    f = F // k
    dense = m["dense_total_B"] * 1e9
    other = dense - L * oracle.dense_ffn_params(d, F)     # embeddings, attention, norms
    tot, act = oracle.moe_ffn_params(d, f, E, k)
    total = other + L * tot
    active = other + L * act
    assert round(total / 1e9, 2) == m["total_B"]
    assert round(active / 1e9, 3) == m["active_B"]
    assert round(total / dense, 1) == m["total_over_dense"]
    # k experts of width F/k hold exactly the dense FFN's parameters
    assert k * 3 * d * f == oracle.dense_ffn_params(d, F)


def test_sparsity_and_combinatorics_printed_by_the_lesson():
    g = json.load(open(os.path.join(GOLDEN, "param_counts.json")))
    ds = g["deepseek_v3"]
    assert round(100 * ds["active_B"] / ds["total_B"], 1) == ds["active_pct"]
    c = math.comb(g["fine_grained"]["E"], g["fine_grained"]["k"])
    assert round(c / 1e12, -2) == g["fine_grained"]["choose_trillions"]
    # fp16 weights of the 671B model
    assert round(ds["total_B"] * 2 / 1000, 1) == g["deepseek_v3"]["fp16_TB"]
