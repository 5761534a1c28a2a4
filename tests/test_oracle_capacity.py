"""Pins of the oracle's expert capacity (token dropping).

Lesson "专家组合 (MoE)", Load balancing item 2: each expert processes at most
a fixed number of tokens (C x N / E) and the overflow skips the layer.  The
oracle keeps an expert's first `capacity` assignments in token order.  These
tests pin that against a first-come-first-served counter written out token
by token, against the uncapped path (which its own tests pin), and the
backward against finite differences and torch.autograd on an independent
masked formulation."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from workloads import CONFIGS, make_inputs, scaled


def _random_idx(T, k, E, seed, skew=0.0):
    rng = np.random.default_rng(seed)
    p = np.exp(-skew * np.arange(E))
    p /= p.sum()
    return np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(T)])


def _decode(row_of):
    return np.where(row_of >= 0, row_of, ~row_of)


def _first_come(idx, E, cap):
    """Kept mask by a running per-expert counter, tokens in order."""
    T, k = idx.shape
    used = [0] * E
    kept = np.zeros((T, k), bool)
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            if used[e] < cap:
                kept[t, j] = True
            used[e] += 1
    return kept


@pytest.mark.parametrize("seed,skew", [(0, 0.0), (1, 0.4), (2, 1.5)])
def test_capacity_is_first_come_first_served(seed, skew):
    T, k, E = 97, 3, 11
    idx = _random_idx(T, k, E, seed, skew)
    for cap in (0, 1, 5, 17, 40):
        counts, offsets, row_of, token_of = oracle.permute(idx, E, cap)
        assert np.array_equal(row_of >= 0, _first_come(idx, E, cap))
        assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=E))
        assert np.array_equal(np.diff(offsets), np.minimum(counts, cap))


@pytest.mark.parametrize("seed", [0, 3])
def test_capacity_layout(seed):
    T, k, E = 120, 4, 9
    idx = _random_idx(T, k, E, seed, skew=0.8)
    cap = 30
    counts, offsets, row_of, token_of = oracle.permute(idx, E, cap)
    A = T * k
    rows = _decode(row_of)
    assert np.array_equal(np.sort(rows.ravel()), np.arange(A))            # every row used once
    tt = np.repeat(np.arange(T)[:, None], k, 1)
    assert np.array_equal(token_of[rows], tt)
    kept_total = offsets[-1]
    assert np.all(rows[row_of >= 0] < kept_total) and np.all(rows[row_of < 0] >= kept_total)
    drop_start = kept_total
    for e in range(E):
        seg = token_of[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0) and np.all(idx[seg].__eq__(e).any(1))
        nd = counts[e] - (offsets[e + 1] - offsets[e])
        dseg = token_of[drop_start:drop_start + nd]
        assert np.all(np.diff(dseg) > 0) and (len(dseg) == 0 or dseg[0] > seg[-1])
        drop_start += nd
    assert drop_start == A


def test_capacity_at_or_above_the_largest_count_changes_nothing():
    idx = _random_idx(80, 2, 7, 4, skew=1.0)
    ref = oracle.permute(idx, 7)
    for cap in (int(np.bincount(idx.ravel()).max()), 160, None, -1):
        got = oracle.permute(idx, 7, cap)
        for a, b in zip(got, ref):
            assert np.array_equal(a, b)


def _cfg(score="softmax", **kw):
    return scaled(CONFIGS["tiny"], T=40, score=score, **kw)


@pytest.mark.parametrize("score", oracle.SCORE_FNS)
def test_capped_output_is_uncapped_output_without_the_dropped_slots(score):
    cfg = _cfg(score)
    inp = make_inputs(cfg)
    a = (inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"], cfg.k, score, False)
    free = oracle.forward(*a, sel_bias=inp["bias"])
    cap = 6
    capped = oracle.forward(*a, sel_bias=inp["bias"], capacity=cap)
    kept = _first_come(free["idx"], cfg.E, cap)
    assert (~kept).sum() > 0
    want = np.zeros_like(free["out"])
    for j in range(cfg.k):
        y = free["y_perm"][free["row_of"][:, j]]
        want += (kept[:, j] * free["gates"][:, j])[:, None] * y
    np.testing.assert_allclose(capped["out"], want, rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(capped["gates"], free["gates"])         # gates are not renormalised


def test_top1_overflow_tokens_skip_the_layer():
    """k = 1 and the lesson's C x N / E: a dropped token's layer output is 0
    (the residual carries it); a kept token's is its expert's FFN output."""
    cfg = _cfg(k=1)
    inp = make_inputs(cfg)
    C = 1.0
    cap = int(np.ceil(C * cfg.T / cfg.E))
    o = oracle.forward(inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"], 1, "softmax", False,
                       sel_bias=inp["bias"], capacity=cap)
    dropped = o["row_of"][:, 0] < 0
    assert dropped.any() and np.all(np.diff(o["offsets"]) <= cap)
    assert np.all(o["out"][dropped] == 0.0)
    for t in np.nonzero(~dropped)[0]:
        e = o["idx"][t, 0]
        ref = oracle.expert_ffn(np.asarray(inp["x"][t:t + 1], np.float64), inp["w_gate_up"][e], inp["w_down"][e],
                                False)["Y"][0]
        np.testing.assert_allclose(o["out"][t], ref, rtol=1e-12, atol=1e-14)   # k = 1: the gate is 1


def test_capacity_zero_leaves_only_the_shared_expert():
    cfg = _cfg(shared=1, f_shared=24)
    inp = make_inputs(cfg)
    o = oracle.forward(inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"], cfg.k, "sigmoid", False,
                       w_gate_up_shared=inp["w_gate_up_shared"], w_down_shared=inp["w_down_shared"], capacity=0)
    assert np.all(o["row_of"] < 0) and o["offsets"][-1] == 0
    np.testing.assert_array_equal(o["out"], o["shared_y"])


# ---------------------------------------------------------------------------- backward

def _setup_bwd(seed=0):
    cfg = scaled(CONFIGS["tiny"], T=24, seed=seed)
    inp = make_inputs(cfg)
    dy = np.random.default_rng(11).standard_normal((cfg.T, cfg.d))
    p = {k: np.asarray(inp[k], np.float64) for k in ("x", "w_router", "w_gate_up", "w_down")}
    return cfg, inp, p, dy


@pytest.mark.parametrize("fn", oracle.SCORE_FNS)
def test_capped_backward_matches_finite_differences(fn):
    cfg, inp, p, dy = _setup_bwd()
    cap = 4
    fwd = oracle.forward(p["x"], p["w_router"], p["w_gate_up"], p["w_down"], cfg.k, fn, False,
                         sel_bias=inp["bias"], capacity=cap)
    assert fwd["margin"].min() > 1e-5 and (fwd["row_of"] < 0).any()
    g = oracle.backward(fwd, dy, p["x"], p["w_router"], p["w_gate_up"], p["w_down"], fn, False)

    def loss():
        o = oracle.forward(p["x"], p["w_router"], p["w_gate_up"], p["w_down"], cfg.k, fn, False,
                           sel_bias=inp["bias"], capacity=cap)
        assert np.array_equal(o["row_of"], fwd["row_of"])
        return float(np.sum(o["out"] * dy))

    rng = np.random.default_rng(6)
    h = 1e-6
    for name, gname in (("x", "dx"), ("w_router", "dw_router"), ("w_gate_up", "dw_gate_up"), ("w_down", "dw_down")):
        arr, grad = p[name], g[gname]
        for _ in range(10):
            i = tuple(int(rng.integers(0, s)) for s in arr.shape)
            old = arr[i]
            arr[i] = old + h
            lp = loss()
            arr[i] = old - h
            lm = loss()
            arr[i] = old
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grad[i]) <= 1e-7 + 1e-6 * abs(fd), (name, i, fd, grad[i])


@pytest.mark.parametrize("fn", oracle.SCORE_FNS)
def test_capped_backward_matches_torch_autograd(fn):
    cfg, inp, p, dy = _setup_bwd(seed=2)
    cap = 5
    fwd = oracle.forward(p["x"], p["w_router"], p["w_gate_up"], p["w_down"], cfg.k, fn, False,
                         sel_bias=inp["bias"], capacity=cap)
    g = oracle.backward(fwd, dy, p["x"], p["w_router"], p["w_gate_up"], p["w_down"], fn, False)
    t = {k: torch.tensor(v, requires_grad=True) for k, v in p.items()}
    idx = torch.from_numpy(fwd["idx"])
    keep = torch.from_numpy((fwd["row_of"] >= 0).astype(np.float64))
    l = t["x"] @ t["w_router"].T
    if fn == "softmax":
        gate = torch.softmax(torch.gather(l, 1, idx), dim=1)
    else:
        s = torch.sigmoid(l) if fn == "sigmoid" else torch.sqrt(F.softplus(l, threshold=1000.0))
        sc = torch.gather(s, 1, idx)
        gate = sc / sc.sum(dim=1, keepdim=True)
    f = t["w_down"].shape[2]
    out = torch.zeros_like(t["x"])
    for j in range(cfg.k):
        e = idx[:, j]
        gt = torch.einsum("td,tfd->tf", t["x"], t["w_gate_up"][e, :f])
        up = torch.einsum("td,tfd->tf", t["x"], t["w_gate_up"][e, f:])
        y = torch.einsum("tf,tdf->td", F.silu(gt) * up, t["w_down"][e])
        out = out + (keep[:, j] * gate[:, j])[:, None] * y
    np.testing.assert_allclose(out.detach().numpy(), fwd["out"], rtol=1e-12, atol=1e-13)
    (out * torch.from_numpy(dy)).sum().backward()
    for k, gk in (("x", "dx"), ("w_router", "dw_router"), ("w_gate_up", "dw_gate_up"), ("w_down", "dw_down")):
        np.testing.assert_allclose(g[gk], t[k].grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=k)
