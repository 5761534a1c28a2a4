"""GPU parity of moe_backward against the oracle's chain rule.

Weight gradients depend on every token of an expert, so they are compared
stage-isolated: the oracle is fed the GPU's expert choice (index parity of
that choice is covered by the routing tests).  The router weight gradient at
full size is compared with the oracle's router backward fed the GPU's logit
gradient, which is itself compared on sampled tokens."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import as_f64, check_close, dev, host, say
from workloads import CONFIGS, make_inputs, scaled

pytestmark = pytest.mark.gpu


def _layer(cfg, inp, capacity=None, aux_alpha=0.0, fuse_permute=True):
    from mixture_experts_layer_free_amd.layer import MoELayer, Shape
    s = Shape(cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, torch.bfloat16, cfg.score, 0, 0, False, cfg.gamma, True,
              capacity=capacity, aux_alpha=aux_alpha, fuse_permute=fuse_permute)
    return MoELayer(s, dev(inp["w_router"]), dev(inp["w_gate_up"]), dev(inp["w_down"]), dev(inp["bias"].copy()),
                    dev(inp["logit_offset"]))


def _run(cfg, inp, capacity=None, aux_alpha=0.0, fuse_permute=True):
    layer = _layer(cfg, inp, capacity, aux_alpha, fuse_permute)
    x = dev(inp["x"])
    layer.forward(x)
    layer.backward(x, dev(inp["dy"]))
    torch.cuda.synchronize()
    return layer


@pytest.mark.parametrize("score", oracle.SCORE_FNS)
@pytest.mark.parametrize("T,d,E,k,f", [(700, 256, 24, 3, 128), (257, 128, 8, 8, 64), (96, 192, 40, 2, 192),
                                       (1100, 256, 4, 2, 256), (900, 384, 3, 3, 384),   # 256x256 tiles
                                       (600, 128, 4, 2, 128)])                          # 300 rows per group: 128x128 tiles
def test_backward_small(score, T, d, E, k, f):
    say(f"[backward small {score} T={T} d={d} E={E} k={k} f={f}]")
    cfg = scaled(CONFIGS["train"], T=T, d=d, E=E, k=k, f=f, score=score, bias="uniform")
    inp = make_inputs(cfg)
    layer = _run(cfg, inp)
    idx = host(layer.idx).astype(np.int64)
    fwd = oracle.forward(inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"], k, score, True,
                         sel_bias=inp["bias"], logit_offset=inp["logit_offset"], idx=idx)
    g = oracle.backward(fwd, inp["dy"], inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"], score, True)
    check_close(host(layer.dgate), g["dg"], "bf16", "dg")
    check_close(host(layer.dlogit), g["dl"], "bf16", "dl")
    check_close(host(layer.dx), g["dx"], "bf16", "dx")
    check_close(host(layer.dw_router), g["dw_router"], "bf16", "dW_router")
    check_close(host(layer.dw_down), g["dw_down"], "bf16", "dW_down")
    check_close(host(layer.dw_gate_up), g["dw_gate_up"], "bf16", "dW_gate_up")


@pytest.mark.parametrize("score", oracle.SCORE_FNS)
@pytest.mark.parametrize("T,d,E,k,f,cap", [(700, 256, 24, 3, 128, 40), (257, 128, 8, 8, 64, 100),
                                           (1100, 256, 4, 2, 256, 300), (300, 128, 16, 4, 64, 0)])
def test_backward_capacity(score, T, d, E, k, f, cap):
    """Expert capacity in training: dropped slots get dg = 0 and no expert
    gradient, their logits still get dl, and dW_r covers the dropped rows."""
    say(f"[backward capacity {score} T={T} d={d} E={E} k={k} f={f} cap={cap}]")
    cfg = scaled(CONFIGS["train"], T=T, d=d, E=E, k=k, f=f, score=score, bias="uniform")
    inp = make_inputs(cfg)
    layer = _run(cfg, inp, capacity=cap)
    idx = host(layer.idx).astype(np.int64)
    fwd = oracle.forward(inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"], k, score, True,
                         sel_bias=inp["bias"], logit_offset=inp["logit_offset"], idx=idx, capacity=cap)
    assert np.array_equal(host(layer.row_of), fwd["row_of"]) and (fwd["row_of"] < 0).any()
    g = oracle.backward(fwd, inp["dy"], inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"], score, True)
    check_close(host(layer.dgate), g["dg"], "bf16", "dg")
    check_close(host(layer.dlogit), g["dl"], "bf16", "dl")
    check_close(host(layer.dx), g["dx"], "bf16", "dx")
    check_close(host(layer.dw_router), g["dw_router"], "bf16", "dW_router")
    check_close(host(layer.dw_down), g["dw_down"], "bf16", "dW_down")
    check_close(host(layer.dw_gate_up), g["dw_gate_up"], "bf16", "dW_gate_up")


@pytest.mark.parametrize("score", oracle.SCORE_FNS)
@pytest.mark.parametrize("T,d,E,k,f,cap", [(700, 256, 24, 3, 128, None), (257, 128, 8, 8, 64, 100),
                                           (600, 128, 40, 4, 64, 40)])
def test_backward_aux_loss(score, T, d, E, k, f, cap):
    """With the auxiliary loss on, every logit has a gradient: dW_r and dx use
    the dense logit gradient.  Compared with the oracle's backward (same alpha)
    fed the GPU's routing; also with an expert capacity."""
    say(f"[backward aux {score} T={T} d={d} E={E} k={k} f={f} cap={cap}]")
    cfg = scaled(CONFIGS["train"], T=T, d=d, E=E, k=k, f=f, score=score, bias="uniform")
    inp = make_inputs(cfg)
    alpha = 0.5
    layer = _run(cfg, inp, capacity=cap, aux_alpha=alpha)
    idx = host(layer.idx).astype(np.int64)
    fwd = oracle.forward(inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"], k, score, True,
                         sel_bias=inp["bias"], logit_offset=inp["logit_offset"], idx=idx, capacity=cap)
    g = oracle.backward(fwd, inp["dy"], inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"], score, True,
                        aux_alpha=alpha)
    want = oracle.aux_loss(fwd["logits"], fwd["counts"], k, score, alpha)
    assert abs(float(host(layer.aux_loss)[0]) - want) <= 1e-5 * abs(want)
    check_close(host(layer.dlogit), g["dl"], "bf16", "dl (main loss)")
    check_close(host(layer.dw_router), g["dw_router"], "bf16", "dW_router")
    check_close(host(layer.dx), g["dx"], "bf16", "dx")
    check_close(host(layer.dw_gate_up), g["dw_gate_up"], "bf16", "dW_gate_up")


@pytest.mark.parametrize("score", oracle.SCORE_FNS)
def test_backward_aux_loss_contribution(score):
    """The aux loss's own share of dW_r and dx: the GPU's (with alpha) minus
    (without) against the oracle's dense aux logit gradient pushed through
    the router, alpha large enough that this share is of order one."""
    say(f"[backward aux share {score}]")
    cfg = scaled(CONFIGS["train"], T=900, d=128, E=32, k=4, f=64, score=score, bias="uniform")
    inp = make_inputs(cfg)
    alpha = 0.5 * cfg.T
    on = _run(cfg, inp, aux_alpha=alpha)
    dw_on, dx_on = host(on.dw_router).astype(np.float64), host(on.dx).astype(np.float64)
    off = _run(cfg, inp)
    assert np.array_equal(host(on.idx), host(off.idx))
    lg = host(on.logits).astype(np.float64)
    dl_aux = oracle.aux_grad_logits(lg, host(on.counts), cfg.k, score, alpha)
    x64 = as_f64(inp["x"])
    want_dw = dl_aux.T @ x64
    want_dx = dl_aux @ np.asarray(inp["w_router"], np.float64)
    say(f"  aux share of dW_r: {np.linalg.norm(want_dw) / np.linalg.norm(dw_on):.2f}")
    check_close(dw_on - host(off.dw_router), want_dw, "bf16", "dW_r aux share")
    check_close(dx_on - host(off.dx), want_dx, "bf16", "dx aux share")


def test_backward_hash_router():
    """Training with the hash router: constant gates, so dl = 0, dW_r = 0, and
    dx has no router term; the expert gradients are the usual ones."""
    say("[backward hash router]")
    cfg = scaled(CONFIGS["train"], T=700, d=256, E=24, k=3, f=128)
    inp = make_inputs(cfg)
    ids = np.random.default_rng(4).integers(0, 50000, cfg.T).astype(np.int32)
    from mixture_experts_layer_free_amd.layer import MoELayer, Shape
    sh = Shape(cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, torch.bfloat16, cfg.score, train=True, router="hash")
    layer = MoELayer(sh, None, dev(inp["w_gate_up"]), dev(inp["w_down"]))
    x = dev(inp["x"])
    layer.forward(x, token_ids=dev(ids))
    layer.backward(x, dev(inp["dy"]))
    torch.cuda.synchronize()
    idx = oracle.hash_route(ids, cfg.E, cfg.k)["idx"]
    fwd = oracle.forward(inp["x"], None, inp["w_gate_up"], inp["w_down"], cfg.k, "uniform", True, idx=idx)
    g = oracle.backward(fwd, inp["dy"], inp["x"], None, inp["w_gate_up"], inp["w_down"], "uniform", True)
    assert np.all(host(layer.dlogit) == 0) and np.all(host(layer.dw_router) == 0)
    check_close(host(layer.dgate), g["dg"], "bf16", "dg")
    check_close(host(layer.dx), g["dx"], "bf16", "dx")
    check_close(host(layer.dw_down), g["dw_down"], "bf16", "dW_down")
    check_close(host(layer.dw_gate_up), g["dw_gate_up"], "bf16", "dW_gate_up")


@pytest.mark.parametrize("T,d,E,k,f,cap", [(700, 256, 24, 3, 128, None), (1100, 256, 4, 2, 256, None),
                                           (257, 128, 8, 8, 64, None), (600, 128, 6, 2, 128, 180)])
def test_backward_gathered_rows_equal_x_perm(T, d, E, k, f, cap):
    """W_gate_up's weight gradient reading x through token_of (no X_perm)
    adds the same products in the same order as the one reading X_perm, on
    both tile shapes, ragged group ends and with dropped slots: every output
    is bit-identical."""
    say(f"[backward gathered vs X_perm T={T} d={d} E={E} k={k} f={f} cap={cap}]")
    cfg = scaled(CONFIGS["train"], T=T, d=d, E=E, k=k, f=f, score="sqrt_softplus", bias="uniform")
    inp = make_inputs(cfg)
    a = _run(cfg, inp, capacity=cap, fuse_permute=True)
    b = _run(cfg, inp, capacity=cap, fuse_permute=False)
    assert a.x_perm is None and b.x_perm is not None
    for name in ("dw_gate_up", "dw_down", "dw_router", "dx", "dgate"):
        u, v = host(getattr(a, name)), host(getattr(b, name))
        assert np.array_equal(u.view(np.uint32), v.view(np.uint32)), name


@pytest.mark.parametrize("f", [64, 128])
def test_backward_empty_and_skewed_experts(f):
    """Experts that receive no token get exactly zero weight gradients; one
    expert holding most rows spans many K tiles.  f = 128 puts the data
    gradients on 256x256 tiles, the few-row experts on half tiles."""
    say(f"[backward skew f={f}]")
    cfg = scaled(CONFIGS["train"], T=600, d=128, E=16, k=2, f=f, score="sigmoid")
    inp = make_inputs(cfg)
    off = np.zeros(cfg.E, np.float32)
    off[3], off[7] = 6.0, 5.0          # nearly every token picks experts 3 and 7
    off[10:] = -30.0                   # experts 10.. never picked
    inp["logit_offset"] = off
    layer = _run(cfg, inp)
    counts = host(layer.counts)
    assert counts[10:].sum() == 0 and counts[3] > 500
    idx = host(layer.idx).astype(np.int64)
    fwd = oracle.forward(inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"], cfg.k, cfg.score, True,
                         logit_offset=off, idx=idx)
    g = oracle.backward(fwd, inp["dy"], inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"], cfg.score, True)
    dwd = host(layer.dw_down)
    assert np.all(dwd[10:] == 0) and np.all(host(layer.dw_gate_up)[10:] == 0) and np.all(host(layer.dw_router)[10:] == 0)
    check_close(dwd, g["dw_down"], "bf16", "dW_down")
    check_close(host(layer.dw_gate_up), g["dw_gate_up"], "bf16", "dW_gate_up")
    check_close(host(layer.dx), g["dx"], "bf16", "dx")
    check_close(host(layer.dw_router), g["dw_router"], "bf16", "dW_router")


def test_backward_full_training_shape():
    cfg = CONFIGS["train"]
    say(f"[backward full train T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} f={cfg.f}]")
    inp = make_inputs(cfg)
    layer = _run(cfg, inp)
    k = cfg.k
    idx = host(layer.idx).astype(np.int64)
    gates = host(layer.gate)
    offsets = host(layer.offsets)
    token_of = host(layer.token_of)
    row_of = host(layer.row_of)
    x64 = as_f64(inp["x"])
    dy64 = as_f64(inp["dy"])
    rng = np.random.default_rng(0)
    # --- sampled tokens: dg, dl, dx
    toks = np.sort(rng.choice(cfg.T, 24, replace=False))
    fw = oracle.forward(inp["x"][toks], inp["w_router"], inp["w_gate_up"], inp["w_down"], k, cfg.score, True,
                        idx=idx[toks])
    gb = oracle.backward(fw, inp["dy"][toks], inp["x"][toks], inp["w_router"], inp["w_gate_up"], inp["w_down"],
                         cfg.score, True)
    check_close(host(layer.dgate)[toks], gb["dg"], "bf16", "dg (sampled tokens)")
    check_close(host(layer.dlogit)[toks], gb["dl"], "bf16", "dl (sampled tokens)")
    check_close(host(layer.dx)[toks], gb["dx"], "bf16", "dx (sampled tokens)")
    # --- router weight gradient: the oracle's router backward fed the GPU's dl
    dwr, _ = oracle.router_backward(host(layer.dlogit).astype(np.float64), idx, inp["x"], inp["w_router"])
    check_close(host(layer.dw_router), dwr, "bf16", "dW_router (GPU dl)")
    # --- expert weight gradients of sampled experts, over all of their rows
    counts = np.diff(offsets)
    for e in sorted({int(counts.argmin()), int(counts.argmax()), int(rng.integers(0, cfg.E))}):
        a, b = int(offsets[e]), int(offsets[e + 1])
        rows = np.arange(a, b)
        tk = token_of[rows]
        slot = np.array([np.nonzero(row_of[t] == r)[0][0] for t, r in zip(tk, rows)])
        ex = oracle.expert_ffn(x64[tk], inp["w_gate_up"][e], inp["w_down"][e], True)
        dyp = oracle.bf16_round(gates[tk, slot][:, None].astype(np.float64) * dy64[tk])
        r = oracle.expert_backward_rows(dyp, x64[tk], ex["G"], ex["U"], ex["H"], inp["w_gate_up"][e],
                                        inp["w_down"][e], True)
        say(f"  expert {e}: {b - a} rows")
        check_close(host(layer.dw_down[e]), r["dW_down"], "bf16", f"dW_down[{e}]")
        check_close(host(layer.dw_gate_up[e]), r["dW_gate_up"], "bf16", f"dW_gate_up[{e}]")


@pytest.mark.parametrize("score", oracle.SCORE_FNS)
def test_backward_replay_invalid_ids(score):
    """Training on a replayed choice in which some expert ids lie outside
    [0, E): those slots have gate 0, no row and no gradient, and every other
    gradient is the oracle's for the same choice."""
    say(f"[backward replay with invalid ids {score}]")
    cfg = scaled(CONFIGS["train"], T=500, d=128, E=16, k=4, f=64, score=score, bias="uniform")
    inp = make_inputs(cfg)
    rng = np.random.default_rng(7)
    ridx = np.stack([rng.permutation(cfg.E)[:cfg.k] for _ in range(cfg.T)]).astype(np.int64)
    bad = rng.random(ridx.shape) < 0.2
    ridx[bad] = rng.choice([-1, -100, cfg.E, 1 << 20], int(bad.sum()))
    ridx[:3] = -1                                   # tokens with no valid slot
    layer = _layer(cfg, inp)
    x = dev(inp["x"])
    layer.forward(x, replay_idx=dev(ridx.astype(np.int32)))
    layer.backward(x, dev(inp["dy"]))
    torch.cuda.synchronize()
    fwd = oracle.forward(inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"], cfg.k, score, True,
                         logit_offset=inp["logit_offset"], idx=ridx)
    g = oracle.backward(fwd, inp["dy"], inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"], score, True)
    valid = (ridx >= 0) & (ridx < cfg.E)
    assert np.all(host(layer.gate)[~valid] == 0) and np.all(host(layer.dlogit)[~valid] == 0)
    assert np.all(host(layer.dgate)[~valid] == 0)
    check_close(host(layer.out), fwd["out"], "bf16", "out")
    check_close(host(layer.dgate), g["dg"], "bf16", "dg")
    check_close(host(layer.dlogit), g["dl"], "bf16", "dl")
    check_close(host(layer.dx), g["dx"], "bf16", "dx")
    check_close(host(layer.dw_router), g["dw_router"], "bf16", "dW_router")
    check_close(host(layer.dw_down), g["dw_down"], "bf16", "dW_down")
    check_close(host(layer.dw_gate_up), g["dw_gate_up"], "bf16", "dW_gate_up")
