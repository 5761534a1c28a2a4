"""Replaying a captured HIP graph of the layer step gives, on every replay,
exactly the eager result (the kernels are deterministic), with eager work and
synchronisations between replays."""
import numpy as np
import pytest
import torch

from gpu_helpers import dev, host, say
from workloads import CONFIGS, make_inputs, scaled

pytestmark = pytest.mark.gpu


def _layer(cfg, inp, train, packed=False):
    from mixture_experts_layer_free_amd.layer import MoELayer, Shape
    s = Shape(cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, torch.bfloat16, cfg.score, cfg.shared, cfg.f_shared,
              cfg.bias_update, cfg.gamma, train, packed_weights=packed)
    return MoELayer(s, dev(inp["w_router"]), dev(inp["w_gate_up"]), dev(inp["w_down"]), dev(inp["bias"].copy()),
                    dev(inp["logit_offset"]), dev(inp.get("w_gate_up_shared")), dev(inp.get("w_down_shared")))


@pytest.mark.parametrize("train,packed", [(False, False), (True, False), (False, True)])
def test_graph_replays_match_eager(train, packed):
    """packed: a forward-only layer on expert weights packed in tile order
    (the configuration the forward-only lines of the benchmark replay)."""
    say(f"[graph replay train={train} packed weights={packed}]")
    cfg = scaled(CONFIGS["train"], T=1024, d=256, E=16, k=4, f=128, score="sigmoid", bias_update=True)
    if not train:
        cfg = scaled(cfg, shared=1, f_shared=128)
    inp = make_inputs(cfg)
    x = dev(inp["x"])
    dy = dev(inp["dy"]) if train else None
    g_layer = _layer(cfg, inp, train, packed)
    e_layer = _layer(cfg, inp, train, packed)
    assert (g_layer.packed is not None) == packed
    graph = g_layer.capture(x, dy)
    # capture ran one eager warm-up step on g_layer (bias updated once): match it
    e_layer.forward(x)
    if train:
        e_layer.backward(x, dy)
    for rep in range(4):
        graph.replay()
        e_layer.forward(x)
        if train:
            e_layer.backward(x, dy)
        torch.cuda.synchronize()
        junk = torch.randn(1000, device="cuda").sum().item()   # unrelated eager work between replays
        assert np.array_equal(host(g_layer.out), host(e_layer.out)), rep
        assert np.array_equal(host(g_layer.sel_bias), host(e_layer.sel_bias)), rep
        assert np.array_equal(host(g_layer.counts), host(e_layer.counts)), rep
        if train:
            for name in ("dx", "dw_router", "dw_gate_up", "dw_down"):
                assert np.array_equal(host(getattr(g_layer, name)), host(getattr(e_layer, name))), (rep, name)
    say("  4 replays bit-identical to eager")
