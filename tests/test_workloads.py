"""The seeded input generators: determinism, shapes, distributions, the
per-expert seeding that lets one expert be regenerated alone, and the skew
of the Zipf logit offset."""
import hashlib

import numpy as np
import pytest

import oracle
from workloads import CONFIGS, bf16_bits_to_f32, expert_weights, f32_to_bf16_bits, make_inputs, scaled


def _digest(inp):
    h = hashlib.sha256()
    for k in sorted(inp):
        if inp[k] is not None:
            h.update(k.encode())
            h.update(np.ascontiguousarray(inp[k]).tobytes())
    return h.hexdigest()


def test_generation_is_deterministic():
    cfg = scaled(CONFIGS["fine"], T=64, d=64, f=32)
    assert _digest(make_inputs(cfg)) == _digest(make_inputs(cfg, workers=1))
    assert _digest(make_inputs(cfg)) != _digest(make_inputs(scaled(cfg, seed=9)))


@pytest.mark.parametrize("name", ["tiny", "tiny_dense"])
def test_tiny_shapes_and_types(name):
    cfg = CONFIGS[name]
    inp = make_inputs(cfg)
    assert inp["x"].shape == (cfg.T, cfg.d) and inp["x"].dtype == np.float32
    assert inp["w_gate_up"].shape == (cfg.E, 2 * cfg.f, cfg.d)
    assert inp["w_down"].shape == (cfg.E, cfg.d, cfg.f)
    assert np.all(np.abs(inp["bias"]) <= 0.05) and np.any(inp["bias"] != 0)


def test_one_expert_regenerates_alone():
    cfg = scaled(CONFIGS["dsv3"], T=8, d=64, E=16, f=32, f_shared=32)
    inp = make_inputs(cfg)
    for e in (0, 7, 15):
        gu, dn = expert_weights(cfg, e)
        assert np.array_equal(gu, inp["w_gate_up"][e]) and np.array_equal(dn, inp["w_down"][e])
    assert inp["w_gate_up_shared"].shape == (1, 64, 64)


def test_bf16_packing_matches_oracle_rounding():
    v = np.random.default_rng(3).standard_normal(5000).astype(np.float32)
    bits = f32_to_bf16_bits(v)
    assert np.array_equal(bf16_bits_to_f32(bits).astype(np.float64), oracle.bf16_round(v.astype(np.float64)))


def test_distributions():
    cfg = scaled(CONFIGS["dsv3"], T=256, d=512, E=8, f=64, f_shared=64)
    inp = make_inputs(cfg)
    x = bf16_bits_to_f32(inp["x"])
    assert abs(x.std() - 1.0) < 0.02
    w = bf16_bits_to_f32(inp["w_gate_up"])
    assert abs(w.std() - 0.006) < 0.0002
    assert abs(inp["w_router"].std() - 0.006) < 0.0003


def test_zipf_offset_gives_skewed_load():
    """The fine-grained workload's offset makes the routed load uneven
    (max/mean well above 1) without collapsing it onto one expert."""
    cfg = scaled(CONFIGS["fine"], T=2048)
    inp = make_inputs(cfg, experts=False)
    o = inp["logit_offset"]
    np.testing.assert_allclose(np.sort(-o / (0.5 * 1.2)), np.log(np.arange(1, 65)), rtol=1e-6, atol=1e-6)
    r = oracle.route(inp["x"], inp["w_router"], cfg.k, cfg.score, logit_offset=o)
    c = np.bincount(r["idx"].reshape(-1), minlength=cfg.E)
    assert 3.0 < c.max() / c.mean() < 12.0
    assert c.max() < cfg.T
