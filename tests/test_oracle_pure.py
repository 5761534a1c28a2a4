"""The pure-Python forward (oracle/pure.py: per-token loops, experts applied
to the token itself, top-k by repeated selection) against the numpy oracle
(matrix products, stable argsort, permute -> grouped experts -> combine) on
the tiny workloads, every score function, bf16 storage points, a shared
expert, a logit offset and exact ties.  Two independent codings of the same
definition: a dropped term, a wrong index or a transposed weight in either
one shows up as a mismatch here."""
import numpy as np
import pytest

import oracle
from oracle import pure
from workloads import CONFIGS, make_inputs, scaled


def _lists(a):
    return None if a is None else oracle.bf16_from_bits(a).tolist() if np.asarray(a).dtype == np.uint16 \
        else np.asarray(a, np.float64).tolist()


def _both(inp, k, fn, bf16, shared=False, offset=False):
    args = dict(sel_bias=inp.get("bias"), logit_offset=inp.get("logit_offset") if offset else None)
    sh = dict(w_gate_up_shared=inp.get("w_gate_up_shared"), w_down_shared=inp.get("w_down_shared")) if shared else {}
    ref = oracle.forward(inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"], k, fn, bf16, **args, **sh)
    got = pure.forward(_lists(inp["x"]), _lists(inp["w_router"]), _lists(inp["w_gate_up"]), _lists(inp["w_down"]),
                       k, fn, bf16, **{a: _lists(v) for a, v in args.items()},
                       **{a: _lists(v) for a, v in sh.items()})
    return ref, got


def _check(ref, got, out_rel=1e-12):
    assert np.array_equal(np.asarray(got["idx"]), ref["idx"])
    np.testing.assert_allclose(np.asarray(got["gates"]), ref["gates"], rtol=1e-13, atol=1e-15)
    out = np.asarray(got["out"])
    scale = np.abs(ref["out"]).max()
    assert np.abs(out - ref["out"]).max() <= out_rel * scale


@pytest.mark.parametrize("fn", oracle.SCORE_FNS)
def test_pure_python_equals_numpy_oracle_tiny(fn):
    """Config 1 (T=64, d=32, 8 experts top-2, fp32, selection bias)."""
    cfg = CONFIGS["tiny"]
    ref, got = _both(make_inputs(cfg), cfg.k, fn, False)
    _check(ref, got)


def test_pure_python_equals_numpy_oracle_dense_case():
    """Config 1's one-expert, k=1 variant: every gate is 1."""
    cfg = CONFIGS["tiny_dense"]
    ref, got = _both(make_inputs(cfg), 1, "softmax", False)
    _check(ref, got)
    assert all(g == [1.0] for g in got["gates"])


@pytest.mark.parametrize("fn", ["sigmoid", "sqrt_softplus"])
def test_pure_python_equals_numpy_oracle_bf16_shared_offset(fn):
    """bf16 inputs and storage points (H rounded to bf16), one shared expert,
    a per-expert logit offset (the skewed workloads'), top-3 of 6."""
    cfg = scaled(CONFIGS["dsv3"], T=24, d=16, E=6, k=3, f=16, f_shared=32)
    inp = make_inputs(cfg)
    inp["logit_offset"] = np.linspace(-0.3, 0.3, cfg.E).astype(np.float32)
    ref, got = _both(inp, cfg.k, fn, True, shared=True, offset=True)
    _check(ref, got, out_rel=1e-11)


def test_pure_python_ties_go_to_the_lower_index():
    """Duplicated router rows give equal keys: both codings pick the lower
    expert first and agree on the gates."""
    cfg = scaled(CONFIGS["tiny"], T=16, E=6, k=3)
    inp = make_inputs(cfg)
    w = np.array(inp["w_router"])
    w[4] = w[1]
    w[5] = w[2]
    inp["w_router"] = w
    inp["bias"] = None
    for fn in oracle.SCORE_FNS:
        ref, got = _both(inp, cfg.k, fn, False)
        _check(ref, got)
        for chosen in got["idx"]:
            assert not (4 in chosen and 1 not in chosen) and not (5 in chosen and 2 not in chosen)
