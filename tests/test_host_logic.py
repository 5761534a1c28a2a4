"""Host-side helpers of the layer (no GPU needed)."""
from fractions import Fraction
from math import ceil

import pytest

from mixture_experts_layer_free_amd.layer import expert_capacity


@pytest.mark.parametrize("C,T,k,E,want", [
    (1.0, 8192, 8, 64, 1024),      # 64 experts top-8: T*k/E
    (1.25, 8192, 8, 64, 1280),
    (1.0, 100, 1, 8, 13),          # the lesson's C x N / E for top-1, rounded up
    (0.0, 100, 2, 8, 0),
    (2.0, 7, 3, 5, 9),             # ceil(8.4)
])
def test_expert_capacity(C, T, k, E, want):
    assert expert_capacity(C, T, k, E) == want


def test_expert_capacity_is_exact_on_the_float_factor():
    # 1.1 as a double is slightly above 11/10, so 1.1 * 10 rounds up to 12
    assert Fraction(1.1) > Fraction(11, 10)
    assert expert_capacity(1.1, 10, 1, 1) == 12
    assert expert_capacity(1.1, 10, 1, 1) == ceil(Fraction(1.1) * 10)


def test_rounding_ambiguity_flags_exactly_the_values_near_a_bf16_midpoint():
    """gpu_helpers.rounding_ambiguous against the oracle's bf16 rounding: a
    value is flagged exactly when moving it by the relative margin down or up
    changes its rounded bf16 value, and the reported unit is the spacing of
    bf16 values at it (8 significant bits)."""
    import numpy as np

    import oracle
    from gpu_helpers import rounding_ambiguous
    rel = 2.0 ** -12                                   # wide enough to flag many random values
    rng = np.random.default_rng(0)
    near = oracle.bf16_round(rng.uniform(0.3, 9.0, 3000))
    near = near + np.ldexp(1.0, np.frexp(near)[1] - 9) * (1 + rng.uniform(-3, 3, near.size) * rel)
    v = np.abs(np.concatenate([rng.standard_normal(30000) * 3, near,
                               oracle.bf16_round(rng.standard_normal(500)), [1.0 + 2.0 ** -8, 0.0]]))
    amb, ulp = rounding_ambiguous(v, rel)
    flips = oracle.bf16_round(v * (1 - rel)) != oracle.bf16_round(v * (1 + rel))
    assert np.array_equal(amb[v > 0], flips[v > 0])
    assert amb.sum() > 100 and (~amb).sum() > 100
    assert amb[-2] and not amb[-1]                     # an exact midpoint is ambiguous, 0 is not
    nz = v > 0
    e = np.frexp(v[nz])[1]
    assert np.all(ulp[nz] == np.ldexp(1.0, e - 8))
    assert np.all((ulp[nz] <= v[nz] * 2.0 ** -7) & (ulp[nz] > v[nz] * 2.0 ** -8))
