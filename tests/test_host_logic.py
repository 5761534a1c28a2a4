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
