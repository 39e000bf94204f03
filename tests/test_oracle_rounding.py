"""Pins for the oracle's round-to-nearest-even into bf16 / f32: against torch's
own float32 -> bfloat16 conversion (a library routine) on values that are
exact in float32, against mpmath's 8-bit rounding on arbitrary float64 values,
and against hand-placed ties."""

import mpmath
import numpy as np
import pytest
import torch

from oracle import round_bf16, round_to


def test_matches_torch_on_float32_values():
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-38).astype(np.float32),      # subnormal range
        (rng.standard_normal(20000) * 1e30).astype(np.float32),
        rng.integers(-(2 ** 31), 2 ** 31, 20000).astype(np.int64).astype(np.uint32).view(np.float32),
    ])
    vals = vals[np.isfinite(vals)]
    want = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float64).numpy()
    got = round_bf16(vals.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_matches_mpmath_8bit_rounding_on_float64():
    rng = np.random.default_rng(1)
    vals = rng.standard_normal(3000) * np.exp2(rng.integers(-60, 60, 3000))
    got = round_bf16(vals)
    for v, g in zip(vals, got):
        with mpmath.workprec(8):          # mpmath rounds to nearest, ties to even
            want = float(+mpmath.mpf(float(v)))
        assert g == want


@pytest.mark.parametrize("x,want", [
    (1.0 + 2.0 ** -8, 1.0),                        # tie -> even (mantissa 0)
    (1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -6),        # tie -> even (round up)
    (1.0 + 2.0 ** -8 + 2.0 ** -40, 1.0 + 2.0 ** -7),   # just above the tie
    (-(1.0 + 2.0 ** -8), -1.0),
    (0.0, 0.0),
    (2.0 ** -133, 2.0 ** -133),                    # smallest subnormal
    (2.0 ** -134, 0.0),                            # tie with zero -> even (zero)
    (3 * 2.0 ** -134, 2.0 ** -132),                # tie -> even
    (3.4e38, np.inf),                              # beyond the largest finite bf16
    (3.3895313892515355e38, 3.3895313892515355e38),   # largest finite bf16
])
def test_hand_placed_cases(x, want):
    assert round_bf16(np.array([x]))[0] == want


def test_non_finite_pass_through():
    got = round_bf16(np.array([np.nan, np.inf, -np.inf]))
    assert np.isnan(got[0]) and got[1] == np.inf and got[2] == -np.inf


def test_f32_rounding_is_numpy_cast():
    x = np.array([1.0 + 2.0 ** -24, 1.0 + 3 * 2.0 ** -24, 0.1])
    np.testing.assert_array_equal(round_to(x, "f32"), [1.0, 1.0 + 2.0 ** -22, np.float32(0.1)])


def test_power_of_two_scaling_commutes():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(10000)
    for k in (-5, 3, 20):
        np.testing.assert_array_equal(round_bf16(x * 2.0 ** k), round_bf16(x) * 2.0 ** k)
