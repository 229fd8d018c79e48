"""The bf16 output allowance of the parity harness: the 1e-2 bar is unchanged wherever a
bf16 output can meet it, and above magnitude 4 exactly bf16's own extra rounding is
allowed, no more."""
import numpy as np
import torch

from _harness import bf16_rounding_excess, max_err


def _bf16(x):
    return torch.tensor(x, dtype=torch.float64).to(torch.bfloat16)


def test_no_allowance_below_four():
    e = np.array([0.0, 1e-3, -0.7, 1.999, 2.0, -3.99])
    assert np.all(bf16_rounding_excess(e) == 0.0)


def test_allowance_is_bf16_half_spacing_minus_two_to_minus_seven():
    e = np.array([4.0, -4.10548, 7.99, 8.0, 15.5])
    want = np.array([2.0**-6 - 2.0**-7] * 3 + [2.0**-5 - 2.0**-7] * 2)
    np.testing.assert_array_equal(bf16_rounding_excess(e), want)


def test_correctly_rounded_output_passes_and_a_neighbour_fails():
    exact = np.array([4.10548, -5.96, 3.49, 0.31])
    good = _bf16(exact.tolist())
    assert max_err(good, exact) <= 1e-2
    # one bf16 step away from the correctly rounded value fails the bar
    bad = good.clone()
    bad[0] = (good[0].float() + 2.0**-5).to(torch.bfloat16)
    assert max_err(bad, exact) > 1e-2
    # below magnitude 4 the plain bar applies: 0.011 off fails
    off = _bf16((exact + np.array([0, 0, 0, 0.011])).tolist())
    assert max_err(off, exact) > 1e-2


def test_float32_outputs_take_no_allowance():
    exact = np.array([5.0])
    out = torch.tensor([5.0 + 0.012], dtype=torch.float32)
    assert abs(max_err(out, exact) - 0.012) < 1e-6
