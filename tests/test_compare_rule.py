"""The parity bar itself (tests/parity.py compare), checked on hand-made bf16
outputs against exact values: no GPU involved."""
import numpy as np
import pytest
import torch

from parity import compare


def bf16(x):
    return torch.tensor(x, dtype=torch.float64).to(torch.bfloat16)


def test_reachable_elements_take_the_absolute_bound():
    ref = np.array([0.5 + 2 ** -10, 3.0 + 0.004])        # bf16 steps 2^-8 and 2^-6 here
    compare(bf16([0.5, 3.0]), ref, "rne")                  # correctly rounded: passes
    # 3.0 + 2^-6 is the other neighbour of 3.004, 0.0116 away: over 1e-2
    with pytest.raises(AssertionError):
        compare(bf16([0.5, 3.0 + 2 ** -6]), ref, "far neighbour", mean_abs=1.0)


def test_unreachable_elements_need_a_bf16_neighbour():
    ref = np.array([5.0 + 0.0125])                         # step 2^-5: RNE error 0.0125 > 1e-2
    compare(bf16([5.0]), ref, "lower neighbour", mean_abs=1.0)
    compare(bf16([5.0 + 2 ** -5]), ref, "upper neighbour", mean_abs=1.0)
    with pytest.raises(AssertionError):
        compare(bf16([5.0 + 2 ** -4]), ref, "two steps away", mean_abs=1.0)


def test_mean_bound_against_fp64_when_reachable():
    ref = np.full(1000, 0.25)
    compare(bf16(np.full(1000, 0.25)), ref, "exact")
    with pytest.raises(AssertionError):
        compare(bf16(np.full(1000, 0.25 + 2 ** -9)), ref, "biased")   # mean 2e-3


def test_relative_mode_scales_by_magnitude():
    ref = np.array([300.0 + 0.3])
    compare(bf16([300.0]), ref, "relative", relative=True)
    with pytest.raises(AssertionError):
        compare(bf16([304.0]), ref, "relative, far", relative=True, mean_abs=1.0)


def test_term_scale_mode_scales_by_the_terms_magnitude():
    # an output of 4 that cancels terms of magnitude 3000: an error of 2 is
    # 2 / 3000 < 1e-2 of the terms, but half the output
    ref = np.array([4.0])
    compare(bf16([6.0]), ref, "cancellation", term_scale=np.array([3000.0]), mean_abs=1.0)
    with pytest.raises(AssertionError):
        compare(bf16([6.0]), ref, "same error without the terms", relative=True, mean_abs=1.0)
    with pytest.raises(AssertionError):
        compare(bf16([40.0]), ref, "36 / 3000 > 1e-2", term_scale=np.array([3000.0]), mean_abs=1.0)
    # a term scale below |out| cannot be a sum of |terms|
    with pytest.raises(AssertionError):
        compare(bf16([4.0]), ref, "bad term scale", term_scale=np.array([1.0]))
