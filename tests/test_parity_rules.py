"""CPU checks of the comparison rules in tests/parity.py themselves: the
output-spacing rule must accept only what the final rounding of a 16-bit
output can explain, and nothing the stated bars would reject otherwise."""

import numpy as np
import pytest
import torch

from tests.parity import assert_within, errors, output_spacing_check


def _case(ref_vals, gpu_vals):
    o_ref = np.asarray(ref_vals, np.float64).reshape(1, 1, -1, 1)
    o = np.asarray(gpu_vals, np.float64).reshape(1, 1, -1, 1)
    lse = np.zeros((1, 1, o.shape[2]))
    return o, o_ref, errors(o, lse, o_ref, lse)


def _bf16(x):
    return float(torch.tensor(x, dtype=torch.float64).to(torch.bfloat16).to(torch.float64))


def test_far_neighbour_in_2_to_4_is_one_ulp():
    # exact 2.2448: nearest bf16 2.25, far neighbour 2.234375 (0.0104 away)
    ref = [2.2448] + [0.1] * 99
    o, o_ref, st = _case(ref, [2.234375] + [0.1] * 99)
    with pytest.raises(AssertionError):
        assert_within(st, "bf16")
    assert output_spacing_check(o, o_ref, st, "bf16") == 1


def test_two_ulps_rejected():
    ref = [2.2448] + [0.1] * 99
    o, o_ref, st = _case(ref, [2.25 + 2 * 2 ** -6] + [0.1] * 99)
    with pytest.raises(AssertionError, match="ulp"):
        output_spacing_check(o, o_ref, st, "bf16")


def test_small_values_keep_the_bar():
    # |O| < 1: bf16 spacing there cannot reach 1e-2, so a miss is a real error
    ref = [0.5123] + [0.1] * 99
    o, o_ref, st = _case(ref, [0.5123 + 0.011] + [0.1] * 99)
    with pytest.raises(AssertionError, match="below"):
        output_spacing_check(o, o_ref, st, "bf16")


def test_fp16_spacing_is_tighter_than_the_bar():
    # fp16 values in [2, 4) are 2^-9 apart: a 0.0104 miss is many ulps
    ref = [2.2448] + [0.1] * 99
    o, o_ref, st = _case(ref, [2.2448 - 0.0104] + [0.1] * 99)
    with pytest.raises(AssertionError, match="ulp"):
        output_spacing_check(o, o_ref, st, "fp16")


def test_mean_and_lse_bars_still_apply():
    ref = [2.2448] * 100
    o, o_ref, st = _case(ref, [2.234375] * 100)   # every element 0.0104 off
    with pytest.raises(AssertionError, match="mean"):
        output_spacing_check(o, o_ref, st, "bf16")


def test_within_bar_needs_no_rule():
    o, o_ref, st = _case([2.2448] + [0.1] * 99, [_bf16(2.2448)] + [0.1] * 99)
    assert output_spacing_check(o, o_ref, st, "bf16") == 0
