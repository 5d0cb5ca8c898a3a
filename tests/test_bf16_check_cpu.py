"""CPU checks of the bf16-mode hidden-code comparison (tests/bf16_check.py):
it accepts the oracle's own codes, a flip to the neighbour where the exact
value sits at the midpoint, and small-h codes off by more within the
row-scale allowance; it rejects codes whose value is off beyond it."""
import numpy as np
import pytest

import oracle
from tests import bf16_check as B


def _codes(v):
    return oracle.bf16_round(np.asarray(v, np.float64))


def test_identical_codes_pass():
    x = np.random.default_rng(0).standard_normal(512) * 300
    assert B.check_codes(_codes(x), x)[0] == 0


def test_flip_at_midpoint_passes():
    # 1 + 2^-8 is the midpoint of 1 and 1 + 2^-7; nudged a hair above it
    x = np.array([1.0 + 2.0 ** -8 + 2.0 ** -20, -(3.0 + 2.0 ** -7 - 2.0 ** -22), 2.0])
    g = _codes(x)
    g[0] = 1.0                     # the other neighbour of x[0]
    g[1] = -(3.0 + 2.0 ** -6)      # the other neighbour of x[1] (spacing 2^-6 at 2..4)
    n, ex = B.check_codes(g, x)
    assert n == 2 and ex <= B.TAU


def test_small_value_within_row_allowance_passes():
    # the row's largest |h| is 4096; a value of 1e-3 off by 1e-4 (many bf16 steps)
    x = np.array([4096.0, 1.0e-3])
    g = _codes(np.array([4096.0, 1.1e-3]))
    n, ex = B.check_codes(g, x)
    assert n == 1 and ex < B.TAU


def test_large_value_off_by_a_step_far_from_midpoint_fails():
    x = np.array([4096.0 * (1.0 + 2.0 ** -9)])  # a quarter step above 4096: its code is 4096
    g = np.array([4096.0 * (1.0 + 2.0 ** -7)])
    with pytest.raises(AssertionError):
        B.check_codes(g, x)


def test_unrelated_values_fail():
    g0 = np.random.default_rng(1).standard_normal(256) * 300
    x = np.random.default_rng(2).standard_normal(256) * 300
    with pytest.raises(AssertionError):
        B.check_codes(_codes(g0), x)
