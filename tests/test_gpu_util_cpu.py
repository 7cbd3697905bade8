"""The parity helper itself (CPU): a NaN or a stray infinity on either side
must fail a comparison, matching infinities must not."""
import math

import numpy as np
import pytest

from gpu_util import max_err


def test_plain_difference():
    assert max_err([1.0, 2.0, 3.0], [1.0, 2.5, 2.0]) == 1.0
    assert max_err(np.zeros((0, 4)), np.zeros((0, 4))) == 0.0


@pytest.mark.parametrize("side", [0, 1])
def test_nan_on_either_side_fails(side):
    a = np.ones(8)
    b = np.ones(8)
    (a if side == 0 else b)[3] = np.nan
    assert max_err(a, b) == math.inf


def test_nan_on_both_sides_fails():
    a = np.full(4, np.nan)
    assert max_err(a, a.copy()) == math.inf


def test_matching_infinities_are_equal():
    a = np.array([-np.inf, 0.5, -np.inf])
    b = np.array([-np.inf, 0.25, -np.inf])
    assert max_err(a, b) == 0.25
    assert max_err(np.array([-np.inf]), np.array([-np.inf])) == 0.0


@pytest.mark.parametrize("a,b", [([np.inf], [1.0]), ([1.0], [-np.inf]), ([np.inf], [-np.inf])])
def test_mismatched_infinities_fail(a, b):
    assert max_err(np.array(a), np.array(b)) == math.inf


def test_shape_mismatch_raises():
    with pytest.raises(ValueError):
        max_err(np.ones(3), np.ones(4))


def test_no_runtime_warning_on_infinite_rows():
    with np.errstate(all="raise"):
        assert max_err(np.array([-np.inf, 1.0]), np.array([-np.inf, 1.0])) == 0.0
