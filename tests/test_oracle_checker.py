"""Pins of ``oracle.rel_max_err``, the checker every parity test and the smoke
check use: the relative max error of one tensor, max|got - ref| / max|ref|
(the infinity-norm reading of "relative max error", one value per tensor).

The expected values are worked out by hand in the comments; nothing here
re-derives them with the function's own formula."""
import numpy as np
import pytest

import oracle


def test_hand_values():
    # |diff| = (0, 0, 1), max |ref| = 4  ->  1/4
    assert oracle.rel_max_err([1.0, 2.0, 3.0], [1.0, 2.0, 4.0]) == 0.25
    # the largest |ref| is a negative entry: |-8| = 8; max |diff| = 1  ->  1/8
    assert oracle.rel_max_err([-7.0, 2.0], [-8.0, 2.0]) == 0.125
    # the error and the largest reference entry sit at different places:
    # |diff| = (0.5, 0), max |ref| = 10  ->  0.05
    assert oracle.rel_max_err([0.5, 10.0], [0.0, 10.0]) == 0.05
    # identical tensors
    assert oracle.rel_max_err(np.arange(6.0).reshape(2, 3), np.arange(6.0).reshape(2, 3)) == 0.0


def test_denominator_is_the_reference_not_the_result():
    # got has the larger entries; only ref's 2 divides: |diff| max = 98  ->  49
    assert oracle.rel_max_err([100.0, 0.0], [2.0, 0.0]) == 49.0
    assert oracle.rel_max_err([2.0, 0.0], [100.0, 0.0]) == pytest.approx(0.98)


def test_all_zero_reference_gives_the_absolute_error():
    assert oracle.rel_max_err([0.0, -3.0], [0.0, 0.0]) == 3.0
    assert oracle.rel_max_err([0.0], [0.0]) == 0.0


def test_empty_tensors_have_no_error():
    assert oracle.rel_max_err(np.zeros((0, 4)), np.zeros((0, 4))) == 0.0


def test_non_finite_results_never_pass_a_tolerance():
    # a NaN or an infinity in the result must make every "err <= tol" check fail
    for bad in (np.nan, np.inf, -np.inf):
        e = oracle.rel_max_err([1.0, bad], [1.0, 2.0])
        assert not (e <= 1.0)


def test_float32_inputs_are_compared_in_float64():
    # 1 + 2^-23 and 1 differ by one float32 ulp; in float64 the difference is exact
    got = np.array([1.0 + 2.0 ** -23], dtype=np.float32)
    ref = np.array([1.0], dtype=np.float32)
    assert oracle.rel_max_err(got, ref) == 2.0 ** -23


def test_broadcast_shapes_are_not_accepted_silently():
    # the checker compares like with like: mismatched shapes raise
    with pytest.raises(ValueError):
        oracle.rel_max_err(np.zeros((2, 3)), np.zeros((3, 2)))
    with pytest.raises(ValueError):
        oracle.rel_max_err(np.zeros((2, 3)), np.zeros(3))      # would broadcast
