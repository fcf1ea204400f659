"""Pins of the comparator that decides every floating-point parity verdict:
rel_err_floor(got, ref) = max_i |got_i - ref_i| / max(|ref_i|, RMS(ref)).

The tolerance metric reads the north-star's "max relative error" with the
denominator floored at the reference's RMS, because elementwise relative
error is ill-posed where the aclnnWeightQuantMatmulAllReduceAddRmsNorm
page's y (Formula) passes near zero. Every expected value below is worked by
hand from that definition (the arithmetic is in the comment beside it); a
comparator with a dropped floor, a floor taken from the wrong argument, a
mean instead of a max, or a self-comparison fails at least one of them."""
import math

import numpy as np
import pytest
import torch

import oracle


def test_element_above_the_floor_uses_its_own_magnitude():
    # ref [3, 4]: RMS = sqrt((9 + 16) / 2) = 3.5355; the error 0.1 sits on
    # the element 4 > RMS, so the ratio is 0.1 / 4 = 0.025
    assert oracle.rel_err_floor([3.0, 4.1], [3.0, 4.0]) == pytest.approx(0.025, rel=1e-12)


def test_element_below_the_floor_uses_the_rms():
    # ref [0.5, 7]: RMS = sqrt((0.25 + 49) / 2) = sqrt(24.625); the error 0.1
    # sits on 0.5 < RMS, so the ratio is 0.1 / sqrt(24.625) = 0.020152...,
    # not the raw relative error 0.1 / 0.5 = 0.2
    e = oracle.rel_err_floor([0.6, 7.0], [0.5, 7.0])
    assert e == pytest.approx(0.1 / math.sqrt(24.625), rel=1e-12)
    assert e < 0.0202


def test_the_floor_comes_from_the_reference_not_the_result():
    # ref [1, 1] (RMS 1), got [1, 3]: |3 - 1| / max(1, 1) = 2 exactly. Taking
    # the RMS or the magnitude from got would give 2 / 3 instead.
    assert oracle.rel_err_floor([1.0, 3.0], [1.0, 1.0]) == 2.0
    assert oracle.rel_err_floor([1.0, 1.0], [1.0, 3.0]) == pytest.approx(2.0 / 3.0, rel=1e-12)


def test_a_single_outlier_is_the_maximum_not_the_mean():
    # ref [1, 1, 1, 100]: RMS = sqrt((3 + 10000) / 4) = 50.0075; got misses
    # the first element by 0.5, the rest exactly: 0.5 / 50.0075 = 0.0099985
    ref = [1.0, 1.0, 1.0, 100.0]
    got = [1.5, 1.0, 1.0, 100.0]
    assert oracle.rel_err_floor(got, ref) == pytest.approx(0.5 / math.sqrt(10003 / 4), rel=1e-12)
    # one bad element among many good ones still decides the verdict
    ref2 = np.ones(10000)
    got2 = ref2.copy()
    got2[1234] = 1.02
    assert oracle.rel_err_floor(got2, ref2) == pytest.approx(0.02, rel=1e-9)


def test_all_zero_reference_falls_back_to_the_absolute_error():
    # RMS(ref) = 0: the denominator of a zero element is then 1, so the
    # measure is the absolute error (and exact zeros pass with 0)
    assert oracle.rel_err_floor([0.0, 0.0], [0.0, 0.0]) == 0.0
    assert oracle.rel_err_floor([0.0, 1e-3], [0.0, 0.0]) == pytest.approx(1e-3, rel=1e-12)


def test_shapes_dtypes_and_empty():
    # any shape is flattened; torch tensors convert exactly to float64
    ref = np.array([[3.0, 4.0], [0.0, 0.0]])             # RMS = sqrt(25 / 4) = 2.5
    got = torch.tensor([[3.0, 4.0], [0.5, 0.0]], dtype=torch.bfloat16)
    assert oracle.rel_err_floor(got, ref) == pytest.approx(0.5 / 2.5, rel=1e-12)
    assert oracle.rel_err_floor(np.zeros(0), np.zeros(0)) == 0.0


def test_a_non_finite_result_never_passes():
    # NaN propagates through the max, so `err <= tol` is False
    e = oracle.rel_err_floor([float("nan"), 1.0], [1.0, 1.0])
    assert not (e <= 1e-2)
    e = oracle.rel_err_floor([float("inf"), 1.0], [1.0, 1.0])
    assert not (e <= 1e-2)


def test_identical_inputs_score_zero_and_any_change_scores_above_zero():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal(257)
    assert oracle.rel_err_floor(ref.copy(), ref) == 0.0
    got = ref.copy()
    got[100] = np.nextafter(got[100], np.inf)
    assert oracle.rel_err_floor(got, ref) > 0.0
