"""Pins of the oracle's unfused chain (aclnnWeightQuantMatmulAllReduceAddRmsNorm
page: the deprecation note names a weight-quantized matmul followed by
AddRmsNorm as the replacement; Formula): ``weight_quant_matmul`` and
``add_rms_norm`` against exact rational arithmetic, closed forms and the fused
operator."""
import math

import numpy as np
import pytest

import oracle
from tests import exact
from tests.test_oracle_wq_matmul import _case


@pytest.mark.parametrize("seed,gran,group,offset,bias", [
    (20, "tensor", 0, True, True), (21, "channel", 0, False, True), (22, "group", 32, True, False),
    (23, "group", 64, True, True)])
def test_matmul_against_exact_rationals(seed, gran, group, offset, bias):
    x1, w, s, o, g, b, res, gam = _case(96, 5, 4, gran, group, offset, bias, seed=seed)
    mm = oracle.weight_quant_matmul(x1, w, s, o, g, b)
    emm, _, _ = exact.wq_matmul(x1, w, s, o, g, b, res, gam, eps=1e-6)
    assert mm.shape == (4, 5)
    np.testing.assert_allclose(mm, emm, rtol=1e-13, atol=1e-13)


def test_add_rms_norm_against_exact_rationals():
    # exact y and normOut of the fused exact reference, fed its exact mm
    x1, w, s, o, g, b, res, gam = _case(64, 7, 3, "group", 32, True, True, seed=24)
    emm, ey, enorm = exact.wq_matmul(x1, w, s, o, g, b, res, gam, eps=1e-5)
    y, norm = oracle.add_rms_norm(emm, res, gam, 1e-5)
    np.testing.assert_allclose(y, ey, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(norm, enorm, rtol=1e-12, atol=1e-12)


def test_add_rms_norm_closed_forms():
    # a row of [3, 4] (sum of x and residual) with eps 0: RMS = sqrt(25 / 2)
    y, norm = oracle.add_rms_norm(np.array([[1.0, 5.0]]), np.array([[2.0, -1.0]]),
                                  np.array([1.0, 2.0]), 0.0)
    np.testing.assert_array_equal(y, [[3.0, 4.0]])
    np.testing.assert_allclose(norm, [[3 / math.sqrt(12.5), 2 * 4 / math.sqrt(12.5)]], rtol=1e-15)
    # a constant row c: normOut = c / sqrt(c^2 + eps) * gamma
    c, eps = -0.75, 0.0625
    g = np.array([0.5, 1.0, 2.0, 4.0])
    _, norm = oracle.add_rms_norm(np.full((1, 4), c), np.zeros((1, 4)), g, eps)
    np.testing.assert_allclose(norm, [c / math.sqrt(c * c + eps) * g], rtol=1e-15)
    # a zero row stays zero (eps > 0)
    _, norm = oracle.add_rms_norm(np.zeros((2, 3)), np.zeros((2, 3)), np.ones(3), 1e-6)
    np.testing.assert_array_equal(norm, np.zeros((2, 3)))


def test_add_rms_norm_invariants():
    rng = np.random.default_rng(25)
    x, r = rng.standard_normal((6, 40)), rng.standard_normal((6, 40))
    g = rng.uniform(0.5, 2, 40)
    eps = 1e-3
    y, norm = oracle.add_rms_norm(x, r, g, eps)
    ms = np.mean(y * y, axis=1)
    np.testing.assert_allclose(np.mean((norm / g) ** 2, axis=1), ms / (ms + eps), rtol=1e-12)
    # with eps = 0, scaling x and residual by a > 0 leaves normOut unchanged
    _, n1 = oracle.add_rms_norm(x, r, g, 0.0)
    _, n2 = oracle.add_rms_norm(3.5 * x, 3.5 * r, g, 0.0)
    np.testing.assert_allclose(n1, n2, rtol=1e-13)
    # residual and x enter symmetrically
    np.testing.assert_array_equal(oracle.add_rms_norm(r, x, g, eps)[1], norm)


def test_chain_equals_fused_operator():
    x1, w, s, o, g, b, res, gam = _case(128, 9, 5, "group", 64, True, True, seed=26)
    mm, y, norm = oracle.wq_matmul_add_rmsnorm(x1, w, s, o, g, b, res, gam, 1e-6)
    cm = oracle.weight_quant_matmul(x1, w, s, o, g, b)
    cy, cn = oracle.add_rms_norm(cm, res, gam, 1e-6)
    np.testing.assert_allclose(cm, mm, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(cy, y, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(cn, norm, rtol=1e-13, atol=1e-13)
