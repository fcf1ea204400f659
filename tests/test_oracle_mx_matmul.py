"""Pins of the oracle's MX block-32 matmul with in-place add."""
import numpy as np
import pytest

import oracle
from tests import exact


def _codes(rng, k, m, n, s_lo=120, s_hi=134):
    x1 = rng.integers(0, 256, (k, m)).astype(np.uint8)
    x1[(x1 & 0x7F) == 0x7F] = 0x00                      # no NaN codes
    x2 = rng.integers(0, 16, (k, n)).astype(np.uint8)
    kb = -(-k // 32)
    s1 = rng.integers(s_lo, s_hi, (m, kb)).astype(np.uint8)
    s2 = rng.integers(s_lo, s_hi, (kb, n)).astype(np.uint8)
    return x1, x2, s1, s2


@pytest.mark.parametrize("k", [32, 80, 96, 7])
def test_against_exact_rationals(k):
    rng = np.random.default_rng(k)
    m, n = 3, 4
    x1, x2, s1, s2 = _codes(rng, k, m, n)
    y = rng.standard_normal((m, n))
    got = oracle.mx_quant_matmul_inplace_add(x1, x2, s1, s2, y)
    want = exact.mx_matmul(x1, x2, s1, s2, y)
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)


def test_unit_scales_equal_textbook_matmul():
    rng = np.random.default_rng(2)
    k, m, n = 64, 3, 5
    x1, x2, _, _ = _codes(rng, k, m, n)
    s1 = np.full((m, 2), 127, np.uint8)
    s2 = np.full((2, n), 127, np.uint8)
    got = oracle.mx_quant_matmul_inplace_add(x1, x2, s1, s2, np.zeros((m, n)))
    for i in range(m):
        for j in range(n):
            t = sum(float(exact.e4m3_value(int(x1[kk, i])) * exact.e2m1_value(int(x2[kk, j])))
                    for kk in range(k))
            assert got[i, j] == t                         # exact: sums stay far below 2^53


def test_one_hot_pins_scale_indexing():
    k, m, n = 96, 4, 6
    rng = np.random.default_rng(3)
    _, x2, s1, s2 = _codes(rng, k, m, n)
    for (kk, mm) in [(0, 0), (33, 2), (95, 3), (64, 1)]:
        x1 = np.zeros((k, m), np.uint8)
        x1[kk, mm] = 0x38                                  # E4M3 1.0
        got = oracle.mx_quant_matmul_inplace_add(x1, x2, s1, s2, np.zeros((m, n)))
        want = np.zeros((m, n))
        j = kk // 32
        want[mm] = (oracle.e2m1_decode(x2[kk]) * 2.0 ** (int(s1[mm, j]) - 127)
                    * 2.0 ** (s2[j].astype(np.int64) - 127))
        np.testing.assert_array_equal(got, want)


def test_linearity_and_integer_exactness():
    rng = np.random.default_rng(4)
    k, m, n = 80, 5, 7
    x1, x2, _, _ = _codes(rng, k, m, n)
    s1 = np.full((m, 3), 127, np.uint8)
    s2 = np.full((3, n), 127, np.uint8)
    y0 = np.zeros((m, n))
    y1 = oracle.mx_quant_matmul_inplace_add(x1, x2, s1, s2, y0)
    y2 = oracle.mx_quant_matmul_inplace_add(x1, x2, s1, s2, y1)
    assert np.array_equal(y2, 2 * y1)
    assert np.all(y1 * 1024 == np.round(y1 * 1024))       # multiples of 2^-10


def test_group_size_decoding():
    packed = 32 | (1 << 16) | (1 << 32)
    assert packed == 4295032864
    assert oracle.decode_group_size(packed, 4096, 8192, 4096, 4096, 256, 4096) == (1, 1, 32)
    assert oracle.decode_group_size(0, 4096, 8192, 4096, 4096, 256, 4096) == (1, 1, 32)
    assert oracle.decode_group_size(0, 8, 80, 4, 8, 3, 4) == (1, 1, 32)
    assert oracle.decode_group_size(0, 8, 34, 4, 8, 2, 4) == (1, 1, 32)
    assert oracle.decode_group_size(0, 8, 64, 4, 4, 2, 4) == (2, 1, 32)
    with pytest.raises(ValueError):
        oracle.decode_group_size(0, 9, 64, 4, 4, 2, 4)


def test_rejects_wrong_scale_shapes():
    rng = np.random.default_rng(5)
    x1, x2, s1, s2 = _codes(rng, 64, 3, 5)
    with pytest.raises(ValueError):
        oracle.mx_quant_matmul_inplace_add(x1, x2, s1.T, s2, np.zeros((3, 5)))
    with pytest.raises(ValueError):
        oracle.mx_quant_matmul_inplace_add(x1, x2, s1, s2.T, np.zeros((3, 5)))
