"""Pins of the oracle's MXFP4 x MXFP4 matmul (aclnnQuantBatchMatmulInplaceAdd
page, Formula, mx quantization, with both operands E2M1) and of the FLOAT ->
FLOAT4_E2M1 pack (aclnnConvertWeightToINT4Pack page), against exact
arithmetic, the hand-written E2M1 table under tests/golden/ and the already
pinned E4M3 x E2M1 oracle."""
import os

import numpy as np
import pytest

import oracle
from tests import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e2m1_values.txt")


def _golden():
    vals, ties = {}, []
    for ln in open(GOLDEN):
        if ln.startswith("#") or not ln.strip():
            continue
        f = ln.split()
        if f[0] == "tie":
            ties.append((float(f[1]), float(f[2])))
        else:
            vals[int(f[0])] = float(f[1])
    return vals, ties


def _codes(rng, m, k, n, s_lo=120, s_hi=134):
    x1 = rng.integers(0, 16, (m, k)).astype(np.uint8)
    x2 = rng.integers(0, 16, (k, n)).astype(np.uint8)
    kb = -(-k // 32)
    s1 = rng.integers(s_lo, s_hi, (m, kb)).astype(np.uint8)
    s2 = rng.integers(s_lo, s_hi, (kb, n)).astype(np.uint8)
    return x1, x2, s1, s2


def test_unit_scales_equal_textbook_matmul():
    rng = np.random.default_rng(40)
    m, k, n = 3, 64, 5
    x1, x2, _, _ = _codes(rng, m, k, n)
    got = oracle.mxfp4_quant_matmul_inplace_add(x1, x2, np.full((m, 2), 127, np.uint8),
                                                np.full((2, n), 127, np.uint8), np.zeros((m, n)))
    for i in range(m):
        for j in range(n):
            t = sum(exact.e2m1_value(int(x1[i, kk])) * exact.e2m1_value(int(x2[kk, j]))
                    for kk in range(k))
            assert got[i, j] == float(t)                  # exact: small dyadic sums


@pytest.mark.parametrize("k", [32, 96, 80, 7])
def test_against_exact_rationals_through_e4m3(k):
    # every E2M1 value is an E4M3 value, so the operand re-encoded as E4M3 and
    # stored (K, M) must give the same result in the exact rational reference
    rng = np.random.default_rng(41 + k)
    m, n = 4, 3
    x1, x2, s1, s2 = _codes(rng, m, k, n)
    y = rng.standard_normal((m, n))
    x1_e4m3_t = oracle.e4m3_encode(oracle.e2m1_decode(x1)).T
    got = oracle.mxfp4_quant_matmul_inplace_add(x1, x2, s1, s2, y)
    want = exact.mx_matmul(x1_e4m3_t, x2, s1, s2, y)
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(got, oracle.mx_quant_matmul_inplace_add(x1_e4m3_t, x2, s1, s2, y))


def test_one_hot_pins_scale_indexing():
    m, k, n = 4, 96, 6
    rng = np.random.default_rng(42)
    _, x2, s1, s2 = _codes(rng, m, k, n)
    for (mm, kk) in [(0, 0), (2, 33), (3, 95), (1, 64)]:
        x1 = np.zeros((m, k), np.uint8)
        x1[mm, kk] = 0x2                                   # E2M1 1.0
        got = oracle.mxfp4_quant_matmul_inplace_add(x1, x2, s1, s2, np.zeros((m, n)))
        want = np.zeros((m, n))
        j = kk // 32
        want[mm] = (oracle.e2m1_decode(x2[kk]) * 2.0 ** (int(s1[mm, j]) - 127)
                    * 2.0 ** (s2[j].astype(np.int64) - 127))
        np.testing.assert_array_equal(got, want)


def test_pack_float_e2m1_every_value_and_tie():
    vals, ties = _golden()
    codes = np.arange(16).reshape(1, 16)
    w = np.array([[vals[c] for c in range(16)]], dtype=np.float32)
    assert np.signbit(w[0, 8])                             # -0.0 keeps its sign
    nd = oracle.pack_float_e2m1(w, "nd")
    np.testing.assert_array_equal(nd, (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8))
    for v, want in ties:
        got = oracle.e2m1_decode(oracle.pack_float_e2m1(np.array([[v, 0.0]], np.float32), "nd") & 0xF)
        assert got[0, 0] == want, (v, got, want)


def _nd_codes(packed):
    b = np.asarray(packed).astype(np.int64)
    out = np.empty((b.shape[0], 2 * b.shape[1]), np.int64)
    out[:, 0::2], out[:, 1::2] = b & 0xF, b >> 4
    return out


def test_pack_float_e2m1_saturates():
    w = np.array([[6.5, 7.0, 1e30, np.inf, -6.1, -np.inf, 5.99, 0.24]], np.float32)
    got = oracle.e2m1_decode(_nd_codes(oracle.pack_float_e2m1(w, "nd")))
    np.testing.assert_array_equal(got, [[6.0, 6.0, 6.0, 6.0, -6.0, -6.0, 6.0, 0.0]])
    with pytest.raises(ValueError):
        oracle.pack_float_e2m1(np.array([[np.nan, 0.0]], np.float32), "nd")


def test_pack_float_layouts_agree_with_the_code_pack():
    rng = np.random.default_rng(43)
    k, n = 200, 48
    codes = rng.integers(0, 16, (k, n))
    w = oracle.e2m1_decode(codes).astype(np.float32)
    w[codes == 8] = -0.0
    np.testing.assert_array_equal(oracle.pack_float_e2m1(w, "gfx950b"),
                                  oracle.pack_codes_gfx950b(codes, k, n))
    np.testing.assert_array_equal(oracle.pack_float_e2m1(w.T.copy(), "gfx950b", transpose=True),
                                  oracle.pack_codes_gfx950b(codes, k, n))
    np.testing.assert_array_equal(
        oracle.pack_float_e2m1(w, "nd"),
        (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8))
