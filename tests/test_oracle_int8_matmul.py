"""Pins of oracle.quant_matmul_inplace_add_int8 (aclnnQuantBatchMatmulInplaceAdd
page, Formula, read for INT8 with one K group and per-token / per-channel
scales) against values that do not come from the oracle: brute force with
Python integers and an independently written float32 rounding, closed forms,
special cases and a transposition invariant."""
import struct

import numpy as np
import pytest

import oracle


def f32(x: float) -> float:
    """Round a Python float (binary64) to the nearest binary32, ties to even
    (struct's conversion), returned as a Python float."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def brute(x1, x2_t, s1, s2, y):
    """Loop over (m, n, k) in the formula's index order; integers exact, each
    float32 step rounded separately. Products of two binary32 values are exact
    in binary64, so f32(a * b) is the correctly rounded binary32 product."""
    M, K = len(x1), len(x1[0])
    N = len(x2_t)
    out = [[0.0] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = 0
            for k in range(K):
                acc += int(x1[m][k]) * int(x2_t[n][k])
            s = f32(float(s1[m]) * float(s2[n]))
            t = f32(f32(float(acc)) * s)
            out[m][n] = f32(float(y[m][n]) + t)
    return np.array(out, dtype=np.float32)


@pytest.mark.parametrize("M,N,K,seed", [(1, 1, 1, 0), (3, 5, 7, 1), (4, 2, 64, 2), (5, 6, 33, 3)])
def test_matches_brute_force(M, N, K, seed):
    rng = np.random.default_rng(seed)
    x1 = rng.integers(-128, 128, size=(M, K))
    x2_t = rng.integers(-128, 128, size=(N, K))
    s1 = rng.uniform(1e-3, 1e-1, size=M).astype(np.float32)
    s2 = rng.uniform(1e-3, 1e-1, size=N).astype(np.float32)
    y = rng.normal(size=(M, N)).astype(np.float32)
    got = oracle.quant_matmul_inplace_add_int8(x1, x2_t, s1, s2, y)
    want = brute(x1.tolist(), x2_t.tolist(), s1.tolist(), s2.tolist(), y.tolist())
    assert got.dtype == np.float32
    assert np.array_equal(got, want)


def test_ones_closed_form():
    # every product is 1, so the sum is K; power-of-two scales keep it exact
    M, N, K = 3, 4, 100
    s1 = np.full(M, 2.0 ** -3, np.float32)
    s2 = np.full(N, 2.0 ** -4, np.float32)
    y = np.arange(M * N, dtype=np.float32).reshape(M, N)
    got = oracle.quant_matmul_inplace_add_int8(np.ones((M, K)), np.ones((N, K)), s1, s2, y)
    assert np.array_equal(got, y + np.float32(K * 2.0 ** -7))


def test_one_hot_row_picks_a_weight_column():
    # x1 row m is one-hot at k0: y[m, n] += x2_t[n, k0] * s1[m] * s2[n]
    rng = np.random.default_rng(5)
    M, N, K, k0 = 2, 6, 9, 4
    x1 = np.zeros((M, K), np.int64)
    x1[1, k0] = 1
    x2_t = rng.integers(-128, 128, size=(N, K))
    s1 = np.array([0.5, 0.25], np.float32)
    s2 = np.full(N, 2.0, np.float32)
    got = oracle.quant_matmul_inplace_add_int8(x1, x2_t, s1, s2, np.zeros((M, N), np.float32))
    assert np.array_equal(got[0], np.zeros(N, np.float32))
    assert np.array_equal(got[1], (x2_t[:, k0] * 0.5).astype(np.float32))


def test_zero_scale_leaves_y():
    rng = np.random.default_rng(6)
    x1 = rng.integers(-128, 128, size=(3, 20))
    x2_t = rng.integers(-128, 128, size=(4, 20))
    y = rng.normal(size=(3, 4)).astype(np.float32)
    got = oracle.quant_matmul_inplace_add_int8(x1, x2_t, np.zeros(3, np.float32),
                                               np.ones(4, np.float32), y)
    assert np.array_equal(got, y)


def test_swapping_operands_transposes_the_result():
    rng = np.random.default_rng(7)
    x1 = rng.integers(-128, 128, size=(5, 40))
    x2_t = rng.integers(-128, 128, size=(3, 40))
    s1 = rng.uniform(0.01, 1, 5).astype(np.float32)
    s2 = rng.uniform(0.01, 1, 3).astype(np.float32)
    a = oracle.quant_matmul_inplace_add_int8(x1, x2_t, s1, s2, np.zeros((5, 3), np.float32))
    b = oracle.quant_matmul_inplace_add_int8(x2_t, x1, s2, s1, np.zeros((3, 5), np.float32))
    assert np.array_equal(a, b.T)


def test_extreme_sum_is_exact():
    # K = 65535 products of (-128) * (-128): 1,073,725,440, inside int32 and
    # rounded once to float32 (a multiple of 64 at this magnitude)
    K = 65535
    got = oracle.quant_matmul_inplace_add_int8(np.full((1, K), -128), np.full((1, K), -128),
                                               np.ones(1, np.float32), np.ones(1, np.float32),
                                               np.zeros((1, 1), np.float32))
    exact = K * 128 * 128
    assert exact < 2 ** 31
    assert got[0, 0] == np.float32(f32(float(exact)))
    assert abs(float(got[0, 0]) - exact) <= 32
