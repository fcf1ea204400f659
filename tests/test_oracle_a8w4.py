"""Pins of oracle.quant_matmul_inplace_add_w4 (aclnnQuantBatchMatmulInplaceAdd
page, Formula, read for an INT8 x1 and an INT4 weight with one K group and
per-token / per-channel scales) against values that do not come from the
oracle: the brute-force loop of the INT8 pins (Python integers, an
independently written float32 rounding), closed forms at the code range's
ends, and the packed storage round trip."""
import numpy as np
import pytest

import oracle
from tests.test_oracle_int8_matmul import brute, f32


@pytest.mark.parametrize("M,N,K,seed", [(1, 1, 1, 0), (3, 5, 7, 1), (4, 2, 64, 2), (5, 6, 33, 3)])
def test_matches_brute_force(M, N, K, seed):
    rng = np.random.default_rng(100 + seed)
    x1 = rng.integers(-128, 128, size=(M, K))
    codes = rng.integers(-8, 8, size=(K, N))
    s1 = rng.uniform(1e-3, 1e-1, size=M).astype(np.float32)
    s2 = rng.uniform(1e-3, 1e-1, size=N).astype(np.float32)
    y = rng.normal(size=(M, N)).astype(np.float32)
    got = oracle.quant_matmul_inplace_add_w4(x1, codes, s1, s2, y)
    want = brute(x1.tolist(), codes.T.tolist(), s1.tolist(), s2.tolist(), y.tolist())
    assert got.dtype == np.float32
    assert np.array_equal(got, want)


def test_codes_outside_int4_are_rejected():
    x1 = np.ones((1, 2))
    one = np.ones(1, np.float32)
    for bad in (8, -9):
        with pytest.raises(ValueError):
            oracle.quant_matmul_inplace_add_w4(x1, np.array([[bad], [0]]), one, one,
                                               np.zeros((1, 1), np.float32))


@pytest.mark.parametrize("code", [-8, 7])
def test_code_range_ends_closed_form(code):
    # x1 all -128 and every code at one end of [-8, 7]: the sum is -128 * code * K
    M, N, K = 2, 3, 65535
    got = oracle.quant_matmul_inplace_add_w4(np.full((M, K), -128), np.full((K, N), code),
                                             np.ones(M, np.float32), np.ones(N, np.float32),
                                             np.zeros((M, N), np.float32))
    exact = -128 * code * K
    assert np.all(got == np.float32(f32(float(exact))))
    if code == -8:                     # 65535 * 1024: sixteen significant bits, exact
        assert np.all(got == exact)


def test_the_packed_weight_holds_the_codes():
    # the weight reaches the GEMM packed in GFX950_B; unpacking the pack gives
    # the codes back, so the oracle's (K, N) codes are what the kernel reads
    rng = np.random.default_rng(9)
    codes = rng.integers(-8, 8, size=(200, 40))
    packed = oracle.pack_int4_gfx950b(codes)
    np.testing.assert_array_equal(oracle.unpack_int4_gfx950b(packed, 200, 40), codes)
