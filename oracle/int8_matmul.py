"""INT8 quantized matmul with in-place add (oracle; exact integers, float32
epilogue).

Follows the aclnnQuantBatchMatmulInplaceAdd page, Formula: for every output
(m, n), ``y[m,n] += sum_j (sum over the j-th K slice of x1 * x2) *
(scale1[m, j] * scale2[j, n])``. The page prints this formula for mx
quantization only; here it is read for INT8 operands with a single K group
(groupSizeK = K, so one slice, j = 0), a scale per row of x1 (per token, the
output of DynamicQuant's per-token mode, aclnnDynamicQuant page, Formula) and a
scale per column of x2 (per channel):

    y[m, n] = (sum_k x1[m, k] * x2[k, n]) * (scale1[m] * scale2[n]) + y[m, n]

Readings:
* x1 is stored (M, K) row-major, as DynamicQuant writes it; x2 is stored
  (N, K) (transposed: each output column's K values contiguous); scale1 and
  scale2 are float32 vectors (M) and (N); y is float32 (M, N).
* The integer sum is exact (|x| <= 128 and K < 2^17 keep it inside int32).
* The float part is taken in float32 in the formula's grouping, each step
  rounded to nearest even: s = fl(scale1[m] * scale2[n]), t = fl(fl(acc) * s),
  y = fl(y + t). Both sides of a parity check take these roundings in this
  order, so the result is bit-exact.
"""
from __future__ import annotations

import numpy as np


def quant_matmul_inplace_add_int8(x1, x2_t, scale1, scale2, y):
    """x1 (M, K) int8 values; x2_t (N, K) int8 values; scale1 (M) and scale2
    (N) float32; y (M, N) float32. Returns the updated y as float32."""
    a = np.asarray(x1, dtype=np.int64)
    b = np.asarray(x2_t, dtype=np.int64)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[1]:
        raise ValueError("x1 is (M, K) and x2_t is (N, K)")
    acc = a @ b.T                                    # exact: int64 sums of int8 products
    s1 = np.asarray(scale1, dtype=np.float32).reshape(-1)
    s2 = np.asarray(scale2, dtype=np.float32).reshape(-1)
    s = (s1[:, None] * s2[None, :]).astype(np.float32)          # fl(scale1 * scale2)
    # int64 -> float64 is exact below 2^53, so this is one rounding to float32
    t = (acc.astype(np.float64).astype(np.float32) * s).astype(np.float32)
    return (np.asarray(y, dtype=np.float32) + t).astype(np.float32)


def quant_matmul_inplace_add_w4(x1, x2_codes, scale1, scale2, y):
    """A8W4: the same formula and roundings with x2 an INT4 weight. x1 (M, K)
    int8 values; x2_codes (K, N) the INT4 codes in [-8, 7] as the pack takes
    them (aclnnConvertWeightToINT4Pack page: the packed layout is storage
    only, the values are the codes); scale1 (M), scale2 (N) float32; y (M, N)
    float32. Returns the updated y as float32."""
    q = np.asarray(x2_codes, dtype=np.int64)
    if q.ndim != 2:
        raise ValueError("x2_codes is (K, N)")
    if q.size and (q.min() < -8 or q.max() > 7):
        raise ValueError("INT4 codes lie in [-8, 7]")
    return quant_matmul_inplace_add_int8(x1, q.T, scale1, scale2, y)
