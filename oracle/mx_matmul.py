"""MX block-32 quantized matmul with in-place add (oracle; float64).

Follows the aclnnQuantBatchMatmulInplaceAdd page:

* Formula (mx quantization): for every output (m, n),
  ``y[m,n] += sum_j (sum over the j-th 32-long K slice of x1 * x2) *
  (scale1[m, j] * scale2[j, n])`` with j over ceil(K / 32) slices, the last
  possibly shorter.
* Constraints: only transposeX1 = true and transposeX2 = false, so x1 arrives
  stored (K, M) and x2 stored (K, N); the group size packs
  ``K | N << 16 | M << 32`` and a zero field is inferred from the shapes
  (groupSizeM = m / scaleM and alike, exact division required).

Readings: scale1 is stored (M, ceil(K/32)) and scale2 (ceil(K/32), N), in the
index order the formula writes them; elements are E4M3 (x1) and E2M1 (x2)
codes and scales are E8M0 codes (formats in :mod:`oracle.formats`). Each slice
sum is exact in float64 (every product is a multiple of 2^-10 and a slice sum
stays below 2^17), the scaling by a power of two is exact, and only the
accumulation over slices and into y rounds.
"""
from __future__ import annotations

import numpy as np

from .formats import e2m1_decode, e4m3_decode, e8m0_decode


def decode_group_size(group_size: int, m: int, k: int, n: int, scale_m: int,
                      scale_k: int, scale_n: int):
    """Split ``K | N << 16 | M << 32`` and infer each zero field from the
    shapes. Returns (gm, gn, gk).

    M and N follow the page's stated principle, ``size / scale_size`` with
    exact division. For K the Formula fixes gsK = 32 for mx and lets the last
    slice be shorter, so a zero K field is read as 32 whenever ``ceil(K / 32)``
    slices match the scale shape, and by exact division otherwise."""
    gk = group_size & 0xFFFF
    gn = (group_size >> 16) & 0xFFFF
    gm = (group_size >> 32) & 0xFFFF

    def infer(size, scale_size):
        if scale_size <= 0 or size % scale_size:
            raise ValueError("group size cannot be inferred: inexact division")
        return size // scale_size

    if not gm:
        gm = infer(m, scale_m)
    if not gn:
        gn = infer(n, scale_n)
    if not gk:
        gk = 32 if -(-k // 32) == scale_k else infer(k, scale_k)
    return gm, gn, gk


def mx_quant_matmul_inplace_add(x1_t_codes, x2_codes, scale1, scale2, y):
    """x1_t_codes (K, M) E4M3 codes; x2_codes (K, N) E2M1 codes (0..15);
    scale1 (M, ceil(K/32)) and scale2 (ceil(K/32), N) E8M0 codes; y (M, N).
    Returns the updated y as float64."""
    a = e4m3_decode(np.asarray(x1_t_codes)).T          # (M, K)
    b = e2m1_decode(np.asarray(x2_codes))               # (K, N)
    s1 = e8m0_decode(scale1)
    s2 = e8m0_decode(scale2)
    m, k = a.shape
    n = b.shape[1]
    k_loops = -(-k // 32)
    if s1.shape != (m, k_loops) or s2.shape != (k_loops, n):
        raise ValueError("scale shapes must be (M, ceil(K/32)) and (ceil(K/32), N)")
    out = np.array(y, dtype=np.float64, copy=True)
    for j in range(k_loops):
        sl = slice(32 * j, min(k, 32 * j + 32))
        block_sum = a[:, sl] @ b[sl, :]
        out += block_sum * (s1[:, j:j + 1] * s2[j:j + 1, :])
    return out


def mxfp4_quant_matmul_inplace_add(x1_codes, x2_codes, scale1, scale2, y):
    """The same Formula (mx quantization) with both operands MXFP4:
    x1_codes (M, K) E2M1 codes (0..15), stored row-major (not transposed: the
    layout in which the block-32 dynamic quant writes E2M1 activations, K
    contiguous); x2_codes (K, N) E2M1 codes; scale1 (M, ceil(K/32)) and
    scale2 (ceil(K/32), N) E8M0 codes; y (M, N). Returns the updated y as
    float64. Every slice sum is exact in float64 (products are multiples of
    2^-2 below 2^6), so only the accumulation over slices and into y rounds."""
    a = e2m1_decode(np.asarray(x1_codes))               # (M, K)
    b = e2m1_decode(np.asarray(x2_codes))               # (K, N)
    s1 = e8m0_decode(scale1)
    s2 = e8m0_decode(scale2)
    m, k = a.shape
    if b.shape[0] != k:
        raise ValueError("x1 is (M, K) and x2 is (K, N)")
    n = b.shape[1]
    k_loops = -(-k // 32)
    if s1.shape != (m, k_loops) or s2.shape != (k_loops, n):
        raise ValueError("scale shapes must be (M, ceil(K/32)) and (ceil(K/32), N)")
    out = np.array(y, dtype=np.float64, copy=True)
    for j in range(k_loops):
        sl = slice(32 * j, min(k, 32 * j + 32))
        out += (a[:, sl] @ b[sl, :]) * (s1[:, j:j + 1] * s2[j:j + 1, :])
    return out
