"""Element formats of the MX path (oracle; test infrastructure only).

The aclnnQuantBatchMatmulInplaceAdd page names "mx quantization" with 32-long
K blocks but does not define the element formats; aclnnConvertWeightToINT4Pack
names FLOAT4_E2M1. Their definitions are taken from the OCP Microscaling
Formats (MX) v1.0 specification:

* E4M3 (the "FN" variant): sign, 4 exponent bits with bias 7, 3 mantissa bits;
  subnormals m * 2^-9 (m = 1..7); largest finite 448; S.1111.111 is NaN; no
  infinities.
* E2M1: sign, 2 exponent bits with bias 1, 1 mantissa bit; magnitudes
  {0, 0.5, 1, 1.5, 2, 3, 4, 6}; no NaN or infinity.
* E8M0: an unsigned biased exponent, value 2^(c - 127); c = 255 is NaN.

Encoding is round-to-nearest, ties to even, and keeps the sign of zero.
Inputs whose rounded magnitude exceeds the format's largest value are outside
the contract here (the quantizer's scale choice never produces them) and raise.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E2M1_MAX = 6.0


def _round_to_grid(a: np.ndarray, min_normal_exp: int, mant_bits: int) -> np.ndarray:
    """Round non-negative ``a`` to the nearest value of a binary floating-point
    format with ``mant_bits`` stored mantissa bits whose smallest normal binade
    starts at 2**min_normal_exp (subnormals share that binade's spacing)."""
    f, ex = np.frexp(a)                        # a = f * 2**ex, f in [0.5, 1)
    binade = np.maximum(ex - 1, min_normal_exp)
    quantum = np.ldexp(1.0, binade - mant_bits)
    return np.rint(a / quantum) * quantum      # a/quantum is exact; rint is RNE


def e4m3_decode(code) -> np.ndarray:
    c = np.asarray(code).astype(np.int64)
    s = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp((8 + m).astype(np.float64), e - 10))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return s * mag


def e4m3_encode(v) -> np.ndarray:
    """Round-to-nearest-even float -> E4M3 code (uint8)."""
    v = np.asarray(v, dtype=np.float64)
    neg = np.signbit(v)
    r = _round_to_grid(np.abs(v), -6, 3)
    if np.any(r > E4M3_MAX):
        raise ValueError("value outside the E4M3 range")
    f, ex = np.frexp(r)
    normal = r >= 2.0 ** -6
    e_field = np.where(normal, ex - 1 + 7, 0)
    m_field = np.where(normal, np.ldexp(r, -(ex - 1) + 3) - 8, np.ldexp(r, 9))
    code = (neg.astype(np.int64) << 7) | (e_field.astype(np.int64) << 3) | m_field.astype(np.int64)
    return code.astype(np.uint8)


def e2m1_decode(code) -> np.ndarray:
    c = np.asarray(code).astype(np.int64)
    s = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = c & 0x1
    mag = np.where(e == 0, 0.5 * m, np.ldexp((2 + m).astype(np.float64), e - 2))
    return s * mag


def e2m1_encode(v) -> np.ndarray:
    """Round-to-nearest-even float -> E2M1 code (0..15, uint8)."""
    v = np.asarray(v, dtype=np.float64)
    neg = np.signbit(v)
    r = _round_to_grid(np.abs(v), 0, 1)
    if np.any(r > E2M1_MAX):
        raise ValueError("value outside the E2M1 range")
    f, ex = np.frexp(r)
    normal = r >= 1.0
    e_field = np.where(normal, ex, 0)
    m_field = np.where(normal, np.ldexp(r, -(ex - 1) + 1) - 2, np.ldexp(r, 1))
    code = (neg.astype(np.int64) << 3) | (e_field.astype(np.int64) << 1) | m_field.astype(np.int64)
    return code.astype(np.uint8)


def e8m0_decode(code) -> np.ndarray:
    c = np.asarray(code).astype(np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - 127))
