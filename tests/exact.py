"""Exact rational brute force for pinning the oracle on tiny inputs.

Pure Python loops over ``fractions.Fraction``: no numpy arithmetic and no
code from ``oracle/``. Used only by the CPU tests.
"""
from __future__ import annotations

import decimal
from fractions import Fraction

import numpy as np


def fr(v) -> Fraction:
    return Fraction(float(v))


def pow2(e: int) -> Fraction:
    return Fraction(2) ** e


def binade(a: Fraction) -> int:
    """floor(log2(a)) for a > 0."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while pow2(e) > a:
        e -= 1
    while pow2(e + 1) <= a:
        e += 1
    return e


def round_to_format(v: Fraction, mant_bits: int, min_exp: int) -> Fraction:
    """Nearest value, ties to even, of a binary format with ``mant_bits``
    fraction bits and smallest normal binade 2**min_exp (no overflow)."""
    if v == 0:
        return Fraction(0)
    a = abs(v)
    e = max(binade(a), min_exp)
    quantum = pow2(e - mant_bits)
    n = round(a / quantum)            # Fraction.__round__ rounds half to even
    r = n * quantum
    return r if v > 0 else -r


def f32(v: Fraction) -> Fraction:
    """Correctly rounded float32 (normal and subnormal range)."""
    return round_to_format(v, 23, -126)


def round_half_even(v: Fraction) -> int:
    return round(v)


def per_token_quant(row, smooth, dmax: int):
    """The DynamicQuant formula with float32 decisions, exactly."""
    vals = [fr(x) * (fr(s) if smooth is not None else 1) for x, s in
            zip(row, smooth if smooth is not None else [1] * len(row))]
    vals = [f32(v) for v in vals]
    a = max(abs(v) for v in vals)
    scale = f32(a / dmax)
    if scale == 0:
        return [0] * len(vals), scale
    q = [max(-dmax, min(dmax, round_half_even(f32(v / scale)))) for v in vals]
    return q, scale


def mx_block(vals, dmax: int, mant_bits: int, min_exp: int):
    """(exponent e, rounded values) of one MX block, exactly."""
    vals = [Fraction(v) for v in vals]
    a = max(abs(v) for v in vals)
    if a == 0:
        return 0, [Fraction(0)] * len(vals)
    e = -200
    while dmax * pow2(e) < a:
        e += 1
    e = max(-127, min(127, e))
    return e, [round_to_format(v / pow2(e), mant_bits, min_exp) for v in vals]


def wq_matmul(x1, w, scale, offset, group_size, bias, residual, gamma, eps,
              rows=None):
    """mm, y and normOut (normOut to ~40 digits) by exact rational loops."""
    x1 = np.asarray(x1, dtype=np.float64)
    w = np.asarray(w)
    k, n = w.shape
    x = x1.reshape(-1, k)
    res = np.asarray(residual, dtype=np.float64).reshape(-1, n)
    s = np.asarray(scale, dtype=np.float64)
    o = None if offset is None else np.asarray(offset, dtype=np.float64)

    def at(t, kk, nn):
        if t.size == 1:
            return fr(t.reshape(-1)[0])
        if t.ndim == 1 or t.shape[0] == 1:
            return fr(t.reshape(-1)[nn])
        return fr(t[kk // group_size, nn])

    rows = range(x.shape[0]) if rows is None else rows
    decimal.getcontext().prec = 40
    out_mm, out_y, out_norm = [], [], []
    for r in rows:
        mm_row, y_row = [], []
        for nn in range(n):
            acc = Fraction(0)
            for kk in range(k):
                wv = int(w[kk, nn]) * at(s, kk, nn)
                if o is not None:
                    wv += at(o, kk, nn)
                acc += fr(x[r, kk]) * wv
            if bias is not None:
                acc += fr(np.asarray(bias, dtype=np.float64)[nn])
            mm_row.append(acc)
            y_row.append(acc + fr(res[r, nn]))
        ms = sum(v * v for v in y_row) / n
        den = (decimal.Decimal(ms.numerator) / decimal.Decimal(ms.denominator)
               + decimal.Decimal(Fraction(eps).numerator) / decimal.Decimal(Fraction(eps).denominator)).sqrt()
        g = np.asarray(gamma, dtype=np.float64)
        norm_row = [float(decimal.Decimal(v.numerator) / decimal.Decimal(v.denominator) / den
                          * decimal.Decimal(float(g[nn]))) for nn, v in enumerate(y_row)]
        out_mm.append([float(v) for v in mm_row])
        out_y.append([float(v) for v in y_row])
        out_norm.append(norm_row)
    return np.array(out_mm), np.array(out_y), np.array(out_norm)


def e4m3_value(code: int) -> Fraction:
    s = -1 if code & 0x80 else 1
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 0:
        return s * Fraction(m, 512)
    return s * (1 + Fraction(m, 8)) * pow2(e - 7)


def e2m1_value(code: int) -> Fraction:
    s = -1 if code & 0x8 else 1
    e = (code >> 1) & 0x3
    m = code & 1
    if e == 0:
        return s * Fraction(m, 2)
    return s * (1 + Fraction(m, 2)) * pow2(e - 1)


def mx_matmul(x1_t, x2, s1, s2, y):
    """y + sum_j (slice sum) * 2^(s1-127) * 2^(s2-127), exactly."""
    k, m = x1_t.shape
    n = x2.shape[1]
    out = np.zeros((m, n))
    for mm in range(m):
        for nn in range(n):
            acc = fr(y[mm, nn])
            for j in range(-(-k // 32)):
                part = Fraction(0)
                for kk in range(32 * j, min(k, 32 * j + 32)):
                    part += e4m3_value(int(x1_t[kk, mm])) * e2m1_value(int(x2[kk, nn]))
                acc += part * pow2(int(s1[mm, j]) - 127) * pow2(int(s2[j, nn]) - 127)
            out[mm, nn] = float(acc)
    return out
