"""Pins of the oracle's dynamic quantization (per-token and MX)."""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.quant import encode_quant_output, mx_exponent
from tests import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fp16(a):
    return np.asarray(a, dtype=np.float16).astype(np.float64)


def test_tie_rule_golden():
    with open(os.path.join(GOLDEN, "dynamic_quant_ties.txt")) as f:
        rows = [l.split("#")[0].strip() for l in f if l.split("#")[0].strip()]
    assert len(rows) == 3
    for row in rows:
        kind, rest = row.split(":")
        xs, scale, qs = rest.split("->")
        x = np.array([[float(v) for v in xs.split()]])
        q, s = oracle.dynamic_quant_per_token(x, None, kind)
        assert s[0] == float(scale.split()[1])
        assert q[0].tolist() == [int(v) for v in qs.split()]


@pytest.mark.parametrize("out", ["int8", "int4", "int32"])
def test_per_token_against_exact_and_invariants(out):
    rng = np.random.default_rng({"int8": 1, "int4": 2, "int32": 3}[out])
    dmax = {"int8": 127, "int4": 7, "int32": 7}[out]
    x = _fp16(rng.standard_normal((24, 16)) * np.exp2(rng.integers(-6, 6, (24, 1))))
    smooth = _fp16(rng.uniform(0.5, 2.0, 16))
    q, s = oracle.dynamic_quant_per_token(x, smooth, out)
    for r in range(x.shape[0]):
        eq, es = exact.per_token_quant(x[r], smooth, dmax)
        assert Fraction(float(s[r])) == es
        assert q[r].tolist() == eq
    assert np.all(np.abs(q) <= dmax)
    v = x * smooth
    arg = np.argmax(np.abs(v), axis=1)
    assert np.array_equal(np.abs(q[np.arange(24), arg]), np.full(24, dmax))
    # reconstruction within half a step (plus float32 rounding of the quotient)
    err = np.abs(q * s[:, None].astype(np.float64) - v)
    assert np.all(err <= s[:, None] * 0.5 * (1 + 2.0 ** -22) + 1e-30)


def test_per_token_zero_row_and_leading_dims():
    x = np.zeros((2, 3, 8))
    x[1, 2, 5] = -3.0
    q, s = oracle.dynamic_quant_per_token(x, None, "int8")
    assert q.shape == (6, 8) and s.shape == (6,)
    assert np.all(s[:5] == 0) and np.all(q[:5] == 0)
    assert s[5] == np.float32(3.0) / np.float32(127) and q[5, 5] == -127


def test_per_token_scale_is_float32_division():
    # The scale is the correctly rounded float32 quotient: compare with the
    # float64 quotient rounded once to float32 (innocuous double rounding for
    # division since 53 >= 2*24 + 2).
    rng = np.random.default_rng(9)
    x = _fp16(rng.standard_normal((200, 32)))
    _, s = oracle.dynamic_quant_per_token(x, None, "int8")
    a = np.max(np.abs(x), axis=1)
    assert np.array_equal(s, (a / 127.0).astype(np.float32))


def test_quant_output_encodings():
    q = np.array([[1, 2, 3, 4, 5, 6, 7, -8, 0, -1, 0, 0, 0, 0, 0, 7]])
    i4 = encode_quant_output(q, "int4")
    assert i4[0, :4].tolist() == [0x21, 0x43, 0x65, 0x87]
    i32 = encode_quant_output(q, "int32")
    assert i32.view(np.uint32)[0].tolist() == [0x87654321, 0x700000F0]
    for out in ("int8", "int4", "int32"):
        assert np.array_equal(oracle.unpack_quant_output(encode_quant_output(q, out), out, 16), q)


def test_mx_scale_golden():
    with open(os.path.join(GOLDEN, "mx_scale_examples.txt")) as f:
        lines = [l.split("#")[0].split() for l in f]
    lines = [l for l in lines if l]
    assert len(lines) == 11
    for fmt, amax, _, e, code in lines:
        dmax = 448.0 if fmt == "e4m3" else 6.0
        assert mx_exponent(np.array([float(amax)]), dmax)[0] == int(e)
        x = np.zeros((1, 32))
        x[0, 7] = float(amax)
        _, sc = oracle.dynamic_quant_mx(x, None, fmt)
        assert sc[0, 0] == int(code)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_mx_against_exact_and_invariants(fmt):
    dmax, mb, me = (448, 3, -6) if fmt == "e4m3" else (6, 1, 0)
    dec = oracle.e4m3_decode if fmt == "e4m3" else oracle.e2m1_decode
    rng = np.random.default_rng(11)
    x = _fp16(rng.standard_normal((6, 80)) * np.exp2(rng.integers(-10, 10, (6, 1))))
    smooth = _fp16(rng.uniform(0.5, 2.0, 80))
    codes, sc = oracle.dynamic_quant_mx(x, smooth, fmt)
    assert codes.shape == (6, 80) and sc.shape == (6, 3)       # 80 = 32 + 32 + 16
    v = x * smooth
    for r in range(6):
        for j in range(3):
            blk = v[r, 32 * j:32 * j + 32]
            e, vals = exact.mx_block([Fraction(float(t)) for t in blk], dmax, mb, me)
            assert sc[r, j] == e + 127
            got = dec(codes[r, 32 * j:32 * j + 32])
            assert [Fraction(float(g)) for g in got] == vals
            assert np.max(np.abs(got)) <= dmax
            assert np.max(np.abs(got)) >= dmax / 2


def test_mx_zero_block_and_one_binade():
    x = np.zeros((1, 64))
    x[0, 40] = 1.0
    codes, sc = oracle.dynamic_quant_mx(x, None, "e4m3")
    assert sc[0].tolist() == [127, 119]
    assert np.all(codes[0, :32] == 0)
    assert oracle.e4m3_decode(codes[0, 40]) * 2.0 ** -8 == 1.0
