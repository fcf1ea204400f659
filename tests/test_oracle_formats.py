"""Pins of the oracle's element formats (E4M3, E2M1, E8M0)."""
import os
from fractions import Fraction

import numpy as np
import torch

import oracle
from tests import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e4m3_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2                          # S.1111.111 only
    assert np.array_equal(ours[~nan], lib[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(lib[~nan]))
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9


def test_e4m3_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_decode(codes)), codes)


def test_e4m3_encode_matches_torch_on_midpoints_and_random():
    # float32 inputs: torch converts through float32, and so do the kernels
    vals = np.sort(np.unique(oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))))
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)   # every tie, exact in fp32
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)),
                           np.nextafter(mids, np.float32(1000))])
    rng = np.random.default_rng(5)
    rand = (rng.uniform(-448, 448, 20000) * np.exp2(rng.integers(-14, 1, 20000))).astype(np.float32)
    for v in (near, -near, rand):
        ours = oracle.e4m3_encode(v.astype(np.float64))
        lib = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(ours, lib)


def test_e4m3_encode_against_exact_rounding():
    rng = np.random.default_rng(6)
    v = rng.uniform(-448, 448, 500) * np.exp2(rng.integers(-12, 1, 500))
    for x in v:
        want = exact.round_to_format(Fraction(float(x)), 3, -6)
        got = oracle.e4m3_decode(oracle.e4m3_encode(x))
        assert Fraction(float(got)) == want


def test_e4m3_sign_of_zero_kept():
    assert oracle.e4m3_encode(np.array([-0.0, -1e-12, 0.0])).tolist() == [0x80, 0x80, 0x00]


def test_e2m1_table_and_ties_from_golden():
    codes, values, ties = [], [], []
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        for line in f:
            line = line.split("#")[0].split()
            if not line:
                continue
            if line[0] == "tie":
                ties.append((float(line[1]), float(line[2])))
            else:
                codes.append(int(line[0]))
                values.append(float(line[1]))
    dec = oracle.e2m1_decode(np.array(codes))
    assert np.array_equal(dec, np.array(values))
    assert np.array_equal(np.signbit(dec), np.signbit(np.array(values)))
    assert np.array_equal(oracle.e2m1_encode(np.array(values)), np.array(codes, dtype=np.uint8))
    for x, want in ties:
        assert oracle.e2m1_decode(oracle.e2m1_encode(x)) == want


def test_e2m1_encode_against_exact_rounding():
    rng = np.random.default_rng(7)
    v = rng.uniform(-6, 6, 2000)
    got = oracle.e2m1_decode(oracle.e2m1_encode(v))
    for x, g in zip(v, got):
        assert Fraction(float(g)) == exact.round_to_format(Fraction(float(x)), 1, 0)


def test_e8m0_decode():
    d = oracle.e8m0_decode(np.array([0, 1, 126, 127, 128, 254, 255]))
    assert d[:6].tolist() == [2.0 ** -127, 2.0 ** -126, 0.5, 1.0, 2.0, 2.0 ** 127]
    assert np.isnan(d[6])
