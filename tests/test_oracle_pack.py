"""Pins of the oracle's INT4 packing (ND and GFX950_B)."""
import itertools
import os

import numpy as np
import pytest

import oracle
from oracle.pack import pack_codes_gfx950b

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_word():
    d = {}
    with open(os.path.join(GOLDEN, "pack_int4_word.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                key, val = line.split(":")
                d[key.strip()] = val.split()
    return d


def test_nd_word_example():
    g = _golden_word()
    vals = np.array([[int(v) for v in g["values"]]], dtype=np.int32)
    packed = oracle.pack_int4_nd(vals)
    assert packed.reshape(-1).tolist() == [int(b, 16) for b in g["bytes"]]
    assert packed.view(np.uint32)[0, 0] == int(g["word"][0], 16)


def test_nd_round_trip_every_value_every_position():
    base = np.zeros((3, 8), dtype=np.int32)
    for (r, c), v in itertools.product(itertools.product(range(3), range(8)), range(-8, 8)):
        w = base.copy()
        w[r, c] = v
        p = oracle.pack_int4_nd(w)
        assert np.array_equal(oracle.unpack_int4_nd(p, 8), w)
        # only the byte that holds (r, c) is non-zero, in the expected nibble
        nz = np.argwhere(p)
        if v:
            assert nz.tolist() == [[r, c // 2]]
            assert (p[r, c // 2] >> (4 * (c % 2))) & 0xF == v & 0xF


def test_nd_transposed_input():
    rng = np.random.default_rng(1)
    w = rng.integers(-8, 8, size=(6, 10), dtype=np.int32)
    assert np.array_equal(oracle.pack_int4_nd(w.T.copy(), transpose=True), oracle.pack_int4_nd(w))


def test_rejects_out_of_range_and_odd_width():
    with pytest.raises(ValueError):
        oracle.pack_int4_nd(np.array([[8, 0]], dtype=np.int32))
    with pytest.raises(ValueError):
        oracle.pack_int4_nd(np.array([[-9, 0]], dtype=np.int32))
    with pytest.raises(ValueError):
        oracle.pack_int4_nd(np.zeros((2, 3), dtype=np.int32))


def test_gfx950b_golden_bytes():
    cases = []
    with open(os.path.join(GOLDEN, "gfx950b_layout.txt")) as f:
        for line in f:
            line = line.split("#")[0].split()
            if not line:
                continue
            if line[0] == "case":
                cases.append(((int(line[1]), int(line[2])), []))
            else:
                k, n, v, _, byte, hexv = line
                cases[-1][1].append((int(k), int(n), int(v), int(byte), int(hexv, 16)))
    assert len(cases) == 2
    for (K, N), plants in cases:
        w = np.zeros((K, N), dtype=np.int32)
        for k, n, v, _, _ in plants:
            w[k, n] = v
        p = oracle.pack_int4_gfx950b(w)
        assert p.size == oracle.gfx950b_bytes(K, N)
        want = {byte: hexv for _, _, _, byte, hexv in plants}
        for byte, hexv in want.items():
            assert p[byte] == hexv, (K, N, byte)
        assert np.count_nonzero(p) == len(want)


@pytest.mark.parametrize("k,n", [(128, 16), (256, 128), (80, 20), (1, 2), (300, 50)])
def test_gfx950b_round_trip_and_permutation(k, n):
    rng = np.random.default_rng(k * 1000 + n)
    w = rng.integers(-8, 8, size=(k, n), dtype=np.int32)
    p = oracle.pack_int4_gfx950b(w)
    assert np.array_equal(oracle.unpack_int4_gfx950b(p, k, n), w)
    # a permutation of the ND nibbles plus zero padding: same nibble histogram
    nib = np.concatenate([p & 0xF, p >> 4])
    hist = np.bincount(nib, minlength=16)
    want = np.bincount((w & 0xF).reshape(-1), minlength=16)
    want[0] += nib.size - w.size
    assert np.array_equal(hist, want)


def test_gfx950b_column_runs_are_contiguous():
    # Each column's 32 K values of one block occupy 16 contiguous bytes.
    k, n = 256, 32
    codes = np.tile(np.arange(32) % 16, (k // 32, 1)).reshape(k, 1) * np.ones((1, n), dtype=np.int64)
    p = pack_codes_gfx950b(codes, k, n)
    run = bytes([(2 * i) % 16 | (((2 * i + 1) % 16) << 4) for i in range(16)])
    for c in range(0, p.size, 16):
        assert p[c:c + 16].tobytes() == run
