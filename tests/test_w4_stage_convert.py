"""CPU check of the INT8 tile's INT4 staging conversion (wq_gemm_w8.hip,
convert_n16): 16 consecutive K codes of one column, two dwords of nibbles in
the GFX950_B byte order (low nibble first), become 16 exact 16-bit values q
in K order.

v_perm_b32 is emulated from its definition in the CDNA ISA (byte i of the
result is the byte of the 64-bit value {S0, S1}, S1 in bytes 0..3, named by
byte i of the selector); the packed half subtraction from IEEE fp16
arithmetic (numpy float16: the difference of two fp16 values in [1024, 2048)
and 1032 is exact); the bf16 path from its float32 steps."""
import numpy as np


def perm(s0: int, s1: int, sel: int) -> int:
    both = (s0 << 32) | s1
    out = 0
    for i in range(4):
        b = (sel >> (8 * i)) & 0xFF
        assert b < 8
        out |= ((both >> (8 * b)) & 0xFF) << (8 * i)
    return out


def halves(v: int):
    return np.array([v & 0xFFFF, v >> 16], dtype=np.uint16).view(np.float16)


def convert_f16(w0: int, w1: int):
    out = []
    for w in (w0, w1):
        u = w ^ 0x88888888
        ev, od = u & 0x0F0F0F0F, (u >> 4) & 0x0F0F0F0F
        p0, p1 = perm(od, ev, 0x05010400), perm(od, ev, 0x07030602)
        for p in (p0, p1):
            for sel in (0x04010400, 0x04030402):
                h = halves(perm(0x64646464, p, sel))
                out += list((h - np.float16(1032.0)).astype(np.float64))
    return out


def convert_bf16(w0: int, w1: int):
    out = []
    for w in (w0, w1):
        u = w ^ 0x88888888
        ev, od = u & 0x0F0F0F0F, (u >> 4) & 0x0F0F0F0F
        p0, p1 = perm(od, ev, 0x05010400), perm(od, ev, 0x07030602)
        for p in (p0, p1):
            for j in range(4):
                q = np.float32((p >> (8 * j)) & 0xFF) - np.float32(8.0)
                out.append(float(q))          # |q| <= 8: exact in bf16
    return out


def codes_of(w0: int, w1: int):
    nib = [((w >> (4 * i)) & 0xF) for w in (w0, w1) for i in range(8)]
    return [n - 16 if n >= 8 else n for n in nib]


def test_every_code_in_every_position():
    for pos in range(16):
        for c in range(-8, 8):
            codes = [(5 * i + 3) % 16 - 8 for i in range(16)]
            codes[pos] = c
            w = [0, 0]
            for i, q in enumerate(codes):
                w[i // 8] |= (q & 0xF) << (4 * (i % 8))
            assert convert_f16(*w) == codes
            assert convert_bf16(*w) == codes


def test_random_dwords():
    rng = np.random.default_rng(1)
    for w0, w1 in rng.integers(0, 2 ** 32, size=(1000, 2), dtype=np.uint64):
        w0, w1 = int(w0), int(w1)
        assert convert_f16(w0, w1) == codes_of(w0, w1)
        assert convert_bf16(w0, w1) == codes_of(w0, w1)


# Row-major ND INT4 (convert_rows4_n): four K rows of four columns, each row
# 16 bits (nibble j = column j) -> per column the four K values as 16-bit q,
# {rows 0-1, rows 2-3}.
def convert_rows_f16(r):
    u = [x ^ 0x8888 for x in r]
    out = []
    for j in range(4):
        col = []
        for a, b in ((0, 1), (2, 3)):
            h = (0x6400 | ((u[a] >> (4 * j)) & 0xF)) | ((0x6400 | ((u[b] >> (4 * j)) & 0xF)) << 16)
            col += list((halves(h) - np.float16(1032.0)).astype(np.float64))
        out.append(col)
    return out


def convert_rows_bf16(r):
    u = [x ^ 0x8888 for x in r]
    return [[float(np.float32((u[i] >> (4 * j)) & 0xF) - np.float32(8.0)) for i in range(4)] for j in range(4)]


def test_row_major_nibbles_every_code_in_every_position():
    for pos in range(16):
        for c in range(-8, 8):
            codes = [[(3 * i + 5 * j + 1) % 16 - 8 for j in range(4)] for i in range(4)]   # [row][col]
            codes[pos // 4][pos % 4] = c
            r = [sum((codes[i][j] & 0xF) << (4 * j) for j in range(4)) for i in range(4)]
            want = [[codes[i][j] for i in range(4)] for j in range(4)]
            assert convert_rows_f16(r) == want
            assert convert_rows_bf16(r) == want
