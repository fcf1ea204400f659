"""CPU check of the INT4 -> 16-bit MFMA operand unpack that the GFX950_B
weight-quantized GEMM kernels share (csrc/wq_unpack.h).

A packed dword holds eight INT4 codes (two's complement, even K in the low
nibble, as the aclnnConvertWeightToINT4Pack page orders them). The kernels
turn it into four dwords whose 16-bit halves are the exact values q + 24
(bf16 or fp16), codes (2j, 2j+1) in dword j, by the bit operations emulated
here from their ISA definitions:
  - v_perm_b32: byte i of the result is the byte of the 64-bit value
    {S0, S1} (S1 in bytes 0..3) named by byte i of the selector; selector
    value 0x0C gives 0x00;
  - v_bitop3_b32 with truth table 0x6A: S2 ^ (S0 & S1);
  - shifts and v_lshl_or_b32: (S0 << S1) | S2.
The constants are the kernel's. A zero-scale column uses zeroed keys and
must give zeros."""
import numpy as np

M32 = 0xFFFFFFFF


def perm(s0: int, s1: int, sel: int) -> int:
    both = (s0 << 32) | s1
    out = 0
    for i in range(4):
        b = (sel >> (8 * i)) & 0xFF
        if b == 0x0C:
            v = 0
        else:
            assert b < 8
            v = (both >> (8 * b)) & 0xFF
        out |= v << (8 * i)
    return out


def bitop3_6a(p: int, m: int, c: int) -> int:
    return (c ^ (m & p)) & M32


def unpack_bf16(w: int, on: bool = True):
    m2, c2 = (0x00780078, 0x41C041C0) if on else (0, 0)
    a, b = (w << 3) & M32, w >> 1
    return [bitop3_6a(perm(b, a, 0x0C040C00 + 0x00010001 * j), m2, c2) for j in range(4)]


def unpack_f16(w: int, on: bool = True):
    m1, c1, e = (0x0F0F0F0F, 0x08080808, 0x4C004C00) if on else (0, 0, 0)
    a, b = bitop3_6a(w, m1, c1), bitop3_6a(w >> 4, m1, c1)
    return [((perm(b, a, 0x0C040C00 + 0x00010001 * j) << 6) & M32) | e for j in range(4)]


def halves(dwords, fmt):
    out = []
    for d in dwords:
        for h in (d & 0xFFFF, d >> 16):
            if fmt == "bf16":
                out.append(float(np.array([h << 16], dtype=np.uint32).view(np.float32)[0]))
            else:
                out.append(float(np.array([h], dtype=np.uint16).view(np.float16)[0]))
    return out


def pack_codes(codes):
    w = 0
    for i, c in enumerate(codes):
        w |= (c & 0xF) << (4 * i)
    return w


def test_every_code_pair_in_every_position():
    for fmt, fn in (("bf16", unpack_bf16), ("f16", unpack_f16)):
        for a in range(-8, 8):
            for b in range(-8, 8):
                for pos in range(0, 8, 2):
                    codes = [(5 * i + 3) % 16 - 8 for i in range(8)]
                    codes[pos], codes[pos + 1] = a, b
                    got = halves(fn(pack_codes(codes)), fmt)
                    assert got == [c + 24.0 for c in codes], (fmt, codes, got)


def test_random_dwords_and_zeroed_keys():
    rng = np.random.default_rng(0)
    for w in rng.integers(0, 2 ** 32, size=3000, dtype=np.uint64):
        w = int(w)
        codes = [((w >> (4 * i)) & 0xF) - (16 if (w >> (4 * i)) & 0x8 else 0) for i in range(8)]
        for fmt, fn in (("bf16", unpack_bf16), ("f16", unpack_f16)):
            assert halves(fn(w), fmt) == [c + 24.0 for c in codes]
            assert fn(w, on=False) == [0, 0, 0, 0]


def test_operand_range_is_exact_and_positive():
    # 16 .. 31: every value is an integer with at most 5 significant bits, so
    # x * B is exact in float32 for any 16-bit x
    vals = halves(unpack_bf16(pack_codes(list(range(-8, 0)))), "bf16") + \
        halves(unpack_f16(pack_codes(list(range(0, 8)))), "f16")
    assert vals == [float(v) for v in range(16, 32)]


def unpack_low(w: int, fmt: str):
    """The decode kernel's 9-operation form: nibble in the low mantissa bits,
    q + 136 (bf16, exponent bits 0x4300) or q + 1032 (fp16, 0x6400)."""
    c = 0x43084308 if fmt == "bf16" else 0x64086408
    w4 = w >> 4
    return [bitop3_6a(perm(w4, w, 0x0C040C00 + 0x00010001 * j), 0x000F000F, c) for j in range(4)]


def test_low_mantissa_form_every_code_pair():
    for fmt, bias in (("bf16", 136.0), ("f16", 1032.0)):
        for a in range(-8, 8):
            for b in range(-8, 8):
                for pos in range(0, 8, 2):
                    codes = [(7 * i + 1) % 16 - 8 for i in range(8)]
                    codes[pos], codes[pos + 1] = a, b
                    got = halves(unpack_low(pack_codes(codes), fmt), fmt)
                    assert got == [c + bias for c in codes], (fmt, codes, got)
