"""CPU check of the A8W4 tile's weight unpack (a8w4_gemm.hip, w4_unpack):
two packed bytes of INT4 codes (even code in the low nibble, as the
aclnnConvertWeightToINT4Pack page's pack orders them) become four int8 bytes
16 * q, in code order, by one byte permute and one mask per output word.

v_perm_b32 is emulated from its definition in the CDNA ISA: byte i of the
result is the byte of the 64-bit value {S0, S1} (S1 in bytes 0..3, S0 in
bytes 4..7) named by byte i of the selector (values 0..7 here)."""
import numpy as np


def perm(s0: int, s1: int, sel: int) -> int:
    both = (s0 << 32) | s1
    out = 0
    for i in range(4):
        b = (sel >> (8 * i)) & 0xFF
        assert b < 8
        out |= ((both >> (8 * b)) & 0xFF) << (8 * i)
    return out


def unpack_word(w: int):
    """The kernel's arithmetic for one packed dword: eight codes -> two
    output dwords of four int8 bytes each."""
    s = (w << 4) & 0xFFFFFFFF
    lo = perm(s, w, 0x01050004) & 0xF0F0F0F0
    hi = perm(s, w, 0x03070206) & 0xF0F0F0F0
    return lo, hi


def as_int8_bytes(v: int):
    return [int(np.int8(np.uint8((v >> (8 * i)) & 0xFF))) for i in range(4)]


def test_every_pair_of_codes_in_every_position():
    codes_all = np.arange(-8, 8)
    for a in codes_all:
        for b in codes_all:
            # place the pair (a, b) at every code position 0..7 of a dword,
            # the other codes fixed and distinct from 0
            for pos in range(0, 8, 2):
                codes = [(3 * i + 1) % 16 - 8 for i in range(8)]
                codes[pos], codes[pos + 1] = int(a), int(b)
                w = 0
                for i, c in enumerate(codes):
                    w |= (c & 0xF) << (4 * i)
                lo, hi = unpack_word(w)
                got = as_int8_bytes(lo) + as_int8_bytes(hi)
                assert got == [16 * c for c in codes], (codes, got)


def test_random_dwords():
    rng = np.random.default_rng(0)
    for w in rng.integers(0, 2 ** 32, size=2000, dtype=np.uint64):
        w = int(w)
        codes = [((w >> (4 * i)) & 0xF) - (16 if (w >> (4 * i)) & 0x8 else 0) for i in range(8)]
        lo, hi = unpack_word(w)
        assert as_int8_bytes(lo) + as_int8_bytes(hi) == [16 * c for c in codes]
