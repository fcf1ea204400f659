"""INT4 weight packing (oracle; test infrastructure only).

Follows the aclnnConvertWeightToINT4Pack page (operator description): weights
stored one 4-bit value per INT32 ("sparse") become tightly packed nibbles
("dense"). The page shows no byte example, so two readings are taken:

* a value is stored as its 4-bit two's complement, ``v & 0xF``;
* within a byte the element with the even index along the packed axis takes
  the low nibble (bits 0..3), which fits the DynamicQuant page's rule that an
  INT4 output needs an even last dimension and an INT32 output one divisible
  by 8 (eight nibbles per word, lowest first).

The ND layout packs along the last axis: a (k, n) weight becomes (k, n/2)
bytes. The GFX950_B layout is this library's own MFMA-operand order (the pages'
FRACTAL_NZ is an Ascend cube layout and is not used). For a logical (K, N)
matrix of 4-bit codes, with Kp = 128*ceil(K/128) and Np = 16*ceil(N/16), the
code at (k, n) (zero for the padding k >= K or n >= N) sits in

    byte   ((k // 128) * Np + n) * 64 + ((k // 32) % 4) * 16 + (k % 32) // 2
    nibble k % 2   (0 = low)

so each column's 32 consecutive K values of one 32-block are 16 contiguous
bytes, and the four blocks of a 128-deep K slab of one column are 64
contiguous bytes. The oracle builds it by reshaping, not by the byte formula.
"""
from __future__ import annotations

import numpy as np


def _check_int4(w: np.ndarray) -> np.ndarray:
    w = np.asarray(w)
    if w.dtype.kind not in "iu":
        raise TypeError("int4 weights must be integers")
    if np.any(w < -8) or np.any(w > 7):
        raise ValueError("int4 values must lie in [-8, 7]")
    return w.astype(np.int64)


def pack_int4_nd(w, transpose: bool = False) -> np.ndarray:
    """(k, n) int32 values in [-8, 7] -> (k, n/2) uint8, even column low.

    ``transpose=True`` means ``w`` is stored (n, k) and the logical weight is
    its transpose (the x2-transposed input of the AddRmsNorm page)."""
    w = _check_int4(w)
    if transpose:
        w = w.T
    k, n = w.shape
    if n % 2:
        raise ValueError("the packed axis must have even length")
    nib = w & 0xF
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


def unpack_int4_nd(packed, n: int) -> np.ndarray:
    """Inverse of :func:`pack_int4_nd` to signed values."""
    b = np.asarray(packed, dtype=np.uint8).astype(np.int64)
    out = np.empty((b.shape[0], n), dtype=np.int64)
    out[:, 0::2] = b & 0xF
    out[:, 1::2] = b >> 4
    return np.where(out >= 8, out - 16, out)


def gfx950b_bytes(k: int, n: int) -> int:
    kp = 128 * -(-k // 128)
    np_ = 16 * -(-n // 16)
    return kp * np_ // 2


def pack_codes_gfx950b(codes, k: int, n: int) -> np.ndarray:
    """(K, N) 4-bit codes (0..15) -> GFX950_B bytes (flat uint8)."""
    kp = 128 * -(-k // 128)
    np_ = 16 * -(-n // 16)
    full = np.zeros((kp, np_), dtype=np.int64)
    full[:k, :n] = np.asarray(codes, dtype=np.int64) & 0xF
    # k = slab*128 + blk*32 + pair*2 + half
    t = full.reshape(kp // 128, 4, 16, 2, np_)
    # storage order: slab, column, blk, pair, half
    t = t.transpose(0, 4, 1, 2, 3)
    return (t[..., 0] | (t[..., 1] << 4)).astype(np.uint8).reshape(-1)


def pack_int4_gfx950b(w, transpose: bool = False) -> np.ndarray:
    """(k, n) int32 values in [-8, 7] -> GFX950_B bytes (flat uint8)."""
    w = _check_int4(w)
    if transpose:
        w = w.T
    k, n = w.shape
    return pack_codes_gfx950b(w & 0xF, k, n)


def unpack_int4_gfx950b(packed, k: int, n: int, signed: bool = True) -> np.ndarray:
    """Inverse of :func:`pack_int4_gfx950b`, dropping the padding."""
    kp = 128 * -(-k // 128)
    np_ = 16 * -(-n // 16)
    b = np.asarray(packed, dtype=np.uint8).astype(np.int64).reshape(kp // 128, np_, 4, 16)
    t = np.stack([b & 0xF, b >> 4], axis=-1)          # slab, col, blk, pair, half
    full = t.transpose(0, 2, 3, 4, 1).reshape(kp, np_)
    out = full[:k, :n]
    return np.where(out >= 8, out - 16, out) if signed else out


def pack_float_e2m1(w, layout: str = "gfx950b", transpose: bool = False) -> np.ndarray:
    """FLOAT -> tightly packed FLOAT4_E2M1 (aclnnConvertWeightToINT4Pack page:
    on the newer chips the pack also takes FLOAT weights and writes packed
    E2M1). ``w`` is (k, n) float32 (or (n, k) with ``transpose``).

    Reading: each value goes to the nearest E2M1 value, ties to even, the sign
    of zero kept; magnitudes beyond 6 (the largest E2M1) saturate to +-6.
    NaN is outside the contract. The codes are then packed exactly as INT4
    codes are (``layout`` "nd": (k, n/2) bytes, even column low; "gfx950b")."""
    from .formats import E2M1_MAX, e2m1_encode
    v = np.asarray(w, dtype=np.float64)
    if np.any(np.isnan(v)):
        raise ValueError("NaN has no E2M1 code")
    if transpose:
        v = v.T
    k, n = v.shape
    codes = e2m1_encode(np.clip(v, -E2M1_MAX, E2M1_MAX)).astype(np.int64)
    if layout == "nd":
        if n % 2:
            raise ValueError("the packed axis must have even length")
        return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    if layout == "gfx950b":
        return pack_codes_gfx950b(codes, k, n)
    raise ValueError(layout)
