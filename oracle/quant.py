"""Dynamic quantization (oracle; test infrastructure only).

Per-token mode follows the aclnnDynamicQuant page (Formula): with the optional
smooth scales, ``input = x * smooth``; ``scale = row_max(|input|) / dtypeMax``;
``y = round(input / scale)``; a row is every leading dimension flattened.

Readings where the page is silent:

* the quantized code is decided in float32: the product ``x * smooth`` (exact
  in float32 for fp16 and bf16 inputs), the row maximum (exact), the scale as
  the correctly rounded float32 quotient ``a / dtypeMax`` and the code as the
  correctly rounded float32 quotient ``input / scale`` rounded half to even;
* dtypeMax is 127 for INT8 and 7 for INT4 and for INT32 (eight INT4 codes per
  word, lowest nibble first); codes are clamped to [-dtypeMax, dtypeMax];
* an all-zero row gets scale 0 and codes 0;
* the scale output is float32, one per row.

MX mode (block 32 along the last axis) applies the same formula per
(row, 32-block), the K blocking of the aclnnQuantBatchMatmulInplaceAdd page
(Formula: gsK = 32, the last block may be shorter). The pages do not say how an
MX scale is chosen; the reading here rounds the page's ``max / dtypeMax`` up
to a power of two, ``2^e`` with ``e = ceil(log2(a / dtypeMax))`` clamped to
[-127, 127] and stored as the E8M0 code ``e + 127``; codes are
``RNE_fmt(input / 2^e)``, whose magnitude then never exceeds dtypeMax
(448 for E4M3, 6 for E2M1). An all-zero block gets code 127 and zero values.
"""
from __future__ import annotations

import numpy as np

from .formats import E2M1_MAX, E4M3_MAX, e2m1_encode, e4m3_encode

DTYPE_MAX = {"int8": 127, "int4": 7, "int32": 7}


def _rows(x, smooth):
    x = np.asarray(x, dtype=np.float64)
    cols = x.shape[-1]
    v = x.reshape(-1, cols)
    if smooth is not None:
        v = v * np.asarray(smooth, dtype=np.float64).reshape(1, cols)
    return v


def dynamic_quant_per_token(x, smooth=None, out: str = "int8"):
    """Returns (codes int64 (rows, cols), scale float32 (rows,))."""
    dmax = DTYPE_MAX[out]
    v64 = _rows(x, smooth)
    v = v64.astype(np.float32)
    if not np.array_equal(v.astype(np.float64), v64):
        raise ValueError("x*smooth is not exact in float32 (outside the contract)")
    a = np.max(np.abs(v), axis=1) if v.shape[1] else np.zeros(v.shape[0], np.float32)
    scale = (a / np.float32(dmax)).astype(np.float32)
    safe = np.where(scale == 0, np.float32(1), scale).astype(np.float32)
    q = np.rint((v / safe[:, None]).astype(np.float32))
    q = np.where(scale[:, None] == 0, 0, q)
    q = np.clip(q, -dmax, dmax).astype(np.int64)
    return q, scale


def encode_quant_output(q, out: str) -> np.ndarray:
    """Store per-token codes as the operator outputs them: INT8 bytes, INT4
    nibbles two per byte (even column low), INT32 words of eight nibbles."""
    q = np.asarray(q, dtype=np.int64)
    if out == "int8":
        return q.astype(np.int8)
    nib = q & 0xF
    if out == "int4":
        return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    if out == "int32":
        word = np.zeros((q.shape[0], q.shape[1] // 8), dtype=np.int64)
        for i in range(8):
            word |= nib[:, i::8] << (4 * i)
        return word.astype(np.uint32).view(np.int32)
    raise ValueError(out)


def unpack_quant_output(stored, out: str, cols: int) -> np.ndarray:
    """Inverse of :func:`encode_quant_output` back to signed codes."""
    s = np.asarray(stored)
    if out == "int8":
        return s.astype(np.int64)
    if out == "int4":
        b = s.astype(np.uint8).astype(np.int64)
        nib = np.empty((b.shape[0], cols), dtype=np.int64)
        nib[:, 0::2] = b & 0xF
        nib[:, 1::2] = b >> 4
    elif out == "int32":
        w = s.astype(np.int32).view(np.uint32).astype(np.int64)
        nib = np.empty((w.shape[0], cols), dtype=np.int64)
        for i in range(8):
            nib[:, i::8] = (w >> (4 * i)) & 0xF
    else:
        raise ValueError(out)
    return np.where(nib >= 8, nib - 16, nib)


def mx_exponent(a, dmax: float) -> np.ndarray:
    """Smallest integer e with dmax * 2^e >= a (a > 0), clamped to [-127, 127];
    0 where a == 0. Exact: only powers of two and comparisons are used."""
    a = np.asarray(a, dtype=np.float64)
    pos = a > 0
    _, ex = np.frexp(np.where(pos, a, 1.0))      # a < 2^ex
    e = ex.astype(np.int64) - 12                 # dmax * 2^e < a here (dmax < 2^12)
    for _ in range(16):
        low = np.ldexp(dmax, e) < a
        e = np.where(low & pos, e + 1, e)
    e = np.where(pos, e, 0)
    return np.clip(e, -127, 127)


def dynamic_quant_mx(x, smooth=None, fmt: str = "e4m3", block: int = 32):
    """Returns (codes uint8 (rows, cols) in the logical layout, E8M0 scale codes
    uint8 (rows, ceil(cols/block)))."""
    dmax = {"e4m3": E4M3_MAX, "e2m1": E2M1_MAX}[fmt]
    enc = {"e4m3": e4m3_encode, "e2m1": e2m1_encode}[fmt]
    v = _rows(x, smooth)
    rows, cols = v.shape
    nb = -(-cols // block)
    codes = np.zeros((rows, cols), dtype=np.uint8)
    scales = np.zeros((rows, nb), dtype=np.uint8)
    for j in range(nb):
        blk = v[:, j * block:min(cols, (j + 1) * block)]
        a = np.max(np.abs(blk), axis=1)
        e = mx_exponent(a, dmax)
        scales[:, j] = (e + 127).astype(np.uint8)
        codes[:, j * block:j * block + blk.shape[1]] = enc(np.ldexp(blk, -e[:, None]))
    return codes, scales
