"""Weight-quantized matmul + residual add + RMSNorm (oracle; float64).

Follows the aclnnWeightQuantMatmulAllReduceAddRmsNorm page:

* Formula: ``mm = x1 @ (x2 * antiquantScale + antiquantOffset) + bias``;
  ``y = mm + residual``; ``normOut = y / RMS(y) * gamma`` with
  ``RMS(y) = sqrt(mean over the last dimension of y^2 + epsilon)``. The
  AllReduce of that formula is the identity on one device and is left out.
* Constraints: per-tensor scale shape (1), per-channel (1, n) or (n),
  per-group (ceil(k / G), n) with G the group size; the offset, when given,
  has the scale's shape; bias (n); residual (b, s, n) with b*s the rows of x1.

Readings: the offset is added after the scaling (as the formula is written);
k index i belongs to group floor(i / G), the last group possibly partial; a
missing offset or bias is zero; every input is converted exactly to float64
and nothing is rounded until the end (the HIP path rounds the dequantized
weight and the outputs to the activation dtype; the tolerance absorbs that).
"""
from __future__ import annotations

import numpy as np


def dequantize_weight(w, scale, offset=None, group_size: int = 0) -> np.ndarray:
    """(k, n) integer weight -> float64 ``w * s[g(i), j] + o[g(i), j]``."""
    q = np.asarray(w, dtype=np.float64)
    k, n = q.shape
    s = np.asarray(scale, dtype=np.float64)
    o = None if offset is None else np.asarray(offset, dtype=np.float64)
    if o is not None and o.shape != s.shape:
        raise ValueError("offset must have the scale's shape")

    def expand(t):
        if t.size == 1:                                   # per tensor
            return np.full((k, n), t.reshape(()))
        if t.ndim == 1 or t.shape[0] == 1:                # per channel
            if t.size != n:
                raise ValueError("per-channel scale needs n entries")
            return np.broadcast_to(t.reshape(1, n), (k, n))
        g = group_size                                    # per group
        if g <= 0 or t.shape != (-(-k // g), n):
            raise ValueError("per-group scale must be (ceil(k/G), n)")
        return t[np.arange(k) // g, :]

    deq = q * expand(s)
    if o is not None:
        deq = deq + expand(o)
    return deq


def wq_matmul_add_rmsnorm(x1, w, scale, offset, group_size, bias, residual,
                          gamma, eps: float):
    """Returns (mm, y, norm_out) as float64 arrays of shape (rows, n)."""
    q = np.asarray(w)
    k, n = q.shape
    x = np.asarray(x1, dtype=np.float64).reshape(-1, k)
    mm = x @ dequantize_weight(q, scale, offset, group_size)
    if bias is not None:
        mm = mm + np.asarray(bias, dtype=np.float64).reshape(1, n)
    y = mm + np.asarray(residual, dtype=np.float64).reshape(-1, n)
    ms = np.mean(y * y, axis=1, keepdims=True)
    norm_out = y / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64).reshape(1, n)
    return mm, y, norm_out


def weight_quant_matmul(x1, w, scale, offset, group_size, bias):
    """The Formula's first line alone, ``mm = x1 @ (x2 * antiquantScale +
    antiquantOffset) + bias`` (AllReduce the identity on one device): the
    standalone weight-quantized matmul that the page's deprecation note names
    as the replacement's first half. Returns float64 (rows, n)."""
    q = np.asarray(w)
    k, n = q.shape
    x = np.asarray(x1, dtype=np.float64).reshape(-1, k)
    mm = x @ dequantize_weight(q, scale, offset, group_size)
    if bias is not None:
        mm = mm + np.asarray(bias, dtype=np.float64).reshape(1, n)
    return mm


def add_rms_norm(x, residual, gamma, eps: float):
    """The Formula's second and third lines alone (the replacement's second
    half, AddRmsNorm): ``y = x + residual`` and ``normOut = y / RMS(y) *
    gamma`` with ``RMS(y) = sqrt(mean of y^2 over the last dimension +
    epsilon)``. ``x`` and ``residual`` are (rows, d) (or anything reshaping to
    it), gamma (d). Returns (y, norm_out) as float64 (rows, d)."""
    g = np.asarray(gamma, dtype=np.float64).reshape(-1)
    d = g.size
    y = (np.asarray(x, dtype=np.float64).reshape(-1, d)
         + np.asarray(residual, dtype=np.float64).reshape(-1, d))
    rms = np.sqrt(np.sum(y * y, axis=1, keepdims=True) / d + eps)
    return y, y / rms * g.reshape(1, d)
