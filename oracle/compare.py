"""Comparison helpers for checking a result against the oracle (test
infrastructure only)."""
from __future__ import annotations

import numpy as np
import torch


def as_f64(t) -> np.ndarray:
    """A tensor or array converted exactly to float64 numpy (any device)."""
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def rel_err_floor(got, ref) -> float:
    """max_i |got_i - ref_i| / max(|ref_i|, RMS(ref)).

    The relative error of each element with its denominator floored at the
    tensor's RMS, so elements near zero are judged against the tensor's scale
    rather than against themselves."""
    g = as_f64(got).reshape(-1)
    r = as_f64(ref).reshape(-1)
    if r.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(r * r)))
    den = np.maximum(np.abs(r), rms)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(g - r) / den))
