"""Helpers for the GPU parity tests: run a workload through the C ABI and run
the same inputs through the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import bit_quantized_gemm_int4_amd as wq
import oracle
from oracle import as_f64

DEV = "cuda"


def note(msg: str) -> None:
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print(msg, flush=True)
    sys.stdout.flush()


def wq_on_gpu(case, layout=wq.WQ_LAYOUT_GFX950_B, inplace=False, transpose_x2=False):
    """Run wq_matmul_add_rmsnorm on ``case``; returns (y, norm_out) on the CPU."""
    m, k, n = case.mkn
    x1 = case.x1.to(DEV)
    if case.w_bits == 4:
        w = case.w.to(DEV)
        if transpose_x2:
            # the transposed weight (n, k), packed along its last dimension:
            # (n, k/2) bytes, even k in the low nibble
            assert layout == wq.WQ_LAYOUT_ND
            x2 = wq.pack_int4(w.t().contiguous(), layout)
        else:
            x2 = wq.pack_int4(w, layout)
        wdt = wq.WQ_INT4
    else:
        w8 = case.w.to(torch.int8)
        x2 = (w8.t().contiguous() if transpose_x2 else w8).to(DEV)
        wdt = wq.WQ_INT8
        layout = wq.WQ_LAYOUT_ND
    dev = lambda t: None if t is None else t.to(DEV)
    residual = case.residual.to(DEV).clone()
    y, norm = wq.matmul_add_rmsnorm(x1, x2, k, n, wdt, dev(case.scale), dev(case.offset),
                                    case.group_size, dev(case.bias), residual, dev(case.gamma),
                                    case.eps, layout=layout, transpose_x2=transpose_x2,
                                    inplace=inplace)
    torch.cuda.synchronize()
    if inplace:
        assert y.data_ptr() == residual.data_ptr()
    return y.cpu(), norm.cpu()


def wq_oracle(case, rows=None):
    """Oracle (mm, y, norm_out) as float64 numpy, optionally for some rows."""
    m, k, n = case.mkn
    x1 = as_f64(case.x1).reshape(m, k)
    res = as_f64(case.residual).reshape(m, n)
    if rows is not None:
        x1, res = x1[rows], res[rows]
    f = lambda t: None if t is None else as_f64(t)
    return oracle.wq_matmul_add_rmsnorm(x1, case.w.numpy(), f(case.scale), f(case.offset),
                                        case.group_size, f(case.bias), res, f(case.gamma),
                                        case.eps)


def check_wq(case, y, norm, rows=None, tol=1e-2):
    m, k, n = case.mkn
    _, oy, on = wq_oracle(case, rows)
    gy = as_f64(y).reshape(m, n)
    gn = as_f64(norm).reshape(m, n)
    if rows is not None:
        gy, gn = gy[rows], gn[rows]
    ey = oracle.rel_err_floor(gy, oy)
    en = oracle.rel_err_floor(gn, on)
    note(f"  {case.name}: y rel err {ey:.3e}, normOut rel err {en:.3e}")
    if ey > tol or en > tol:
        bad = np.argsort(-np.max(np.abs(gn - on) / np.maximum(np.abs(on), 1e-3), axis=1))[:8]
        note(f"  worst rows {bad.tolist()}")
    assert np.all(np.isfinite(gy)) and np.all(np.isfinite(gn))
    assert ey <= tol, f"{case.name}: y rel err {ey}"
    assert en <= tol, f"{case.name}: normOut rel err {en}"
    return ey, en
