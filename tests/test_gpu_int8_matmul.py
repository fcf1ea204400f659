"""GPU parity: wq_quant_matmul_inplace_add (INT8 x INT8, exact int32 sums,
float32 epilogue) against the oracle, bit for bit: both sides take the same
float32 roundings in the same order."""
import numpy as np
import pytest
import torch

import bit_quantized_gemm_int4_amd as wq
import oracle
from oracle import as_f64
from tests.gpu_util import DEV, note

pytestmark = pytest.mark.gpu


def _inputs(m, k, n, seed, lo=-128):
    rng = np.random.default_rng(seed)
    x1 = rng.integers(lo, 128, size=(m, k), dtype=np.int8)
    x2t = rng.integers(lo, 128, size=(n, k), dtype=np.int8)
    s1 = rng.uniform(1e-4, 2e-2, size=m).astype(np.float32)
    s2 = rng.uniform(1e-4, 2e-2, size=n).astype(np.float32)
    y = rng.normal(size=(m, n)).astype(np.float32)
    return x1, x2t, s1, s2, y


def _gpu(x1, x2t, s1, s2, y):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    yd = t(y)
    wq.quant_matmul_inplace_add(t(x1), t(x2t), t(s1), t(s2), yd)
    torch.cuda.synchronize()
    return yd.cpu().numpy()


@pytest.mark.parametrize("m,k,n", [(1, 16, 1), (17, 16, 33), (256, 128, 256), (300, 48, 270),
                                   (513, 272, 1000), (64, 4096, 96), (257, 1040, 513)])
def test_int8_matmul_bit_exact(m, k, n):
    note(f"int8 matmul {m}x{k}x{n}")
    x1, x2t, s1, s2, y = _inputs(m, k, n, m + 3 * k + 7 * n)
    got = _gpu(x1, x2t, s1, s2, y)
    want = oracle.quant_matmul_inplace_add_int8(x1, x2t, s1, s2, y)
    assert np.array_equal(got, want)


def test_int8_extremes_and_zero_scales():
    # all -128: the largest sums; zero scales for some rows and columns leave y
    note("int8 matmul extremes")
    m, k, n = 40, 8192, 72
    x1 = np.full((m, k), -128, np.int8)
    x2t = np.full((n, k), -128, np.int8)
    s1 = np.full(m, 2.0 ** -20, np.float32)
    s2 = np.full(n, 2.0 ** -3, np.float32)
    s1[5] = 0
    s2[7] = 0
    y = np.random.default_rng(9).normal(size=(m, n)).astype(np.float32)
    got = _gpu(x1, x2t, s1, s2, y)
    assert np.array_equal(got, oracle.quant_matmul_inplace_add_int8(x1, x2t, s1, s2, y))
    assert np.array_equal(got[5], y[5]) and np.array_equal(got[:, 7], y[:, 7])


def test_dynamic_quant_feeds_int8_matmul():
    # the A8W8 chain: per-token INT8 DynamicQuant of x, then the INT8 matmul
    note("dynamic quant -> int8 matmul chain")
    rng = np.random.default_rng(11)
    m, k, n = 96, 512, 160
    x = torch.from_numpy(rng.normal(size=(m, k))).to(torch.float16)
    xq, xs = wq.dynamic_quant(x.to(DEV), None, wq.WQ_INT8)
    q, s = oracle.dynamic_quant_per_token(as_f64(x), None, "int8")
    assert np.array_equal(xq.cpu().numpy(), q.astype(np.int8)) and np.array_equal(xs.cpu().numpy(), s)
    w = rng.integers(-127, 128, size=(n, k), dtype=np.int8)
    ws = rng.uniform(1e-3, 1e-2, size=n).astype(np.float32)
    y = rng.normal(size=(m, n)).astype(np.float32)
    yd = torch.from_numpy(y).to(DEV)
    wq.quant_matmul_inplace_add(xq, torch.from_numpy(w).to(DEV), xs, torch.from_numpy(ws).to(DEV), yd)
    torch.cuda.synchronize()
    want = oracle.quant_matmul_inplace_add_int8(q, w, s, ws, y)
    assert np.array_equal(yd.cpu().numpy(), want)
    # and it stays within the quantizer's bound of x @ (w * ws).T + y: each
    # |x - q * s| <= s / 2, so |error[m, n]| <= s[m] / 2 * sum_k |w[n, k] * ws[n]|
    # (plus float32 rounding of the epilogue)
    exact = as_f64(x) @ (w.astype(np.float64) * ws[:, None]).T + y
    bound = 0.5 * s.astype(np.float64)[:, None] * (np.abs(w.astype(np.float64)) * ws[:, None]).sum(1)[None, :]
    err = np.abs(yd.cpu().numpy().astype(np.float64) - exact)
    assert np.all(err <= bound * (1 + 1e-5) + 1e-5 * np.abs(exact) + 1e-6)


def test_int8_matmul_full_size_sampled_rows():
    # the bench shape (4096 x 8192 x 4096): every output of 48 rows spread
    # over the tiles, bit for bit
    note("int8 matmul full size 4096x8192x4096 (sampled rows)")
    m, k, n = 4096, 8192, 4096
    x1, x2t, s1, s2, y = _inputs(m, k, n, 21)
    got = _gpu(x1, x2t, s1, s2, y)
    rows = np.random.default_rng(22).choice(m, size=48, replace=False)
    want = oracle.quant_matmul_inplace_add_int8(x1[rows], x2t, s1[rows], s2, y[rows])
    assert np.array_equal(got[rows], want)
