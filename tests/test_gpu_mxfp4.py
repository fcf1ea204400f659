"""GPU parity: the FLOAT -> E2M1 pack (wq_pack_fp4, bit for bit) and the
MXFP4 x MXFP4 matmul with in-place add (mx_fp4_quant_matmul_inplace_add)
against the oracle.

The oracle runs on the same E2M1 codes and E8M0 scales as the GPU; every
slice sum is exact on both sides, so only the float32 accumulation order
differs: tolerance 2e-2 (relative, RMS floored, as for the E4M3 path), and
bit-exact y where every partial sum is a float32 integer."""
import numpy as np
import pytest
import torch

import bit_quantized_gemm_int4_amd as wq
import oracle
import workloads
from oracle import as_f64
from tests.gpu_util import DEV, note

pytestmark = pytest.mark.gpu

B, ND = wq.WQ_LAYOUT_GFX950_B, wq.WQ_LAYOUT_ND


def _pack_rows(codes):
    """(m, k) E2M1 codes -> (m, k/2) bytes, even k in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def _run(x1_codes, x2_codes, s1, s2, y):
    m, k = x1_codes.shape
    n = x2_codes.shape[1]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    x2p = wq.pack_int4(t(x2_codes.astype(np.int32)), B)
    yd = t(y.astype(np.float32))
    wq.mxfp4_matmul_inplace_add(t(_pack_rows(x1_codes)), x2p, t(s1), t(s2), yd, m, k, n)
    torch.cuda.synchronize()
    return yd.cpu().numpy().astype(np.float64)


def _codes(rng, m, k, n, s_lo=118, s_hi=134):
    x1 = rng.integers(0, 16, (m, k)).astype(np.uint8)
    x2 = rng.integers(0, 16, (k, n)).astype(np.uint8)
    kb = k // 32
    s1 = rng.integers(s_lo, s_hi, (m, kb)).astype(np.uint8)
    s2 = rng.integers(s_lo, s_hi, (kb, n)).astype(np.uint8)
    return x1, x2, s1, s2


@pytest.mark.parametrize("m,k,n", [(256, 128, 256), (512, 1024, 768), (300, 416, 270), (1, 32, 2),
                                   (64, 96, 48), (257, 160, 513), (1000, 2048, 1000), (33, 4096, 17)])
def test_random_codes(m, k, n):
    note(f"mxfp4 random codes {m}x{k}x{n}")
    rng = np.random.default_rng(m * 7 + k + 3 * n)
    x1, x2, s1, s2 = _codes(rng, m, k, n)
    y = rng.standard_normal((m, n)).astype(np.float32)
    got = _run(x1, x2, s1, s2, y)
    want = oracle.mxfp4_quant_matmul_inplace_add(x1, x2, s1, s2, y.astype(np.float64))
    err = oracle.rel_err_floor(got, want)
    note(f"  rel err {err:.3e}")
    assert np.all(np.isfinite(got))
    assert err <= 2e-2


def test_integer_valued_case_is_bit_exact():
    # unit scales and E2M1 values {0, +-1, +-2, +-3, +-4, +-6}: every partial
    # sum is an integer far below 2^24, so both sides are exact
    note("mxfp4 integer-valued 384x512x320")
    rng = np.random.default_rng(7)
    m, k, n = 384, 512, 320
    ints = np.array([0, 2, 4, 5, 6, 7, 10, 12, 13, 14, 15], np.uint8)
    x1 = rng.choice(ints, (m, k))
    x2 = rng.choice(ints, (k, n))
    s1 = np.full((m, k // 32), 127, np.uint8)
    s2 = np.full((k // 32, n), 127, np.uint8)
    y = rng.integers(-50, 50, (m, n)).astype(np.float32)
    got = _run(x1, x2, s1, s2, y)
    want = oracle.mxfp4_quant_matmul_inplace_add(x1, x2, s1, s2, y.astype(np.float64))
    assert np.array_equal(got, want)


def test_scale_indexing_one_hot_rows():
    # one nonzero x1 code per row, at a different slice per row: each output
    # row is that slice's scaled weight row
    note("mxfp4 one-hot rows")
    rng = np.random.default_rng(8)
    m, k, n = 64, 256, 96
    x1 = np.zeros((m, k), np.uint8)
    for r in range(m):
        x1[r, (37 * r) % k] = 2                          # 1.0
    _, x2, s1, s2 = _codes(rng, m, k, n, 110, 140)
    got = _run(x1, x2, s1, s2, np.zeros((m, n), np.float32))
    want = oracle.mxfp4_quant_matmul_inplace_add(x1, x2, s1, s2, np.zeros((m, n)))
    assert np.array_equal(got, want)


def test_full_size_sampled_rows():
    note("mxfp4 4096x8192x4096 (sampled rows)")
    rng = np.random.default_rng(9)
    m, k, n = 4096, 8192, 4096
    x1, x2, s1, s2 = _codes(rng, m, k, n)
    y = rng.standard_normal((m, n)).astype(np.float32)
    got = _run(x1, x2, s1, s2, y)
    rows = rng.choice(m, 24, replace=False)
    want = oracle.mxfp4_quant_matmul_inplace_add(x1[rows], x2, s1[rows], s2, y[rows].astype(np.float64))
    err = oracle.rel_err_floor(got[rows], want)
    note(f"  rel err {err:.3e}")
    assert err <= 2e-2


@pytest.mark.parametrize("k,n,layout,transpose", [(128, 256, B, False), (200, 530, B, False),
                                                  (1031, 300, B, True), (256, 64, ND, False),
                                                  (96, 34, ND, True), (4096, 4096, B, False)])
def test_pack_fp4_bit_exact(k, n, layout, transpose):
    note(f"pack fp4 {k}x{n} layout={layout} transpose={transpose}")
    rng = np.random.default_rng(k + n)
    w = (rng.standard_normal((n, k) if transpose else (k, n)) * 3).astype(np.float32)
    # the E2M1 ties, saturation and signed zeros somewhere in every case
    special = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -2.5, 6.5, 1e30, -np.inf, -0.0, 0.0],
                       np.float32)
    w.reshape(-1)[:special.size] = special
    got = wq.pack_fp4(torch.from_numpy(w).to(DEV), layout, transpose)
    torch.cuda.synchronize()
    want = oracle.pack_float_e2m1(w, "gfx950b" if layout == B else "nd", transpose)
    assert np.array_equal(got.cpu().numpy().reshape(-1), want.reshape(-1))


def test_quant_pack_gemm_chain():
    # E2M1 block-32 quant of the activations (wq_dynamic_quant), the weight
    # MX-quantized along K by the oracle and packed from its E2M1 values by
    # wq_pack_fp4, then the FP4 GEMM; against the oracle on the same codes
    note("mxfp4 chain: quant E2M1 -> pack fp4 -> GEMM (512x1024x384)")
    c = workloads.mx(512, 1024, 384, seed=3)
    m, k, n = c.mkn
    q, s1 = wq.dynamic_quant(c.x.to(DEV), c.smooth.to(DEV), wq.WQ_FP4_E2M1, 32, False)
    oq, os1 = oracle.dynamic_quant_mx(as_f64(c.x), as_f64(c.smooth), "e2m1")
    assert np.array_equal(s1.cpu().numpy(), os1)
    assert np.array_equal(q.cpu().numpy(), _pack_rows(oq))
    codes_w, s2t = oracle.dynamic_quant_mx(c.w.numpy().T.astype(np.float64), None, "e2m1")
    w_vals = np.ascontiguousarray(oracle.e2m1_decode(codes_w.T), dtype=np.float32)  # (k, n)
    x2p = wq.pack_fp4(torch.from_numpy(w_vals).to(DEV), B)
    s2 = np.ascontiguousarray(s2t.T)
    y = c.y.to(DEV).clone()
    wq.mxfp4_matmul_inplace_add(q, x2p, s1, torch.from_numpy(s2).to(DEV), y, m, k, n)
    torch.cuda.synchronize()
    want = oracle.mxfp4_quant_matmul_inplace_add(oq, codes_w.T, os1, s2, as_f64(c.y))
    err = oracle.rel_err_floor(y.cpu().numpy().astype(np.float64), want)
    note(f"  rel err {err:.3e}")
    assert err <= 2e-2
