"""GPU parity: wq_quant_matmul_inplace_add_w4 (INT8 or INT4 x packed INT4, exact int32
sums, float32 epilogue) against the oracle, bit for bit: both sides take the
same float32 roundings in the same order. The weight reaches the GPU as
INT32 codes packed on the device by wq_pack_int4 (GFX950_B)."""
import numpy as np
import pytest
import torch

import bit_quantized_gemm_int4_amd as wq
import oracle
from oracle import as_f64
from tests.gpu_util import DEV, note

pytestmark = pytest.mark.gpu


def _inputs(m, k, n, seed):
    rng = np.random.default_rng(seed)
    x1 = rng.integers(-128, 128, size=(m, k), dtype=np.int8)
    codes = rng.integers(-8, 8, size=(k, n)).astype(np.int32)
    s1 = rng.uniform(1e-4, 2e-2, size=m).astype(np.float32)
    s2 = rng.uniform(1e-4, 2e-2, size=n).astype(np.float32)
    y = rng.normal(size=(m, n)).astype(np.float32)
    return x1, codes, s1, s2, y


def _gpu(x1, codes, s1, s2, y):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    n = codes.shape[1]
    x2 = wq.pack_int4(t(codes), wq.WQ_LAYOUT_GFX950_B)
    yd = t(y)
    wq.quant_matmul_inplace_add_w4(t(x1), x2, n, t(s1), t(s2), yd)
    torch.cuda.synchronize()
    return yd.cpu().numpy()


@pytest.mark.parametrize("m,k,n", [(1, 16, 1), (17, 16, 33), (256, 128, 256), (300, 48, 270),
                                   (513, 272, 1000), (64, 4096, 96), (257, 1040, 513),
                                   (512, 2048, 512), (33, 208, 17)])
def test_a8w4_bit_exact(m, k, n):
    note(f"a8w4 matmul {m}x{k}x{n}")
    x1, codes, s1, s2, y = _inputs(m, k, n, m + 5 * k + 3 * n)
    got = _gpu(x1, codes, s1, s2, y)
    want = oracle.quant_matmul_inplace_add_w4(x1, codes, s1, s2, y)
    assert np.array_equal(got, want)


def test_a8w4_extremes_and_zero_scales():
    # x1 all -128 and every code -8 over k = 65520: 16 times the sum is
    # 1,073,479,680, the largest the accumulator meets; zero scales leave y
    note("a8w4 extremes k=65520")
    m, k, n = 16, 65520, 20
    x1 = np.full((m, k), -128, np.int8)
    codes = np.full((k, n), -8, np.int32)
    codes[:, 3] = 7
    s1 = np.full(m, 2.0 ** -20, np.float32)
    s2 = np.full(n, 2.0 ** -3, np.float32)
    s1[5] = 0
    s2[7] = 0
    y = np.random.default_rng(9).normal(size=(m, n)).astype(np.float32)
    got = _gpu(x1, codes, s1, s2, y)
    assert np.array_equal(got, oracle.quant_matmul_inplace_add_w4(x1, codes, s1, s2, y))
    assert np.array_equal(got[5], y[5]) and np.array_equal(got[:, 7], y[:, 7])


def test_dynamic_quant_feeds_a8w4():
    # the A8W4 chain: per-token INT8 DynamicQuant of x, then the INT8 x INT4
    # matmul on a weight packed on the device
    note("dynamic quant -> a8w4 matmul chain")
    rng = np.random.default_rng(12)
    m, k, n = 96, 512, 160
    x = torch.from_numpy(rng.normal(size=(m, k))).to(torch.float16)
    xq, xs = wq.dynamic_quant(x.to(DEV), None, wq.WQ_INT8)
    q, s = oracle.dynamic_quant_per_token(as_f64(x), None, "int8")
    assert np.array_equal(xq.cpu().numpy(), q.astype(np.int8)) and np.array_equal(xs.cpu().numpy(), s)
    codes = rng.integers(-8, 8, size=(k, n)).astype(np.int32)
    ws = rng.uniform(1e-3, 1e-2, size=n).astype(np.float32)
    y = rng.normal(size=(m, n)).astype(np.float32)
    yd = torch.from_numpy(y).to(DEV)
    x2 = wq.pack_int4(torch.from_numpy(codes).to(DEV), wq.WQ_LAYOUT_GFX950_B)
    wq.quant_matmul_inplace_add_w4(xq, x2, n, xs, torch.from_numpy(ws).to(DEV), yd)
    torch.cuda.synchronize()
    assert np.array_equal(yd.cpu().numpy(), oracle.quant_matmul_inplace_add_w4(q, codes, s, ws, y))


def test_a8w4_full_size_sampled_rows():
    # the bench shape (4096 x 8192 x 4096): every output of 48 rows spread
    # over the tiles, bit for bit
    note("a8w4 matmul full size 4096x8192x4096 (sampled rows)")
    m, k, n = 4096, 8192, 4096
    x1, codes, s1, s2, y = _inputs(m, k, n, 23)
    got = _gpu(x1, codes, s1, s2, y)
    rows = np.random.default_rng(24).choice(m, size=48, replace=False)
    want = oracle.quant_matmul_inplace_add_w4(x1[rows], codes, s1[rows], s2, y[rows])
    assert np.array_equal(got[rows], want)


# ---- INT4 activations (A4W4): x1 as the per-token quant's INT4 output ----

def _pack_rows(codes):
    """(m, k) INT4 codes -> (m, k/2) bytes, even k in the low nibble."""
    c = np.asarray(codes, dtype=np.int64) & 0xF
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def _gpu_a4(a_codes, codes, s1, s2, y):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    n = codes.shape[1]
    x2 = wq.pack_int4(t(codes), wq.WQ_LAYOUT_GFX950_B)
    yd = t(y)
    wq.quant_matmul_inplace_add_w4(t(_pack_rows(a_codes)), x2, n, t(s1), t(s2), yd, x1_int4=True)
    torch.cuda.synchronize()
    return yd.cpu().numpy()


@pytest.mark.parametrize("m,k,n", [(1, 32, 1), (17, 32, 33), (256, 128, 256), (300, 96, 270),
                                   (513, 288, 1000), (64, 4096, 96), (257, 1056, 513)])
def test_a4w4_bit_exact(m, k, n):
    note(f"a4w4 matmul {m}x{k}x{n}")
    rng = np.random.default_rng(m + 7 * k + n)
    a = rng.integers(-8, 8, size=(m, k))
    codes = rng.integers(-8, 8, size=(k, n)).astype(np.int32)
    s1 = rng.uniform(1e-3, 2e-1, size=m).astype(np.float32)
    s2 = rng.uniform(1e-3, 2e-2, size=n).astype(np.float32)
    y = rng.normal(size=(m, n)).astype(np.float32)
    got = _gpu_a4(a, codes, s1, s2, y)
    assert np.array_equal(got, oracle.quant_matmul_inplace_add_w4(a, codes, s1, s2, y))


def test_a4w4_extremes():
    # every code -8 on both sides over k = 65504: 256 times the sum is
    # 1,073,807,360, the largest the accumulator meets
    note("a4w4 extremes k=65504")
    m, k, n = 16, 65504, 20
    a = np.full((m, k), -8)
    a[3] = 7
    codes = np.full((k, n), -8, np.int32)
    s1 = np.full(m, 2.0 ** -10, np.float32)
    s2 = np.full(n, 2.0 ** -3, np.float32)
    y = np.random.default_rng(10).normal(size=(m, n)).astype(np.float32)
    got = _gpu_a4(a, codes, s1, s2, y)
    assert np.array_equal(got, oracle.quant_matmul_inplace_add_w4(a, codes, s1, s2, y))


def test_dynamic_quant_int4_feeds_a4w4():
    # the A4W4 chain: per-token INT4 DynamicQuant of x (its stored output,
    # two codes per byte), then the INT4 x INT4 matmul
    note("dynamic quant int4 -> a4w4 matmul chain")
    rng = np.random.default_rng(13)
    m, k, n = 96, 512, 160
    x = torch.from_numpy(rng.normal(size=(m, k))).to(torch.float16)
    xq, xs = wq.dynamic_quant(x.to(DEV), None, wq.WQ_INT4)
    q, s = oracle.dynamic_quant_per_token(as_f64(x), None, "int4")
    assert np.array_equal(xq.cpu().numpy(), oracle.encode_quant_output(q, "int4"))
    assert np.array_equal(xs.cpu().numpy(), s)
    codes = rng.integers(-8, 8, size=(k, n)).astype(np.int32)
    ws = rng.uniform(1e-3, 1e-2, size=n).astype(np.float32)
    y = rng.normal(size=(m, n)).astype(np.float32)
    yd = torch.from_numpy(y).to(DEV)
    x2 = wq.pack_int4(torch.from_numpy(codes).to(DEV), wq.WQ_LAYOUT_GFX950_B)
    wq.quant_matmul_inplace_add_w4(xq, x2, n, xs, torch.from_numpy(ws).to(DEV), yd, x1_int4=True)
    torch.cuda.synchronize()
    assert np.array_equal(yd.cpu().numpy(), oracle.quant_matmul_inplace_add_w4(q, codes, s, ws, y))


def test_a4w4_full_size_sampled_rows():
    # the bench shape (4096 x 8192 x 4096) with INT4 activations: every output
    # of 48 rows spread over the tiles, bit for bit
    note("a4w4 matmul full size 4096x8192x4096 (sampled rows)")
    m, k, n = 4096, 8192, 4096
    rng = np.random.default_rng(25)
    a = rng.integers(-8, 8, size=(m, k))
    codes = rng.integers(-8, 8, size=(k, n)).astype(np.int32)
    s1 = rng.uniform(1e-3, 2e-1, size=m).astype(np.float32)
    s2 = rng.uniform(1e-3, 2e-2, size=n).astype(np.float32)
    y = rng.normal(size=(m, n)).astype(np.float32)
    got = _gpu_a4(a, codes, s1, s2, y)
    rows = rng.choice(m, size=48, replace=False)
    want = oracle.quant_matmul_inplace_add_w4(a[rows], codes, s1[rows], s2, y[rows])
    assert np.array_equal(got[rows], want)


def test_dynamic_quant_int32_feeds_a4w4():
    # the INT32 output (eight nibbles per word, lowest first) holds the same
    # bytes as the INT4 output, so it feeds the INT4-activation GEMM as is
    note("dynamic quant int32 -> a4w4 matmul chain")
    rng = np.random.default_rng(14)
    m, k, n = 64, 256, 96
    x = torch.from_numpy(rng.normal(size=(m, k))).to(torch.bfloat16)
    x32, xs = wq.dynamic_quant(x.to(DEV), None, wq.WQ_INT32)
    x4, xs4 = wq.dynamic_quant(x.to(DEV), None, wq.WQ_INT4)
    assert torch.equal(x32.view(torch.uint8).reshape(m, k // 2), x4) and torch.equal(xs, xs4)
    q, s = oracle.dynamic_quant_per_token(as_f64(x), None, "int32")
    codes = rng.integers(-8, 8, size=(k, n)).astype(np.int32)
    ws = rng.uniform(1e-3, 1e-2, size=n).astype(np.float32)
    y = rng.normal(size=(m, n)).astype(np.float32)
    yd = torch.from_numpy(y).to(DEV)
    x2 = wq.pack_int4(torch.from_numpy(codes).to(DEV), wq.WQ_LAYOUT_GFX950_B)
    wq.quant_matmul_inplace_add_w4(x32.view(torch.uint8).reshape(m, k // 2), x2, n, xs,
                                   torch.from_numpy(ws).to(DEV), yd, x1_int4=True)
    torch.cuda.synchronize()
    assert np.array_equal(yd.cpu().numpy(), oracle.quant_matmul_inplace_add_w4(q, codes, s, ws, y))
