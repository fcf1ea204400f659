"""GPU parity: wq_dynamic_quant against the oracle, bit for bit (codes and
scales)."""
import numpy as np
import pytest
import torch

import bit_quantized_gemm_int4_amd as wq
import oracle
import workloads
from oracle import as_f64
from oracle.quant import encode_quant_output
from tests.gpu_util import DEV, note

pytestmark = pytest.mark.gpu

OUT = {wq.WQ_INT8: "int8", wq.WQ_INT4: "int4", wq.WQ_INT32: "int32"}


def _x(rows, cols, dtype, seed, spread=True):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((rows, cols))
    if spread:
        v = v * np.exp2(rng.integers(-8, 8, (rows, 1)))
    return workloads.cast(v, dtype)


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("y_dtype", [wq.WQ_INT8, wq.WQ_INT4, wq.WQ_INT32])
@pytest.mark.parametrize("rows,cols,smooth", [(7, 64, True), (33, 2056, False), (5, 24, True),
                                              (3, 4104, True), (2, 16, False), (4, 30, True),
                                              (6, 8202, False), (3, 16400, True), (2, 8194, True)])
def test_per_token_bit_exact(dtype, y_dtype, rows, cols, smooth):
    if y_dtype == wq.WQ_INT32 and cols % 8:
        pytest.skip("INT32 needs cols % 8 == 0")
    note(f"quant per-token {dtype} {OUT[y_dtype]} {rows}x{cols} smooth={smooth}")
    x = _x(rows, cols, dtype, rows * cols)
    sm = workloads.cast(np.random.default_rng(1).uniform(0.5, 2.0, cols), dtype) if smooth else None
    y, scale = wq.dynamic_quant(x.to(DEV), None if sm is None else sm.to(DEV), y_dtype)
    q, s = oracle.dynamic_quant_per_token(as_f64(x), None if sm is None else as_f64(sm), OUT[y_dtype])
    assert np.array_equal(scale.cpu().numpy(), s)
    assert np.array_equal(y.cpu().numpy(), encode_quant_output(q, OUT[y_dtype]))


def test_per_token_zero_rows_and_ties():
    note("quant per-token zero row and exact ties")
    x = torch.zeros((3, 16), dtype=torch.float16)
    x[1, :4] = torch.tensor([7.0, 3.5, -0.5, 2.5])
    x[2, :4] = torch.tensor([127.0, 0.5, 1.5, -2.5])
    y4, s4 = wq.dynamic_quant(x.to(DEV), None, wq.WQ_INT4)
    q4 = oracle.unpack_quant_output(y4.cpu().numpy(), "int4", 16)
    assert s4.cpu().tolist()[:2] == [0.0, 1.0]
    assert q4[0].tolist() == [0] * 16 and q4[1, :4].tolist() == [7, 4, 0, 2]
    y8, s8 = wq.dynamic_quant(x.to(DEV), None, wq.WQ_INT8)
    assert s8.cpu()[2].item() == 1.0 and y8.cpu()[2, :4].tolist() == [127, 0, 2, -2]


def _all_values_up_to(dtype, amax_bits):
    """Every finite non-negative value of the 16-bit type up to the one with
    bits amax_bits, both signs, as float32 (exact)."""
    if dtype == torch.float16:
        v = np.arange(0, amax_bits + 1, dtype=np.uint16).view(np.float16).astype(np.float32)
    else:
        v = (np.arange(0, amax_bits + 1, dtype=np.uint32) << 16).view(np.float32)
    return np.concatenate([v, -v[1:]])


# Row scales where v * (1 / scale) and the correctly rounded v / scale round
# to different integers for a few v (found by enumeration), so every such
# quotient is checked against the division the operator defines.
@pytest.mark.parametrize("dtype,amax_bits,y_dtype", [
    (torch.float16, 0x63D0, wq.WQ_INT4),      # amax 1000, dmax 7
    (torch.float16, 0x1F45, wq.WQ_INT8),      # amax 0.0071, dmax 127
    (torch.bfloat16, 0x3C15, wq.WQ_INT8),
    (torch.bfloat16, 0x3C23, wq.WQ_INT4)])
def test_per_token_every_value_near_half_quotients(dtype, amax_bits, y_dtype):
    note(f"quant per-token every value up to 0x{amax_bits:04x} {dtype} {OUT[y_dtype]}")
    v = _all_values_up_to(dtype, amax_bits)
    v = np.concatenate([v, np.zeros((-v.size) % 8, np.float32)])   # 16-byte rows as well
    for x_np in (v[None, :], v[None, : v.size - 6]):
        x = torch.from_numpy(np.ascontiguousarray(x_np)).to(dtype)
        assert np.array_equal(x.float().numpy(), x_np)
        y, scale = wq.dynamic_quant(x.to(DEV), None, y_dtype)
        q, sc = oracle.dynamic_quant_per_token(as_f64(x), None, OUT[y_dtype])
        assert np.array_equal(scale.cpu().numpy(), sc)
        assert np.array_equal(y.cpu().numpy(), encode_quant_output(q, OUT[y_dtype]))


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("fmt,transpose", [("e4m3", False), ("e4m3", True), ("e2m1", False)])
@pytest.mark.parametrize("rows,cols,smooth", [(128, 64, True), (200, 96, True), (37, 80, True),
                                              (5, 8, True), (130, 200, True), (129, 90, True),
                                              (37, 20, False), (260, 136, False)])
def test_mx_bit_exact(dtype, fmt, transpose, rows, cols, smooth):
    note(f"quant mx {fmt} transpose={transpose} {dtype} {rows}x{cols} smooth={smooth}")
    x = _x(rows, cols, dtype, rows + cols)
    sm = workloads.cast(np.random.default_rng(2).uniform(0.5, 2.0, cols), dtype) if smooth else None
    ydt = wq.WQ_FP8_E4M3 if fmt == "e4m3" else wq.WQ_FP4_E2M1
    y, sc = wq.dynamic_quant(x.to(DEV), None if sm is None else sm.to(DEV), ydt, 32, transpose)
    codes, scales = oracle.dynamic_quant_mx(as_f64(x), None if sm is None else as_f64(sm), fmt)
    assert np.array_equal(sc.cpu().numpy(), scales)
    got = y.cpu().numpy()
    if fmt == "e2m1":
        want = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    else:
        want = codes.T if transpose else codes
    assert np.array_equal(got, want)


def test_mx_e4m3_every_tie_and_signed_zero():
    note("quant mx e4m3 all halfway points")
    vals = np.unique(np.abs(oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))))
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float16)          # exact in fp16
    below = np.nextafter(mids, np.float16(0))
    above = np.nextafter(mids, np.float16(1000))
    pool = np.concatenate([mids, below, above, -mids, -above, vals.astype(np.float16),
                           np.array([-0.0, 2.0 ** -12, -(2.0 ** -12)], np.float16)])
    pool = pool.astype(np.float64)
    # every row: 448 first (block scale exactly 1), then 31 pool values
    n = -(-pool.size // 31)
    fill = np.zeros(n * 31)
    fill[:pool.size] = pool
    x = np.zeros((n, 32))
    x[:, 0] = 448.0
    x[:, 1:] = fill.reshape(n, 31)
    xt = workloads.cast(x, torch.float16)
    assert np.array_equal(as_f64(xt), x)
    y, sc = wq.dynamic_quant(xt.to(DEV), None, wq.WQ_FP8_E4M3, 32, False)
    codes, scales = oracle.dynamic_quant_mx(as_f64(xt), None, "e4m3")
    assert np.all(scales == 127)
    assert np.array_equal(sc.cpu().numpy(), scales)
    assert np.array_equal(y.cpu().numpy(), codes)


def test_mx_full_size_transposed():
    c = workloads.mx(draw_w=False)
    m, k, n = c.mkn
    note(f"quant mx full size {m}x{k} e4m3 transposed")
    y, sc = wq.dynamic_quant(c.x.to(DEV), c.smooth.to(DEV), wq.WQ_FP8_E4M3, 32, True)
    codes, scales = oracle.dynamic_quant_mx(as_f64(c.x), as_f64(c.smooth), "e4m3")
    assert np.array_equal(sc.cpu().numpy(), scales)
    assert np.array_equal(y.cpu().numpy(), codes.T)


def test_per_token_full_size():
    c = workloads.mx(draw_w=False)
    m, k, n = c.mkn
    note(f"quant per-token full size {m}x{k} int8")
    y, s = wq.dynamic_quant(c.x.to(DEV), c.smooth.to(DEV), wq.WQ_INT8)
    q, so = oracle.dynamic_quant_per_token(as_f64(c.x), as_f64(c.smooth), "int8")
    assert np.array_equal(s.cpu().numpy(), so)
    assert np.array_equal(y.cpu().numpy(), q.astype(np.int8))


def test_mx_full_size_e2m1():
    # the E2M1 mode (row-major (M, K/2) bytes, 16 x 512 tiles) at the bench size
    c = workloads.mx(draw_w=False)
    m, k, n = c.mkn
    note(f"quant mx full size {m}x{k} e2m1")
    y, sc = wq.dynamic_quant(c.x.to(DEV), c.smooth.to(DEV), wq.WQ_FP4_E2M1, 32, False)
    codes, scales = oracle.dynamic_quant_mx(as_f64(c.x), as_f64(c.smooth), "e2m1")
    assert np.array_equal(sc.cpu().numpy(), scales)
    c8 = np.asarray(codes, dtype=np.int64)
    assert np.array_equal(y.cpu().numpy(), (c8[:, 0::2] | (c8[:, 1::2] << 4)).astype(np.uint8))


def test_per_token_int4_full_size():
    # the INT4 output that feeds the A4W4 GEMM, at the bench size
    c = workloads.mx(draw_w=False)
    m, k, n = c.mkn
    note(f"quant per-token full size {m}x{k} int4")
    y, s = wq.dynamic_quant(c.x.to(DEV), c.smooth.to(DEV), wq.WQ_INT4)
    q, so = oracle.dynamic_quant_per_token(as_f64(c.x), as_f64(c.smooth), "int4")
    assert np.array_equal(s.cpu().numpy(), so)
    assert np.array_equal(y.cpu().numpy(), oracle.encode_quant_output(q, "int4"))
