"""GPU parity: mx_quant_matmul_inplace_add against the float64 oracle.

The oracle runs on the same E4M3/E2M1 codes and E8M0 scales as the GPU, so
only the float32 accumulation order differs: tolerance 2e-2 (relative, RMS
floored), bit-exact y in the integer-valued case."""
import numpy as np
import pytest
import torch

import bit_quantized_gemm_int4_amd as wq
import oracle
import workloads
from oracle import as_f64
from tests.gpu_util import DEV, note

pytestmark = pytest.mark.gpu


def _run(x1_t, x2_codes, s1, s2, y, group=wq.MX_GROUP_SIZE):
    """x1_t (k, m) uint8, x2_codes (k, n) int codes 0..15, s1 (m, kb), s2 (kb, n)."""
    k, m = x1_t.shape
    n = x2_codes.shape[1]
    x2p = wq.pack_int4(torch.from_numpy(np.ascontiguousarray(x2_codes, dtype=np.int32)).to(DEV),
                       wq.WQ_LAYOUT_GFX950_B)
    yd = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32)).to(DEV)
    wq.mx_matmul_inplace_add(torch.from_numpy(np.ascontiguousarray(x1_t)).to(DEV), x2p,
                             torch.from_numpy(np.ascontiguousarray(s1)).to(DEV),
                             torch.from_numpy(np.ascontiguousarray(s2)).to(DEV), yd, m, k, n,
                             group)
    torch.cuda.synchronize()
    return yd.cpu().numpy().astype(np.float64)


def _codes(rng, k, m, n, s_lo=118, s_hi=134):
    x1 = rng.integers(0, 256, (k, m)).astype(np.uint8)
    x1[(x1 & 0x7F) == 0x7F] = 0
    x2 = rng.integers(0, 16, (k, n)).astype(np.uint8)
    kb = -(-k // 32)
    s1 = rng.integers(s_lo, s_hi, (m, kb)).astype(np.uint8)
    s2 = rng.integers(s_lo, s_hi, (kb, n)).astype(np.uint8)
    return x1, x2, s1, s2


# the last four shapes take the 256 x 256 tile (M, N multiples of 256, K of 128),
# with one, three (odd) and many 128-deep steps
@pytest.mark.parametrize("m,k,n", [(64, 128, 64), (16, 256, 16), (70, 80, 20), (130, 416, 96),
                                   (1, 32, 2), (33, 7, 17), (256, 1024, 256), (256, 128, 512),
                                   (512, 384, 768), (768, 2048, 256)])
def test_random_codes(m, k, n):
    note(f"mx random codes {m}x{k}x{n}")
    rng = np.random.default_rng(m * k + n)
    x1, x2, s1, s2 = _codes(rng, k, m, n)
    y = rng.standard_normal((m, n)).astype(np.float32)
    got = _run(x1, x2, s1, s2, y)
    want = oracle.mx_quant_matmul_inplace_add(x1, x2, s1, s2, y.astype(np.float64))
    err = oracle.rel_err_floor(got, want)
    note(f"  rel err {err:.3e}")
    assert err <= 2e-2
    # tighter check: the scaled MFMA's internal sum is near float32 accuracy
    # (measured up to ~6e-4 when products span ~30 binades, as here; the
    # 256 x 256 tile starts its accumulators at y_old, and each 128-deep
    # block sum is then aligned with a running sum that already holds y_old:
    # measured up to ~1.1e-3)
    assert err <= 2e-3


def test_group_size_zero_same_as_explicit():
    rng = np.random.default_rng(1)
    x1, x2, s1, s2 = _codes(rng, 96, 32, 32)
    y = rng.standard_normal((32, 32)).astype(np.float32)
    note("mx group size 0 vs explicit")
    a = _run(x1, x2, s1, s2, y, wq.MX_GROUP_SIZE)
    b = _run(x1, x2, s1, s2, y, 0)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("k,m,n,hots", [
    (256, 32, 48, [(0, 0), (33, 2), (95, 31), (130, 17), (255, 5)]),
    # 256 x 256 tile: rows in each 64-row wave block, K in both steps
    (256, 256, 256, [(0, 0), (40, 70), (127, 255), (128, 129), (200, 191), (255, 64)]),
])
def test_one_hot_pins_scale_indexing(k, m, n, hots):
    rng = np.random.default_rng(3)
    _, x2, s1, s2 = _codes(rng, k, m, n)
    for kk, mm in hots:
        x1 = np.zeros((k, m), np.uint8)
        x1[kk, mm] = 0x38                                      # E4M3 1.0
        note(f"mx one-hot k={kk} m={mm}")
        got = _run(x1, x2, s1, s2, np.zeros((m, n)))
        want = oracle.mx_quant_matmul_inplace_add(x1, x2, s1, s2, np.zeros((m, n)))
        assert np.array_equal(got, want)


@pytest.mark.parametrize("k,m,n", [(160, 48, 40), (384, 256, 512)])
def test_integer_valued_and_linear(k, m, n):
    # Unit scales and integer-valued elements (E4M3 integers in [-16, 16],
    # E2M1 values in {0, +-1, +-2, +-3, +-4, +-6}): every product and partial
    # sum is an integer below 2^24, so y is exact. (With products spread over
    # many binades the MFMA's internal sum may drop the lowest bits; measured
    # deviations stay near 1e-5 relative, see the random-code test.)
    rng = np.random.default_rng(4 + k)
    ints = oracle.e4m3_encode(np.arange(-16, 17).astype(np.float64))
    x1 = ints[rng.integers(0, ints.size, (k, m))]
    x2 = np.array([0, 2, 4, 5, 6, 7, 10, 12, 13, 14, 15], np.uint8)[rng.integers(0, 11, (k, n))]
    kb = -(-k // 32)
    s1 = np.full((m, kb), 127, np.uint8)
    s2 = np.full((kb, n), 127, np.uint8)
    note(f"mx integer-valued {m}x{k}x{n}")
    y1 = _run(x1, x2, s1, s2, np.zeros((m, n)))
    want = oracle.mx_quant_matmul_inplace_add(x1, x2, s1, s2, np.zeros((m, n)))
    assert np.all(want == np.round(want)) and np.all(np.abs(want) < 2 ** 24)
    assert np.array_equal(y1, want)
    y2 = _run(x1, x2, s1, s2, y1)
    assert np.array_equal(y2, 2 * want)


def test_full_pipeline_from_float_inputs():
    """x (4096, 8192) fp16 with smooth scales -> MX E4M3 (transposed) on the
    GPU; W (8192, 4096) N(0,1) quantized to MXFP4 by the oracle; y += on the
    GPU; every output checked against the oracle on the same codes (the
    oracle runs over 16 row blocks in parallel threads), then a second call
    on the same inputs reproduces the first bit for bit."""
    c = workloads.mx()
    m, k, n = c.mkn
    note(f"mx full pipeline {m}x{k}x{n}")
    x1q, s1 = wq.dynamic_quant(c.x.to(DEV), c.smooth.to(DEV), wq.WQ_FP8_E4M3, 32, True)
    codes_w, s2_t = oracle.dynamic_quant_mx(c.w.numpy().T.astype(np.float64), None, "e2m1")
    x2_codes = codes_w.T.copy()                                # (k, n)
    s2 = s2_t.T.copy()                                         # (kb, n)
    x2p = wq.pack_int4(torch.from_numpy(x2_codes.astype(np.int32)).to(DEV), wq.WQ_LAYOUT_GFX950_B)
    y = c.y.to(DEV)
    s2d = torch.from_numpy(s2).to(DEV)
    wq.mx_matmul_inplace_add(x1q, x2p, s1, s2d, y, m, k, n)
    y2 = c.y.to(DEV)
    wq.mx_matmul_inplace_add(x1q, x2p, s1, s2d, y2, m, k, n)
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "two calls on the same inputs differ"
    x1_codes = x1q.cpu().numpy()                               # (k, m): GPU-quantized, checked
    codes_x, s1_o = oracle.dynamic_quant_mx(as_f64(c.x), as_f64(c.smooth), "e4m3")
    assert np.array_equal(s1.cpu().numpy(), s1_o) and np.array_equal(x1_codes, codes_x.T)
    y0 = as_f64(c.y)
    from concurrent.futures import ThreadPoolExecutor
    blocks = [np.arange(r, r + 256) for r in range(0, m, 256)]
    with ThreadPoolExecutor(max_workers=8) as ex:
        want = np.concatenate(list(ex.map(
            lambda rows: oracle.mx_quant_matmul_inplace_add(codes_x.T[:, rows], x2_codes, s1_o[rows], s2,
                                                            y0[rows]), blocks)))
    got = y.cpu().numpy().astype(np.float64)
    err = oracle.rel_err_floor(got, want)
    note(f"  rel err {err:.3e} over all {m * n} outputs")
    assert err <= 2e-2
    assert np.all(np.isfinite(got))
