"""Pins of the oracle's weight-quantized matmul + AddRmsNorm."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import exact


def _case(k, n, m, gran, group=0, offset=True, bias=True, seed=0):
    rng = np.random.default_rng(seed)
    f16 = lambda a: np.asarray(a, dtype=np.float16).astype(np.float64)
    x1 = f16(rng.standard_normal((m, k)))
    w = rng.integers(-8, 8, size=(k, n))
    shape = {"tensor": (1,), "channel": (n,), "group": (-(-k // max(group, 1)), n)}[gran]
    s = f16(rng.uniform(0.005, 0.02, shape))
    o = f16(rng.uniform(-0.5, 0.5, shape)) if offset else None
    b = f16(rng.normal(0, 0.1, n)) if bias else None
    res = f16(rng.standard_normal((1, m, n)))
    g = f16(rng.uniform(0.9, 1.1, n))
    return x1, w, s, o, group, b, res, g


@pytest.mark.parametrize("seed,gran,group,offset,bias", [
    (10, "tensor", 0, True, True), (11, "channel", 0, True, False), (12, "group", 32, True, True),
    (13, "group", 32, False, True), (14, "group", 64, True, False)])
def test_against_exact_rationals(seed, gran, group, offset, bias):
    args = _case(80, 6, 3, gran, group, offset, bias, seed=seed)
    mm, y, norm = oracle.wq_matmul_add_rmsnorm(*args, eps=1e-6)
    emm, ey, enorm = exact.wq_matmul(*args, eps=1e-6)
    np.testing.assert_allclose(mm, emm, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(y, ey, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(norm, enorm, rtol=1e-12, atol=1e-12)


def test_tiny_workload_rows_against_exact_rationals():
    c = workloads.tiny()
    f = lambda t: None if t is None else t.to(torch.float64).numpy()
    args = (f(c.x1), c.w.numpy(), f(c.scale), f(c.offset), c.group_size, f(c.bias),
            f(c.residual), f(c.gamma))
    mm, y, norm = oracle.wq_matmul_add_rmsnorm(*args, eps=c.eps)
    emm, ey, enorm = exact.wq_matmul(*args, eps=c.eps, rows=[0, 15])
    np.testing.assert_allclose(mm[[0, 15]], emm, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(norm[[0, 15]], enorm, rtol=1e-12, atol=1e-12)
    # magnitude sanity: sigma(mm) near 1 for this workload
    assert 0.5 < np.std(mm) < 2.0


def test_one_hot_rows_select_dequantized_weight_rows():
    k, n, G = 96, 5, 32
    rng = np.random.default_rng(3)
    w = rng.integers(-8, 8, size=(k, n))
    w[40] = 0                                      # a zero row reads back the offset
    s = rng.uniform(0.5, 2, (3, n))
    o = rng.uniform(-1, 1, (3, n))
    x1 = np.eye(k)
    mm, _, _ = oracle.wq_matmul_add_rmsnorm(x1, w, s, o, G, None, np.zeros((k, n)), np.ones(n), 1e-6)
    for i in (0, 31, 32, 40, 63, 64, 95):
        np.testing.assert_array_equal(mm[i], w[i] * s[i // G] + o[i // G])
    np.testing.assert_array_equal(mm[40], o[1])    # offset added after scaling


def test_closed_form_constant_inputs():
    k, n, c, s, o, b = 200, 7, -3, 0.25, 0.5, 1.5
    mm, y, _ = oracle.wq_matmul_add_rmsnorm(
        np.ones((2, k)), np.full((k, n), c), np.array([s]), np.array([o]), 0,
        np.full(n, b), np.zeros((2, n)), np.ones(n), 1e-6)
    assert np.all(mm == k * (c * s + o) + b)


def test_rms_invariant_and_scale_invariance():
    args = list(_case(64, 40, 4, "group", 32, seed=4))
    eps = 1e-6
    _, y, norm = oracle.wq_matmul_add_rmsnorm(*args, eps=eps)
    ms = np.mean(y * y, axis=1)
    rms = np.sqrt(np.mean((norm / args[7]) ** 2, axis=1))
    np.testing.assert_allclose(rms, np.sqrt(ms / (ms + eps)), rtol=1e-12)
    # scaling every additive term by 4 scales y by 4; normOut changes only via eps
    args4 = list(args)
    args4[0] = args[0] * 2
    args4[2] = args[2] * 2
    args4[3] = args[3] * 2
    args4[5] = args[5] * 4
    args4[6] = args[6] * 4
    _, y4, norm4 = oracle.wq_matmul_add_rmsnorm(*args4, eps=0.0)
    _, _, norm0 = oracle.wq_matmul_add_rmsnorm(*args, eps=0.0)
    np.testing.assert_allclose(y4, 4 * y, rtol=1e-12)
    np.testing.assert_allclose(norm4, norm0, rtol=1e-12)


def test_equal_group_scales_equal_per_channel():
    x1, w, s, o, _, b, res, g = _case(128, 9, 3, "channel", seed=5)
    sg = np.tile(s.reshape(1, -1), (4, 1))
    og = np.tile(o.reshape(1, -1), (4, 1))
    a = oracle.wq_matmul_add_rmsnorm(x1, w, s, o, 0, b, res, g, 1e-6)
    bgrp = oracle.wq_matmul_add_rmsnorm(x1, w, sg, og, 32, b, res, g, 1e-6)
    c2d = oracle.wq_matmul_add_rmsnorm(x1, w, s.reshape(1, -1), o.reshape(1, -1), 0, b, res, g, 1e-6)
    for u, v, t in zip(a, bgrp, c2d):
        np.testing.assert_array_equal(u, v)
        np.testing.assert_array_equal(u, t)


def test_integer_valued_case_is_exact():
    # Integer x1, unit scale, zero offset and bias: mm is an exact integer sum.
    rng = np.random.default_rng(6)
    x1 = rng.integers(-2, 3, (5, 256)).astype(np.float64)
    w = rng.integers(-8, 8, (256, 16))
    res = rng.integers(-4, 5, (5, 16)).astype(np.float64)
    mm, y, _ = oracle.wq_matmul_add_rmsnorm(x1, w, np.ones(1), None, 0, None, res, np.ones(16), 1e-6)
    want = (x1.astype(np.int64) @ w) + res.astype(np.int64)
    assert np.array_equal(y, want)


def test_rejects_bad_scale_shapes():
    x1, w, s, o, _, b, res, g = _case(64, 4, 2, "group", 32, seed=7)
    s3 = np.vstack([s, s[:1]])                    # 3 groups for k=64, G=32
    with pytest.raises(ValueError):
        oracle.wq_matmul_add_rmsnorm(x1, w, s3, np.vstack([o, o[:1]]), 32, b, res, g, 1e-6)
    with pytest.raises(ValueError):
        oracle.wq_matmul_add_rmsnorm(x1, w, s[:1, :2], o[:1, :2], 0, b, res, g, 1e-6)
    with pytest.raises(ValueError):
        oracle.wq_matmul_add_rmsnorm(x1, w, s, o[:, :2], 32, b, res, g, 1e-6)
