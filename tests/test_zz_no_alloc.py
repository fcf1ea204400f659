"""The allocation-free fused call (wq_matmul_add_rmsnorm_noalloc): the same
kernels as wq_matmul_add_rmsnorm with the library's per-GPU device array as
their workspace. Checked through the C ABI against the workspace entry point
(bit for bit) and the float64 oracle, on two calls in a row, the second
smaller, so the array is reused with the first call's contents left in it."""
import numpy as np
import pytest
import torch

import bit_quantized_gemm_int4_amd as wq
import oracle
import workloads
from tests.gpu_util import DEV, check_wq, note

pytestmark = pytest.mark.gpu


def _noalloc_fn():
    # the C entry point itself (argument types declared by the binding)
    return wq.lib().wq_matmul_add_rmsnorm_noalloc, wq.WQ_NOALLOC_MAX_WORKSPACE


def _inputs(c):
    m, k, n = c.mkn
    x1 = c.x1.to(DEV).reshape(m, k).contiguous()
    x2 = wq.pack_int4(c.w.to(DEV), wq.WQ_LAYOUT_GFX950_B)
    dev = lambda t: None if t is None else t.to(DEV).contiguous()
    return x1, x2, dev(c.scale), dev(c.offset), dev(c.bias), dev(c.residual).reshape(m, n), dev(c.gamma)


def _run_both(c, fn):
    m, k, n = c.mkn
    x1, x2, sc, of, bi, res, ga = _inputs(c)
    act = wq.act_code(c.act_dtype)
    srows, scols = (sc.shape[0], sc.shape[1]) if sc.dim() == 2 else (1, sc.numel())
    p = lambda t: None if t is None else t.data_ptr()
    s = torch.cuda.current_stream().cuda_stream
    y0, n0 = torch.empty_like(res), torch.empty_like(res)
    wsn = wq.wq_matmul_add_rmsnorm_workspace_size(m, k, n)
    ws = torch.zeros(wsn, dtype=torch.uint8, device=DEV)
    st = wq.lib().wq_matmul_add_rmsnorm(p(x1), m, k, act, p(x2), n, wq.WQ_INT4, wq.WQ_LAYOUT_GFX950_B, 0,
                                        p(sc), srows, scols, p(of), c.group_size, p(bi), p(res), p(ga),
                                        c.eps, p(y0), p(n0), p(ws), wsn, s)
    assert st == wq.WQ_OK
    y1, n1 = torch.full_like(res, 7.0), torch.full_like(res, 7.0)
    st = fn(p(x1), m, k, act, p(x2), n, wq.WQ_INT4, wq.WQ_LAYOUT_GFX950_B, 0, p(sc), srows, scols, p(of),
            c.group_size, p(bi), p(res), p(ga), c.eps, p(y1), p(n1), s)
    assert st == wq.WQ_OK
    torch.cuda.synchronize()
    return y0.cpu(), n0.cpu(), y1.cpu(), n1.cpu()


def test_noalloc_matches_the_workspace_call_twice_in_a_row():
    fn, cap = _noalloc_fn()
    assert cap == 32 << 20
    cases = [
        # prefill tile (pre-pass, MFMA tile, finish): the larger workspace first
        workloads.wq_case("noalloc prefill", 300, 2048, 700, act=torch.bfloat16, w_bits=4,
                          granularity="group", group_size=128, offset_range=(-0.5, 0.5)),
        # then the decode kernel on a smaller problem, over the first call's leftovers
        workloads.wq_case("noalloc decode", 8, 1024, 520, act=torch.float16, w_bits=4,
                          granularity="group", group_size=256, offset_range=(-0.5, 0.5), seed=1),
    ]
    for c in cases:
        note(f"noalloc {c.name} {c.mkn}")
        y0, n0, y1, n1 = _run_both(c, fn)
        assert torch.equal(y0, y1) and torch.equal(n0, n1), c.name
        check_wq(c, y1, n1)


def test_noalloc_rejects_a_problem_beyond_the_array():
    fn, cap = _noalloc_fn()
    m, k, n = 65536, 8192, 8192
    assert wq.wq_matmul_add_rmsnorm_workspace_size(m, k, n) > cap
    F = 0x7F0000000000
    st = fn(F, m, k, wq.WQ_BF16, F + (1 << 32), n, wq.WQ_INT4, wq.WQ_LAYOUT_GFX950_B, 0, F + (2 << 32), 64,
            n, None, 128, None, F + (3 << 32), F + (4 << 32), 1e-6, F + (5 << 32), F + (6 << 32), 0)
    assert st == wq.WQ_ERR_WORKSPACE
