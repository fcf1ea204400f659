"""Guard bands: every output of a ragged launch is written inside its bounds.

Each output (and each workspace) is placed inside a larger buffer whose
leading and trailing 256 bytes hold a canary pattern; after the call the
canaries must be untouched. In-place outputs (y of the in-place add, y
written into residual's memory, which the aclnnWeightQuantMatmulAllReduceAddRmsNorm
page's in-place variant allows) start from their input values. Shapes are
ragged on purpose: rows past a tile, columns past a 16- or 64-column tile, K
not a multiple of the block. The values themselves are checked against the
oracle by the other GPU tests; the last test here checks the one shape class
those do not reach (more rows than one launch covers) on sampled rows."""
import numpy as np
import pytest
import torch

import bit_quantized_gemm_int4_amd as wq
import oracle
import workloads
from oracle import as_f64
from tests.gpu_util import DEV, note

pytestmark = pytest.mark.gpu

PAD = 256
CANARY = 0xA5


class Guarded:
    """A device region of ``nbytes`` between two canary bands."""

    def __init__(self, nbytes: int, init: torch.Tensor = None):
        self.nbytes = nbytes
        self.buf = torch.full((nbytes + 2 * PAD,), CANARY, dtype=torch.uint8, device=DEV)
        if init is not None:
            src = init.contiguous().view(torch.uint8).reshape(-1)
            assert src.numel() == nbytes
            self.buf[PAD:PAD + nbytes].copy_(src)

    @property
    def ptr(self) -> int:
        return self.buf.data_ptr() + PAD

    def body(self, dtype) -> torch.Tensor:
        return self.buf[PAD:PAD + self.nbytes].view(dtype)

    def check(self, what: str):
        torch.cuda.synchronize()
        head = self.buf[:PAD].cpu().numpy()
        tail = self.buf[PAD + self.nbytes:].cpu().numpy()
        assert np.all(head == CANARY), f"{what}: bytes before the output written"
        assert np.all(tail == CANARY), f"{what}: bytes after the output written"


WQ_CASES = [  # m, k, n, act, granularity, group, layout, transpose, inplace
    (17, 256, 40, torch.float16, "group", 32, wq.WQ_LAYOUT_GFX950_B, False, False),   # decode kernel, group 32
    (5, 384, 130, torch.bfloat16, "group", 128, wq.WQ_LAYOUT_GFX950_B, False, True),  # decode kernel
    (21, 512, 200, torch.float16, "channel", 0, wq.WQ_LAYOUT_GFX950_B, False, False), # decode, 2 launches
    (130, 512, 520, torch.bfloat16, "group", 128, wq.WQ_LAYOUT_GFX950_B, False, True),  # prefill, masked strip
    (33, 256, 90, torch.bfloat16, "group", 64, wq.WQ_LAYOUT_ND, False, False),        # ND, n % 4 != 0: generic
    (70, 256, 48, torch.float16, "channel", 0, wq.WQ_LAYOUT_ND, True, False),          # INT4 ND transposed
    (70, 336, 132, torch.bfloat16, "group", 32, wq.WQ_LAYOUT_GFX950_B, False, True),   # INT8 tile, INT4 weight
    (70, 512, 132, torch.float16, "group", 64, wq.WQ_LAYOUT_ND, False, True),          # INT8 tile, INT4 ND
    (36, 2048, 132, torch.bfloat16, "group", 32, wq.WQ_LAYOUT_GFX950_B, False, True),  # INT8 tile, K split 4
    (36, 2048, 70, torch.float16, "group", 64, wq.WQ_LAYOUT_ND, True, True),           # K split 4, n % 4 != 0
]


@pytest.mark.parametrize("case", WQ_CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}-{c[4]}{c[5]}-l{c[6]}" for c in WQ_CASES])
def test_wq_matmul_add_rmsnorm_guards(case):
    m, k, n, act, gran, G, layout, tr, inplace = case
    c = workloads.wq_case(f"guard {m}x{k}x{n}", m, k, n, act=act, w_bits=4, granularity=gran,
                          group_size=G, offset_range=(-0.5, 0.5))
    note(f"guards wq {case}")
    w = c.w.to(DEV)
    x2 = wq.pack_int4(w.t().contiguous() if tr else w, layout)
    x1 = c.x1.to(DEV).reshape(m, k)
    sc, of, bi, ga = (t.to(DEV) for t in (c.scale, c.offset, c.bias, c.gamma))
    srows, scols = (sc.shape[0], sc.shape[1]) if sc.dim() == 2 else (1, sc.numel())
    res = Guarded(m * n * 2, c.residual.to(DEV).reshape(m, n))
    y = res if inplace else Guarded(m * n * 2)
    norm = Guarded(m * n * 2)
    wsn = wq.wq_matmul_add_rmsnorm_workspace_size(m, k, n)
    ws = Guarded(wsn)
    wq.wq_matmul_add_rmsnorm(x1, m, k, wq.act_code(act), x2, n, wq.WQ_INT4, layout, tr, sc, srows,
                             scols, of, G, bi, res.ptr, ga, c.eps, y.ptr, norm.ptr, ws.ptr, wsn)
    for g, what in ((y, "y"), (norm, "normOut"), (ws, "workspace"), (res, "residual")):
        g.check(what)
    assert not torch.all(norm.body(torch.uint8) == CANARY)


@pytest.mark.parametrize("y_dtype,cols", [(wq.WQ_INT8, 136), (wq.WQ_INT4, 136), (wq.WQ_INT32, 136),
                                          (wq.WQ_INT8, 37)])
def test_per_token_quant_guards(y_dtype, cols):
    rows = 33
    g = torch.Generator().manual_seed(5)
    x = torch.randn(rows, cols, generator=g).to(torch.float16).to(DEV)
    sm = (torch.rand(cols, generator=g) + 0.5).to(torch.float16).to(DEV)
    note(f"guards per-token quant dtype={y_dtype} cols={cols}")
    ybytes = {wq.WQ_INT8: rows * cols, wq.WQ_INT4: rows * cols // 2, wq.WQ_INT32: rows * cols // 2}[y_dtype]
    y, s = Guarded(ybytes), Guarded(rows * 4)
    wq.wq_dynamic_quant(x, wq.WQ_F16, rows, cols, sm, y_dtype, 0, 0, y.ptr, s.ptr)
    y.check("q")
    s.check("scale")


@pytest.mark.parametrize("y_dtype,transpose,rows,cols", [(wq.WQ_FP8_E4M3, 1, 130, 80),
                                                         (wq.WQ_FP8_E4M3, 0, 17, 200),
                                                         (wq.WQ_FP4_E2M1, 0, 33, 80)])
def test_mx_quant_guards(y_dtype, transpose, rows, cols):
    g = torch.Generator().manual_seed(6)
    x = torch.randn(rows, cols, generator=g).to(torch.bfloat16).to(DEV)
    note(f"guards mx quant dtype={y_dtype} transpose={transpose} {rows}x{cols}")
    ybytes = rows * cols if y_dtype == wq.WQ_FP8_E4M3 else rows * cols // 2
    y, s = Guarded(ybytes), Guarded(rows * ((cols + 31) // 32))
    wq.wq_dynamic_quant(x, wq.WQ_BF16, rows, cols, None, y_dtype, 32, transpose, y.ptr, s.ptr)
    y.check("q")
    s.check("scale")


def _e4m3_codes(shape, gen):
    c = torch.randint(0, 256, shape, generator=gen, dtype=torch.int32)
    c[(c & 0x7F) == 0x7F] = 0x38                     # no NaN codes
    return c.to(torch.uint8)


@pytest.mark.parametrize("m,k,n", [(80, 80, 48), (256, 128, 256), (80, 80, 50), (272, 200, 263)])
def test_mx_gemm_guards(m, k, n):
    gen = torch.Generator().manual_seed(7)
    kb = (k + 31) // 32
    x1 = _e4m3_codes((k, m), gen).to(DEV)
    x2 = wq.pack_int4(torch.randint(0, 16, (k, n), generator=gen, dtype=torch.int32).to(DEV))
    s1 = torch.randint(120, 135, (m, kb), generator=gen, dtype=torch.int32).to(torch.uint8).to(DEV)
    s2 = torch.randint(120, 135, (kb, n), generator=gen, dtype=torch.int32).to(torch.uint8).to(DEV)
    y = Guarded(m * n * 4, torch.randn(m, n, generator=gen).to(DEV))
    note(f"guards mx gemm {m}x{k}x{n}")
    wq.mx_quant_matmul_inplace_add(x1, x2, wq.WQ_LAYOUT_GFX950_B, s1, s2, m, k, n, 1, 0,
                                   wq.MX_GROUP_SIZE, y.ptr)
    y.check("y")


@pytest.mark.parametrize("kind", ["int8", "a8w4", "a4w4", "mxfp4"])
def test_inplace_gemm_guards(kind):
    gen = torch.Generator().manual_seed(8)
    m, k, n = 33, 64, 40
    y = Guarded(m * n * 4, torch.randn(m, n, generator=gen).to(DEV))
    s1 = (torch.rand(m, generator=gen) + 0.5).to(DEV)
    s2 = (torch.rand(n, generator=gen) + 0.5).to(DEV)
    note(f"guards in-place gemm {kind} {m}x{k}x{n}")
    if kind == "int8":
        x1 = torch.randint(-127, 128, (m, k), generator=gen, dtype=torch.int8).to(DEV)
        x2t = torch.randint(-127, 128, (n, k), generator=gen, dtype=torch.int8).to(DEV)
        wq.wq_quant_matmul_inplace_add(x1, x2t, s1, s2, m, k, n, y.ptr)
    elif kind in ("a8w4", "a4w4"):
        x2 = wq.pack_int4(torch.randint(-8, 8, (k, n), generator=gen, dtype=torch.int32).to(DEV))
        if kind == "a8w4":
            x1 = torch.randint(-127, 128, (m, k), generator=gen, dtype=torch.int8).to(DEV)
            wq.wq_quant_matmul_inplace_add_w4(x1, wq.WQ_INT8, x2, wq.WQ_LAYOUT_GFX950_B, s1, s2, m, k, n, y.ptr)
        else:
            x1 = torch.randint(0, 256, (m, k // 2), generator=gen, dtype=torch.int32).to(torch.uint8).to(DEV)
            wq.wq_quant_matmul_inplace_add_w4(x1, wq.WQ_INT4, x2, wq.WQ_LAYOUT_GFX950_B, s1, s2, m, k, n, y.ptr)
    else:
        kb = k // 32
        x1 = torch.randint(0, 256, (m, k // 2), generator=gen, dtype=torch.int32).to(torch.uint8).to(DEV)
        x2 = wq.pack_int4(torch.randint(0, 16, (k, n), generator=gen, dtype=torch.int32).to(DEV))
        sa = torch.randint(120, 135, (m, kb), generator=gen, dtype=torch.int32).to(torch.uint8).to(DEV)
        sb = torch.randint(120, 135, (kb, n), generator=gen, dtype=torch.int32).to(torch.uint8).to(DEV)
        wsn = wq.mx_fp4_quant_matmul_inplace_add_workspace_size(m, k, n)
        ws = Guarded(wsn)
        wq.mx_fp4_quant_matmul_inplace_add(x1, x2, wq.WQ_LAYOUT_GFX950_B, sa, sb, m, k, n,
                                           wq.MX_GROUP_SIZE, y.ptr, ws.ptr, wsn)
        ws.check("workspace")
    y.check("y")


@pytest.mark.parametrize("layout,k,n,transpose", [(wq.WQ_LAYOUT_ND, 80, 20, 0), (wq.WQ_LAYOUT_GFX950_B, 80, 20, 0),
                                                  (wq.WQ_LAYOUT_GFX950_B, 200, 36, 1)])
@pytest.mark.parametrize("fp4", [False, True])
def test_pack_guards(layout, k, n, transpose, fp4):
    gen = torch.Generator().manual_seed(9)
    shape = (n, k) if transpose else (k, n)
    if fp4:
        w = (torch.randn(shape, generator=gen) * 3).to(DEV)
    else:
        w = torch.randint(-8, 8, shape, generator=gen, dtype=torch.int32).to(DEV)
    out = Guarded(wq.wq_pack_int4_bytes(k, n, layout))
    note(f"guards pack fp4={fp4} layout={layout} {k}x{n} transpose={transpose}")
    if fp4:
        wq.wq_pack_fp4(w, k, n, transpose, layout, out.ptr)
    else:
        wq.wq_pack_int4(w, k, n, transpose, layout, out.ptr)
    out.check("packed weight")


@pytest.mark.parametrize("rows,cols", [(3, 24), (5, 64), (2, 20000)])
def test_add_rms_norm_guards(rows, cols):
    gen = torch.Generator().manual_seed(10)
    x = torch.randn(rows, cols, generator=gen).to(torch.bfloat16).to(DEV)
    r = torch.randn(rows, cols, generator=gen).to(torch.bfloat16).to(DEV)
    ga = (torch.rand(cols, generator=gen) + 0.5).to(torch.bfloat16).to(DEV)
    y, nrm = Guarded(rows * cols * 2), Guarded(rows * cols * 2)
    note(f"guards add_rms_norm {rows}x{cols}")
    wq.wq_add_rms_norm(x, r, ga, rows, cols, wq.WQ_BF16, 1e-6, y.ptr, nrm.ptr)
    y.check("y")
    nrm.check("normOut")


ROW_CHUNK = 1 << 20          # rows per launch of the row-parallel kernels


def test_more_rows_than_one_launch():
    """The pages allow up to 2^31 - 1 rows; row-parallel kernels run them in
    chunks of 2^20. Rows on both sides of the chunk boundary, the first and
    the last, against the oracle: per-token quant, AddRmsNorm and the fused
    operator (prefill tile)."""
    rows = ROW_CHUNK + 37
    pick = np.array([0, 1, ROW_CHUNK - 2, ROW_CHUNK - 1, ROW_CHUNK, ROW_CHUNK + 1, rows - 1])
    gen = torch.Generator(device=DEV).manual_seed(11)
    note(f"tall per-token quant {rows} x 16")
    x = torch.randn(rows, 16, generator=gen, device=DEV).to(torch.float16)
    q, s = wq.dynamic_quant(x, None, wq.WQ_INT8)
    torch.cuda.synchronize()
    oq, os_ = oracle.dynamic_quant_per_token(as_f64(x[pick]), None, "int8")
    assert np.array_equal(q[pick].cpu().numpy().astype(np.int64), oq)
    assert np.array_equal(s[pick].cpu().numpy(), os_)

    note(f"tall add_rms_norm {rows} x 8")
    a = torch.randn(rows, 8, generator=gen, device=DEV).to(torch.bfloat16)
    b = torch.randn(rows, 8, generator=gen, device=DEV).to(torch.bfloat16)
    ga = torch.ones(8, dtype=torch.bfloat16, device=DEV)
    y, nrm = wq.add_rms_norm(a, b, ga, 1e-6)
    torch.cuda.synchronize()
    oy, on = oracle.add_rms_norm(as_f64(a[pick]), as_f64(b[pick]), as_f64(ga), 1e-6)
    assert oracle.rel_err_floor(y[pick], oy) <= 1e-2
    assert oracle.rel_err_floor(nrm[pick], on) <= 1e-2

    m, k, n = ROW_CHUNK + 3, 128, 16
    note(f"tall fused wq {m}x{k}x{n}")
    x1 = torch.randn(m, k, generator=gen, device=DEV).to(torch.bfloat16)
    w = torch.randint(-8, 8, (k, n), generator=gen, device=DEV, dtype=torch.int32)
    sc = (torch.rand(n, generator=gen, device=DEV) * 0.02 + 0.002).to(torch.bfloat16)
    res = torch.randn(m, n, generator=gen, device=DEV).to(torch.bfloat16)
    gam = torch.ones(n, dtype=torch.bfloat16, device=DEV)
    yy, nn = wq.matmul_add_rmsnorm(x1, wq.pack_int4(w), k, n, wq.WQ_INT4, sc, None, 0, None, res, gam, 1e-6)
    torch.cuda.synchronize()
    pick = np.array([0, ROW_CHUNK - 1, ROW_CHUNK, m - 1])
    _, oy, on = oracle.wq_matmul_add_rmsnorm(as_f64(x1[pick]), w.cpu().numpy(), as_f64(sc), None, 0,
                                             None, as_f64(res[pick]), as_f64(gam), 1e-6)
    assert oracle.rel_err_floor(yy[pick], oy) <= 1e-2
    assert oracle.rel_err_floor(nn[pick], on) <= 1e-2
