"""GPU parity: the unfused chain (wq_weight_quant_matmul, then wq_add_rms_norm)
against the oracle's weight_quant_matmul and add_rms_norm.

Tolerance: max_i |gpu_i - oracle_i| / max(|oracle_i|, RMS(oracle)) <= 1e-2
(fp16/bf16 outputs). The standalone matmul runs the fused operator's kernels
with the residual read as zero, so it equals the fused call's y on a zero
residual bit for bit."""
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


def _operands(c, layout=B):
    m, k, n = c.mkn
    d = lambda t: None if t is None else t.to(DEV)
    if c.w_bits == 4:
        x2, wdt = wq.pack_int4(c.w.to(DEV), layout), wq.WQ_INT4
    else:
        x2, wdt, layout = c.w.to(torch.int8).to(DEV), wq.WQ_INT8, ND
    return dict(x1=c.x1.to(DEV).reshape(m, k), x2=x2, k=k, n=n, w_dtype=wdt, layout=layout,
                scale=d(c.scale), offset=d(c.offset), group_size=c.group_size, bias=d(c.bias))


def _oracle_mm(c, rows=None):
    m, k, n = c.mkn
    x1 = as_f64(c.x1).reshape(m, k)
    if rows is not None:
        x1 = x1[rows]
    f = lambda t: None if t is None else as_f64(t)
    return oracle.weight_quant_matmul(x1, c.w.numpy(), f(c.scale), f(c.offset), c.group_size, f(c.bias))


def _check(got, want, what, tol=1e-2):
    err = oracle.rel_err_floor(as_f64(got).reshape(want.shape), want)
    note(f"  {what}: rel err {err:.3e}")
    assert np.all(np.isfinite(as_f64(got)))
    assert err <= tol, f"{what}: {err}"


CASES = [  # m, k, n, granularity, group, offset, bias, act, layout  (path)
    (1, 4096, 11008, "group", 128, (-0.5, 0.5), 0.1, torch.bfloat16, B),      # decode
    (16, 4096, 4096, "group", 128, "none", 0.1, torch.float16, B),            # decode, fp16, no offset
    (256, 1024, 1024, "group", 128, (-0.5, 0.5), 0.1, torch.bfloat16, B),     # prefill tile
    (300, 2048, 700, "channel", 0, (-0.5, 0.5), None, torch.bfloat16, B),     # prefill, ragged
    (96, 512, 640, "group", 32, (-0.5, 0.5), 0.1, torch.bfloat16, B),         # generic
    (33, 256, 130, "group", 64, None, 0.1, torch.float16, ND),                # generic, ND
    (5, 100, 48, "tensor", 0, (-1.0, 1.0), 0.1, torch.bfloat16, B),           # generic, ragged k
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}-{c[3]}{c[4]}" for c in CASES])
def test_weight_quant_matmul(case):
    m, k, n, gran, g, off, bias, act, layout = case
    c = workloads.wq_case(f"wqbmm{m}x{k}x{n}", m, k, n, act=act, w_bits=4, granularity=gran,
                          group_size=g, offset_range=off, bias_std=bias, seed=m + 3 * k + n)
    note(f"standalone wq matmul {c.name} {gran} g={g} layout={layout}")
    ops = _operands(c, layout)
    out = wq.weight_quant_matmul(**ops)
    torch.cuda.synchronize()
    _check(out.cpu(), _oracle_mm(c), c.name)
    # equals the fused call's y on a zero residual, bit for bit
    zero = torch.zeros((m, n), dtype=act, device=DEV)
    y, _ = wq.matmul_add_rmsnorm(ops["x1"], ops["x2"], k, n, ops["w_dtype"], ops["scale"],
                                 ops["offset"], g, ops["bias"], zero,
                                 torch.ones(n, dtype=act, device=DEV), 1e-6, layout=ops["layout"])
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), y.cpu().reshape(m, n))


@pytest.mark.parametrize("act", [torch.bfloat16, torch.float16])
def test_weight_quant_matmul_int4_transposed(act):
    # x2 given transposed: (n, k) INT4 codes packed along k, ND layout
    c = workloads.wq_case("wqbmmT", 70, 640, 150, act=act, w_bits=4, granularity="group",
                          group_size=64, offset_range=(-0.5, 0.5), bias_std=0.1, seed=77)
    m, k, n = c.mkn
    note(f"standalone wq matmul int4 transposed ND {m}x{k}x{n} {act}")
    x2 = wq.pack_int4(c.w.to(DEV).t().contiguous(), ND)
    assert x2.numel() == n * k // 2
    d = lambda t: None if t is None else t.to(DEV)
    out = wq.weight_quant_matmul(c.x1.to(DEV).reshape(m, k), x2, k, n, wq.WQ_INT4, d(c.scale),
                                 d(c.offset), c.group_size, d(c.bias), layout=ND, transpose_x2=True)
    torch.cuda.synchronize()
    _check(out.cpu(), _oracle_mm(c), "int4 transposed")


def test_weight_quant_matmul_w8():
    c = workloads.w8()
    note("standalone wq matmul w8 per-channel")
    ops = _operands(c)
    out = wq.weight_quant_matmul(**ops)
    torch.cuda.synchronize()
    _check(out.cpu(), _oracle_mm(c), "w8")


@pytest.mark.parametrize("m,k,n", [(40, 4096, 1028), (64, 1536, 1000)])
def test_weight_quant_matmul_int8_k_split(m, k, n):
    # small grids over a long K split K across workgroups (four splits, then
    # two), with the split finish writing y and no norm
    c = workloads.wq_case(f"wqbmm8s{m}x{k}x{n}", m, k, n, act=torch.float16, w_bits=8,
                          granularity="group", group_size=128, offset_range=(-0.5, 0.5),
                          bias_std=0.1, seed=m + k + n)
    note(f"standalone wq matmul int8 k split {m}x{k}x{n}")
    ops = _operands(c)
    out = wq.weight_quant_matmul(**ops)
    torch.cuda.synchronize()
    _check(out.cpu(), _oracle_mm(c), c.name)
    zero = torch.zeros((m, n), dtype=torch.float16, device=DEV)
    y, _ = wq.matmul_add_rmsnorm(ops["x1"], ops["x2"], k, n, ops["w_dtype"], ops["scale"],
                                 ops["offset"], 128, ops["bias"], zero,
                                 torch.ones(n, dtype=torch.float16, device=DEV), 1e-6, layout=ops["layout"])
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), y.cpu().reshape(m, n))


def test_weight_quant_matmul_prefill_full_size_sampled_rows():
    c = workloads.prefill()
    m, k, n = c.mkn
    note(f"standalone wq matmul {m}x{k}x{n} (sampled rows)")
    out = wq.weight_quant_matmul(**_operands(c))
    torch.cuda.synchronize()
    rows = np.random.default_rng(31).choice(m, size=24, replace=False)
    _check(out.cpu()[rows], _oracle_mm(c, rows), "prefill rows")


def _arn_inputs(rows, d, act, seed):
    rng = np.random.default_rng(seed)
    t = lambda a: torch.from_numpy(a).to(act).to(DEV)
    return (t(rng.standard_normal((rows, d))), t(rng.standard_normal((rows, d))),
            t(rng.uniform(0.5, 1.5, d)))


@pytest.mark.parametrize("rows,d,act", [(1, 11008, torch.bfloat16), (16, 11008, torch.float16),
                                        (300, 8192, torch.bfloat16), (7, 100, torch.float16),
                                        (3, 20000, torch.bfloat16), (2, 65528, torch.bfloat16),
                                        (5, 1, torch.float16), (1, 8, torch.bfloat16)])
def test_add_rms_norm(rows, d, act):
    note(f"add_rms_norm {rows}x{d} {act}")
    x, r, g = _arn_inputs(rows, d, act, rows + d)
    y, nrm = wq.add_rms_norm(x, r, g, 1e-6)
    torch.cuda.synchronize()
    oy, on = oracle.add_rms_norm(as_f64(x.cpu()), as_f64(r.cpu()), as_f64(g.cpu()), 1e-6)
    _check(y.cpu(), oy, "y")
    _check(nrm.cpu(), on, "normOut")
    # y is x + residual rounded once: exact against a float32 sum rounded the same way
    want_y = (x.float() + r.float()).to(act)
    assert torch.equal(y, want_y)


@pytest.mark.parametrize("target", ["x", "residual"])
@pytest.mark.parametrize("d", [4096, 20000, 100])
def test_add_rms_norm_in_place(target, d):
    note(f"add_rms_norm in place on {target}, d={d}")
    x, r, g = _arn_inputs(4, d, torch.bfloat16, 7 + d)
    y0, n0 = wq.add_rms_norm(x, r, g, 1e-5)
    torch.cuda.synchronize()
    y0, n0 = y0.clone(), n0.clone()
    dst = x if target == "x" else r
    y, nrm = wq.add_rms_norm(x, r, g, 1e-5, y=dst)
    torch.cuda.synchronize()
    assert y.data_ptr() == dst.data_ptr()
    assert torch.equal(y, y0) and torch.equal(nrm, n0)


def test_chain_matches_fused_operator():
    # decode shape: matmul, then AddRmsNorm on a residual. Each stage against
    # its own oracle on the inputs it received; end to end against the fused
    # oracle with one more rounding in the budget: the chain stores mm in the
    # activation dtype (relative error <= 2^-8 for bf16) where the fused
    # operator keeps it in float32.
    c = workloads.decode(8)
    m, k, n = c.mkn
    note("chain: standalone matmul -> add_rms_norm, decode m=8")
    ops = _operands(c)
    mm = wq.weight_quant_matmul(**ops)
    res = c.residual.to(DEV).reshape(m, n)
    y, nrm = wq.add_rms_norm(mm, res, c.gamma.to(DEV), c.eps)
    torch.cuda.synchronize()
    _check(mm.cpu(), _oracle_mm(c), "chain mm")
    sy, sn = oracle.add_rms_norm(as_f64(mm.cpu()), as_f64(c.residual).reshape(m, n),
                                 as_f64(c.gamma), c.eps)
    _check(y.cpu(), sy, "chain y (stage 2 on the stored mm)")
    _check(nrm.cpu(), sn, "chain normOut (stage 2 on the stored mm)")
    f = lambda t: None if t is None else as_f64(t)
    _, oy, on = oracle.wq_matmul_add_rmsnorm(as_f64(c.x1).reshape(m, k), c.w.numpy(), f(c.scale),
                                             f(c.offset), c.group_size, f(c.bias),
                                             as_f64(c.residual).reshape(m, n), f(c.gamma), c.eps)
    tol = 1e-2 + 2.0 ** -8
    _check(y.cpu(), oy, "chain y vs fused", tol)
    _check(nrm.cpu(), on, "chain normOut vs fused", tol)
