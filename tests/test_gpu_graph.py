"""HIP graph capture of the library's entry points.

Every entry point only enqueues kernels on the caller's stream: no
allocation, memset, host synchronization or event (profiling off), so a call
can be captured into a graph and replayed, as a serving loop does with its
decode layers. Each test captures calls, replays the graph several times with
eager work and synchronizations between the replays, and checks every replay
against the eager result bit for bit (the same kernels on the same inputs).
The eager results themselves are checked against the oracle by the other GPU
tests."""
import numpy as np
import pytest
import torch

import bit_quantized_gemm_int4_amd as wq
import workloads
from tests.gpu_util import DEV, note

pytestmark = pytest.mark.gpu

B = wq.WQ_LAYOUT_GFX950_B


def _capture(fn) -> torch.cuda.CUDAGraph:
    """Warm up ``fn`` once on a side stream (as capture requires), then
    capture one call of it."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _eager_noise():
    """Unrelated eager work between replays (a library call and torch ops)."""
    x = torch.randn(64, 256, dtype=torch.float16, device=DEV)
    wq.dynamic_quant(x, None, wq.WQ_INT8)
    (x.float() @ x.float().t()).sum().item()
    torch.cuda.synchronize()


class _WQCall:
    """One wq_matmul_add_rmsnorm call on device buffers it owns."""

    def __init__(self, case, layout=B):
        m, k, n = case.mkn
        self.m, self.k, self.n = m, k, n
        self.case = case
        self.x1 = case.x1.to(DEV)
        if case.w_bits == 4:
            self.x2 = wq.pack_int4(case.w.to(DEV), layout)
            self.wdt, self.layout = wq.WQ_INT4, layout
        else:
            self.x2 = case.w.to(torch.int8).to(DEV)
            self.wdt, self.layout = wq.WQ_INT8, wq.WQ_LAYOUT_ND
        d = lambda t: None if t is None else t.to(DEV)
        self.scale, self.offset, self.bias = d(case.scale), d(case.offset), d(case.bias)
        self.residual, self.gamma = d(case.residual), d(case.gamma)
        self.y = torch.empty_like(self.residual)
        self.norm = torch.empty_like(self.residual)
        self.ws_n = wq.wq_matmul_add_rmsnorm_workspace_size(m, k, n)
        self.ws = torch.zeros(max(self.ws_n, 1), dtype=torch.uint8, device=DEV)

    def __call__(self):
        s = self.scale
        s_rows, s_cols = (s.shape if s.dim() == 2 else (1, s.numel()))
        wq.wq_matmul_add_rmsnorm(self.x1, self.m, self.k, wq.act_code(self.x1.dtype), self.x2, self.n,
                                 self.wdt, self.layout, 0, s, s_rows, s_cols, self.offset,
                                 self.case.group_size, self.bias, self.residual, self.gamma,
                                 self.case.eps, self.y, self.norm, self.ws, self.ws_n)

    def outputs(self):
        return self.y.clone(), self.norm.clone()

    def poison(self):
        self.y.fill_(float("nan"))
        self.norm.fill_(float("nan"))


def _check_replays(call, replays=3):
    call()
    torch.cuda.synchronize()
    want = call.outputs()
    g = _capture(call)
    for r in range(replays):
        call.poison()
        _eager_noise()
        g.replay()
        torch.cuda.synchronize()
        got = call.outputs()
        for a, b in zip(got, want):
            assert torch.equal(a, b), f"replay {r} differs from the eager call"


@pytest.mark.parametrize("m", [1, 16])
def test_decode_call_replays(m):
    note(f"graph: wq decode m={m}")
    _check_replays(_WQCall(workloads.decode(m)))


def test_decode_graph_of_rotating_weights():
    # a decode step of 4 layers with their own weights captured as one graph
    note("graph: 4 decode calls, own weights each, one graph")
    calls = [_WQCall(workloads.wq_case(f"layer{i}", 8, 4096, 11008, act=torch.bfloat16, w_bits=4,
                                       granularity="group", group_size=128,
                                       offset_range=(-0.5, 0.5), bias_std=0.1, seed=40 + i))
             for i in range(4)]
    wants = []
    for c in calls:
        c()
    torch.cuda.synchronize()
    wants = [c.outputs() for c in calls]

    def step():
        for c in calls:
            c()
    g = _capture(step)
    for r in range(3):
        for c in calls:
            c.poison()
        _eager_noise()
        g.replay()
        torch.cuda.synchronize()
        for c, w in zip(calls, wants):
            for a, b in zip(c.outputs(), w):
                assert torch.equal(a, b), f"replay {r}"


@pytest.mark.parametrize("shape", [(256, 1024, 1024, 128), (96, 512, 640, 32)],
                         ids=["prefill-tile-g128", "int8-tile-int4-g32"])
def test_prefill_and_generic_call_replays(shape):
    m, k, n, g = shape
    note(f"graph: wq {m}x{k}x{n} g={g}")
    c = workloads.wq_case(f"graph{m}x{k}x{n}", m, k, n, act=torch.bfloat16, w_bits=4,
                          granularity="group", group_size=g, offset_range=(-0.5, 0.5),
                          bias_std=0.1, seed=7)
    _check_replays(_WQCall(c))


def test_w8_call_replays():
    note("graph: wq w8 per-channel")
    _check_replays(_WQCall(workloads.w8()))


def test_w8_four_way_k_split_replays():
    # a small grid over a long K: the INT8 tile in four K splits, then the
    # split finish (float32 sums through the workspace)
    c = workloads.wq_case("graph w8 split4", 40, 4096, 1028, act=torch.float16, w_bits=8,
                          granularity="group", group_size=128, offset_range=(-0.5, 0.5),
                          bias_std=0.1, seed=11)
    note("graph: wq w8 40x4096x1028 g128 (four K splits)")
    _check_replays(_WQCall(c))


def test_dynamic_quant_and_pack_replay():
    note("graph: dynamic quant (per token int8, MX e4m3 and e2m1) and pack (int4, fp4)")
    rng = np.random.default_rng(3)
    x = torch.from_numpy(rng.standard_normal((300, 1024))).to(torch.float16).to(DEV)
    sm = torch.from_numpy(rng.uniform(0.5, 2, 1024)).to(torch.float16).to(DEV)
    w = torch.from_numpy(rng.integers(-8, 8, (512, 768), dtype=np.int32)).to(DEV)
    q8 = torch.empty((300, 1024), dtype=torch.int8, device=DEV)
    s8 = torch.empty(300, dtype=torch.float32, device=DEV)
    qmx = torch.empty((1024, 300), dtype=torch.uint8, device=DEV)
    smx = torch.empty((300, 32), dtype=torch.uint8, device=DEV)
    pk = torch.empty(wq.wq_pack_int4_bytes(512, 768, B), dtype=torch.uint8, device=DEV)
    q4 = torch.empty((300, 512), dtype=torch.uint8, device=DEV)
    s4 = torch.empty((300, 32), dtype=torch.uint8, device=DEV)
    wf = torch.from_numpy(rng.standard_normal((512, 768)).astype(np.float32) * 3).to(DEV)
    pf = torch.empty(wq.wq_pack_int4_bytes(512, 768, B), dtype=torch.uint8, device=DEV)

    def fn():
        wq.wq_dynamic_quant(x, wq.WQ_F16, 300, 1024, sm, wq.WQ_INT8, 0, 0, q8, s8)
        wq.wq_dynamic_quant(x, wq.WQ_F16, 300, 1024, sm, wq.WQ_FP8_E4M3, 32, 1, qmx, smx)
        wq.wq_dynamic_quant(x, wq.WQ_F16, 300, 1024, sm, wq.WQ_FP4_E2M1, 32, 0, q4, s4)
        wq.wq_pack_int4(w, 512, 768, 0, B, pk)
        wq.wq_pack_fp4(wf, 512, 768, 0, B, pf)
    outs = (q8, s8, qmx, smx, q4, s4, pk, pf)
    fn()
    torch.cuda.synchronize()
    want = [t.clone() for t in outs]
    g = _capture(fn)
    for r in range(3):
        for t in outs:
            if t is s8:
                t.fill_(float("nan"))
            else:
                t.fill_(0x55)
        _eager_noise()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, want):
            assert torch.equal(a, b), f"replay {r}"


def test_inplace_accumulators_replay():
    # MX, INT8, INT8 x INT4 and MXFP4 add into y: replay r must equal r + 1 eager
    # calls from the same start (the warm-up before capture is the first)
    note("graph: MX, INT8, A8W4 and MXFP4 in-place add, replays accumulate")
    rng = np.random.default_rng(5)
    m, k, n = 256, 512, 384
    x1 = torch.from_numpy(rng.integers(-127, 128, (m, k), dtype=np.int8)).to(DEV)
    x2 = torch.from_numpy(rng.integers(-127, 128, (n, k), dtype=np.int8)).to(DEV)
    s1 = torch.from_numpy(rng.uniform(1e-3, 1e-2, m).astype(np.float32)).to(DEV)
    s2 = torch.from_numpy(rng.uniform(1e-3, 1e-2, n).astype(np.float32)).to(DEV)
    y0 = torch.from_numpy(rng.standard_normal((m, n)).astype(np.float32)).to(DEV)

    mx_x1 = torch.from_numpy(rng.integers(0, 256, (k, m), dtype=np.uint8))
    mx_x1[(mx_x1 & 0x7F) == 0x7F] = 0
    mx_x1 = mx_x1.to(DEV)
    mx_x2 = wq.pack_int4(torch.from_numpy(rng.integers(0, 16, (k, n), dtype=np.int32)).to(DEV), B)
    mx_s1 = torch.from_numpy(rng.integers(120, 128, (m, k // 32), dtype=np.uint8)).to(DEV)
    mx_s2 = torch.from_numpy(rng.integers(120, 128, (k // 32, n), dtype=np.uint8)).to(DEV)

    # MXFP4: E2M1 x1 (m, k/2) bytes and a workspace of its own
    f4_x1 = torch.from_numpy(rng.integers(0, 256, (m, k // 2), dtype=np.uint8)).to(DEV)
    ws4 = torch.empty(wq.mx_fp4_quant_matmul_inplace_add_workspace_size(m, k, n), dtype=torch.uint8,
                      device=DEV)

    y_i8, y_mx, y_w4, y_f4 = y0.clone(), y0.clone(), y0.clone(), y0.clone()

    def fn():
        wq.quant_matmul_inplace_add(x1, x2, s1, s2, y_i8)
        wq.mx_matmul_inplace_add(mx_x1, mx_x2, mx_s1, mx_s2, y_mx, m, k, n)
        # the packed nibbles of mx_x2 read as INT4 codes
        wq.quant_matmul_inplace_add_w4(x1, mx_x2, n, s1, s2, y_w4)
        wq.mxfp4_matmul_inplace_add(f4_x1, mx_x2, mx_s1, mx_s2, y_f4, m, k, n, workspace=ws4)

    # eager sequence on copies
    e_i8, e_mx, e_w4, e_f4 = y0.clone(), y0.clone(), y0.clone(), y0.clone()
    seq = []
    for _ in range(4):
        wq.quant_matmul_inplace_add(x1, x2, s1, s2, e_i8)
        wq.mx_matmul_inplace_add(mx_x1, mx_x2, mx_s1, mx_s2, e_mx, m, k, n)
        wq.quant_matmul_inplace_add_w4(x1, mx_x2, n, s1, s2, e_w4)
        wq.mxfp4_matmul_inplace_add(f4_x1, mx_x2, mx_s1, mx_s2, e_f4, m, k, n, workspace=ws4)
        seq.append((e_i8.clone(), e_mx.clone(), e_w4.clone(), e_f4.clone()))
    torch.cuda.synchronize()
    g = _capture(fn)                       # the warm-up ran once on y_i8 / y_mx
    for r in range(3):
        _eager_noise()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_i8, seq[r + 1][0]), f"int8 replay {r}"
        assert torch.equal(y_mx, seq[r + 1][1]), f"mx replay {r}"
        assert torch.equal(y_w4, seq[r + 1][2]), f"a8w4 replay {r}"
        assert torch.equal(y_f4, seq[r + 1][3]), f"mxfp4 replay {r}"


def test_mx_misaligned_n_replays():
    # the MX tile's form for N not a multiple of 4 (scale2 by byte loads, y in
    # unaligned 16-byte runs and element-wise across N) accumulates replay by
    # replay exactly as eager calls do
    note("graph: MX in-place add, n % 4 != 0")
    rng = np.random.default_rng(11)
    m, k, n = 272, 200, 262
    x1 = torch.from_numpy(rng.integers(0, 256, (k, m), dtype=np.uint8))
    x1[(x1 & 0x7F) == 0x7F] = 0
    x1 = x1.to(DEV)
    x2 = wq.pack_int4(torch.from_numpy(rng.integers(0, 16, (k, n), dtype=np.int32)).to(DEV), B)
    kb = -(-k // 32)
    s1 = torch.from_numpy(rng.integers(120, 128, (m, kb), dtype=np.uint8)).to(DEV)
    s2 = torch.from_numpy(rng.integers(120, 128, (kb, n), dtype=np.uint8)).to(DEV)
    y0 = torch.from_numpy(rng.standard_normal((m, n)).astype(np.float32)).to(DEV)
    y = y0.clone()
    e = y0.clone()
    seq = []
    for _ in range(4):
        wq.mx_matmul_inplace_add(x1, x2, s1, s2, e, m, k, n)
        seq.append(e.clone())
    torch.cuda.synchronize()
    g = _capture(lambda: wq.mx_matmul_inplace_add(x1, x2, s1, s2, y, m, k, n))
    for r in range(3):
        _eager_noise()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, seq[r + 1]), f"replay {r}"


def test_unfused_chain_replays():
    note("graph: standalone matmul -> add_rms_norm (decode m=4)")
    c = workloads.decode(4)
    m, k, n = c.mkn
    x1 = c.x1.to(DEV).reshape(m, k)
    x2 = wq.pack_int4(c.w.to(DEV), B)
    sc, off, bias = c.scale.to(DEV), c.offset.to(DEV), c.bias.to(DEV)
    res, gam = c.residual.to(DEV).reshape(m, n), c.gamma.to(DEV)
    mm = torch.empty((m, n), dtype=x1.dtype, device=DEV)
    y, nrm = torch.empty_like(mm), torch.empty_like(mm)
    ws = torch.zeros(wq.wq_weight_quant_matmul_workspace_size(m, k, n), dtype=torch.uint8, device=DEV)

    def fn():
        wq.weight_quant_matmul(x1, x2, k, n, wq.WQ_INT4, sc, off, c.group_size, bias, out=mm,
                               workspace=ws)
        wq.add_rms_norm(mm, res, gam, c.eps, y=y, norm_out=nrm)
    fn()
    torch.cuda.synchronize()
    want = [t.clone() for t in (mm, y, nrm)]
    g = _capture(fn)
    for r in range(3):
        for t in (mm, y, nrm):
            t.fill_(float("nan"))
        _eager_noise()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((mm, y, nrm), want):
            assert torch.equal(a, b), f"replay {r}"
