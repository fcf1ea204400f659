"""GPU parity: wq_matmul_add_rmsnorm against the float64 oracle.

Tolerance: max_i |gpu_i - oracle_i| / max(|oracle_i|, RMS(oracle)) <= 1e-2
for the fp16/bf16 outputs y and normOut; bit-exact y for integer-valued
inputs whose partial sums are all exactly representable."""
import numpy as np
import pytest
import torch

import bit_quantized_gemm_int4_amd as wq
import oracle
import workloads
from oracle import as_f64
from tests.gpu_util import DEV, check_wq, note, wq_on_gpu

pytestmark = pytest.mark.gpu

B, ND = wq.WQ_LAYOUT_GFX950_B, wq.WQ_LAYOUT_ND


def test_tiny_workload():
    c = workloads.tiny()
    for layout in (B, ND):
        note(f"wq tiny fp16 g32 layout={layout}")
        y, n = wq_on_gpu(c, layout)
        check_wq(c, y, n)


def test_w8_workload():
    c = workloads.w8()
    for t in (False, True):
        note(f"wq w8 per-channel transpose_x2={t}")
        y, n = wq_on_gpu(c, transpose_x2=t)
        check_wq(c, y, n)


@pytest.mark.parametrize("m", [1, 8, 16])
def test_decode_workload(m):
    c = workloads.decode(m)
    note(f"wq decode m={m}")
    y, n = wq_on_gpu(c)
    check_wq(c, y, n)


def test_prefill_workload_all_rows():
    c = workloads.prefill()
    note("wq prefill 4096x8192x8192 (all rows against the full oracle)")
    y, n = wq_on_gpu(c)
    check_wq(c, y, n)
    # invariant on every row: RMS(normOut / gamma) = sqrt(ms / (ms + eps)) ~ 1
    nn = as_f64(n).reshape(-1, 8192) / as_f64(c.gamma)[None, :]
    rms = np.sqrt(np.mean(nn * nn, axis=1))
    assert np.all(np.abs(rms - 1) < 1e-2)


SHAPES = [  # m, k, n, granularity, group, offset, bias, act
    (17, 80, 20, "group", 32, (-0.5, 0.5), 0.1, torch.float16),
    (1, 64, 2, "tensor", 0, (-0.5, 0.5), 0.1, torch.bfloat16),
    (33, 100, 70, "channel", 0, "none", None, torch.bfloat16),
    (65, 257, 48, "channel2d", 0, (-0.5, 0.5), 0.1, torch.float16),
    (130, 512, 96, "group", 64, None, 0.1, torch.bfloat16),
    (5, 384, 130, "group", 128, (-1.0, 1.0), None, torch.bfloat16),
    (3, 32, 16, "tensor", 0, "none", 0.1, torch.float16),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{s[0]}x{s[1]}x{s[2]}-{s[3]}" for s in SHAPES])
@pytest.mark.parametrize("layout", [B, ND])
def test_edge_shapes_int4(shape, layout):
    m, k, n, gran, g, off, bias, act = shape
    if layout == ND and n % 2:
        pytest.skip("ND packs pairs along n")
    c = workloads.wq_case(f"edge{m}x{k}x{n}", m, k, n, act=act, w_bits=4, granularity=gran,
                          group_size=g, offset_range=off, bias_std=bias, seed=m + k + n)
    note(f"wq edge int4 {c.name} {gran} g={g} layout={layout}")
    y, nrm = wq_on_gpu(c, layout)
    check_wq(c, y, nrm)


@pytest.mark.parametrize("shape", SHAPES + [(300, 1024, 200, "group", 128, (-0.5, 0.5), 0.1,
                                              torch.bfloat16)],
                         ids=[f"{s[0]}x{s[1]}x{s[2]}-{s[3]}" for s in SHAPES] + ["300x1024x200"])
def test_edge_shapes_int4_transposed(shape):
    # x2 given transposed, (n, k) packed along k (ND only)
    m, k, n, gran, g, off, bias, act = shape
    if k % 2:
        pytest.skip("the transposed ND weight packs pairs along k")
    c = workloads.wq_case(f"edgeT{m}x{k}x{n}", m, k, n, act=act, w_bits=4, granularity=gran,
                          group_size=g, offset_range=off, bias_std=bias, seed=3 * m + k + n)
    note(f"wq edge int4 transposed ND {c.name} {gran} g={g}")
    y, nrm = wq_on_gpu(c, ND, transpose_x2=True)
    check_wq(c, y, nrm)


@pytest.mark.parametrize("shape", SHAPES[:4], ids=[f"{s[0]}x{s[1]}x{s[2]}" for s in SHAPES[:4]])
@pytest.mark.parametrize("transpose", [False, True])
def test_edge_shapes_int8(shape, transpose):
    m, k, n, gran, g, off, bias, act = shape
    c = workloads.wq_case(f"edge8_{m}x{k}x{n}", m, k, n, act=act, w_bits=8, granularity=gran,
                          group_size=g, scale_range=(0.001, 0.01), offset_range=off,
                          bias_std=bias, seed=m * k + n)
    note(f"wq edge int8 {c.name} transpose={transpose}")
    y, nrm = wq_on_gpu(c, transpose_x2=transpose)
    check_wq(c, y, nrm)


def test_inplace_matches_out_of_place():
    c = workloads.tiny()
    note("wq inplace tiny")
    y0, n0 = wq_on_gpu(c)
    y1, n1 = wq_on_gpu(c, inplace=True)
    assert torch.equal(y0, y1) and torch.equal(n0, n1)


def test_deterministic():
    c = workloads.decode(16)
    note("wq determinism decode m=16")
    y0, n0 = wq_on_gpu(c)
    y1, n1 = wq_on_gpu(c)
    assert torch.equal(y0, y1) and torch.equal(n0, n1)


@pytest.mark.parametrize("act", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("k,G", [(256, 32), (512, 128), (384, 0)])
def test_integer_valued_y_is_bit_exact(act, k, G):
    # Sparse x1 in {-1,0,1}, int4 weights, scale 1, offset 0, bias 0 and an
    # integer residual: every partial sum is an integer far below 2^24 and
    # |y| <= 256, so y is exact in fp16 and bf16 alike.
    m, n = 20, 64
    rng = np.random.default_rng(k + G)
    xv = rng.integers(-1, 2, (m, k)) * (rng.random((m, k)) < 0.25)
    x1 = torch.from_numpy(xv.astype(np.float32)).to(act)
    w = torch.from_numpy(rng.integers(-8, 8, (k, n), dtype=np.int32))
    srows = (k + G - 1) // G if G else 1
    scale = torch.ones((srows, n) if G else (1,), dtype=act)
    res = torch.from_numpy(rng.integers(-4, 5, (1, m, n)).astype(np.float32)).to(act)
    c = workloads.WQCase("intexact", x1, w, 4, scale, torch.zeros_like(scale), G,
                         torch.zeros(n, dtype=act), res, torch.ones(n, dtype=act), 1e-6)
    _, oy, on = oracle.wq_matmul_add_rmsnorm(as_f64(x1), w.numpy(), as_f64(scale), None, G, None,
                                             as_f64(res).reshape(m, n), np.ones(n), 1e-6)
    assert np.max(np.abs(oy)) <= 256            # the case's own precondition
    note(f"wq integer-exact {act} k={k} G={G}")
    y, nrm = wq_on_gpu(c)
    assert np.array_equal(as_f64(y).reshape(m, n), oy)
    assert oracle.rel_err_floor(nrm, on) <= 1e-2


def test_one_hot_rows_pin_group_indexing():
    k, n, G = 256, 32, 32
    m = 8
    rows = [0, 31, 32, 100, 128, 200, 224, 255]
    x1 = torch.zeros((m, k), dtype=torch.bfloat16)
    for i, r in enumerate(rows):
        x1[i, r] = 1.0
    c = workloads.wq_case("onehot", m, k, n, act=torch.bfloat16, w_bits=4, granularity="group",
                          group_size=G, offset_range=(-1, 1), bias_std=None, seed=5)
    c.x1 = x1
    c.residual = torch.zeros_like(c.residual)
    note("wq one-hot rows")
    y, nrm = wq_on_gpu(c)
    _, oy, _ = oracle.wq_matmul_add_rmsnorm(as_f64(x1), c.w.numpy(), as_f64(c.scale),
                                            as_f64(c.offset), G, None, np.zeros((m, n)),
                                            np.ones(n), 1e-6)
    # y is the dequantized weight row q * s + o, rounded once to bf16
    assert oracle.rel_err_floor(y.reshape(m, n), oy) <= 2.0 ** -8


FAST = [  # m, k, n, granularity, group, offset, bias, act: the large-m GFX950_B tile
    (300, 384, 200, "group", 128, (-1.0, 1.0), 0.1, torch.bfloat16),
    (257, 1024, 136, "channel", 0, (-0.5, 0.5), None, torch.bfloat16),
    (65, 256, 48, "tensor", 0, "none", 0.1, torch.float16),
    (512, 1024, 256, "group", 256, (-0.5, 0.5), 0.1, torch.float16),
    (33, 128, 18, "channel2d", 0, None, 0.1, torch.bfloat16),
    (520, 2048, 300, "group", 128, "none", None, torch.bfloat16),
    # whole 512-column strips (the unmasked tile), next to a ragged one
    (256, 512, 1024, "group", 128, (-1.0, 1.0), 0.1, torch.bfloat16),
    (384, 1024, 1536, "group", 256, (-0.5, 0.5), None, torch.float16),
    (200, 640, 1100, "channel", 0, (-0.5, 0.5), 0.1, torch.bfloat16),
]


@pytest.mark.parametrize("shape", FAST, ids=[f"{s[0]}x{s[1]}x{s[2]}-{s[3]}{s[4]}" for s in FAST])
def test_fast_tile_shapes(shape):
    m, k, n, gran, g, off, bias, act = shape
    c = workloads.wq_case(f"fast{m}x{k}x{n}", m, k, n, act=act, w_bits=4, granularity=gran,
                          group_size=g, scale_range=(0.002, 0.02), offset_range=off,
                          bias_std=bias, seed=3 * m + k + n)
    note(f"wq fast tile {c.name} {gran} g={g} {act}")
    y, nrm = wq_on_gpu(c)
    check_wq(c, y, nrm)
    y2, n2 = wq_on_gpu(c, inplace=True)
    assert torch.equal(y, y2) and torch.equal(nrm, n2)


DECODE = [  # m, k, n, granularity, group, offset, bias, act: the m <= 32 weight stream
    (1, 128, 16, "tensor", 0, "none", None, torch.bfloat16),
    (2, 384, 48, "group", 128, (-1.0, 1.0), 0.1, torch.bfloat16),
    (7, 1024, 130, "channel", 0, (-0.5, 0.5), 0.1, torch.float16),
    (9, 256, 777, "group", 128, (-1.0, 1.0), 0.1, torch.bfloat16),
    (16, 4096, 4100, "group", 128, (-1.0, 1.0), 0.1, torch.bfloat16),
    (17, 2048, 8210, "group", 256, None, None, torch.bfloat16),
    (31, 640, 13000, "group", 128, "none", 0.1, torch.bfloat16),
    (32, 8192, 1000, "channel2d", 0, (-0.5, 0.5), 0.1, torch.float16),
    (5, 1152, 2000, "group", 384, (-1.0, 1.0), None, torch.float16),
]


@pytest.mark.parametrize("shape", DECODE, ids=[f"{s[0]}x{s[1]}x{s[2]}-{s[3]}{s[4]}" for s in DECODE])
def test_decode_kernel_shapes(shape):
    m, k, n, gran, g, off, bias, act = shape
    c = workloads.wq_case(f"dec{m}x{k}x{n}", m, k, n, act=act, w_bits=4, granularity=gran,
                          group_size=g, scale_range=(0.002, 0.02), offset_range=off,
                          bias_std=bias, seed=7 * m + k + n)
    note(f"wq decode kernel {c.name} {gran} g={g} {act}")
    y, nrm = wq_on_gpu(c)
    check_wq(c, y, nrm)
    y2, n2 = wq_on_gpu(c, inplace=True)
    assert torch.equal(y, y2) and torch.equal(nrm, n2)


@pytest.mark.parametrize("G", [128, 256])
def test_fast_zero_scale_in_one_strip(G):
    # zero group scales inside one 512-column strip only: that strip's tiles
    # zero the weight operand, the other strips run unmasked
    m, k, n = 160, 512, 1536
    c = workloads.wq_case(f"fast_zero_scale_g{G}", m, k, n, act=torch.bfloat16, w_bits=4,
                          granularity="group", group_size=G, scale_range=(0.002, 0.02),
                          offset_range=(-1.0, 1.0), bias_std=0.1, seed=13 + G)
    c.scale[1, 600:610] = 0
    c.scale[:, 700] = 0
    note(f"wq fast tile zero-scale strip g={G}")
    y, nrm = wq_on_gpu(c)
    check_wq(c, y, nrm)


@pytest.mark.parametrize("m,k,n", [(300, 1024, 700), (4096, 2048, 1024)])
def test_fast_tile_fp16_group128(m, k, n):
    # the prefill tile's fp16 form (codes enter as q + 1032) with the group-128
    # specialization, ragged and at a full-height m
    c = workloads.wq_case(f"fast_f16_{m}x{k}x{n}", m, k, n, act=torch.float16, w_bits=4,
                          granularity="group", group_size=128, offset_range=(-0.5, 0.5),
                          bias_std=0.1, seed=m + k)
    note(f"wq fast tile fp16 g128 {m}x{k}x{n}")
    y, nrm = wq_on_gpu(c)
    rows = None if m <= 512 else np.random.default_rng(3).choice(m, size=32, replace=False)
    check_wq(c, y, nrm, rows=rows)


def test_fast_zero_scale_in_a_later_group_tile():
    # k = 8192 at group 128: 64 groups, so the correction pass flags two
    # 32-group tiles per 64 columns; zero scales only in groups 40 and 63
    # must still send their strips down the masked path
    m, k, n = 160, 8192, 1024
    c = workloads.wq_case("fast_zero_scale_late", m, k, n, act=torch.bfloat16, w_bits=4,
                          granularity="group", group_size=128, scale_range=(0.002, 0.02),
                          offset_range=(-1.0, 1.0), bias_std=0.1, seed=17)
    c.scale[40, 300:303] = 0
    c.scale[63, 900] = 0
    note("wq fast tile zero scales in groups 40 and 63")
    y, nrm = wq_on_gpu(c)
    check_wq(c, y, nrm)


def test_decode_zero_scale_columns():
    # a zero group scale leaves only the offset: w = o for that group
    m, k, n, G = 4, 512, 64, 128
    c = workloads.wq_case("dec_zero_scale", m, k, n, act=torch.bfloat16, w_bits=4,
                          granularity="group", group_size=G, scale_range=(0.002, 0.02),
                          offset_range=(-1.0, 1.0), bias_std=0.1, seed=11)
    c.scale[1, :] = 0
    c.scale[:, 5] = 0
    note("wq decode zero-scale groups and columns")
    y, nrm = wq_on_gpu(c)
    check_wq(c, y, nrm)


@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 7, 8, 9, 12, 15, 16, 17, 19, 21, 24, 28, 31, 32])
def test_decode_every_row_count(m):
    # the decode kernel computes 16 rows per launch (absent rows read zeros),
    # rows 17..32 in a second launch: every count of rows, against the oracle
    c = workloads.wq_case(f"dec{m}", m, 1024, 640, act=torch.bfloat16, w_bits=4,
                          granularity="group", group_size=128, offset_range=(-0.5, 0.5),
                          bias_std=0.1, seed=100 + m)
    note(f"wq decode rows m={m} 1024x640 g128")
    y, n = wq_on_gpu(c)
    check_wq(c, y, n)


@pytest.mark.parametrize("m,k,n,g", [(40, 1024, 65535, 128),     # widest n: ragged, masked strips
                                     (48, 65408, 256, 128),      # deepest k on the fast path
                                     (3, 65408, 640, 128),       # the same k on the decode kernel
                                     (24, 2048, 65535, 0)],      # widest n, decode, per channel
                         ids=["n65535-prefill", "k65408-prefill", "k65408-decode", "n65535-decode"])
def test_maximum_sizes_sampled_rows(m, k, n, g):
    # the largest n and k the call takes (n <= 65535, k <= 65535 and a multiple
    # of 128 for the fast kernels), checked on sampled rows (the full rows:
    # normOut needs the whole row)
    gran = "group" if g else "channel"
    c = workloads.wq_case(f"max{m}x{k}x{n}", m, k, n, act=torch.bfloat16, w_bits=4, granularity=gran,
                          group_size=g, offset_range=(-0.5, 0.5), bias_std=0.1, seed=k + n)
    note(f"wq maximum size {m}x{k}x{n} g={g}")
    y, nrm = wq_on_gpu(c)
    rows = np.random.default_rng(5).choice(m, size=min(m, 4), replace=False)
    check_wq(c, y, nrm, rows=rows)
