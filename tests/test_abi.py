"""The C ABI: the library loads, exports every entry point declared in
include/wq.h, and its host-side validation rejects bad arguments before any
launch. No test here launches a kernel: each call breaks a rule that is
checked on the host, and the fake device addresses are never dereferenced."""
import ctypes
import os
import re

import pytest

import bit_quantized_gemm_int4_amd as wq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wq.h")

pytestmark = pytest.mark.skipif(not os.path.exists(wq.LIB_PATH),
                                reason="libwq.so not built (run __graft_entry__.build())")

FAKE = 0x7F0000000000          # 16-byte aligned fake device address, never touched
FAKE2 = 0x7F0000100000
FAKE3 = 0x7F0000200000


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:wq|mx)_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) == 23, names
    L = wq.lib()
    for name in names:
        assert hasattr(L, name), name
    assert sorted(wq.EXPORTS) == names


def test_version_and_status_strings():
    assert wq.lib().wq_abi_version() == 1
    for code in range(9):
        s = wq.lib().wq_status_string(code).decode()
        assert s.startswith("WQ_")
    assert wq.lib().wq_status_string(99).decode() == "unknown wq_status"


def test_profile_read_without_a_record():
    # nothing recorded yet: zero time, zero launches, no device call needed
    assert wq.wq_profile_read() == []
    assert wq.lib().wq_profile_read(None, 0, None) == wq.WQ_ERR_NULLPTR
    n = ctypes.c_int64(0)
    assert wq.lib().wq_profile_read(None, 4, ctypes.byref(n)) == wq.WQ_ERR_NULLPTR  # no buffer


def test_size_queries():
    assert wq.wq_pack_int4_bytes(256, 128, wq.WQ_LAYOUT_ND) == 256 * 64
    assert wq.wq_pack_int4_bytes(256, 128, wq.WQ_LAYOUT_GFX950_B) == 256 * 128 // 2
    assert wq.wq_pack_int4_bytes(80, 20, wq.WQ_LAYOUT_GFX950_B) == 128 * 32 // 2
    assert wq.wq_pack_int4_bytes(4, 3, wq.WQ_LAYOUT_ND) == 0
    assert wq.wq_pack_int4_bytes(-1, 3, wq.WQ_LAYOUT_GFX950_B) == 0
    ws = wq.wq_matmul_add_rmsnorm_workspace_size(4096, 8192, 8192)
    assert ws >= 4096 * (8192 // 32) * 4
    # small grids over a long K: room for the float32 sums of every K split
    # (two at 512 x 1024 x 1024, four at 1 x 4096 x 4096 and 36 x 2048 x 250)
    assert wq.wq_matmul_add_rmsnorm_workspace_size(512, 1024, 1024) >= 2 * 512 * 1024 * 4
    assert wq.wq_matmul_add_rmsnorm_workspace_size(1, 4096, 4096) >= 4 * 4096 * 4
    assert wq.wq_matmul_add_rmsnorm_workspace_size(36, 2048, 250) >= 4 * 36 * 250 * 4
    # a grid of one workgroup per CU or more takes no split
    assert wq.wq_matmul_add_rmsnorm_workspace_size(1024, 1024, 4096) < 2 * 1024 * 4096 * 4
    assert wq.mx_quant_matmul_inplace_add_workspace_size(4096, 8192, 4096) == 0
    # m % 16 != 0: room for x1 with rows padded to 16 bytes (k x 16 ceil(m/16)), 256-byte rounded
    assert wq.mx_quant_matmul_inplace_add_workspace_size(4100, 8192, 4100) == 8192 * 4112
    # m % 16 != 0 with n % 4 != 0: the tile on a padded x1 copy, 7 x 48 bytes rounded to 256
    assert wq.mx_quant_matmul_inplace_add_workspace_size(33, 7, 17) == 512
    assert wq.mx_quant_matmul_inplace_add_workspace_size(33, 7, 16) == 512        # 7 x 48 = 336 -> 512
    assert wq.mx_quant_matmul_inplace_add_workspace_size(0, 7, 16) == 0


def _pack(**kw):
    a = dict(weight=FAKE, k=64, n=64, transpose=0, layout=wq.WQ_LAYOUT_ND, out=FAKE2, stream=0)
    a.update(kw)
    return wq.lib().wq_pack_int4(a["weight"], a["k"], a["n"], a["transpose"], a["layout"],
                                 a["out"], a["stream"])


def test_pack_validation():
    assert _pack(n=63) == wq.WQ_ERR_SHAPE
    assert _pack(k=-1) == wq.WQ_ERR_SHAPE
    assert _pack(layout=7) == wq.WQ_ERR_UNSUPPORTED
    assert _pack(weight=None) == wq.WQ_ERR_NULLPTR
    assert _pack(out=None, layout=wq.WQ_LAYOUT_GFX950_B) == wq.WQ_ERR_NULLPTR
    assert _pack(out=FAKE2 + 4) == wq.WQ_ERR_SHAPE                 # misaligned output
    assert _pack(out=FAKE + 64) == wq.WQ_ERR_ALIAS                 # overlaps the input
    assert _pack(k=0) == wq.WQ_OK and _pack(n=0) == wq.WQ_OK       # empty: no-op
    # GFX950_B tiles use 32-bit byte offsets: n < 2^22, or k < 2^21 transposed
    assert _pack(layout=wq.WQ_LAYOUT_GFX950_B, n=1 << 22) == wq.WQ_ERR_SHAPE
    assert _pack(layout=wq.WQ_LAYOUT_GFX950_B, k=1 << 21, transpose=1) == wq.WQ_ERR_SHAPE


def _quant(**kw):
    a = dict(x=FAKE, x_dtype=wq.WQ_F16, rows=4, cols=64, smooth=None, y_dtype=wq.WQ_INT8,
             block_k=0, transpose_y=0, y=FAKE2, scale=FAKE3, stream=0)
    a.update(kw)
    return wq.lib().wq_dynamic_quant(a["x"], a["x_dtype"], a["rows"], a["cols"], a["smooth"],
                                     a["y_dtype"], a["block_k"], a["transpose_y"], a["y"],
                                     a["scale"], a["stream"])


def test_dynamic_quant_validation():
    assert _quant(x_dtype=wq.WQ_F32) == wq.WQ_ERR_DTYPE
    assert _quant(y_dtype=wq.WQ_FP8_E4M3) == wq.WQ_ERR_DTYPE        # per-token
    assert _quant(y_dtype=wq.WQ_INT4, cols=63) == wq.WQ_ERR_SHAPE   # INT4: even cols
    assert _quant(y_dtype=wq.WQ_INT32, cols=60) == wq.WQ_ERR_SHAPE  # INT32: cols % 8
    assert _quant(transpose_y=1) == wq.WQ_ERR_UNSUPPORTED
    assert _quant(block_k=16) == wq.WQ_ERR_UNSUPPORTED
    assert _quant(block_k=32, y_dtype=wq.WQ_INT8) == wq.WQ_ERR_DTYPE
    assert _quant(block_k=32, y_dtype=wq.WQ_FP4_E2M1, transpose_y=1) == wq.WQ_ERR_UNSUPPORTED
    assert _quant(block_k=32, y_dtype=wq.WQ_FP4_E2M1, cols=63) == wq.WQ_ERR_SHAPE
    assert _quant(rows=-1) == wq.WQ_ERR_SHAPE
    assert _quant(scale=None) == wq.WQ_ERR_NULLPTR
    assert _quant(x=FAKE + 2) == wq.WQ_ERR_SHAPE
    assert _quant(rows=0) == wq.WQ_OK and _quant(cols=0) == wq.WQ_OK
    assert _quant(cols=1 << 30) == wq.WQ_ERR_SHAPE                 # per-token row offsets


def _wqmm(**kw):
    m, k, n = kw.pop("m", 16), kw.pop("k", 256), kw.pop("n", 128)
    a = dict(x1=FAKE, act=wq.WQ_F16, x2=FAKE + 0x10000, w=wq.WQ_INT4,
             layout=wq.WQ_LAYOUT_GFX950_B, tx2=0, scale=FAKE + 0x20000, srows=8, scols=n,
             offset=None, group=32, bias=None, residual=FAKE + 0x30000, gamma=FAKE + 0x40000,
             eps=1e-6, y=FAKE + 0x50000, norm=FAKE + 0x60000, ws=FAKE + 0x70000,
             ws_size=1 << 20)
    a.update(kw)
    return wq.lib().wq_matmul_add_rmsnorm(
        a["x1"], m, k, a["act"], a["x2"], n, a["w"], a["layout"], a["tx2"], a["scale"],
        a["srows"], a["scols"], a["offset"], a["group"], a["bias"], a["residual"], a["gamma"],
        a["eps"], a["y"], a["norm"], a["ws"], a["ws_size"], 0)


def test_wq_matmul_validation_dtypes_and_layouts():
    assert _wqmm(act=wq.WQ_F32) == wq.WQ_ERR_DTYPE
    assert _wqmm(w=wq.WQ_FP8_E4M3) == wq.WQ_ERR_DTYPE
    assert _wqmm(layout=5) == wq.WQ_ERR_UNSUPPORTED
    assert _wqmm(tx2=1) == wq.WQ_ERR_UNSUPPORTED                    # GFX950_B: pack the transpose
    assert _wqmm(tx2=1, layout=wq.WQ_LAYOUT_ND, k=255) == wq.WQ_ERR_SHAPE   # (n, k/2) needs k even
    assert _wqmm(w=wq.WQ_INT8) == wq.WQ_ERR_UNSUPPORTED             # int8 in GFX950_B


def test_wq_matmul_validation_shapes():
    assert _wqmm(k=0) == wq.WQ_ERR_SHAPE                             # k = 0 is not supported
    assert _wqmm(k=65536, srows=2048) == wq.WQ_ERR_SHAPE
    assert _wqmm(n=65536) == wq.WQ_ERR_SHAPE
    assert _wqmm(m=-1) == wq.WQ_ERR_SHAPE
    assert _wqmm(m=2 ** 31) == wq.WQ_ERR_SHAPE
    assert _wqmm(n=127, layout=wq.WQ_LAYOUT_ND, scols=127) == wq.WQ_ERR_SHAPE
    assert _wqmm(eps=-1.0) == wq.WQ_ERR_SHAPE
    assert _wqmm(eps=float("nan")) == wq.WQ_ERR_SHAPE
    assert _wqmm(x1=FAKE + 8) == wq.WQ_ERR_SHAPE                     # misaligned


def test_wq_matmul_validation_groups():
    assert _wqmm(group=16, srows=16) == wq.WQ_ERR_GROUP              # below 32
    assert _wqmm(group=48, srows=6) == wq.WQ_ERR_GROUP               # not a multiple of 32
    assert _wqmm(group=256, srows=1) == wq.WQ_ERR_GROUP              # G > k - 1
    assert _wqmm(group=32, srows=7) == wq.WQ_ERR_GROUP               # rows != ceil(k/G)
    assert _wqmm(group=32, scols=64) == wq.WQ_ERR_GROUP
    assert _wqmm(group=0, srows=8) == wq.WQ_ERR_GROUP                # 2-D scale without G
    assert _wqmm(group=0, srows=1, scols=7) == wq.WQ_ERR_GROUP


def test_wq_matmul_validation_pointers_workspace_alias():
    assert _wqmm(m=0) == wq.WQ_OK and _wqmm(n=0, scols=0) == wq.WQ_OK   # empty
    assert _wqmm(gamma=None) == wq.WQ_ERR_NULLPTR
    assert _wqmm(residual=None) == wq.WQ_ERR_NULLPTR
    assert _wqmm(ws=None) == wq.WQ_ERR_WORKSPACE
    assert _wqmm(ws_size=16) == wq.WQ_ERR_WORKSPACE
    assert _wqmm(norm=FAKE + 0x30000) == wq.WQ_ERR_ALIAS             # norm_out == residual
    assert _wqmm(norm=FAKE + 0x50000) == wq.WQ_ERR_ALIAS             # norm_out == y
    assert _wqmm(y=FAKE + 0x30010) == wq.WQ_ERR_ALIAS                # y partially over residual
    assert _wqmm(y=FAKE, m=16) == wq.WQ_ERR_ALIAS                    # y over x1
    # the workspace is written before the inputs are read: it may overlap none
    assert _wqmm(ws=FAKE) == wq.WQ_ERR_ALIAS                         # over x1
    assert _wqmm(ws=FAKE + 0x10000) == wq.WQ_ERR_ALIAS               # over x2
    assert _wqmm(ws=FAKE + 0x20000) == wq.WQ_ERR_ALIAS               # over the scale
    assert _wqmm(ws=FAKE + 0x30000) == wq.WQ_ERR_ALIAS               # over residual
    assert _wqmm(ws=FAKE + 0x40000) == wq.WQ_ERR_ALIAS               # over gamma
    assert _wqmm(ws=FAKE + 0x80000, offset=FAKE + 0x80000) == wq.WQ_ERR_ALIAS  # over the offset
    assert _wqmm(ws=FAKE + 0x80000, bias=FAKE + 0x80000) == wq.WQ_ERR_ALIAS    # over bias


def test_noalloc_validation_without_a_device():
    # the size rule is checked first, on the host: nothing touches the GPU
    F = FAKE
    assert wq.wq_matmul_add_rmsnorm_workspace_size(65536, 8192, 8192) > wq.WQ_NOALLOC_MAX_WORKSPACE
    st = wq.lib().wq_matmul_add_rmsnorm_noalloc(
        F, 65536, 8192, wq.WQ_BF16, F + (1 << 32), 8192, wq.WQ_INT4, wq.WQ_LAYOUT_GFX950_B, 0,
        F + (2 << 32), 64, 8192, None, 128, None, F + (3 << 32), F + (4 << 32), 1e-6,
        F + (5 << 32), F + (6 << 32), 0)
    assert st == wq.WQ_ERR_WORKSPACE
    # the workspace call's rules apply unchanged; an empty problem is a no-op
    L = wq.lib()
    args = lambda m, act, G: (F, m, 256, act, F + 0x10000, 128, wq.WQ_INT4, wq.WQ_LAYOUT_GFX950_B, 0,
                              F + 0x20000, 8, 128, None, G, None, F + 0x30000, F + 0x40000, 1e-6,
                              F + 0x50000, F + 0x60000, 0)
    assert L.wq_matmul_add_rmsnorm_noalloc(*args(0, wq.WQ_BF16, 32)) == wq.WQ_OK
    assert L.wq_matmul_add_rmsnorm_noalloc(*args(16, wq.WQ_F32, 32)) == wq.WQ_ERR_DTYPE
    assert L.wq_matmul_add_rmsnorm_noalloc(*args(16, wq.WQ_BF16, 48)) == wq.WQ_ERR_GROUP


def _mx(**kw):
    a = dict(x1=FAKE, x2=FAKE2, layout=wq.WQ_LAYOUT_GFX950_B, s1=FAKE3, s2=FAKE3 + 0x10000,
             m=64, k=256, n=64, t1=1, t2=0, group=wq.MX_GROUP_SIZE, y=FAKE3 + 0x100000, ws=None,
             wsn=0)
    a.update(kw)
    return wq.lib().mx_quant_matmul_inplace_add(a["x1"], a["x2"], a["layout"], a["s1"], a["s2"],
                                                a["m"], a["k"], a["n"], a["t1"], a["t2"],
                                                a["group"], a["y"], a["ws"], a["wsn"], 0)


def test_mx_matmul_validation():
    assert wq.MX_GROUP_SIZE == 4295032864
    assert _mx(t1=0) == wq.WQ_ERR_UNSUPPORTED                        # only transposeX1 = true
    assert _mx(t2=1) == wq.WQ_ERR_UNSUPPORTED                        # only transposeX2 = false
    assert _mx(layout=wq.WQ_LAYOUT_ND) == wq.WQ_ERR_UNSUPPORTED
    assert _mx(group=64) == wq.WQ_ERR_GROUP
    assert _mx(group=32 | (2 << 16)) == wq.WQ_ERR_GROUP
    assert _mx(group=-1) == wq.WQ_ERR_GROUP
    assert _mx(m=-3) == wq.WQ_ERR_SHAPE
    assert _mx(y=None) == wq.WQ_ERR_NULLPTR
    assert _mx(y=FAKE2 + 4) == wq.WQ_ERR_SHAPE
    assert _mx(y=FAKE2 + 16) == wq.WQ_ERR_ALIAS                      # y over x2
    # the tiled kernel copies x1 in 16-byte and the scales in 4-byte pieces
    assert _mx(x1=FAKE + 8) == wq.WQ_ERR_SHAPE
    assert _mx(s1=FAKE3 + 1) == wq.WQ_ERR_SHAPE
    assert _mx(s2=FAKE3 + 0x10002) == wq.WQ_ERR_SHAPE
    assert _mx(m=0) == wq.WQ_OK and _mx(k=0) == wq.WQ_OK
    # the optional workspace (m % 16 != 0): checked only when it is large enough to be used
    need = wq.mx_quant_matmul_inplace_add_workspace_size(60, 256, 64)
    assert need == 256 * 64
    assert _mx(m=60, ws=FAKE3 + 0x200008, wsn=need) == wq.WQ_ERR_SHAPE         # misaligned
    assert _mx(m=60, ws=FAKE3 + 0x100000, wsn=need) == wq.WQ_ERR_ALIAS         # over y
    assert _mx(m=60, ws=FAKE + 0x10, wsn=need) == wq.WQ_ERR_ALIAS              # over x1


def _qmm(**kw):
    a = dict(x1=FAKE, x2=FAKE2, s1=FAKE3, s2=FAKE3 + 0x4000, m=32, k=64, n=48, y=FAKE + 0x40000000,
             stream=0)
    a.update(kw)
    return wq.lib().wq_quant_matmul_inplace_add(a["x1"], a["x2"], a["s1"], a["s2"], a["m"], a["k"],
                                                a["n"], a["y"], a["stream"])


def test_int8_matmul_validation():
    assert _qmm(k=0) == wq.WQ_ERR_SHAPE
    assert _qmm(k=40) == wq.WQ_ERR_SHAPE                   # k % 16
    assert _qmm(k=65536) == wq.WQ_ERR_SHAPE
    assert _qmm(n=65536) == wq.WQ_ERR_SHAPE
    assert _qmm(m=-1) == wq.WQ_ERR_SHAPE
    assert _qmm(x1=None) == wq.WQ_ERR_NULLPTR
    assert _qmm(s2=None) == wq.WQ_ERR_NULLPTR
    assert _qmm(x2=FAKE2 + 8) == wq.WQ_ERR_SHAPE           # 16-byte operand rows
    assert _qmm(y=FAKE + 0x40000002) == wq.WQ_ERR_SHAPE    # float alignment
    assert _qmm(y=FAKE + 64) == wq.WQ_ERR_ALIAS            # y over x1
    assert _qmm(m=0) == wq.WQ_OK and _qmm(n=0) == wq.WQ_OK


def _w4mm(**kw):
    a = dict(x1=FAKE, dt=wq.WQ_INT8, x2=FAKE2, layout=wq.WQ_LAYOUT_GFX950_B, s1=FAKE3,
             s2=FAKE3 + 0x4000, m=32, k=64, n=48, y=FAKE + 0x40000000, stream=0)
    a.update(kw)
    return wq.lib().wq_quant_matmul_inplace_add_w4(a["x1"], a["dt"], a["x2"], a["layout"], a["s1"],
                                                   a["s2"], a["m"], a["k"], a["n"], a["y"], a["stream"])


def test_a8w4_matmul_validation():
    assert _w4mm(dt=wq.WQ_FP8_E4M3) == wq.WQ_ERR_DTYPE
    assert _w4mm(dt=wq.WQ_INT4, k=48) == wq.WQ_ERR_SHAPE    # INT4 x1: k % 32
    assert _w4mm(dt=wq.WQ_INT4, m=0) == wq.WQ_OK
    assert _w4mm(layout=wq.WQ_LAYOUT_ND) == wq.WQ_ERR_UNSUPPORTED
    assert _w4mm(k=0) == wq.WQ_ERR_SHAPE
    assert _w4mm(k=40) == wq.WQ_ERR_SHAPE                  # k % 16
    assert _w4mm(k=65536) == wq.WQ_ERR_SHAPE
    assert _w4mm(n=65536) == wq.WQ_ERR_SHAPE
    assert _w4mm(m=-1) == wq.WQ_ERR_SHAPE
    assert _w4mm(x1=None) == wq.WQ_ERR_NULLPTR
    assert _w4mm(s1=None) == wq.WQ_ERR_NULLPTR
    assert _w4mm(x2=FAKE2 + 8) == wq.WQ_ERR_SHAPE          # 16-byte weight records
    assert _w4mm(y=FAKE + 0x40000002) == wq.WQ_ERR_SHAPE   # float alignment
    # the packed weight of k = 65520, n = 65535 is 512 * 65536 * 64 = 2^31 bytes
    assert wq.wq_pack_int4_bytes(65520, 65535, wq.WQ_LAYOUT_GFX950_B) == 1 << 31
    assert _w4mm(k=65520, n=65535) == wq.WQ_ERR_SHAPE
    assert _w4mm(y=FAKE2 + 64) == wq.WQ_ERR_ALIAS          # y over x2
    assert _w4mm(m=0) == wq.WQ_OK and _w4mm(n=0) == wq.WQ_OK


def _wqbmm(**kw):
    # the standalone matmul on the fused call's defaults (no residual, gamma,
    # epsilon or norm_out); out where the fused call has y
    m, k, n = kw.pop("m", 64), kw.pop("k", 256), kw.pop("n", 128)
    a = dict(x1=FAKE, act=wq.WQ_BF16, x2=FAKE + 0x10000, w=wq.WQ_INT4,
             layout=wq.WQ_LAYOUT_GFX950_B, tx2=0, scale=FAKE + 0x20000, srows=8, scols=n,
             offset=None, group=32, bias=None, out=FAKE + 0x50000, ws=FAKE2,
             ws_size=wq.wq_weight_quant_matmul_workspace_size(m, k, n))
    a.update(kw)
    return wq.lib().wq_weight_quant_matmul(
        a["x1"], m, k, a["act"], a["x2"], n, a["w"], a["layout"], a["tx2"], a["scale"],
        a["srows"], a["scols"], a["offset"], a["group"], a["bias"], a["out"], a["ws"],
        a["ws_size"], 0)


def test_weight_quant_matmul_validation():
    assert wq.wq_weight_quant_matmul_workspace_size(64, 256, 128) == \
        wq.wq_matmul_add_rmsnorm_workspace_size(64, 256, 128)
    assert _wqbmm(act=wq.WQ_F32) == wq.WQ_ERR_DTYPE
    assert _wqbmm(tx2=1) == wq.WQ_ERR_UNSUPPORTED
    assert _wqbmm(k=0) == wq.WQ_ERR_SHAPE
    assert _wqbmm(n=65536) == wq.WQ_ERR_SHAPE
    assert _wqbmm(group=48, srows=6) == wq.WQ_ERR_GROUP
    assert _wqbmm(m=0) == wq.WQ_OK
    assert _wqbmm(out=None) == wq.WQ_ERR_NULLPTR
    assert _wqbmm(ws=None) == wq.WQ_ERR_WORKSPACE
    assert _wqbmm(out=FAKE + 0x50008) == wq.WQ_ERR_SHAPE             # misaligned
    assert _wqbmm(out=FAKE + 0x10000) == wq.WQ_ERR_ALIAS             # out over x2
    assert _wqbmm(out=FAKE2 + 0x100) == wq.WQ_ERR_ALIAS              # out over the workspace
    assert _wqbmm(ws=FAKE) == wq.WQ_ERR_ALIAS                        # workspace over x1
    assert _wqbmm(ws=FAKE + 0x20000) == wq.WQ_ERR_ALIAS              # workspace over the scale


def _arn(**kw):
    # five disjoint regions (each row block is 64 x 1024 x 2 = 0x20000 bytes)
    a = dict(x=FAKE, res=FAKE + 0x100000, gamma=FAKE + 0x200000, rows=64, cols=1024,
             dt=wq.WQ_BF16, eps=1e-6, y=FAKE + 0x300000, norm=FAKE + 0x400000)
    a.update(kw)
    return wq.lib().wq_add_rms_norm(a["x"], a["res"], a["gamma"], a["rows"], a["cols"], a["dt"],
                                    a["eps"], a["y"], a["norm"], 0)


def test_add_rms_norm_validation():
    assert _arn(dt=wq.WQ_INT8) == wq.WQ_ERR_DTYPE
    assert _arn(cols=0) == wq.WQ_ERR_SHAPE
    assert _arn(cols=65536) == wq.WQ_ERR_SHAPE
    assert _arn(rows=-1) == wq.WQ_ERR_SHAPE
    assert _arn(eps=-1.0) == wq.WQ_ERR_SHAPE
    assert _arn(eps=float("inf")) == wq.WQ_ERR_SHAPE
    assert _arn(rows=0) == wq.WQ_OK
    assert _arn(gamma=None) == wq.WQ_ERR_NULLPTR
    assert _arn(x=FAKE + 2) == wq.WQ_ERR_SHAPE                       # misaligned
    assert _arn(y=FAKE + 0x10) == wq.WQ_ERR_ALIAS                    # y partly over x
    assert _arn(norm=FAKE + 0x100000) == wq.WQ_ERR_ALIAS             # norm_out == residual
    assert _arn(norm=FAKE + 0x300000) == wq.WQ_ERR_ALIAS             # norm_out == y
    assert _arn(norm=FAKE + 0x200000 - 0x10) == wq.WQ_ERR_ALIAS      # norm_out over gamma
    assert _arn(y=FAKE + 0x200000 - 0x10) == wq.WQ_ERR_ALIAS         # y over gamma
    # in place is allowed: y == x or y == residual pass every host check (not
    # called here: a valid call would launch)



def test_pack_fp4_validation():
    L = wq.lib()
    assert L.wq_pack_fp4(FAKE, 256, 128, 0, 5, FAKE2, 0) == wq.WQ_ERR_UNSUPPORTED
    assert L.wq_pack_fp4(FAKE, -1, 128, 0, wq.WQ_LAYOUT_GFX950_B, FAKE2, 0) == wq.WQ_ERR_SHAPE
    assert L.wq_pack_fp4(FAKE, 256, 127, 0, wq.WQ_LAYOUT_ND, FAKE2, 0) == wq.WQ_ERR_SHAPE
    assert L.wq_pack_fp4(None, 256, 128, 0, wq.WQ_LAYOUT_GFX950_B, FAKE2, 0) == wq.WQ_ERR_NULLPTR
    assert L.wq_pack_fp4(FAKE, 256, 128, 0, wq.WQ_LAYOUT_GFX950_B, FAKE2 + 8, 0) == wq.WQ_ERR_SHAPE
    assert L.wq_pack_fp4(FAKE, 256, 128, 0, wq.WQ_LAYOUT_GFX950_B, FAKE + 64, 0) == wq.WQ_ERR_ALIAS
    assert L.wq_pack_fp4(FAKE, 0, 128, 0, wq.WQ_LAYOUT_GFX950_B, FAKE2, 0) == wq.WQ_OK


def _mx4(**kw):
    m, k, n = kw.pop("m", 256), kw.pop("k", 512), kw.pop("n", 256)
    a = dict(x1=FAKE, x2=FAKE + 0x100000, layout=wq.WQ_LAYOUT_GFX950_B, s1=FAKE + 0x200000,
             s2=FAKE + 0x300000, group=wq.MX_GROUP_SIZE, y=FAKE + 0x400000, ws=FAKE + 0x800000,
             ws_size=wq.mx_fp4_quant_matmul_inplace_add_workspace_size(m, k, n))
    a.update(kw)
    return wq.lib().mx_fp4_quant_matmul_inplace_add(a["x1"], a["x2"], a["layout"], a["s1"], a["s2"], m, k,
                                                    n, a["group"], a["y"], a["ws"], a["ws_size"], 0)


def test_mx_fp4_matmul_validation():
    # 2 m-tiles + 1 n-tile, 4 steps of 128, 1 KiB each
    assert wq.mx_fp4_quant_matmul_inplace_add_workspace_size(300, 512, 200) == (2 + 1) * 4 * 1024
    assert _mx4(layout=wq.WQ_LAYOUT_ND) == wq.WQ_ERR_UNSUPPORTED
    assert _mx4(k=48) == wq.WQ_ERR_SHAPE                              # k % 32
    assert _mx4(k=0) == wq.WQ_ERR_SHAPE
    assert _mx4(n=65536) == wq.WQ_ERR_SHAPE
    assert _mx4(group=64) == wq.WQ_ERR_GROUP
    assert _mx4(group=0, ws=None) == wq.WQ_ERR_WORKSPACE                # 0 passes the group rule
    assert _mx4(m=0) == wq.WQ_OK
    assert _mx4(y=None) == wq.WQ_ERR_NULLPTR
    assert _mx4(ws=None) == wq.WQ_ERR_WORKSPACE
    assert _mx4(ws_size=1024) == wq.WQ_ERR_WORKSPACE
    assert _mx4(x1=FAKE + 8) == wq.WQ_ERR_SHAPE                       # misaligned
    assert _mx4(y=FAKE + 0x100000) == wq.WQ_ERR_ALIAS                 # y over x2
    assert _mx4(ws=FAKE + 0x200000) == wq.WQ_ERR_ALIAS                # workspace over x1's scales


def test_ceiling_microkernels_validate_on_the_host():
    L = wq.lib()
    assert L.wq_ceiling_stream_read_words(0) == 0
    assert L.wq_ceiling_stream_read_words(24) == 0                # not a multiple of 16
    assert L.wq_ceiling_stream_read_words(16) == 4                # one workgroup, four waves
    assert L.wq_ceiling_stream_read_words(16384) == 4
    assert L.wq_ceiling_stream_read_words(16400) == 8
    assert L.wq_ceiling_stream_read_words(1 << 40) == 0
    assert L.wq_ceiling_stream_read(None, 16, FAKE, None) == wq.WQ_ERR_NULLPTR
    assert L.wq_ceiling_stream_read(FAKE, 16, None, None) == wq.WQ_ERR_NULLPTR
    assert L.wq_ceiling_stream_read(FAKE, 24, FAKE2, None) == wq.WQ_ERR_SHAPE
    assert L.wq_ceiling_stream_read(FAKE + 8, 16, FAKE2, None) == wq.WQ_ERR_SHAPE
    assert L.wq_ceiling_stream_read(FAKE, 16, FAKE2 + 2, None) == wq.WQ_ERR_SHAPE
    assert L.wq_ceiling_stream_read(FAKE, 1 << 20, FAKE + 4096, None) == wq.WQ_ERR_ALIAS
    assert L.wq_ceiling_mfma_loop(1, 1, None, None) == wq.WQ_ERR_NULLPTR
    assert L.wq_ceiling_mfma_loop(0, 1, FAKE, None) == wq.WQ_ERR_SHAPE
    assert L.wq_ceiling_mfma_loop((1 << 20) + 1, 1, FAKE, None) == wq.WQ_ERR_SHAPE
    assert L.wq_ceiling_mfma_loop(1, 0, FAKE, None) == wq.WQ_ERR_SHAPE
    assert L.wq_ceiling_mfma_loop(1, 16385, FAKE, None) == wq.WQ_ERR_SHAPE
