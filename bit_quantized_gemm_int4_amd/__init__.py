"""Python binding of libwq (argument marshalling only).

Every computation runs in the HIP kernels of ``libwq.so``; this module only
turns tensors into device pointers and sizes, calls the C ABI declared in
``include/wq.h`` through ctypes on torch's current stream, and raises
:class:`WqError` on a non-zero status. PyTorch provides device memory and
streams. Importing works without the library; the first call raises
``ImportError`` if ``libwq.so`` has not been built, and nothing falls back
to another implementation.

The C names are exported unchanged (``wq_pack_int4``, ``wq_dynamic_quant``,
``wq_matmul_add_rmsnorm``, ``mx_quant_matmul_inplace_add`` and the size
queries); the lower-case helpers without the prefix allocate outputs with
torch and call them.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwq.so")

# wq_status
WQ_OK, WQ_ERR_NULLPTR, WQ_ERR_SHAPE, WQ_ERR_DTYPE, WQ_ERR_GROUP = 0, 1, 2, 3, 4
WQ_ERR_WORKSPACE, WQ_ERR_UNSUPPORTED, WQ_ERR_LAUNCH, WQ_ERR_ALIAS = 5, 6, 7, 8
# wq_dtype
WQ_F16, WQ_BF16, WQ_F32, WQ_INT8, WQ_INT4 = 1, 2, 3, 4, 5
WQ_INT32, WQ_FP8_E4M3, WQ_FP4_E2M1, WQ_E8M0 = 6, 7, 8, 9
# wq_layout
WQ_LAYOUT_ND, WQ_LAYOUT_GFX950_B = 0, 1

MX_GROUP_SIZE = 32 | (1 << 16) | (1 << 32)
WQ_NOALLOC_MAX_WORKSPACE = 32 << 20      # the allocation-free call's device array

EXPORTS = (
    "wq_status_string", "wq_abi_version",
    "wq_pack_int4_bytes", "wq_pack_int4", "wq_pack_fp4",
    "wq_dynamic_quant",
    "wq_matmul_add_rmsnorm_workspace_size", "wq_matmul_add_rmsnorm",
    "wq_matmul_add_rmsnorm_noalloc",
    "mx_quant_matmul_inplace_add_workspace_size", "mx_quant_matmul_inplace_add",
    "wq_quant_matmul_inplace_add", "wq_quant_matmul_inplace_add_w4",
    "mx_fp4_quant_matmul_inplace_add_workspace_size", "mx_fp4_quant_matmul_inplace_add",
    "wq_weight_quant_matmul_workspace_size", "wq_weight_quant_matmul", "wq_add_rms_norm",
    "wq_profile_enable", "wq_profile_read",
    "wq_ceiling_stream_read_words", "wq_ceiling_stream_read", "wq_ceiling_mfma_loop",
)

_lib = None


class WqError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__(f"{fn}: {lib().wq_status_string(status).decode()}")


def lib() -> ctypes.CDLL:
    """The loaded libwq (declares argument types on first use)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                              "or python -m bit_quantized_gemm_int4_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I, D, S = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_size_t
        sig = {
            "wq_status_string": (ctypes.c_char_p, [I]),
            "wq_abi_version": (I, []),
            "wq_pack_int4_bytes": (S, [I64, I64, I]),
            "wq_pack_int4": (I, [P, I64, I64, I, I, P, P]),
            "wq_pack_fp4": (I, [P, I64, I64, I, I, P, P]),
            "wq_dynamic_quant": (I, [P, I, I64, I64, P, I, I64, I, P, P, P]),
            "wq_matmul_add_rmsnorm_workspace_size": (S, [I64, I64, I64]),
            "wq_matmul_add_rmsnorm": (I, [P, I64, I64, I, P, I64, I, I, I, P, I64, I64, P, I64,
                                          P, P, P, D, P, P, P, S, P]),
            "wq_matmul_add_rmsnorm_noalloc": (I, [P, I64, I64, I, P, I64, I, I, I, P, I64, I64, P,
                                                  I64, P, P, P, D, P, P, P]),
            "mx_quant_matmul_inplace_add_workspace_size": (S, [I64, I64, I64]),
            "mx_quant_matmul_inplace_add": (I, [P, P, I, P, P, I64, I64, I64, I, I, I64, P, P, S, P]),
            "wq_quant_matmul_inplace_add": (I, [P, P, P, P, I64, I64, I64, P, P]),
            "wq_quant_matmul_inplace_add_w4": (I, [P, I, P, I, P, P, I64, I64, I64, P, P]),
            "mx_fp4_quant_matmul_inplace_add_workspace_size": (S, [I64, I64, I64]),
            "mx_fp4_quant_matmul_inplace_add": (I, [P, P, I, P, P, I64, I64, I64, I64, P, P, S, P]),
            "wq_weight_quant_matmul_workspace_size": (S, [I64, I64, I64]),
            "wq_weight_quant_matmul": (I, [P, I64, I64, I, P, I64, I, I, I, P, I64, I64, P, I64,
                                           P, P, P, S, P]),
            "wq_add_rms_norm": (I, [P, P, P, I64, I64, I, D, P, P, P]),
            "wq_profile_enable": (I, [I]),
            "wq_profile_read": (I, [P, I64, ctypes.POINTER(I64)]),
            "wq_ceiling_stream_read_words": (S, [S]),
            "wq_ceiling_stream_read": (I, [P, S, P, P]),
            "wq_ceiling_mfma_loop": (I, [I64, ctypes.c_int32, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(t) -> Optional[int]:
    """A tensor's address for the C ABI, which reads every tensor as dense
    row-major memory: a strided view is refused, not reinterpreted."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("libwq takes contiguous tensors (call .contiguous() first)")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, fn: str, check: bool) -> int:
    if check and status != WQ_OK:
        raise WqError(status, fn)
    return status


def act_code(dtype: torch.dtype) -> int:
    return {torch.float16: WQ_F16, torch.bfloat16: WQ_BF16}[dtype]


# ---- the C entry points, one to one ------------------------------------------

def wq_pack_int4_bytes(k: int, n: int, layout: int) -> int:
    return lib().wq_pack_int4_bytes(k, n, layout)


def wq_pack_int4(weight, k, n, transpose, layout, out, stream=None, check=True) -> int:
    st = lib().wq_pack_int4(_ptr(weight), k, n, int(transpose), layout, _ptr(out), _stream(stream))
    return _check(st, "wq_pack_int4", check)


def wq_dynamic_quant(x, x_dtype, rows, cols, smooth, y_dtype, block_k, transpose_y, y, scale,
                     stream=None, check=True) -> int:
    st = lib().wq_dynamic_quant(_ptr(x), x_dtype, rows, cols, _ptr(smooth), y_dtype, block_k,
                                int(transpose_y), _ptr(y), _ptr(scale), _stream(stream))
    return _check(st, "wq_dynamic_quant", check)


def wq_quant_matmul_inplace_add(x1, x2, x1_scale, x2_scale, m, k, n, y, stream=None,
                                check=True) -> int:
    st = lib().wq_quant_matmul_inplace_add(_ptr(x1), _ptr(x2), _ptr(x1_scale), _ptr(x2_scale), m, k,
                                           n, _ptr(y), _stream(stream))
    return _check(st, "wq_quant_matmul_inplace_add", check)


def wq_quant_matmul_inplace_add_w4(x1, x1_dtype, x2, x2_layout, x1_scale, x2_scale, m, k, n, y,
                                   stream=None, check=True) -> int:
    st = lib().wq_quant_matmul_inplace_add_w4(_ptr(x1), x1_dtype, _ptr(x2), x2_layout, _ptr(x1_scale),
                                              _ptr(x2_scale), m, k, n, _ptr(y), _stream(stream))
    return _check(st, "wq_quant_matmul_inplace_add_w4", check)


def wq_profile_enable(enable: bool, check=True) -> int:
    return _check(lib().wq_profile_enable(int(enable)), "wq_profile_enable", check)


def wq_profile_read(capacity: int = 4096, check=True):
    """Per-launch contraction-kernel times (ms, launch order) recorded since
    the last enable / read."""
    buf = (ctypes.c_float * max(capacity, 1))()
    n = ctypes.c_int64(0)
    _check(lib().wq_profile_read(ctypes.addressof(buf), capacity, ctypes.byref(n)),
           "wq_profile_read", check)
    return [buf[i] for i in range(min(n.value, capacity))]


def wq_ceiling_stream_read_words(nbytes: int) -> int:
    return lib().wq_ceiling_stream_read_words(nbytes)


def wq_ceiling_stream_read(src, nbytes, out, stream=None, check=True) -> int:
    st = lib().wq_ceiling_stream_read(_ptr(src), nbytes, _ptr(out), _stream(stream))
    return _check(st, "wq_ceiling_stream_read", check)


def wq_ceiling_mfma_loop(workgroups, iters, out, stream=None, check=True) -> int:
    st = lib().wq_ceiling_mfma_loop(workgroups, iters, _ptr(out), _stream(stream))
    return _check(st, "wq_ceiling_mfma_loop", check)


def wq_matmul_add_rmsnorm_workspace_size(m: int, k: int, n: int) -> int:
    return lib().wq_matmul_add_rmsnorm_workspace_size(m, k, n)


def wq_matmul_add_rmsnorm(x1, m, k, act_dtype, x2, n, w_dtype, x2_layout, transpose_x2,
                          scale, scale_rows, scale_cols, offset, group_size, bias, residual,
                          gamma, epsilon, y, norm_out, workspace, workspace_size,
                          stream=None, check=True) -> int:
    st = lib().wq_matmul_add_rmsnorm(
        _ptr(x1), m, k, act_dtype, _ptr(x2), n, w_dtype, x2_layout, int(transpose_x2),
        _ptr(scale), scale_rows, scale_cols, _ptr(offset), group_size, _ptr(bias),
        _ptr(residual), _ptr(gamma), float(epsilon), _ptr(y), _ptr(norm_out),
        _ptr(workspace), workspace_size, _stream(stream))
    return _check(st, "wq_matmul_add_rmsnorm", check)


def wq_matmul_add_rmsnorm_noalloc(x1, m, k, act_dtype, x2, n, w_dtype, x2_layout, transpose_x2,
                                  scale, scale_rows, scale_cols, offset, group_size, bias,
                                  residual, gamma, epsilon, y, norm_out, stream=None,
                                  check=True) -> int:
    st = lib().wq_matmul_add_rmsnorm_noalloc(
        _ptr(x1), m, k, act_dtype, _ptr(x2), n, w_dtype, x2_layout, int(transpose_x2),
        _ptr(scale), scale_rows, scale_cols, _ptr(offset), group_size, _ptr(bias),
        _ptr(residual), _ptr(gamma), float(epsilon), _ptr(y), _ptr(norm_out), _stream(stream))
    return _check(st, "wq_matmul_add_rmsnorm_noalloc", check)


def wq_pack_fp4(weight, k, n, transpose, layout, out, stream=None, check=True) -> int:
    st = lib().wq_pack_fp4(_ptr(weight), k, n, int(transpose), layout, _ptr(out), _stream(stream))
    return _check(st, "wq_pack_fp4", check)


def mx_fp4_quant_matmul_inplace_add_workspace_size(m: int, k: int, n: int) -> int:
    return lib().mx_fp4_quant_matmul_inplace_add_workspace_size(m, k, n)


def mx_fp4_quant_matmul_inplace_add(x1, x2, x2_layout, x1_scale, x2_scale, m, k, n, group_size, y,
                                    workspace, workspace_size, stream=None, check=True) -> int:
    st = lib().mx_fp4_quant_matmul_inplace_add(
        _ptr(x1), _ptr(x2), x2_layout, _ptr(x1_scale), _ptr(x2_scale), m, k, n, group_size, _ptr(y),
        _ptr(workspace), workspace_size, _stream(stream))
    return _check(st, "mx_fp4_quant_matmul_inplace_add", check)


def wq_weight_quant_matmul_workspace_size(m: int, k: int, n: int) -> int:
    return lib().wq_weight_quant_matmul_workspace_size(m, k, n)


def wq_weight_quant_matmul(x1, m, k, act_dtype, x2, n, w_dtype, x2_layout, transpose_x2,
                           scale, scale_rows, scale_cols, offset, group_size, bias, out,
                           workspace, workspace_size, stream=None, check=True) -> int:
    st = lib().wq_weight_quant_matmul(
        _ptr(x1), m, k, act_dtype, _ptr(x2), n, w_dtype, x2_layout, int(transpose_x2),
        _ptr(scale), scale_rows, scale_cols, _ptr(offset), group_size, _ptr(bias), _ptr(out),
        _ptr(workspace), workspace_size, _stream(stream))
    return _check(st, "wq_weight_quant_matmul", check)


def wq_add_rms_norm(x, residual, gamma, rows, cols, dtype, epsilon, y, norm_out, stream=None,
                    check=True) -> int:
    st = lib().wq_add_rms_norm(_ptr(x), _ptr(residual), _ptr(gamma), rows, cols, dtype,
                               float(epsilon), _ptr(y), _ptr(norm_out), _stream(stream))
    return _check(st, "wq_add_rms_norm", check)


def mx_quant_matmul_inplace_add_workspace_size(m: int, k: int, n: int) -> int:
    return lib().mx_quant_matmul_inplace_add_workspace_size(m, k, n)


def mx_quant_matmul_inplace_add(x1, x2, x2_layout, x1_scale, x2_scale, m, k, n, transpose_x1,
                                transpose_x2, group_size, y, workspace=None, workspace_size=0,
                                stream=None, check=True) -> int:
    st = lib().mx_quant_matmul_inplace_add(
        _ptr(x1), _ptr(x2), x2_layout, _ptr(x1_scale), _ptr(x2_scale), m, k, n,
        int(transpose_x1), int(transpose_x2), group_size, _ptr(y), _ptr(workspace),
        workspace_size, _stream(stream))
    return _check(st, "mx_quant_matmul_inplace_add", check)


# ---- allocating helpers (torch for memory only) -------------------------------

def pack_int4(weight: torch.Tensor, layout: int = WQ_LAYOUT_GFX950_B, transpose: bool = False,
              stream=None) -> torch.Tensor:
    """Pack a device int32 weight (k, n) (or (n, k) with ``transpose``)."""
    k, n = (weight.shape[1], weight.shape[0]) if transpose else tuple(weight.shape)
    out = torch.empty(wq_pack_int4_bytes(k, n, layout), dtype=torch.uint8, device=weight.device)
    wq_pack_int4(weight, k, n, transpose, layout, out, stream)
    return out


def dynamic_quant(x: torch.Tensor, smooth: Optional[torch.Tensor] = None, y_dtype: int = WQ_INT8,
                  block_k: int = 0, transpose_y: bool = False, stream=None):
    """Returns (y, scale) of the dynamic quantization of ``x`` (rows = all but
    the last dimension)."""
    cols = x.shape[-1]
    rows = x.numel() // cols if cols else 0
    dev = x.device
    if block_k == 0:
        shape = {WQ_INT8: (rows, cols), WQ_INT4: (rows, cols // 2), WQ_INT32: (rows, cols // 8)}[y_dtype]
        dt = {WQ_INT8: torch.int8, WQ_INT4: torch.uint8, WQ_INT32: torch.int32}[y_dtype]
        y = torch.empty(shape, dtype=dt, device=dev)
        scale = torch.empty(rows, dtype=torch.float32, device=dev)
    else:
        if y_dtype == WQ_FP8_E4M3:
            shape = (cols, rows) if transpose_y else (rows, cols)
        else:
            shape = (rows, cols // 2)
        y = torch.empty(shape, dtype=torch.uint8, device=dev)
        scale = torch.empty((rows, (cols + 31) // 32), dtype=torch.uint8, device=dev)
    wq_dynamic_quant(x, act_code(x.dtype), rows, cols, smooth, y_dtype, block_k, transpose_y,
                     y, scale, stream)
    return y, scale


def matmul_add_rmsnorm(x1: torch.Tensor, x2: torch.Tensor, k: int, n: int, w_dtype: int,
                       scale: torch.Tensor, offset: Optional[torch.Tensor], group_size: int,
                       bias: Optional[torch.Tensor], residual: torch.Tensor, gamma: torch.Tensor,
                       eps: float, layout: int = WQ_LAYOUT_GFX950_B, transpose_x2: bool = False,
                       inplace: bool = False, workspace: Optional[torch.Tensor] = None,
                       norm_out: Optional[torch.Tensor] = None, stream=None):
    """Returns (y, norm_out); ``inplace`` writes y into ``residual``."""
    m = x1.numel() // k
    if scale.dim() == 2:
        s_rows, s_cols = scale.shape
    else:
        s_rows, s_cols = 1, scale.numel()
    y = residual if inplace else torch.empty_like(residual)
    if norm_out is None:
        norm_out = torch.empty_like(residual)
    ws = wq_matmul_add_rmsnorm_workspace_size(m, k, n)
    if workspace is None or workspace.numel() < ws:
        workspace = torch.zeros(ws, dtype=torch.uint8, device=x1.device)
    wq_matmul_add_rmsnorm(x1, m, k, act_code(x1.dtype), x2, n, w_dtype, layout, transpose_x2,
                          scale, s_rows, s_cols, offset, group_size, bias, residual, gamma, eps,
                          y, norm_out, workspace, workspace.numel(), stream)
    return y, norm_out


def mx_matmul_inplace_add(x1_t: torch.Tensor, x2_packed: torch.Tensor, x1_scale: torch.Tensor,
                          x2_scale: torch.Tensor, y: torch.Tensor, m: int, k: int, n: int,
                          group_size: int = MX_GROUP_SIZE, stream=None) -> torch.Tensor:
    """y += the MX block-32 product; x1_t is (k, m) E4M3, x2 GFX950_B E2M1.
    Allocates the optional workspace the size query asks for (m not a
    multiple of 16: the large tile on a padded copy of x1)."""
    wsn = mx_quant_matmul_inplace_add_workspace_size(m, k, n)
    ws = torch.empty(wsn, dtype=torch.uint8, device=y.device) if wsn else None
    mx_quant_matmul_inplace_add(x1_t, x2_packed, WQ_LAYOUT_GFX950_B, x1_scale, x2_scale, m, k, n,
                                1, 0, group_size, y, ws, wsn, stream)
    return y


def quant_matmul_inplace_add(x1: torch.Tensor, x2_t: torch.Tensor, x1_scale: torch.Tensor,
                             x2_scale: torch.Tensor, y: torch.Tensor, stream=None) -> torch.Tensor:
    """y += (x1 @ x2_t.T) * x1_scale[:, None] * x2_scale[None, :] with INT8
    x1 (m, k), x2_t (n, k), float32 scales and y (m, n) updated in place."""
    m, k = x1.shape
    n = x2_t.shape[0]
    wq_quant_matmul_inplace_add(x1, x2_t, x1_scale, x2_scale, m, k, n, y, stream)
    return y


def quant_matmul_inplace_add_w4(x1: torch.Tensor, x2_packed: torch.Tensor, n: int,
                                x1_scale: torch.Tensor, x2_scale: torch.Tensor, y: torch.Tensor,
                                x1_int4: bool = False, stream=None) -> torch.Tensor:
    """y += (x1 @ q) * x1_scale[:, None] * x2_scale[None, :] with x1 INT8
    (m, k) or, with ``x1_int4``, INT4 codes packed (m, k/2); INT4 codes q
    (k, n) packed in GFX950_B; float32 scales; y (m, n) updated in place."""
    m = x1.shape[0]
    k = x1.shape[1] * (2 if x1_int4 else 1)
    wq_quant_matmul_inplace_add_w4(x1, WQ_INT4 if x1_int4 else WQ_INT8, x2_packed,
                                   WQ_LAYOUT_GFX950_B, x1_scale, x2_scale, m, k, n, y, stream)
    return y


def weight_quant_matmul(x1: torch.Tensor, x2: torch.Tensor, k: int, n: int, w_dtype: int,
                        scale: torch.Tensor, offset: Optional[torch.Tensor], group_size: int,
                        bias: Optional[torch.Tensor], layout: int = WQ_LAYOUT_GFX950_B,
                        transpose_x2: bool = False, out: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """out = x1 @ (x2 * scale + offset) + bias, (m, n) in x1's dtype."""
    m = x1.numel() // k
    if scale.dim() == 2:
        s_rows, s_cols = scale.shape
    else:
        s_rows, s_cols = 1, scale.numel()
    if out is None:
        out = torch.empty((m, n), dtype=x1.dtype, device=x1.device)
    ws = wq_weight_quant_matmul_workspace_size(m, k, n)
    if workspace is None or workspace.numel() < ws:
        workspace = torch.zeros(max(ws, 1), dtype=torch.uint8, device=x1.device)
    wq_weight_quant_matmul(x1, m, k, act_code(x1.dtype), x2, n, w_dtype, layout, transpose_x2,
                           scale, s_rows, s_cols, offset, group_size, bias, out, workspace,
                           workspace.numel(), stream)
    return out


def add_rms_norm(x: torch.Tensor, residual: torch.Tensor, gamma: torch.Tensor, eps: float,
                 y: Optional[torch.Tensor] = None, norm_out: Optional[torch.Tensor] = None,
                 stream=None):
    """Returns (y, norm_out): y = x + residual, norm_out = y / RMS(y) * gamma
    over the last dimension."""
    cols = gamma.numel()
    rows = x.numel() // cols
    if y is None:
        y = torch.empty_like(x)
    if norm_out is None:
        norm_out = torch.empty_like(x)
    wq_add_rms_norm(x, residual, gamma, rows, cols, act_code(x.dtype), eps, y, norm_out, stream)
    return y, norm_out


def pack_fp4(weight: torch.Tensor, layout: int = WQ_LAYOUT_GFX950_B, transpose: bool = False,
             stream=None) -> torch.Tensor:
    """FLOAT -> packed E2M1 codes; ``weight`` float32 (k, n), or (n, k) with
    ``transpose``."""
    if transpose:
        n, k = weight.shape
    else:
        k, n = weight.shape
    out = torch.empty(wq_pack_int4_bytes(k, n, layout), dtype=torch.uint8, device=weight.device)
    wq_pack_fp4(weight, k, n, transpose, layout, out, stream)
    return out


def mxfp4_matmul_inplace_add(x1: torch.Tensor, x2_packed: torch.Tensor, x1_scale: torch.Tensor,
                             x2_scale: torch.Tensor, y: torch.Tensor, m: int, k: int, n: int,
                             group_size: int = MX_GROUP_SIZE, workspace: Optional[torch.Tensor] = None,
                             stream=None) -> torch.Tensor:
    """y += the MXFP4 x MXFP4 block-32 product; x1 (m, k/2) packed E2M1,
    x2 GFX950_B E2M1."""
    ws = mx_fp4_quant_matmul_inplace_add_workspace_size(m, k, n)
    if workspace is None or workspace.numel() < ws:
        workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=y.device)
    mx_fp4_quant_matmul_inplace_add(x1, x2_packed, WQ_LAYOUT_GFX950_B, x1_scale, x2_scale, m, k, n,
                                    group_size, y, workspace, workspace.numel(), stream)
    return y

