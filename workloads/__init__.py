"""Seeded synthetic inputs for the weight-quantized matmul workloads.

This module only draws random numbers and casts them to the storage dtypes the
operators take (fp16/bf16 by round-to-nearest-even, int32 integers, raw code
bytes). It holds none of the operators' arithmetic, so that the CPU oracle and
the HIP path can both consume it without sharing any of the method.

Every workload uses numpy's PCG64 with one child stream per tensor, spawned from
``SeedSequence(seed)`` in the order the tensors are listed, so a tensor's values
do not depend on the shapes of the tensors drawn before it.

Workloads (shapes and distributions as the weight-quantized matmul operators of
the aclnnWeightQuantMatmulAllReduceAddRmsNorm / aclnnDynamicQuant /
aclnnQuantBatchMatmulInplaceAdd pages are exercised):

* ``tiny``     W4A16 per-group g32, fp16, x1 (16,256), x2 (256,128)
* ``w8``       W8A16 per-channel, fp16, x1 (512,1024), x2 (1024,1024)
* ``decode``   W4A16 g128, bf16, x1 (m,4096) m in {1,8,16}, x2 (4096,11008)
* ``prefill``  W4A16 g128, bf16, x1 (4,1024,8192), x2 (8192,8192)
* ``mx``       x fp16 (4096,8192) with smooth scales, x2 (8192,4096) MXFP4,
               y fp32 (4096,4096)
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch


def streams(seed: int, n: int):
    """``n`` independent numpy generators spawned from one seed, in order."""
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(seed).spawn(n)]


def cast(a: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """Store float draws in ``dtype`` (round-to-nearest-even), on the CPU."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(dtype)


@dataclass
class WQCase:
    """Inputs of one weight-quantized matmul + AddRmsNorm call.

    ``w`` holds the integer weight values as int32 (one value per element,
    before packing). ``scale``/``offset`` keep the shape the caller passes:
    (1,) per tensor, (n,) or (1,n) per channel, (ceil(k/G), n) per group.
    """
    name: str
    x1: torch.Tensor                 # (m,k) or (b,s,k), act dtype
    w: torch.Tensor                  # (k,n) int32
    w_bits: int                      # 4 or 8
    scale: torch.Tensor
    offset: Optional[torch.Tensor]
    group_size: int                  # 0 unless per-group
    bias: Optional[torch.Tensor]     # (n,)
    residual: torch.Tensor           # (b,s,n) (or (1,m,n))
    gamma: torch.Tensor              # (n,)
    eps: float = 1e-6
    meta: dict = field(default_factory=dict)

    @property
    def act_dtype(self) -> torch.dtype:
        return self.x1.dtype

    @property
    def mkn(self):
        k, n = self.w.shape
        m = self.x1.numel() // k
        return m, k, n


def wq_case(name: str, m: int, k: int, n: int, *, act: torch.dtype, w_bits: int,
            granularity: str, group_size: int = 0, scale_range=(0.005, 0.02),
            offset_range=None, bias_std: Optional[float] = 0.1,
            x1_shape=None, seed: int = 0, x1_abs: bool = False, w_range=None) -> WQCase:
    """A generic weight-quantized case with the configs' distributions.

    x1 ~ N(0,1) (|N(0,1)| with ``x1_abs``: activations of one sign); weights
    uniform over the signed range of ``w_bits`` (int4: [-8,7], int8:
    [-127,127]) or over ``w_range`` = (lo, hi) inclusive; scale ~
    U[scale_range]; offset ~ U[offset_range]
    (zeros when ``offset_range`` is None and ``granularity`` asks for one, no
    offset when it is the string "none"); bias ~ N(0, bias_std); residual ~
    N(0,1); gamma ~ U[0.9,1.1].
    """
    g = streams(seed, 7)
    x1d = g[0].standard_normal((m, k))
    x1 = cast(np.abs(x1d) if x1_abs else x1d, act)
    if x1_shape is not None:
        x1 = x1.reshape(x1_shape)
    lo, hi = (-8, 8) if w_bits == 4 else (-127, 128)
    if w_range is not None:
        lo, hi = w_range[0], w_range[1] + 1
    w = torch.from_numpy(g[1].integers(lo, hi, size=(k, n), dtype=np.int32))
    if granularity == "tensor":
        sshape = (1,)
    elif granularity == "channel":
        sshape = (n,)
    elif granularity == "channel2d":
        sshape = (1, n)
    elif granularity == "group":
        sshape = ((k + group_size - 1) // group_size, n)
    else:
        raise ValueError(granularity)
    scale = cast(g[2].uniform(scale_range[0], scale_range[1], size=sshape), act)
    if offset_range == "none":
        offset = None
    elif offset_range is None:
        offset = torch.zeros(sshape, dtype=act)
    else:
        offset = cast(g[3].uniform(offset_range[0], offset_range[1], size=sshape), act)
    bias = None if bias_std is None else cast(g[4].normal(0.0, bias_std, size=(n,)), act)
    residual = cast(g[5].standard_normal((1, m, n)), act)
    gamma = cast(g[6].uniform(0.9, 1.1, size=(n,)), act)
    return WQCase(name, x1, w, w_bits, scale, offset,
                  group_size if granularity == "group" else 0,
                  bias, residual, gamma, 1e-6)


def tiny() -> WQCase:
    """W4A16 per-group (group 32), fp16: x1 (16,256), x2 (256,128), seed 0."""
    return wq_case("tiny", 16, 256, 128, act=torch.float16, w_bits=4,
                   granularity="group", group_size=32, scale_range=(0.005, 0.02),
                   offset_range=None, bias_std=0.1)


def w8() -> WQCase:
    """W8A16 per-channel, fp16: x1 (512,1024), x2 int8 (1024,1024)."""
    return wq_case("w8", 512, 1024, 1024, act=torch.float16, w_bits=8,
                   granularity="channel", scale_range=(0.001, 0.01),
                   offset_range=(-0.5, 0.5), bias_std=0.1)


def decode(m: int = 16) -> WQCase:
    """Decode-shaped W4A16 group 128, bf16: x1 (m,4096), x2 (4096,11008).

    The draws are made at m=16 and the first ``m`` rows kept, so the m=1 row
    is the first row of m=8 and m=16.
    """
    c = wq_case("decode", 16, 4096, 11008, act=torch.bfloat16, w_bits=4,
                granularity="group", group_size=128, scale_range=(0.002, 0.02),
                offset_range=(-1.0, 1.0), bias_std=0.1)
    c.name = f"decode_m{m}"
    c.x1 = c.x1[:m].contiguous()
    c.residual = c.residual[:, :m].contiguous()
    return c


def prefill() -> WQCase:
    """Prefill-shaped W4A16 group 128 + AddRmsNorm, bf16: x1 (4,1024,8192),
    x2 (8192,8192), offset zeros."""
    c = wq_case("prefill", 4096, 8192, 8192, act=torch.bfloat16, w_bits=4,
                granularity="group", group_size=128, scale_range=(0.002, 0.02),
                offset_range=None, bias_std=0.1, x1_shape=(4, 1024, 8192))
    c.residual = c.residual.reshape(4, 1024, 8192)
    return c


@dataclass
class MXCase:
    """Inputs of the MX block-32 path.

    ``x`` (M,K) fp16 and ``smooth`` (K,) fp16 feed the dynamic quantization;
    ``w`` (K,N) fp32 ~ N(0,1) is the float weight that a test quantizes to
    MXFP4; ``x2_codes`` (K,N) int32 e2m1 codes and ``x2_scale`` (ceil(K/32),N)
    uint8 E8M0 codes are a directly drawn MXFP4 weight; ``y`` (M,N) fp32.
    """
    x: torch.Tensor
    smooth: torch.Tensor
    w: torch.Tensor
    x2_codes: torch.Tensor
    x2_scale: torch.Tensor
    y: torch.Tensor

    @property
    def mkn(self):
        m, k = self.x.shape
        return m, k, self.y.shape[1]


def mx(m: int = 4096, k: int = 8192, n: int = 4096, seed: int = 0,
       draw_w: bool = True) -> MXCase:
    """x ~ N(0,1) fp16 (m,k); smooth ~ U[0.5,2] fp16 (k); W ~ N(0,1) fp32 (k,n);
    e2m1 codes uniform over the 16 codes and E8M0 codes uniform in [120,126]
    for the directly drawn weight; y ~ N(0,1) fp32 (m,n)."""
    g = streams(seed, 6)
    x = cast(g[0].standard_normal((m, k)), torch.float16)
    smooth = cast(g[1].uniform(0.5, 2.0, size=(k,)), torch.float16)
    if draw_w:
        w = torch.from_numpy(g[2].standard_normal((k, n)).astype(np.float32))
    else:
        w = torch.empty(0)
    codes = torch.from_numpy(g[3].integers(0, 16, size=(k, n), dtype=np.int32))
    kb = (k + 31) // 32
    sc = torch.from_numpy(g[4].integers(120, 127, size=(kb, n), dtype=np.uint8))
    y = torch.from_numpy(g[5].standard_normal((m, n)).astype(np.float32))
    return MXCase(x, smooth, w, codes, sc, y)


@dataclass
class I8Case:
    w: torch.Tensor          # int8 (n, k): weight, stored transposed (K contiguous)
    w_scale: torch.Tensor    # float32 (n), per channel
    y: torch.Tensor          # float32 (m, n)


def int8_gemm(m: int = 4096, k: int = 8192, n: int = 4096, seed: int = 0) -> I8Case:
    """The INT8 consumer of the per-token quant output of ``mx``'s x: weight
    int8 uniform in [-127, 127] stored (n, k); per-channel scales
    U[0.001, 0.01] fp32; y ~ N(0,1) fp32 (m, n). x1 is the per-token INT8
    quantization of ``mx(m, k, n).x * smooth`` (made on the device)."""
    g = streams(seed + 1, 3)
    w = torch.from_numpy(g[0].integers(-127, 128, size=(n, k), dtype=np.int8))
    ws = torch.from_numpy(g[1].uniform(0.001, 0.01, size=(n,)).astype(np.float32))
    y = torch.from_numpy(g[2].standard_normal((m, n)).astype(np.float32))
    return I8Case(w, ws, y)
