"""Build libwq.so (HIP for gfx950) in-tree with hipcc.

Each source compiles to an object under ``_build/`` in parallel, then one
shared library is linked next to this file. Run ``python -m
bit_quantized_gemm_int4_amd.build`` or call :func:`build`.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libwq.so")

SOURCES = ["wq_api.cpp", "wq_profile.cpp", "wq_pack.hip", "wq_quant.hip", "wq_gemm.hip", "wq_gemm_fast.hip",
           "wq_gemm_decode.hip", "wq_gemm_w8.hip", "mx_gemm.hip", "i8_gemm.hip", "add_rmsnorm.hip",
           "mx4_gemm.hip", "a8w4_gemm.hip", "wq_noalloc.hip", "wq_ceiling.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-FP32 VALU forms are disabled for every device compile.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I" + os.path.join(ROOT, "include"),
]


# Per-file flags: the MFMA-bound tile rescales its accumulators with VALU
# multiplies, and the INT8 tile folds its group sums into them, so their
# MFMAs keep accumulators in ordinary VGPRs (no AGPR copies). Its accumulators are long-lived and updated in place; the decode
# kernel, whose per-block partial sums are short-lived, keeps them in AGPRs.
FILE_FLAGS = {"wq_gemm_fast.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              # the MFMA-loop microkernel: with AGPR accumulators the
              # allocator rotated them into partially overlapping MFMAs
              "wq_ceiling.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              "wq_gemm_w8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              # the INT8 epilogue rounds each float step on its own, as its
              # reading of the formula fixes: no fused multiply-add
              "i8_gemm.hip": ["-ffp-contract=off"], "a8w4_gemm.hip": ["-ffp-contract=off"]}


# Sources with MFMA kernels: their device assembly is checked for MFMA
# destinations that partially overlap a source operand (codegen_check).
MFMA_SOURCES = ["wq_gemm.hip", "wq_gemm_fast.hip", "wq_gemm_decode.hip", "wq_gemm_w8.hip", "mx_gemm.hip",
                "i8_gemm.hip",
                "mx4_gemm.hip", "a8w4_gemm.hip", "wq_ceiling.hip"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def device_asm(src: str) -> str:
    """gfx950 assembly of one source, compiled with the library's flags."""
    out = os.path.join(BUILD_DIR, os.path.basename(src) + ".s")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), "-x", "hip", "--cuda-device-only", "-S",
           os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{r.stderr}")
    with open(out) as f:
        return f.read()


def _check_mfma(src: str) -> list:
    from .codegen_check import partial_overlaps
    return partial_overlaps(device_asm(src))


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=8) as ex:
        objs_f = ex.map(_compile, SOURCES)
        checks = list(ex.map(_check_mfma, MFMA_SOURCES))
        objs = list(objs_f)
    bad = [b for c in checks for b in c]
    if bad:
        raise RuntimeError("MFMA destination partially overlaps a source operand (wrong results "
                           "on gfx950):\n" + "\n".join(bad))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    if __package__ in (None, ""):
        sys.path.insert(0, ROOT)
        __package__ = "bit_quantized_gemm_int4_amd"
    build(verbose=True)
    sys.exit(0)
