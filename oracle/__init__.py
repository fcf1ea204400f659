"""CPU oracle for the weight-quantized matmul operators — TEST INFRASTRUCTURE.

A plain, slow, obviously correct numpy implementation of what the HIP library
computes, written from the operator pages it cites. It shares no code with the
HIP path, and the product path never calls it: only the tests, the smoke check
and the CPU-baseline leg of the benchmark import it.

Precision: float64 for the matmul and normalization; the two quantizers take
their integer decisions in float32 (per-token) or in exact arithmetic (MX),
because a quantized code has exactly one right answer and both sides must take
that decision in the same precision.

Parity pins: every function here is checked by ``tests/test_oracle_*.py``
against values that do not come from this code (hand-worked examples under
``tests/golden/``, exact rational brute force, closed forms, invariants and
library conversions).
"""
from .formats import (e4m3_decode, e4m3_encode, e2m1_decode, e2m1_encode,
                      e8m0_decode, E4M3_MAX, E2M1_MAX)
from .pack import (pack_int4_nd, unpack_int4_nd, pack_int4_gfx950b,
                   unpack_int4_gfx950b, gfx950b_bytes, pack_codes_gfx950b, pack_float_e2m1)
from .quant import dynamic_quant_per_token, dynamic_quant_mx, encode_quant_output, unpack_quant_output
from .wq_matmul import dequantize_weight, wq_matmul_add_rmsnorm, weight_quant_matmul, add_rms_norm
from .mx_matmul import decode_group_size, mx_quant_matmul_inplace_add, mxfp4_quant_matmul_inplace_add
from .int8_matmul import quant_matmul_inplace_add_int8, quant_matmul_inplace_add_w4
from .compare import rel_err_floor, as_f64

__all__ = [
    "e4m3_decode", "e4m3_encode", "e2m1_decode", "e2m1_encode", "e8m0_decode",
    "E4M3_MAX", "E2M1_MAX",
    "pack_int4_nd", "unpack_int4_nd", "pack_int4_gfx950b", "unpack_int4_gfx950b",
    "gfx950b_bytes", "pack_codes_gfx950b", "pack_float_e2m1",
    "dynamic_quant_per_token", "dynamic_quant_mx", "encode_quant_output", "unpack_quant_output",
    "dequantize_weight", "wq_matmul_add_rmsnorm", "weight_quant_matmul", "add_rms_norm",
    "decode_group_size", "mx_quant_matmul_inplace_add", "mxfp4_quant_matmul_inplace_add", "quant_matmul_inplace_add_int8",
    "rel_err_floor", "as_f64",
    "quant_matmul_inplace_add_w4",
]
