"""Static checks of the gfx950 code the kernels compile to (no GPU needed): no
MFMA destination may partially overlap one of its source operands, and no
kernel spills registers or uses scratch memory."""
import shutil

import pytest

from bit_quantized_gemm_int4_amd import build as wqbuild
from bit_quantized_gemm_int4_amd.codegen_check import count_mfma, kernel_resources, partial_overlaps


def test_checker_flags_partial_overlaps():
    asm = "\n".join([
        "kern:",
        "  v_mfma_f32_16x16x32_bf16 v[4:7], v[46:49], v[2:5], v[6:9]",     # C and B partial
        "  v_mfma_f32_16x16x32_bf16 a[14:17], v[54:57], v[2:5], a[16:19]",  # C partial
        "  v_mfma_f32_16x16x32_bf16 v[8:11], v[0:3], v[12:15], v[8:11]",    # in place: fine
        "  v_mfma_f32_16x16x32_bf16 v[8:11], v[8:11], v[12:15], 0",         # D == A: fine
        "  v_mfma_f32_16x16x32_bf16 v[8:11], v[0:3], v[12:15], v[20:23]",   # disjoint: fine
    ])
    bad = partial_overlaps(asm)
    assert len(bad) == 2 and all(b.startswith("kern:") for b in bad)
    assert count_mfma(asm) == 5


@pytest.mark.skipif(shutil.which(wqbuild.HIPCC) is None and not __import__("os").path.exists(wqbuild.HIPCC),
                    reason="hipcc not available")
@pytest.mark.parametrize("src", wqbuild.MFMA_SOURCES)
def test_mfma_operands_never_partially_overlap(src):
    import os
    os.makedirs(wqbuild.BUILD_DIR, exist_ok=True)
    asm = wqbuild.device_asm(src)
    assert count_mfma(asm) > 0
    assert partial_overlaps(asm) == []


# device code without kernels: the allocation-free entry point's device array
KERNEL_FREE = {"wq_noalloc.hip"}


@pytest.mark.skipif(shutil.which(wqbuild.HIPCC) is None and not __import__("os").path.exists(wqbuild.HIPCC),
                    reason="hipcc not available")
@pytest.mark.parametrize("src", [s for s in wqbuild.SOURCES if s.endswith(".hip") and s not in KERNEL_FREE])
def test_no_spills_no_scratch(src):
    import os
    os.makedirs(wqbuild.BUILD_DIR, exist_ok=True)
    res = kernel_resources(wqbuild.device_asm(src))
    kernels = {k: v for k, v in res.items() if "private_segment" in v}
    assert kernels, src
    for name, v in kernels.items():
        # SGPR spills go to VGPR lanes, not memory; VGPR spills would need scratch
        assert v["private_segment"] == 0, (name, v)
        assert v.get("vgpr_spill", 0) == 0, (name, v)
