"""Static check of the compiled GEMM kernels' MFMA register operands.

On gfx950 a 16x16x32 MFMA whose destination registers partially overlap one
of its sources (A, B or the accumulator C) computes wrong results, yet the
compiler's register allocator can emit such an instruction for 4-register
destinations. An exact overlap (destination == C, the in-place accumulate,
or destination == A/B) and disjoint registers are both fine. The kernels are
written so that the allocator has no reason to split an accumulator; this
check makes that a build-time guarantee: it scans the device assembly
(hipcc --cuda-device-only -S) of each MFMA source for partial overlaps.
"""
from __future__ import annotations

import re
from typing import List, Optional, Tuple

_RANGE = re.compile(r"([va])\[(\d+):(\d+)\]|([va])(\d+)")


def _regs(tok: str) -> Optional[Tuple[str, int, int]]:
    m = _RANGE.fullmatch(tok.strip())
    if not m:
        return None
    if m.group(1):
        return m.group(1), int(m.group(2)), int(m.group(3))
    return m.group(4), int(m.group(5)), int(m.group(5))


def _partial(d, s) -> bool:
    if d is None or s is None or d[0] != s[0] or d == s:
        return False
    return not (d[2] < s[1] or s[2] < d[1])


def partial_overlaps(asm_text: str) -> List[str]:
    """MFMA instructions in ``asm_text`` whose destination partially overlaps
    a source operand, each prefixed with the function it belongs to."""
    bad, fn = [], "?"
    for line in asm_text.splitlines():
        if re.match(r"^[A-Za-z_.$][\w.$]*:", line) and not line.startswith("."):
            fn = line.split(":")[0]
        s = line.strip()
        if not s.startswith("v_mfma"):
            continue
        ops = [o.strip() for o in s.split(None, 1)[1].split(",")]
        if len(ops) < 4:
            continue
        d, a, b, c = (_regs(o) for o in ops[:4])
        if any(_partial(d, x) for x in (a, b, c)):
            bad.append(f"{fn}: {s}")
    return bad


def count_mfma(asm_text: str) -> int:
    return sum(1 for line in asm_text.splitlines() if line.strip().startswith("v_mfma"))


def kernel_resources(asm_text: str) -> dict:
    """Per-kernel resource figures from the code-object metadata of an
    assembly listing: {kernel name: {"private_segment": bytes of scratch per
    lane, "vgpr_spill": n, "sgpr_spill": n, "vgpr": n}}."""
    import re
    out = {}
    cur = None
    for line in asm_text.splitlines():
        m = re.match(r"\s*\.amdhsa_kernel\s+(\S+)", line)
        if m:
            cur = m.group(1)
            out.setdefault(cur, {})
            continue
        m = re.match(r"\s*\.amdhsa_private_segment_fixed_size\s+(\d+)", line)
        if m and cur:
            out[cur]["private_segment"] = int(m.group(1))
        m = re.match(r"\s*-?\s*\.name:\s+(\S+)", line)
        if m:
            cur = m.group(1)
            out.setdefault(cur, {})
        for key, field in (("vgpr_spill", "vgpr_spill_count"), ("sgpr_spill", "sgpr_spill_count"),
                           ("vgpr", "vgpr_count")):
            m = re.match(r"\s*\.%s:\s+(\d+)" % field, line)
            if m and cur:
                out[cur][key] = int(m.group(1))
    return out
