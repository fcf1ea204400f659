"""The achievable-ceiling microkernels (measurement aids) compute what their
declarations state: the stream read's per-wave words XOR to the XOR of every
word of the input (a ragged tail included), and every lane of the MFMA loop
ends at iters times its share of the eight 16x16x32 products, rebuilt here
from the operand hash and the MFMA's lane layout (A row l % 16 and B column
l % 16 with K values 8 (l / 16) .. + 7; D column l % 16, rows 4 (l / 16) + i)."""
import numpy as np
import pytest
import torch

import bit_quantized_gemm_int4_amd as wq
from tests.gpu_util import DEV, note

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 16384, 16400, 1 << 20, 22544384])
def test_stream_read_folds_every_word(nbytes):
    note(f"stream read {nbytes}")
    g = np.random.default_rng(nbytes)
    host = g.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32).copy()).to(DEV)
    words = wq.wq_ceiling_stream_read_words(nbytes)
    out = torch.full((words,), -1, dtype=torch.int32, device=DEV)
    wq.wq_ceiling_stream_read(src, nbytes, out)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)


def _ml_dword(lane, s, d):
    m = np.uint64(0xFFFFFFFF)
    x = (np.uint64(lane) * np.uint64(0x9E3779B1) + np.uint64(s) * np.uint64(0x85EBCA77) +
         np.uint64(d) * np.uint64(0xC2B2AE3D) + np.uint64(0x27D4EB2F)) & m
    x ^= x >> np.uint64(15)
    x = (x * np.uint64(0x2C1B3C6D)) & m
    x ^= x >> np.uint64(12)
    x = (x * np.uint64(0x297A2D39)) & m
    x ^= x >> np.uint64(15)
    return int((x & np.uint64(0x80FF80FF)) | np.uint64(0x3F003F00))


def _bf16(bits):
    return float(np.array([bits << 16], dtype=np.uint32).view(np.float32)[0])


def _lane_expect():
    """Per lane: (sum of its accumulator elements after one round, the same
    sum over absolute products), in float64."""
    vals = np.zeros((64, 8, 8))            # lane, set, element (K order in the lane)
    for lane in range(64):
        for s in range(8):
            for d in range(4):
                w = _ml_dword(lane, s, d)
                vals[lane, s, 2 * d] = _bf16(w & 0xFFFF)
                vals[lane, s, 2 * d + 1] = _bf16(w >> 16)
    A = np.zeros((4, 16, 32))
    B = np.zeros((4, 32, 16))
    for s in range(4):
        for r in range(16):
            for k in range(32):
                A[s, r, k] = vals[r + 16 * (k // 8), s, k % 8]
                B[s, k, r] = vals[r + 16 * (k // 8), s + 4, k % 8]
    exp, mag = np.zeros(64), np.zeros(64)
    for j in range(8):
        D = A[j % 4] @ B[j // 2]
        Dabs = np.abs(A[j % 4]) @ np.abs(B[j // 2])
        for lane in range(64):
            for i in range(4):
                exp[lane] += D[4 * (lane // 16) + i, lane % 16]
                mag[lane] += Dabs[4 * (lane // 16) + i, lane % 16]
    return exp, mag


@pytest.mark.parametrize("workgroups,iters", [(1, 1), (512, 64), (3, 16384)])
def test_mfma_loop_sums(workgroups, iters):
    note(f"mfma loop {workgroups} x {iters}")
    out = torch.zeros(workgroups * 256, dtype=torch.float32, device=DEV)
    wq.wq_ceiling_mfma_loop(workgroups, iters, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64).reshape(workgroups * 4, 64)
    exp, mag = _lane_expect()
    # float32 accumulation over `iters` rounds: within 2^-11 of the absolute sum
    assert np.all(np.abs(got - iters * exp) <= iters * mag * 2.0 ** -11)
    assert np.all(got == got[0])            # every wave computes the same thing
