"""GPU parity: wq_pack_int4 against the oracle, bit for bit."""
import numpy as np
import pytest
import torch

import bit_quantized_gemm_int4_amd as wq
import oracle
import workloads
from tests.gpu_util import DEV, note

pytestmark = pytest.mark.gpu


def _oracle_pack(w, layout, transpose):
    if layout == wq.WQ_LAYOUT_ND:
        return oracle.pack_int4_nd(w, transpose).reshape(-1)
    return oracle.pack_int4_gfx950b(w, transpose)


@pytest.mark.parametrize("k,n", [(256, 128), (80, 20), (1, 2), (300, 50), (128, 64), (129, 18),
                                 (200, 530), (1031, 300), (384, 1024)])
@pytest.mark.parametrize("layout", [wq.WQ_LAYOUT_ND, wq.WQ_LAYOUT_GFX950_B])
@pytest.mark.parametrize("transpose", [False, True])
def test_pack_bit_exact(k, n, layout, transpose):
    note(f"pack k={k} n={n} layout={layout} transpose={transpose}")
    rng = np.random.default_rng(k * 7 + n)
    w = rng.integers(-8, 8, size=(k, n), dtype=np.int32)
    stored = w.T.copy() if transpose else w
    got = wq.pack_int4(torch.from_numpy(stored).to(DEV), layout, transpose).cpu().numpy()
    want = _oracle_pack(stored, layout, transpose)
    assert got.shape == want.shape
    assert np.array_equal(got, want)


def test_pack_all_values_every_nibble_position():
    note("pack every value at every nibble position")
    k, n = 128, 16
    w = ((np.arange(k)[:, None] + 3 * np.arange(n)[None, :]) % 16 - 8).astype(np.int32)
    for layout in (wq.WQ_LAYOUT_ND, wq.WQ_LAYOUT_GFX950_B):
        got = wq.pack_int4(torch.from_numpy(w).to(DEV), layout).cpu().numpy()
        assert np.array_equal(got, _oracle_pack(w, layout, False))


def test_pack_fp4_codes_round_trip():
    note("pack e2m1 codes 0..15")
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 16, size=(256, 48), dtype=np.int32)
    got = wq.pack_int4(torch.from_numpy(codes).to(DEV), wq.WQ_LAYOUT_GFX950_B).cpu().numpy()
    assert np.array_equal(oracle.unpack_int4_gfx950b(got, 256, 48, signed=False), codes)


@pytest.mark.parametrize("which", ["decode", "prefill"])
def test_pack_full_size(which):
    c = workloads.decode(1) if which == "decode" else workloads.prefill()
    k, n = c.w.shape
    note(f"pack full size {which} {k}x{n}")
    got = wq.pack_int4(c.w.to(DEV), wq.WQ_LAYOUT_GFX950_B).cpu().numpy()
    assert np.array_equal(got, oracle.pack_int4_gfx950b(c.w.numpy()))
