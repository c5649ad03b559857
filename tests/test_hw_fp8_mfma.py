"""The FP8 matrix instruction's accumulation error, measured on the GPU.

The FP8 parity bound (tests/test_parity_fp8.py) charges every scaled score
eps * scale * sum_k |Q_ik| |K_jk| for the way v_mfma_f32_32x32x64_f8f6f4
adds its 64 products (it does not add them like float32), and its
mean-square model an RMS term rms * (the same magnitude). This test measures
that instruction on in-bounds random operands (tests/hw/fp8_mfma_probe.hip,
one instruction per tile with a zero accumulator) against the exact float64
sums of the decoded codes, and requires the worst relative error to stay
within half of the constant the parity bound uses, and, for the operand
families the kernel feeds the instruction, the RMS relative error within
half of the mean-square model's constant.

Operand families: codes drawn uniformly over every finite E4M3 code (products
spanning 2^-18 .. 2^17.6, the hardest case for alignment), N(0,1) data
quantized like the FP8 inputs (Q K^T), and probability codes 2^3 * p times
quantized values (P V).
"""

import ctypes
import os

import numpy as np
import pytest
import torch

from oracle import e4m3_decode
from test_parity_fp8 import EPS_MFMA8, RMS_MFMA8

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hw", "libfa_probe.so")
TILES = 4096


def probe(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """[T, 32, 64] x [T, 32, 64] codes -> [T, 32, 32] float32 results."""
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB)
    lib.fa_probe_fp8_mfma.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_int, ctypes.c_void_p]
    lib.fa_probe_fp8_mfma.restype = ctypes.c_int
    T = a.shape[0]
    assert a.shape == b.shape == (T, 32, 64) and a.dtype == b.dtype == np.uint8
    ga = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    gb = torch.from_numpy(np.ascontiguousarray(b)).cuda()
    gc = torch.full((T, 32, 32), float("nan"), dtype=torch.float32, device="cuda")
    st = lib.fa_probe_fp8_mfma(ga.data_ptr(), gb.data_ptr(), gc.data_ptr(), T,
                               torch.cuda.current_stream().cuda_stream)
    assert st == 0, st
    torch.cuda.synchronize()
    return gc.cpu().numpy().astype(np.float64)


def finite_codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    return np.where((c & 0x7F) == 0x7F, c & 0xF0, c).astype(np.uint8)  # no NaN codes


def quantized_normal(rng, shape):
    x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32))
    s = x.abs().max() / 448.0
    return (x / s).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def probability_codes(rng, shape):
    p = np.exp(-np.abs(rng.standard_normal(shape)) * 3.0) * 8.0  # 2^3 * p, p in (0, 1]
    return torch.from_numpy(p.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# Families whose RMS the parity bound's mean-square model uses: the
# operands the FP8 kernel feeds the instruction (quantized data for the
# scores, probability codes times quantized values for P V). Codes spread
# over the whole range are checked against the worst-case constant only.
RMS_FAMILIES = ("quantized_normal", "probabilities_x_values")

FAMILIES = {
    "whole_range": lambda rng: (finite_codes(rng, (TILES, 32, 64)),
                                finite_codes(rng, (TILES, 32, 64))),
    "quantized_normal": lambda rng: (quantized_normal(rng, (TILES, 32, 64)),
                                     quantized_normal(rng, (TILES, 32, 64))),
    "probabilities_x_values": lambda rng: (probability_codes(rng, (TILES, 32, 64)),
                                           quantized_normal(rng, (TILES, 32, 64))),
}


@pytest.mark.parametrize("family", list(FAMILIES))
def test_fp8_mfma_accumulation_error_within_half_the_bound(family):
    rng = np.random.default_rng(list(FAMILIES).index(family) + 100)
    a, b = FAMILIES[family](rng)
    got = probe(a, b)
    da, db = e4m3_decode(a), e4m3_decode(b)
    exact = np.einsum("tik,tjk->tij", da, db)           # float64: exact for these sums
    mag = np.einsum("tik,tjk->tij", np.abs(da), np.abs(db))
    assert np.isfinite(got).all()
    nz = mag > 0
    assert (got[~nz] == 0).all()
    rel = np.abs(got - exact)[nz] / mag[nz]
    worst, rms = float(rel.max()), float(np.sqrt((rel ** 2).mean()))
    print(f"\n[fp8 mfma] {family}: worst {worst:.3e} (2^{np.log2(max(worst, 1e-300)):.2f}), "
          f"rms {rms:.3e} (2^{np.log2(max(rms, 1e-300)):.2f}); bound uses eps 2^"
          f"{np.log2(EPS_MFMA8):.0f}, rms 2^{np.log2(RMS_MFMA8):.0f}", flush=True)
    assert worst <= EPS_MFMA8 / 2, f"worst relative error {worst:.3e} > eps/2"
    if family in RMS_FAMILIES:
        assert rms <= RMS_MFMA8 / 2, f"RMS relative error {rms:.3e} > rms/2"


def test_probe_pairs_operands_as_assumed():
    """Exact cases: one-hot codes pick single products, so the probe's
    operand layout (row/column = lane & 31, k-bytes 32 * (lane >> 5) ..) is
    the one the comparison above assumes."""
    rng = np.random.default_rng(7)
    a = np.zeros((64, 32, 64), np.uint8)
    b = np.zeros((64, 32, 64), np.uint8)
    one = 0x38  # E4M3 code of 1.0
    for t in range(64):
        i, j, k = rng.integers(0, 32), rng.integers(0, 32), rng.integers(0, 64)
        a[t, i, k] = one
        b[t, j, k] = 0x40  # 2.0
    got = probe(a, b)
    want = np.einsum("tik,tjk->tij", e4m3_decode(a), e4m3_decode(b))
    assert np.array_equal(got, want)
