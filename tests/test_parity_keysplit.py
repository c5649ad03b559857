"""GPU parity of the key-split forward (fa_fwd_keysplit, and fa_fwd /
fa_fwd_ex where the library picks it) against the CPU oracle, through the C
ABI via the Python binding.

The kernel deals a workgroup's key tiles out over groups of its waves and
merges their partial (O, max, sum) in LDS: the same attention, so the plain
forward's tolerances apply (16-bit O <= 2e-2, LSE <= 1e-3). Cases: ragged N
(rows and key tiles past N), fewer tiles than wave groups, the causal rule,
windows narrower than a workgroup, grouped K/V heads, large scales, a long
head (many tiles per group), the library's own choice of kernel, and
agreement with the row-tiled kernel.
"""

import numpy as np
import pytest
import torch

import exact_attention_120_amd as fa
from fa_inputs import WORKLOADS, make_inputs, to_f64, workload_inputs
from oracle import attention_forward

pytestmark = pytest.mark.gpu

TOL_O = {"f16": 2e-2, "bf16": 2e-2}
TOL_LSE = 1e-3
DEV = "cuda"


def scale_of(d):
    return float(torch.tensor(d ** -0.5, dtype=torch.float32))


def run(inp, causal, scale, window=None):
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    o = torch.full_like(q, float("nan"))  # rows never written would stay NaN
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    fa.fa_fwd_keysplit(q, k, v, o, lse, scale, causal, window)
    torch.cuda.synchronize()
    return o, lse


def check(o, lse, inp, causal, scale, dtype, window=None, tol_o=None):
    ref_o, ref_l = attention_forward(*(to_f64(inp[n]) for n in ("q", "k", "v")), scale, causal,
                                     window=window)
    o64, l64 = to_f64(o), to_f64(lse)
    assert np.isfinite(o64).all() and np.isfinite(l64).all()
    err_o, err_l = np.abs(o64 - ref_o).max(), np.abs(l64 - ref_l).max()
    print(f"  max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}", flush=True)
    assert err_o <= (tol_o or TOL_O[dtype]), f"O max err {err_o:.3e}"
    assert err_l <= TOL_LSE, f"LSE max err {err_l:.3e}"
    return err_o, err_l


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 7, 64, 65, 129, 300, 1000])
def test_small_shapes(dtype, d, causal, N):
    print(f"\n[keysplit] dtype={dtype} d={d} causal={causal} N={N}", flush=True)
    inp = make_inputs(2, 3, N, d, dtype, seed=N + 3 * d)
    scale = scale_of(d)
    o, lse = run(inp, causal, scale)
    check(o, lse, inp, causal, scale, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal,window", [(True, (100, 0)), (False, (64, 200)), (False, (0, 0)),
                                           (True, (5, -1)), (False, (300, 30))])
def test_windows_and_groups(dtype, d, causal, window):
    """Windows narrower than a workgroup's rows (the tile range starts past 0
    and differs between its row groups) with grouped K/V heads."""
    print(f"\n[keysplit opts] dtype={dtype} d={d} causal={causal} window={window}", flush=True)
    inp = make_inputs(2, 4, 1100, d, dtype, seed=41 + d, kv_heads=2)
    scale = scale_of(d)
    o, lse = run(inp, causal, scale, window)
    check(o, lse, inp, causal, scale, dtype, window)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_large_scales(dtype, causal):
    """scale*log2(e) > 1: parts whose tiles hold none of a row's keys keep
    the no-reference max, and the merge must weigh them 0 without overflow."""
    print(f"\n[keysplit large scale] dtype={dtype} causal={causal}", flush=True)
    inp = make_inputs(1, 2, 700, 64, dtype, seed=23)
    for scale, window in [(1.5, (100, 0)), (4.0, (100, 40)), (1.0, None), (3.0, None)]:
        o, lse = run(inp, causal, scale, window)
        check(o, lse, inp, causal, scale, dtype, window)


@pytest.mark.parametrize("causal", [False, True])
def test_long_head_every_row(causal):
    """One head of N = 8192 at d = 128 (64 key tiles per part group at most):
    the key-split kernel on a long chain, every row against the oracle."""
    print(f"\n[keysplit long] causal={causal}", flush=True)
    inp = make_inputs(1, 1, 8192, 128, "bf16", seed=47)
    scale = scale_of(128)
    o, lse = run(inp, causal, scale)
    check(o, lse, inp, causal, scale, "bf16")


def test_causal_bf16_n1k_workload_every_row():
    """The causal B=2 H=8 N=1024 d=64 bf16 workload, for which fa_fwd picks
    this kernel; fa_fwd's result must equal fa_fwd_keysplit's bit for bit."""
    w = WORKLOADS["causal_bf16_n1k"]
    print(f"\n[keysplit workload] {w}", flush=True)
    inp = workload_inputs(w)
    o, lse = run(inp, w.causal, w.scale)
    check(o, lse, inp, w.causal, w.scale, w.dtype)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    o2, l2 = fa.forward(q, k, v, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, l2)


def test_bf16_n4k_d128_workload_every_row():
    """The B=4 H=16 N=4096 d=128 workload (row tiles fill the GPU, so fa_fwd
    does not pick this kernel) through fa_fwd_keysplit: 32 key tiles per wave
    group, every row of every head against the oracle."""
    w = WORKLOADS["bf16_n4k_d128"]
    print(f"\n[keysplit workload] {w}", flush=True)
    inp = workload_inputs(w)
    o, lse = run(inp, w.causal, w.scale)
    check(o, lse, inp, w.causal, w.scale, w.dtype)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_agrees_with_row_tiles(d, causal):
    """Same attention as the row-tiled kernel up to float rounding (the
    partial sums are grouped differently)."""
    inp = make_inputs(2, 4, 777, d, "bf16", seed=51 + d)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    o0, l0 = fa.forward(q, k, v, causal=causal, num_splits=1)
    o1, l1 = fa.forward(q, k, v, causal=causal, key_split=True)
    torch.cuda.synchronize()
    do = (o0.float() - o1.float()).abs().max().item()
    dl = (l0 - l1).abs().max().item()
    print(f"\n[keysplit vs rows] d={d} causal={causal} max|dO|={do:.3e} max|dLSE|={dl:.3e}",
          flush=True)
    assert do <= 2e-2 and dl <= 1e-4


def test_deterministic():
    inp = make_inputs(2, 4, 900, 128, "f16", seed=53)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    a = fa.forward(q, k, v, causal=True, key_split=True)
    b = fa.forward(q, k, v, causal=True, key_split=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_float32_is_unsupported():
    q = torch.zeros(1, 1, 64, 64, device=DEV)
    with pytest.raises(fa.FaError) as e:
        fa.forward(q, q, q, key_split=True)
    assert e.value.status == -2  # FA_ERR_UNSUPPORTED
