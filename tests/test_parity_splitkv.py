"""GPU parity of the split-KV forward (fa_fwd_splitkv) against the CPU
oracle, through the C ABI via the Python binding.

The merged result is the same attention, so the plain forward's tolerances
apply: fp32 O <= 1e-5, 16-bit O <= 2e-2, LSE <= 1e-3. Slices with no tiles
(more slices than key tiles) and rows that see no key of a slice (causal
rule, windows) exercise the empty partials (O = 0, LSE = -inf).
"""

import numpy as np
import pytest
import torch

import exact_attention_120_amd as fa
from fa_inputs import WORKLOADS, make_inputs, to_f64, workload_inputs
from oracle import attention_forward

pytestmark = pytest.mark.gpu

TOL_O = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2}
TOL_LSE = 1e-3
DEV = "cuda"


def scale_of(d):
    return float(torch.tensor(d ** -0.5, dtype=torch.float32))


def run(inp, causal, scale, num_splits, window=None):
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    B, H, N, d = q.shape
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    nbytes = fa.fa_fwd_splitkv_workspace_size(B, H, N, d, q.dtype, num_splits)
    ws = None
    if nbytes:
        ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=DEV)  # NaN pattern
    fa.fa_fwd_splitkv(q, k, v, o, lse, scale, causal, num_splits, ws, window)
    torch.cuda.synchronize()
    return o, lse


def check(o, lse, inp, causal, scale, dtype, window=None):
    ref_o, ref_l = attention_forward(*(to_f64(inp[n]) for n in ("q", "k", "v")), scale, causal,
                                     window=window)
    o64, l64 = to_f64(o), to_f64(lse)
    assert np.isfinite(o64).all() and np.isfinite(l64).all()
    err_o, err_l = np.abs(o64 - ref_o).max(), np.abs(l64 - ref_l).max()
    assert err_o <= TOL_O[dtype], f"O max err {err_o:.3e}"
    assert err_l <= TOL_LSE, f"LSE max err {err_l:.3e}"
    return err_o, err_l


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("num_splits", [2, 3, 5, 16])
@pytest.mark.parametrize("N", [1, 100, 700])
def test_small_shapes(dtype, d, causal, num_splits, N):
    print(f"\n[splitkv] dtype={dtype} d={d} causal={causal} S={num_splits} N={N}", flush=True)
    inp = make_inputs(2, 2, N, d, dtype, seed=N + num_splits)
    scale = scale_of(d)
    o, lse = run(inp, causal, scale, num_splits)
    check(o, lse, inp, causal, scale, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal,window", [(True, (100, 0)), (False, (64, 200)),
                                           (False, (0, 0)), (True, (-1, -1))])
@pytest.mark.parametrize("num_splits", [2, 7])
def test_with_window_and_groups(dtype, causal, window, num_splits):
    print(f"\n[splitkv opts] dtype={dtype} causal={causal} window={window} S={num_splits}",
          flush=True)
    inp = make_inputs(1, 4, 1100, 128, dtype, seed=41, kv_heads=2)
    scale = scale_of(128)
    o, lse = run(inp, causal, scale, num_splits, window)
    check(o, lse, inp, causal, scale, dtype, window)


def test_causal_bf16_n1k_auto_split():
    """The B=2, H=8, N=1024, d=64 causal bf16 workload (64 workgroups
    unsplit): the library's own slice count, checked whole."""
    w = WORKLOADS["causal_bf16_n1k"]
    ns = fa.fa_fwd_num_splits(w.B, w.H, w.N, w.d, w.torch_dtype)
    print(f"\n[splitkv auto] {w} -> {ns} slices", flush=True)
    assert ns == 4
    inp = workload_inputs(w)
    o, lse = run(inp, w.causal, w.scale, 0)
    err = check(o, lse, inp, w.causal, w.scale, w.dtype)
    print(f"[splitkv auto] max|dO|={err[0]:.3e} max|dLSE|={err[1]:.3e}", flush=True)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_one_slice_is_the_plain_forward_bitwise(dtype):
    """One slice is the row-tiled kernel alone, which is what fa_fwd runs for
    a grid of more than 256 row tiles (bf16: B=2 H=128 N=512) and for fp32."""
    H, N = (128, 512) if dtype == "bf16" else (3, 500)
    inp = make_inputs(2, H, N, 64, dtype, seed=43)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    for causal in (False, True):
        o0, l0 = fa.forward(q, k, v, causal=causal)
        o1, l1 = fa.forward(q, k, v, causal=causal, num_splits=1)
        assert torch.equal(o0, o1) and torch.equal(l0, l1)


def test_splits_agree_with_plain_forward():
    """Every slice count gives the plain result up to float rounding (the
    merge reorders the sums, nothing else)."""
    inp = make_inputs(1, 4, 2048, 128, "bf16", seed=44)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    for causal in (False, True):
        o0, l0 = fa.forward(q, k, v, causal=causal)
        for s in (2, 4, 8, 32, 64):
            o1, l1 = fa.forward(q, k, v, causal=causal, num_splits=s)
            torch.cuda.synchronize()
            # Both are roundings of nearly the same float32 value: within
            # two bf16 units in the last place of each other.
            diff = (o0.float() - o1.float()).abs()
            assert (diff <= o0.float().abs() * 2.0 ** -6 + 1e-3).all(), s
            assert (l0 - l1).abs().max().item() <= 1e-4, s


def test_outputs_do_not_spill_and_workspace_reuse():
    B, H, N, d = 1, 2, 300, 64
    inp = make_inputs(B, H, N, d, "f16", seed=45)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    pad = 4096
    obuf = torch.full((pad + B * H * N * d + pad,), 7.0, dtype=torch.float16, device=DEV)
    lbuf = torch.full((pad + B * H * N + pad,), 7.0, dtype=torch.float32, device=DEV)
    o = obuf[pad:pad + B * H * N * d].view(B, H, N, d)
    lse = lbuf[pad:pad + B * H * N].view(B, H, N)
    ws = torch.empty(fa.fa_fwd_splitkv_workspace_size(B, H, N, d, torch.float16, 5),
                     dtype=torch.uint8, device=DEV)
    for causal in (True, False):  # the second call reuses the first's workspace
        fa.fa_fwd_splitkv(q, k, v, o, lse, 0.125, causal, 5, ws)
        torch.cuda.synchronize()
        assert (obuf[:pad] == 7).all() and (obuf[-pad:] == 7).all()
        assert (lbuf[:pad] == 7).all() and (lbuf[-pad:] == 7).all()
        check(o, lse, inp, causal, 0.125, "f16")
