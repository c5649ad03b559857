"""GPU parity of the option variants (fa_fwd_ex, fa_bwd_ex) against the CPU
oracle: grouped K/V heads (multi-query and grouped-query attention) and
local windows, alone and combined with the causal rule, called through the
C ABI via the Python binding.

Tolerances are those of the plain calls: fp32 O <= 1e-5, 16-bit O <= 2e-2,
LSE <= 1e-3; fp32 gradients <= 1e-5, 16-bit gradients <= 5e-2. Grouped dK
and dV sum up to H/Hkv query heads' contributions in float32 before one
rounding, so the bound of the plain call still holds per element.
"""

import numpy as np
import pytest
import torch

import exact_attention_120_amd as fa
from fa_inputs import make_inputs, to_f64
from oracle import attention_backward, attention_forward

pytestmark = pytest.mark.gpu

TOL_O = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2}
TOL_LSE = 1e-3
TOL_G = {"f32": 1e-5, "f16": 5e-2, "bf16": 5e-2}
DEV = "cuda"

# (left, right) bounds; -1 = unbounded on that side. (0, 0): each row sees
# only its own key; (-1, 37) with causal is the causal rule itself.
WINDOWS = [(0, 0), (16, -1), (-1, 37), (50, 50), (100, 0), (300, 200)]


def scale_of(d):
    return float(torch.tensor(d ** -0.5, dtype=torch.float32))


# Forward kernels: "auto" is fa_fwd_ex (the library's choice: the key-split
# kernel for these small 16-bit grids), "rows" the row-tiled kernel alone
# (fa_fwd_splitkv with one slice).
KERNELS = ["auto", "rows"]


def fwd(inp, causal, scale, window, kernel="auto"):
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    if kernel == "rows":
        fa.fa_fwd_splitkv(q, k, v, o, lse, scale, causal, 1, None, window)
    else:
        fa.fa_fwd_ex(q, k, v, o, lse, scale, causal, window)
    torch.cuda.synchronize()
    return o, lse


def one_kernel_for_f32(dtype, kernel):
    if dtype == "f32" and kernel != "auto":
        pytest.skip("float32 has one forward kernel")


def bwd(inp, causal, scale, window):
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale, window=window)
    B, H, N, d = q.shape
    ws = torch.full((fa.fa_bwd_workspace_size(B, H, N, d),), 0xFF, dtype=torch.uint8, device=DEV)
    dq = torch.full_like(q, float("nan"))
    dk, dv = torch.full_like(k, float("nan")), torch.full_like(v, float("nan"))
    fa.fa_bwd_ex(q, k, v, o, do, lse, dq, dk, dv, scale, causal, ws, window)
    torch.cuda.synchronize()
    return dq, dk, dv


def check_fwd(o, lse, inp, causal, scale, window, dtype, rows=None, tol_o=TOL_O):
    q, k, v = (to_f64(inp[n]) for n in ("q", "k", "v"))
    if rows is None:
        ref_o, ref_l = attention_forward(q, k, v, scale, causal, window=window)
        o64, l64 = to_f64(o), to_f64(lse)
    else:
        ref_o, ref_l = attention_forward(q[..., rows, :], k, v, scale, causal, q_positions=rows,
                                         window=window)
        o64, l64 = to_f64(o)[..., rows, :], to_f64(lse)[..., rows]
    assert np.isfinite(o64).all() and np.isfinite(l64).all()
    err_o, err_l = np.abs(o64 - ref_o).max(), np.abs(l64 - ref_l).max()
    assert err_o <= tol_o[dtype], f"O max err {err_o:.3e}"
    assert err_l <= TOL_LSE, f"LSE max err {err_l:.3e}"
    return err_o, err_l


def check_bwd(got, inp, causal, scale, window, dtype):
    ref = attention_backward(*(to_f64(inp[n]) for n in ("q", "k", "v", "do")), scale, causal,
                             window=window)
    errs = {}
    for name, g, r in zip(("dq", "dk", "dv"), got, ref[:3]):
        g64 = to_f64(g)
        assert g64.shape == r.shape, name
        assert np.isfinite(g64).all(), f"{name} has non-finite values"
        errs[name] = float(np.abs(g64 - r).max())
    print(f"  {dtype} gradient max errors: " + ", ".join(f"{k} {e:.3e}" for k, e in errs.items()),
          flush=True)
    bad = {k: e for k, e in errs.items() if not e <= TOL_G[dtype]}
    assert not bad, f"max errors {errs}"
    return errs


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("window", WINDOWS)
@pytest.mark.parametrize("kernel", KERNELS)
def test_window_forward(dtype, d, causal, window, kernel):
    one_kernel_for_f32(dtype, kernel)
    print(f"\n[fwd window] dtype={dtype} d={d} causal={causal} window={window} kernel={kernel}",
          flush=True)
    inp = make_inputs(2, 2, 300, d, dtype, seed=d + window[0] + 7 * window[1])
    scale = scale_of(d)
    o, lse = fwd(inp, causal, scale, window, kernel)
    check_fwd(o, lse, inp, causal, scale, window, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("heads", [(4, 1), (4, 2), (6, 3)])
@pytest.mark.parametrize("N", [129, 300])
@pytest.mark.parametrize("kernel", KERNELS)
def test_grouped_forward(dtype, d, causal, heads, N, kernel):
    one_kernel_for_f32(dtype, kernel)
    H, Hkv = heads
    print(f"\n[fwd grouped] dtype={dtype} d={d} causal={causal} H={H} Hkv={Hkv} N={N} "
          f"kernel={kernel}", flush=True)
    inp = make_inputs(2, H, N, d, dtype, seed=N + H + Hkv, kv_heads=Hkv)
    scale = scale_of(d)
    o, lse = fwd(inp, causal, scale, None, kernel)
    check_fwd(o, lse, inp, causal, scale, None, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kernel", KERNELS)
def test_grouped_window_forward_longer(dtype, causal, kernel):
    """Windows narrower than a workgroup's rows: the key-tile range starts
    past 0 and differs between the waves of one workgroup."""
    one_kernel_for_f32(dtype, kernel)
    print(f"\n[fwd grouped window] dtype={dtype} causal={causal} kernel={kernel}", flush=True)
    inp = make_inputs(1, 4, 2000, 128, dtype, seed=21, kv_heads=2)
    scale = scale_of(128)
    for window in [(256, 0), (70, 130), (5, -1)]:
        o, lse = fwd(inp, causal, scale, window, kernel)
        check_fwd(o, lse, inp, causal, scale, window, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kernel", KERNELS)
def test_window_forward_large_scale(dtype, causal, kernel):
    """scale * log2(e) > 1 with a left window bound: rows whose first visited
    key tile holds none of their keys still have no reference max there
    (-FLT_MAX), whose product with the exponent multiplier overflows. The
    result must stay the finite attention (also split over key slices).

    fp32's 1e-5 is the bound at scale 1/sqrt(d); float32 score errors grow
    with the scores, so at larger scales it is multiplied by scale*sqrt(d)."""
    one_kernel_for_f32(dtype, kernel)
    print(f"\n[fwd window large scale] dtype={dtype} causal={causal} kernel={kernel}", flush=True)
    inp = make_inputs(1, 2, 700, 64, dtype, seed=23)
    for scale, window in [(1.5, (100, 0)), (4.0, (100, 40)), (1.0, (45, -1))]:
        tol = {**TOL_O, "f32": TOL_O["f32"] * max(1.0, scale * 64 ** 0.5)}
        o, lse = fwd(inp, causal, scale, window, kernel)
        check_fwd(o, lse, inp, causal, scale, window, dtype, tol_o=tol)
        q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
        o, lse = fa.forward(q, k, v, causal=causal, scale=scale, window=window, num_splits=3)
        torch.cuda.synchronize()
        check_fwd(o, lse, inp, causal, scale, window, dtype, tol_o=tol)


INT_MAX = 2 ** 31 - 1


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("window", [(0, INT_MAX), (INT_MAX, 0), (INT_MAX, INT_MAX),
                                    (INT_MAX, 5), (7, INT_MAX)])
def test_int_max_window_bounds(dtype, window):
    """A bound of INT_MAX is valid (it hides nothing on its side). The
    kernels add bounds to row indices, so the library maps any bound >= N - 1
    to unbounded; without that the sums overflowed and rows saw no key."""
    print(f"\n[window INT_MAX] dtype={dtype} window={window}", flush=True)
    inp = make_inputs(1, 2, 300, 64, dtype, seed=29, backward=True)
    scale = scale_of(64)
    for causal in (False, True):
        o, lse = fwd(inp, causal, scale, window)
        check_fwd(o, lse, inp, causal, scale, window, dtype)
        check_bwd(bwd(inp, causal, scale, window), inp, causal, scale, window, dtype)
        q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
        o, lse = fa.forward(q, k, v, causal=causal, scale=scale, window=window, num_splits=3)
        torch.cuda.synchronize()
        check_fwd(o, lse, inp, causal, scale, window, dtype)


def sampled_rows(N, n, seed):
    rng = np.random.default_rng(seed)
    extra = rng.choice(N, size=min(n, N), replace=False)
    edge = [0, 1, 31, 32, 63, 64, 255, 256, 1023, 1024, 1025, N - 2, N - 1]
    return np.unique(np.concatenate([[r for r in edge if 0 <= r < N], extra]))


@pytest.mark.parametrize("causal,window", [(True, (1024, 0)), (False, (512, 512)),
                                           (False, None)])
def test_full_size_grouped_window_forward(causal, window):
    """bf16, B=1, H=16 with 4 K/V heads, N=16384, d=128: the full launch,
    checked on sampled rows of every head."""
    print(f"\n[fwd full-size grouped] causal={causal} window={window}", flush=True)
    inp = make_inputs(1, 16, 16384, 128, "bf16", seed=5, kv_heads=4)
    scale = scale_of(128)
    o, lse = fwd(inp, causal, scale, window)
    rows = sampled_rows(16384, 64, 2)
    err = check_fwd(o, lse, inp, causal, scale, window, "bf16", rows)
    print(f"[fwd full-size grouped] max|dO|={err[0]:.3e} max|dLSE|={err[1]:.3e}", flush=True)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("window", WINDOWS)
def test_window_backward(dtype, d, causal, window):
    print(f"\n[bwd window] dtype={dtype} d={d} causal={causal} window={window}", flush=True)
    inp = make_inputs(1, 2, 300, d, dtype, seed=3 + d + window[0], backward=True)
    scale = scale_of(d)
    check_bwd(bwd(inp, causal, scale, window), inp, causal, scale, window, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("heads", [(4, 1), (4, 2), (6, 3)])
@pytest.mark.parametrize("N", [129, 300])
def test_grouped_backward(dtype, d, causal, heads, N):
    H, Hkv = heads
    print(f"\n[bwd grouped] dtype={dtype} d={d} causal={causal} H={H} Hkv={Hkv} N={N}",
          flush=True)
    inp = make_inputs(2, H, N, d, dtype, seed=N + 2 * H + Hkv, backward=True, kv_heads=Hkv)
    scale = scale_of(d)
    check_bwd(bwd(inp, causal, scale, None), inp, causal, scale, None, dtype)


@pytest.mark.parametrize("causal,window", [(True, (256, 0)), (False, (100, 300))])
def test_grouped_window_backward_longer(causal, window):
    print(f"\n[bwd grouped window] causal={causal} window={window}", flush=True)
    inp = make_inputs(1, 4, 1500, 128, "bf16", seed=31, backward=True, kv_heads=2)
    scale = scale_of(128)
    errs = check_bwd(bwd(inp, causal, scale, window), inp, causal, scale, window, "bf16")
    print(f"[bwd grouped window] {errs}", flush=True)


def test_full_size_grouped_window_backward_one_group():
    """bf16, B=1, H=8 with 2 K/V heads, N=8192, d=128, causal with a
    1024-key left window: the full launch; the oracle checks the last K/V
    head's group (its 4 query heads) whole."""
    print("\n[bwd full-size grouped window]", flush=True)
    window = (1024, 0)
    inp = make_inputs(1, 8, 8192, 128, "bf16", seed=8, backward=True, kv_heads=2)
    scale = scale_of(128)
    dq, dk, dv = bwd(inp, True, scale, window)
    part = {"q": inp["q"][:, 4:], "do": inp["do"][:, 4:], "k": inp["k"][:, 1:],
            "v": inp["v"][:, 1:]}
    got = [dq[:, 4:], dk[:, 1:], dv[:, 1:]]
    errs = check_bwd(got, part, True, scale, window, "bf16")
    print(f"[bwd full-size grouped window] {errs}", flush=True)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_options_that_change_nothing_are_bit_identical(dtype):
    """An unbounded window, or one wider than the sequence, and Hkv = H give
    the plain call's outputs bit for bit (same tiles, same arithmetic)."""
    inp = make_inputs(2, 4, 333, 64, dtype, seed=17, backward=True)
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    for causal in (False, True):
        o0, l0 = fa.forward(q, k, v, causal=causal)
        for window in [(-1, -1), (333, 333), (10 ** 6, 10 ** 6)]:
            o1, l1 = fa.forward(q, k, v, causal=causal, window=window)
            assert torch.equal(o0, o1) and torch.equal(l0, l1), window
        g0 = fa.backward(q, k, v, o0, do, l0, causal=causal)
        g1 = fa.backward(q, k, v, o0, do, l0, causal=causal, window=(-1, -1))
        assert torch.equal(g0[1], g1[1]) and torch.equal(g0[2], g1[2])


def test_grouped_forward_equals_repeated_heads_bitwise():
    """Query head h with K/V head h // G computes exactly what the plain call
    computes with that K/V head repeated G times."""
    inp = make_inputs(2, 8, 777, 128, "bf16", seed=19, kv_heads=2)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    for causal in (False, True):
        o1, l1 = fa.forward(q, k, v, causal=causal)
        kr = k.repeat_interleave(4, dim=1).contiguous()
        vr = v.repeat_interleave(4, dim=1).contiguous()
        o0, l0 = fa.forward(q, kr, vr, causal=causal)
        assert torch.equal(o0, o1) and torch.equal(l0, l1)


def test_binding_rejects_bad_group_shapes():
    q = torch.zeros(1, 4, 16, 64, dtype=torch.bfloat16, device=DEV)
    k3 = torch.zeros(1, 3, 16, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        fa.forward(q, k3, k3)
    k2 = torch.zeros(1, 2, 16, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        fa.fa_fwd(q, k2, k2, torch.empty_like(q),
                  torch.empty(1, 4, 16, dtype=torch.float32, device=DEV), 0.125, False)
