"""GPU parity of fa_bwd against the CPU oracle's analytic gradients (float64
on the same rounded inputs), called through the C ABI via the binding.

Tolerances (max abs error, the scope's bounds): bf16/fp16 dQ, dK, dV <= 5e-2;
fp32 dQ, dK, dV <= 1e-5 (the scope's fp32 bound holds for every fp32 result).
Every check prints its measured maxima.
"""

import numpy as np
import pytest
import torch

import exact_attention_120_amd as fa
from fa_inputs import WORKLOADS, make_inputs, to_f64, workload_inputs
from oracle import attention_backward

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 5e-2, "bf16": 5e-2}
DEV = "cuda"


def scale_of(d):
    return float(torch.tensor(d ** -0.5, dtype=torch.float32))


def run(inp, causal, scale, poison_workspace=True):
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale)
    B, H, N, d = q.shape
    ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d), dtype=torch.uint8, device=DEV)
    if poison_workspace:
        ws.fill_(0xFF)  # NaN pattern: the library must clear what it uses
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, scale, causal, ws)
    torch.cuda.synchronize()
    return dq, dk, dv


def check(got, ref, dtype, what=""):
    errs = {}
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        g64 = to_f64(g) if isinstance(g, torch.Tensor) else g
        assert np.isfinite(g64).all(), f"{what} {name} has non-finite values"
        errs[name] = float(np.abs(g64 - r).max())
    print(f"  {what} {dtype} gradient max errors: "
          + ", ".join(f"{k} {e:.3e}" for k, e in errs.items()), flush=True)
    bad = {k: e for k, e in errs.items() if not e <= TOL[dtype]}
    assert not bad, f"{what} max errors {errs}"
    return errs


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 7, 64, 129, 300])
def test_small_shapes_full_compare(dtype, d, causal, N):
    print(f"\n[bwd small] dtype={dtype} d={d} causal={causal} N={N}", flush=True)
    inp = make_inputs(2, 2, N, d, dtype, seed=N + d + 1, backward=True)
    scale = scale_of(d)
    got = run(inp, causal, scale)
    ref = attention_backward(*(to_f64(inp[n]) for n in ("q", "k", "v", "do")), scale, causal)
    check(got, ref[:3], dtype)


def test_fp16_causal_workload_full():
    w = WORKLOADS["f16_n2k_fwdbwd_causal"]
    print(f"\n[bwd workload] {w}", flush=True)
    inp = workload_inputs(w)
    got = run(inp, w.causal, w.scale)
    ref = attention_backward(*(to_f64(inp[n]) for n in ("q", "k", "v", "do")), w.scale, w.causal)
    errs = check(got, ref[:3], w.dtype)
    print(f"[bwd workload] {w.name}: {errs}", flush=True)


_FULL = {}


def _full_size(name):
    """Inputs and GPU gradients of a full-size workload, computed once per
    module (the launch covers every head; the head groups below each check
    part of it)."""
    if name not in _FULL:
        _FULL.clear()
        w = WORKLOADS[name]
        inp = make_inputs(w.B, w.H, w.N, w.d, w.dtype, seed=w.seed, input_scale=w.input_scale,
                          backward=True)
        got = [g.cpu() for g in run(inp, w.causal, w.scale)]
        _FULL[name] = (w, inp, got)
    return _FULL[name]


@pytest.mark.parametrize("name", ["bf16_n4k_d128", "bf16_n16k_d128", "bf16_n16k_d128_causal"])
@pytest.mark.parametrize("part", range(4))
def test_full_size_bf16_every_head(name, part):
    """Full-size launch; the oracle checks every head whole, a quarter of the
    (batch, head) pairs per test case."""
    w, inp, got = _full_size(name)
    print(f"\n[bwd full-size] {w} heads part {part}/4", flush=True)
    pairs = [(b, h) for b in range(w.B) for h in range(w.H)]
    n = len(pairs) // 4
    worst = {}
    for b, h in pairs[part * n:(part + 1) * n]:
        ref = attention_backward(*(to_f64(inp[x][b, h]) for x in ("q", "k", "v", "do")),
                                 w.scale, w.causal)
        errs = check([to_f64(g[b, h]) for g in got], ref[:3], w.dtype, f"{name} b={b} h={h}")
        worst = {k: max(worst.get(k, 0.0), e) for k, e in errs.items()}
    print(f"[bwd full-size] {name} part {part}: {worst}", flush=True)


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_invariants_on_gpu(causal):
    inp = make_inputs(1, 4, 512, 128, "f16", seed=11, backward=True)
    dq, dk, dv = run(inp, causal, scale_of(128))
    dk64, dv64 = to_f64(dk), to_f64(dv)
    # Rows of dS sum to zero -> key gradients sum to ~0; rows of P sum to
    # one -> value gradients sum to the output-gradient sum.
    assert np.abs(dk64.sum(-2)).max() < 5e-2
    np.testing.assert_allclose(dv64.sum(-2), to_f64(inp["do"]).sum(-2), atol=0.25)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_scale_zero(dtype):
    inp = make_inputs(1, 2, 150, 64, dtype, seed=12, backward=True)
    got = run(inp, True, 0.0)
    ref = attention_backward(*(to_f64(inp[n]) for n in ("q", "k", "v", "do")), 0.0, True)
    check(got, ref[:3], dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_16bit_backward_is_deterministic(dtype):
    """The 16-bit backward has no atomics: dQ, dK and dV repeat bit for bit."""
    inp = make_inputs(2, 2, 700, 128, dtype, seed=13, backward=True)
    a = run(inp, True, scale_of(128))
    b = run(inp, True, scale_of(128), poison_workspace=False)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("window", [None, (60, 20)])
def test_many_heads_several_rounds(window):
    """B=1 H=256 N=512 d=64 bf16, non-causal: 512 forward and dQ workgroups
    and 1024 dK/dV workgroups (the kernels launched one after the other, in
    several rounds per XCD). Forward and gradients of every head against the
    oracle."""
    from oracle import attention_forward
    print(f"\n[rounds] window={window}", flush=True)
    inp = make_inputs(1, 256, 512, 64, "bf16", seed=61, backward=True)
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    scale = scale_of(64)
    o, lse = fa.forward(q, k, v, scale=scale, window=window, num_splits=1)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, scale=scale, window=window)
    torch.cuda.synchronize()
    x = [to_f64(inp[n])[0] for n in ("q", "k", "v", "do")]
    ref_o, ref_l = attention_forward(x[0], x[1], x[2], scale, False, window=window)
    err_o = np.abs(to_f64(o)[0] - ref_o).max()
    err_l = np.abs(to_f64(lse)[0] - ref_l).max()
    print(f"  fwd max errors: O {err_o:.3e}, LSE {err_l:.3e}", flush=True)
    assert err_o <= 2e-2 and err_l <= 1e-3
    ref = attention_backward(*x, scale, False, window=window)
    check([to_f64(g)[0] for g in (dq, dk, dv)], ref[:3], "bf16", "rounds")
