"""GPU parity of the backward's one-launch grids over several rounds: 16-bit
grids of more than 256 workgroups and at most 1024 run the dQ and dK/dV
kernels side by side in one launch (bwd_fused16_kernel), and here each
compute unit runs workgroups of both kinds, one after the other.

B=1 H=24 N=1024 gives 96 dQ and 192 dK/dV workgroups (288); with
H/Hkv = 24/3 the grouped heads are split into 8 parts per key tile (192 dK/dV
workgroups, float32 partials summed afterwards). Plain, grouped K/V heads, a
local window and a block mask, each causal and not, against the oracle at
the plain calls' bounds (16-bit gradients <= 5e-2), and repeats bit for bit.
"""
import numpy as np
import pytest
import torch

import exact_attention_120_amd as fa
from fa_inputs import make_block_mask, make_inputs, to_f64
from oracle import attention_backward

pytestmark = pytest.mark.gpu

TOL_G = 5e-2
DEV = "cuda"
B, H, N = 1, 24, 1024


def scale_of(d):
    return float(torch.tensor(d ** -0.5, dtype=torch.float32))


def run(inp, causal, scale, window=None, mask=None, poison=0xFF):
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale, window=window, block_mask=mask)
    ws = torch.full((fa.fa_bwd_workspace_size(*q.shape),), poison, dtype=torch.uint8, device=DEV)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, causal=causal, scale=scale, workspace=ws,
                             window=window, block_mask=mask)
    torch.cuda.synchronize()
    return dq, dk, dv


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("variant", ["plain", "grouped", "window", "sparse"])
def test_fused_rounds_backward(d, causal, variant):
    print(f"\n[bwd fused rounds] d={d} causal={causal} variant={variant}", flush=True)
    kv_heads = 3 if variant == "grouped" else None
    inp = make_inputs(B, H, N, d, "bf16", seed=71 + d + causal, backward=True, kv_heads=kv_heads)
    window = (60, 20) if variant == "window" else None
    mask = make_block_mask(N, "random", seed=9, density=0.5) if variant == "sparse" else None
    scale = scale_of(d)
    got = run(inp, causal, scale, window, None if mask is None else mask.to(DEV))
    ref = attention_backward(*(to_f64(inp[n]) for n in ("q", "k", "v", "do")), scale, causal,
                             window=window, block_mask=None if mask is None else mask.numpy())
    errs = {}
    for name, g, r in zip(("dq", "dk", "dv"), got, ref[:3]):
        g64 = to_f64(g)
        assert g64.shape == r.shape, name
        assert np.isfinite(g64).all(), f"{name} has non-finite values"
        errs[name] = float(np.abs(g64 - r).max())
    print("  gradient max errors: " + ", ".join(f"{k} {e:.3e}" for k, e in errs.items()), flush=True)
    bad = {k: e for k, e in errs.items() if not e <= TOL_G}
    assert not bad, f"max errors {errs}"


@pytest.mark.parametrize("causal", [False, True])
def test_fused_rounds_fp16_repeats_bitwise(causal):
    inp = make_inputs(B, H, N, 128, "f16", seed=83, backward=True)
    scale = scale_of(128)
    a = run(inp, causal, scale, poison=0xFF)
    b = run(inp, causal, scale, poison=0x00)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
