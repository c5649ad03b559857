"""fa_bwd_noalloc (the backward for callers that cannot allocate: its
scratch is the library's static per-GPU array) against fa_bwd, the entry
point with a caller workspace whose kernels it shares.

Two calls in a row on one GPU, the second on a smaller problem, so the
second call starts from the first call's leftovers in the static array.
16-bit results must equal fa_bwd's bit for bit (same kernels, no atomics);
float32 results (whose dQ is accumulated with atomics) within the scope's
float32 bound, 1e-5, of fa_bwd's and of the oracle's.
"""

import numpy as np
import pytest
import torch

import exact_attention_120_amd as fa
from fa_inputs import make_inputs, to_f64
from oracle import attention_backward

pytestmark = pytest.mark.gpu

DEV = "cuda"


def both(inp, causal, scale):
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale)
    B, H, N, d = q.shape
    ws = torch.full((fa.fa_bwd_workspace_size(B, H, N, d),), 0xFF, dtype=torch.uint8, device=DEV)
    ref = [torch.full_like(x, float("nan")) for x in (q, k, v)]
    fa.fa_bwd(q, k, v, o, do, lse, *ref, scale, causal, ws)
    got = [torch.full_like(x, float("nan")) for x in (q, k, v)]
    fa.fa_bwd_noalloc(q, k, v, o, do, lse, *got, scale, causal)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_noalloc_equals_fa_bwd_on_two_calls_second_smaller(dtype):
    for (B, H, N, d, causal, seed) in ((2, 4, 1000, 128, True, 41), (1, 2, 300, 64, False, 42)):
        print(f"\n[noalloc] dtype={dtype} B={B} H={H} N={N} d={d} causal={causal}", flush=True)
        inp = make_inputs(B, H, N, d, dtype, seed=seed, backward=True)
        scale = float(torch.tensor(d ** -0.5, dtype=torch.float32))
        ref, got = both(inp, causal, scale)
        if dtype == "f32":
            oracle = attention_backward(*(to_f64(inp[n]) for n in ("q", "k", "v", "do")), scale,
                                        causal)
            for name, r, g, x in zip(("dq", "dk", "dv"), ref, got, oracle):
                e_ref = float((g - r).abs().max())
                e_orc = float(np.abs(to_f64(g) - x).max())
                print(f"  {name}: |noalloc - fa_bwd| {e_ref:.3e}, |noalloc - oracle| {e_orc:.3e}",
                      flush=True)
                assert e_ref <= 1e-5 and e_orc <= 1e-5, name
        else:
            for name, r, g in zip(("dq", "dk", "dv"), ref, got):
                assert torch.equal(r, g), name


def test_noalloc_rejects_what_does_not_fit():
    """4*B*H*N bytes above 64 MiB: rejected before anything is enqueued."""
    q = torch.zeros(1, 256, 65537, 64, dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros(1, 256, 65537, dtype=torch.float32, device=DEV)
    with pytest.raises(fa.FaError) as e:
        fa.fa_bwd_noalloc(q, q, q, q, q, lse, q, q, q, 0.125, False)
    assert e.value.status == -6
