"""GPU parity at the largest head the library accepts.

One bf16 head of N = 8,384,512 rows at d = 128, so that a head's slab is
N * d * 2 = 2^31 - 2^20 bytes. That is the limit of the kernels' 32-bit
per-head byte offsets, with one tile of overrun kept free. Forward and
backward run with the causal rule and a local window of 127 keys to the
left. Every row then sees at most 128 keys, and the work is O(N) rather
than O(N^2).

Each checked block of n rows [a, a + n) is compared with the float64
oracle run on the self-contained problem over rows and keys [a - 127, a + n).
Under the window, the rows from a on see exactly the same keys there as in
the full head, so O, LSE and dQ of those rows, and dK and dV of the keys
[a, a + n - 127), are the full problem's. Blocks sit at the start of the head
(a = 0, where the sub-problem is the head's own first rows), around the
2^30-byte offset, and at the end, where offsets come closest to 2^31.

Inputs: float32 standard-normal draws from a CUDA torch generator seeded 0 (in
the order Q, K, V, dO, one [1, 1, N, d] tensor each), rounded to bf16 on the
GPU. A CPU draw of four 1.07e9-element tensors would take minutes. The oracle
receives the checked slices, copied back and upcast to float64.

Tolerances are those of the plain calls: O <= 2e-2, LSE <= 1e-3, dQ/dK/dV <= 5e-2.
"""

import numpy as np
import pytest
import torch

import exact_attention_120_amd as fa
from oracle import attention_backward, attention_forward

pytestmark = pytest.mark.gpu

D = 128
N_MAX = ((1 << 31) - (1 << 20)) // (D * 2)   # 8,384,512
LEFT = 127
WINDOW = (LEFT, 0)
BLOCK = 512


def _draw(gen, n):
    x = torch.randn((1, 1, n, D), generator=gen, device="cuda", dtype=torch.float32)
    y = x.to(torch.bfloat16)
    del x
    return y


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def test_max_head_forward_backward():
    assert N_MAX * D * 2 == (1 << 31) - (1 << 20)
    scale = float(torch.tensor(D ** -0.5, dtype=torch.float32))
    print(f"\n[max head] bf16 N={N_MAX} d={D} causal window={WINDOW}: drawing inputs", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(0)
    q, k, v, do = (_draw(gen, N_MAX) for _ in range(4))
    print("[max head] forward", flush=True)
    o, lse = fa.forward(q, k, v, causal=True, scale=scale, window=WINDOW)
    print("[max head] backward", flush=True)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, causal=True, scale=scale, window=WINDOW)
    torch.cuda.synchronize()
    print("[max head] checking blocks against the oracle", flush=True)

    starts = [0, (1 << 30) // (D * 2) - BLOCK // 2, N_MAX - BLOCK]
    for a in starts:
        lo = max(a - LEFT, 0)
        hi = a + BLOCK
        sl = slice(lo, hi)
        qs, ks, vs, dos = (_f64(t[:, :, sl]) for t in (q, k, v, do))
        ref_o, ref_l = attention_forward(qs, ks, vs, scale, True, window=WINDOW)
        ref_dq, ref_dk, ref_dv, _ = attention_backward(qs, ks, vs, dos, scale, True,
                                                       window=WINDOW)
        r = a - lo  # first checked row inside the sub-problem
        err_o = np.abs(_f64(o[:, :, a:hi]) - ref_o[:, :, r:]).max()
        err_l = np.abs(lse[:, :, a:hi].cpu().numpy().astype(np.float64) - ref_l[:, :, r:]).max()
        err_dq = np.abs(_f64(dq[:, :, a:hi]) - ref_dq[:, :, r:]).max()
        # Keys whose every query lies inside the sub-problem: [a, hi - LEFT),
        # and at the head's start all keys up to hi - LEFT.
        kend = hi - LEFT
        err_dk = np.abs(_f64(dk[:, :, a:kend]) - ref_dk[:, :, r:kend - lo]).max()
        err_dv = np.abs(_f64(dv[:, :, a:kend]) - ref_dv[:, :, r:kend - lo]).max()
        print(f"[max head] rows {a}..{hi}: O {err_o:.2e} LSE {err_l:.2e} dQ {err_dq:.2e} "
              f"dK {err_dk:.2e} dV {err_dv:.2e}", flush=True)
        assert err_o <= 2e-2 and err_l <= 1e-3, (a, err_o, err_l)
        assert max(err_dq, err_dk, err_dv) <= 5e-2, (a, err_dq, err_dk, err_dv)
        assert np.isfinite(_f64(o[:, :, a:hi])).all()
