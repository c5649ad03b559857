"""GPU parity of the 8-bit forward (fa_fwd_fp8) against the CPU oracle.

The oracle is exact attention (float64) over the values the E4M3 codes stand
for (code value times the tensor's factor). The kernel's own arithmetic is
float32 except for one rounding: each probability enters the P V product as
an E4M3 code of x = 2^3 * p (p relative to the kernel's reference, at most
the row max), while the normalizer uses the unrounded values. E4M3 rounds a
normal x (>= 2^-6) with error <= 2^-4 * x, a subnormal one with error
<= 2^-10. Since the reference never exceeds the final row max, the kernel's
normalizer is at least 2^3 / max_j w_ij (w = the exact softmax weights), and
the error of O[i, c] is bounded by

    B_ic = 2^-4 * sum_j w_ij |V_jc| + 2^-10 / 2^3 * max_j w_ij * sum_{j seen} |V_jc|

plus the output rounding (bf16: 2^-8 |O|, fp16: 2^-11 |O|) and float32 slack
(1e-5 max |V|). That worst case assumes every rounding error has the same
sign; the errors are in fact spread on both sides, so the tests also bound
the mean square error by twice the variance of that model: RNE errors are
at most uniform over one code step (step <= 2^-3 x for a normal x, 2^-9 for
a subnormal one), giving

    Var_ic <= (2^-6/12) sum_j w_ij^2 V_jc^2
              + (2^-18/12) / 2^6 * (max_j w_ij)^2 * sum_{j seen} V_jc^2
              + (output code step)^2 / 12.

The scores themselves carry one more error: the FP8 matrix instruction does
not add its 64 products like float32. tests/test_hw_fp8_mfma.py measures it
on gfx950 over random operands against exact sums: up to 2^-11.6 of the sum
of the products' magnitudes for codes spread over the whole E4M3 range (RMS
2^-15.0), less for quantized normal data. With eps = 2^-10 (that test
requires the worst measured to stay within eps/2) a scaled score s_ij moves
by at most

    delta_i = eps * scale * max_{j seen} sum_k |Q_ik| |K_jk|,

which moves the LSE by at most delta_i (a log-sum-exp moves by at most its
largest argument's change) and O[i, c] by at most 2 delta_i sum_j w_ij |V_jc|
(the weights change by factors within e^(+-2 delta)). Both terms join the
bounds above; the mean-square model adds (2^-16 * scale * max_j sum_k
|Q_ik| |K_jk| * sum_j w_ij |V_jc|)^2 (the same test requires the RMS over
the operands the kernel feeds the instruction to stay within half of 2^-16). The LSE is
otherwise computed from unrounded values (float32 slack 1e-5 (1 + |LSE|)).
Closed forms that involve no probability rounding (all keys equal: every
row is the mean of the values it sees) are checked to the output rounding
alone.
"""

import numpy as np
import pytest
import torch

import exact_attention_120_amd as fa
from fa_inputs import make_fp8_inputs
from oracle import attention_forward_e4m3, attention_probabilities, e4m3_decode

pytestmark = pytest.mark.gpu

DEV = "cuda"
# FP8 MFMA accumulation error relative to sum |products|: worst case and RMS
# (checked against the instruction by tests/test_hw_fp8_mfma.py).
EPS_MFMA8 = 2.0 ** -10
RMS_MFMA8 = 2.0 ** -16
OUT = {"bf16": torch.bfloat16, "f16": torch.float16}
OUT_REL = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}
OUT_BITS = {"bf16": 8, "f16": 11}  # significant bits of the output type


def scale_of(d):
    return float(torch.tensor(d ** -0.5, dtype=torch.float32))


def run(inp, causal, scale, out="bf16", window=None, descale=None):
    q8, k8, v8 = (inp[n].to(DEV) for n in ("q8", "k8", "v8"))
    B, H, N, d = q8.shape
    o = torch.full((B, H, N, d), float("nan"), dtype=OUT[out], device=DEV)
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=DEV)
    fa.fa_fwd_fp8(q8, k8, v8, o, lse, scale, causal, *(descale or inp["descale"]), window=window)
    torch.cuda.synchronize()
    return o, lse


def dequantized(inp):
    return [e4m3_decode(inp[n].numpy()) * s for n, s in zip(("q8", "k8", "v8"), inp["descale"])]


def bounds(inp, causal, scale, window=None, rows=None):
    """Terms of the module docstring for the checked rows ([B, H, rows, ...]):
    the O bound and variance model (without the output rounding), the score
    error bound delta (as [..., 1]) and max |V|."""
    q, k, v = dequantized(inp)
    if rows is not None:
        q = q[..., rows, :]
    w = attention_probabilities(q, k, scale, causal, window=window, q_positions=rows)
    group = q.shape[1] // v.shape[1]
    v, k = np.repeat(v, group, axis=1), np.repeat(k, group, axis=1)
    seen = (w > 0).astype(np.float64)
    wmax = w.max(axis=-1, keepdims=True)
    av, v2 = np.abs(v), v * v
    mag = np.max(np.where(seen > 0, np.abs(q) @ np.abs(k).swapaxes(-1, -2), 0.0), axis=-1,
                 keepdims=True)  # max_{j seen} sum_k |Q_ik| |K_jk|
    delta = EPS_MFMA8 * scale * mag
    wav = w @ av
    b = 2.0 ** -4 * wav + 2.0 ** -13 * wmax * (seen @ av) + 2.0 * delta * wav
    var = (2.0 ** -6 / 12) * ((w * w) @ v2) + (2.0 ** -24 / 12) * wmax ** 2 * (seen @ v2) \
        + (RMS_MFMA8 * scale * mag * wav) ** 2
    return b, var, delta, float(np.abs(v).max())


def check(o, lse, inp, causal, scale, out, window=None, rows=None):
    ref_o, ref_l = attention_forward_e4m3(inp["q8"].numpy(), inp["k8"].numpy(), inp["v8"].numpy(),
                                          inp["descale"], scale, causal, window=window,
                                          q_positions=rows)
    o64 = o.detach().cpu().to(torch.float64).numpy()
    l64 = lse.detach().cpu().to(torch.float64).numpy()
    if rows is not None:
        o64, l64 = o64[..., rows, :], l64[..., rows]
    assert np.isfinite(o64).all() and np.isfinite(l64).all()
    b, var, delta, vmax = bounds(inp, causal, scale, window, rows)
    err = np.abs(o64 - ref_o)
    rel = OUT_REL[out]
    limit = b + rel * (np.abs(ref_o) + b) + 1e-5 * vmax
    worst = np.unravel_index(np.argmax(err - limit), err.shape)
    assert (err <= limit).all(), (f"O err {err[worst]:.3e} > bound {limit[worst]:.3e} at {worst} "
                                  f"(ref {ref_o[worst]:.4e})")
    step = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref_o), 1e-30))) + 1 - OUT_BITS[out])
    model = var + step ** 2 / 12
    mse, mmodel = float((err ** 2).mean()), float(model.mean())
    assert mse <= 2 * mmodel + (1e-6 * vmax) ** 2, f"mean square err {mse:.3e} > 2 x {mmodel:.3e}"
    err_l = np.abs(l64 - ref_l)
    lim_l = delta[..., 0] + 1e-5 * (1 + np.abs(ref_l))
    assert (err_l <= lim_l).all(), (f"LSE err {err_l.max():.3e} (bound at worst "
                                    f"{lim_l.flat[np.argmax(err_l - lim_l)]:.3e})")
    return float(err.max()), float(np.sqrt(mse)), float(np.sqrt(mmodel)), float(err_l.max())


@pytest.mark.parametrize("out", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 100, 300, 700])
def test_small_shapes(out, d, causal, N):
    print(f"\n[fp8] out={out} d={d} causal={causal} N={N}", flush=True)
    inp = make_fp8_inputs(2, 2, N, d, seed=N + d)
    scale = scale_of(d)
    o, lse = run(inp, causal, scale, out)
    r = check(o, lse, inp, causal, scale, out)
    print(f"[fp8] max|dO|={r[0]:.3e} rms={r[1]:.3e} (model {r[2]:.3e}) max|dLSE|={r[3]:.3e}",
          flush=True)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("heads,window,scale", [((4, 2), None, None), ((4, 1), (100, 0), None),
                                                 ((6, 3), (64, 200), None), ((2, 2), (0, 0), None),
                                                 ((4, 2), (100, 40), 1.5), ((2, 1), (45, -1), 4.0)])
def test_grouped_and_window(causal, heads, window, scale):
    H, Hkv = heads
    print(f"\n[fp8 opts] causal={causal} H={H} Hkv={Hkv} window={window} scale={scale}",
          flush=True)
    inp = make_fp8_inputs(1, H, 700, 128, seed=H + Hkv, kv_heads=Hkv)
    scale = scale_of(128) if scale is None else scale
    o, lse = run(inp, causal, scale, "bf16", window)
    check(o, lse, inp, causal, scale, "bf16", window)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_values(causal):
    """No probability rounding: every visible score of a row is the row max,
    so every probability is exactly 2^3 * 1. O is the mean of the visible V
    rows (prefix means under the causal rule), up to float32 sums and the
    output rounding."""
    B, H, N, d = 1, 2, 1000, 128
    inp = make_fp8_inputs(B, H, N, d, seed=7)
    inp["k8"] = inp["k8"][:, :, :1, :].expand(B, H, N, d).contiguous()
    o, lse = run(inp, causal, 0.7, "bf16")
    v = dequantized(inp)[2]
    want = np.cumsum(v, axis=-2) / np.arange(1, N + 1)[:, None] if causal \
        else np.broadcast_to(v.mean(axis=-2, keepdims=True), v.shape)
    got = o.cpu().to(torch.float64).numpy()
    err = np.abs(got - want)
    assert (err <= 2.0 ** -8 * np.abs(want) + 1e-5 * np.abs(v).max()).all(), err.max()
    ref_o, ref_l = attention_forward_e4m3(inp["q8"].numpy(), inp["k8"].numpy(), inp["v8"].numpy(),
                                          inp["descale"], 0.7, causal)
    delta = bounds(inp, causal, 0.7)[2][..., 0]
    assert (np.abs(lse.cpu().numpy() - ref_l) <= delta + 1e-5 * (1 + np.abs(ref_l))).all()


def test_factors_scale_exactly():
    """Doubling V's factor doubles O exactly; moving a power of two between
    the factors of Q and K (same score scale) changes nothing."""
    inp = make_fp8_inputs(1, 2, 333, 64, seed=8)
    sq, sk, sv = inp["descale"]
    o1, l1 = run(inp, True, 0.125, "bf16")
    o2, l2 = run(inp, True, 0.125, "bf16", descale=(sq, sk, 2 * sv))
    o3, l3 = run(inp, True, 0.125, "bf16", descale=(2 * sq, sk / 2, sv))
    assert torch.equal(o2, 2 * o1) and torch.equal(l1, l2)
    assert torch.equal(o3, o1) and torch.equal(l3, l1)


_FULL = {}


def _full_size(causal):
    """B=1, H=16, N=16384, d=128 (the long-sequence workload), as timed: the
    whole output computed once per causal setting."""
    if causal not in _FULL:
        _FULL.clear()
        inp = make_fp8_inputs(1, 16, 16384, 128, seed=0)
        o, lse = run(inp, causal, scale_of(128), "bf16")
        _FULL[causal] = (inp, o.cpu(), lse.cpu())
    return _FULL[causal]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("part", range(4))
def test_full_size_every_row(causal, part):
    """The full launch; every row of every head is checked against the
    oracle and the bounds above, four heads per test case, 2048 rows at a
    time (the bounds materialize one row block's softmax weights)."""
    inp, o, lse = _full_size(causal)
    N, scale = 16384, scale_of(128)
    print(f"\n[fp8 full] causal={causal} heads {4 * part}..{4 * part + 3}", flush=True)
    worst = [0.0, 0.0, 0.0]
    for h in range(4 * part, 4 * part + 4):
        sub = {"q8": inp["q8"][:, h:h + 1], "k8": inp["k8"][:, h:h + 1],
               "v8": inp["v8"][:, h:h + 1], "descale": inp["descale"]}
        for r0 in range(0, N, 2048):
            rows = np.arange(r0, r0 + 2048)
            r = check(o[:, h:h + 1], lse[:, h:h + 1], sub, causal, scale, "bf16", rows=rows)
            worst = [max(worst[0], r[0]), max(worst[1], r[1]), max(worst[2], r[3])]
    print(f"[fp8 full] max|dO|={worst[0]:.3e} max block rms={worst[1]:.3e} "
          f"max|dLSE|={worst[2]:.3e}", flush=True)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


def test_outputs_do_not_spill():
    B, H, N, d = 1, 2, 300, 64
    inp = make_fp8_inputs(B, H, N, d, seed=10)
    q8, k8, v8 = (inp[n].to(DEV) for n in ("q8", "k8", "v8"))
    pad = 4096
    obuf = torch.full((pad + B * H * N * d + pad,), 7.0, dtype=torch.float16, device=DEV)
    lbuf = torch.full((pad + B * H * N + pad,), 7.0, dtype=torch.float32, device=DEV)
    o = obuf[pad:pad + B * H * N * d].view(B, H, N, d)
    lse = lbuf[pad:pad + B * H * N].view(B, H, N)
    fa.fa_fwd_fp8(q8, k8, v8, o, lse, 0.125, False, *inp["descale"])
    torch.cuda.synchronize()
    assert (obuf[:pad] == 7).all() and (obuf[-pad:] == 7).all()
    assert (lbuf[:pad] == 7).all() and (lbuf[-pad:] == 7).all()
    check(o, lse, inp, False, 0.125, "f16")


def test_binding_accepts_float8_tensors_and_rejects_bad_ones():
    inp = make_fp8_inputs(1, 2, 64, 64, seed=11)
    q8, k8, v8 = (inp[n].to(DEV) for n in ("q8", "k8", "v8"))
    o1, l1 = fa.forward_fp8(q8, k8, v8, inp["descale"], causal=True)
    f8 = [t.view(torch.float8_e4m3fn) for t in (q8, k8, v8)]
    o2, l2 = fa.forward_fp8(*f8, inp["descale"], causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    with pytest.raises(ValueError):
        fa.forward_fp8(q8.to(torch.int8), k8, v8, inp["descale"])
    with pytest.raises(ValueError):
        fa.forward_fp8(q8, k8, v8, inp["descale"], out_dtype=torch.float32)
    with pytest.raises(fa.FaError):
        fa.forward_fp8(q8, k8, v8, (0.0, 1.0, 1.0))
