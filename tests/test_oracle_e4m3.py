"""Pins of the E4M3 part of the oracle (oracle/e4m3.py), on the CPU.

The decoder is pinned to the OCP 8-bit floating point specification's E4M3
values (closed forms of named codes), to an independent library routine
(torch's float8_e4m3fn decoding, all 256 codes) and to the format's
invariants; the dequantized attention to a closed form (identical keys give
the mean of the visible values) and to the linearity of the factors. A copy
of the module with a planted mistake must fail at least one pin.
"""

import os
import types

import numpy as np
import pytest
import torch

import oracle
from fa_inputs import make_fp8_inputs
from oracle import attention_forward

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "e4m3.py")

# Functions under test (replaced by a mutant's in the mutation tests).
e4m3_decode = oracle.e4m3_decode
attention_forward_e4m3 = oracle.attention_forward_e4m3

# Named codes and their values from the format's definition (sign, exponent
# bias 7, three mantissa bits, subnormals M * 2^-9, no infinities).
SPEC = {
    0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x09: 1.125 * 2.0 ** -6,
    0x30: 0.5, 0x38: 1.0, 0x39: 1.125, 0x3F: 1.875, 0x40: 2.0, 0x50: 8.0, 0x68: 64.0, 0x70: 128.0,
    0x77: 240.0, 0x78: 256.0, 0x7E: 448.0, 0x80: -0.0, 0x81: -(2.0 ** -9), 0xB8: -1.0,
    0xC4: -3.0, 0xFE: -448.0,
}


def test_decode_named_codes():
    for code, want in SPEC.items():
        got = e4m3_decode(np.array([code]))[0]
        assert got == want, f"code {code:#04x}: {got} != {want}"
    assert np.signbit(e4m3_decode(np.array([0x80]))[0])
    assert np.isnan(e4m3_decode(np.array([0x7F, 0xFF]))).all()


def test_decode_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.uint8)
    lib = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = e4m3_decode(codes.numpy())
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    ok = ~np.isnan(lib)
    assert np.array_equal(ours[ok], lib[ok])


def test_decode_invariants():
    v = e4m3_decode(np.arange(256))
    assert np.isnan(v).sum() == 2
    pos = v[:127]
    assert (np.diff(pos) > 0).all()  # codes 0..126 increase strictly
    assert np.array_equal(v[128:255], -pos)  # the sign bit negates
    assert pos.max() == 448.0
    # every finite value has at most 4 significant bits and lies on 2^-9 grid
    assert np.array_equal(pos * 2 ** 9, np.round(pos * 2 ** 9))


def test_dequantized_attention_is_attention_of_decoded_values():
    x = make_fp8_inputs(1, 2, 37, 16, seed=3, kv_heads=1)
    desc = x["descale"]
    lib = [x[n].view(torch.float8_e4m3fn).to(torch.float64).numpy() * s
           for n, s in zip(("q8", "k8", "v8"), desc)]
    for causal in (False, True):
        o, lse = attention_forward_e4m3(x["q8"].numpy(), x["k8"].numpy(), x["v8"].numpy(), desc,
                                        0.25, causal, window=(5, 3))
        ro, rl = attention_forward(*lib, 0.25, causal, window=(5, 3))
        np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)
    rows = np.array([0, 5, 36])
    o, lse = attention_forward_e4m3(x["q8"].numpy(), x["k8"].numpy(), x["v8"].numpy(), desc,
                                    0.25, True, q_positions=rows)
    ro, rl = attention_forward(lib[0][..., rows, :], lib[1], lib[2], 0.25, True, q_positions=rows)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)


def test_identical_keys_give_mean_of_dequantized_values():
    rng = np.random.default_rng(0)
    N, d = 9, 8
    q8 = rng.integers(0, 0x7E, size=(1, 1, N, d))
    k8 = np.tile(rng.integers(0, 0x7E, size=(1, 1, 1, d)), (1, 1, N, 1))
    v8 = rng.integers(0, 0x7E, size=(1, 1, N, d)) | (rng.integers(0, 2, size=(1, 1, N, d)) << 7)
    sv = 0.03125
    for causal in (False, True):
        o, _ = attention_forward_e4m3(q8, k8, v8, (0.5, 2.0, sv), 0.3, causal)
        vals = SPEC_TABLE[v8 & 0x7F] * np.where(v8 >> 7, -1.0, 1.0) * sv
        want = np.cumsum(vals, axis=-2) / np.arange(1, N + 1)[:, None] if causal \
            else np.broadcast_to(vals.mean(axis=-2, keepdims=True), vals.shape)
        np.testing.assert_allclose(o, want, rtol=0, atol=1e-12)


def test_factors_are_linear():
    x = make_fp8_inputs(1, 1, 20, 8, seed=4)
    a = (x["q8"].numpy(), x["k8"].numpy(), x["v8"].numpy())
    o1, l1 = attention_forward_e4m3(*a, (0.5, 0.25, 1.0), 1.0, False)
    o2, l2 = attention_forward_e4m3(*a, (1.0, 1.0, 3.0), 0.125, False)  # same score scale
    np.testing.assert_allclose(o2, 3.0 * o1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-12)


def _positive_values_table():
    """|value| of codes 0..127 written out from the definition, code by code."""
    t = np.zeros(128)
    for code in range(128):
        e, m = code >> 3, code & 7
        if e == 15 and m == 7:
            t[code] = np.nan
        elif e == 0:
            t[code] = m / 512.0
        else:
            t[code] = (8 + m) * 2.0 ** (e - 10)
    return t


SPEC_TABLE = _positive_values_table()

PINS = [test_decode_named_codes, test_decode_matches_torch_float8_e4m3fn, test_decode_invariants,
        test_dequantized_attention_is_attention_of_decoded_values,
        test_identical_keys_give_mean_of_dequantized_values, test_factors_are_linear]

MUTATIONS = [
    ("exponent bias 8", "np.exp2(e - 7.0)", "np.exp2(e - 8.0)"),
    ("subnormal step 2^-10", "subnormal = m * 2.0 ** -9", "subnormal = m * 2.0 ** -10"),
    ("mantissa over 16", "(1.0 + m / 8.0)", "(1.0 + m / 16.0)"),
    ("no implicit one", "(1.0 + m / 8.0)", "(m / 8.0)"),
    ("sign ignored", "np.where(sign == 1, -mag, mag)", "mag"),
    ("NaN on the wrong code", "(m == 0x7)", "(m == 0x6)"),
    ("exponent field misread", "e = (c >> 3) & 0xF", "e = (c >> 4) & 0xF"),
    ("V factor dropped", "v = e4m3_decode(v8) * sv", "v = e4m3_decode(v8)"),
    ("K factor dropped", "k = e4m3_decode(k8) * sk", "k = e4m3_decode(k8)"),
    ("query rows not selected", "q = q[..., q_positions, :]", "q = q"),
]


def _mutant(old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique/present: {old!r}"
    src = src.replace(old, new).replace("from .attention import attention_forward", "")
    mod = types.ModuleType("e4m3_mutant")
    mod.__dict__["attention_forward"] = attention_forward
    exec(compile(src, "<e4m3 mutant>", "exec"), mod.__dict__)
    return mod


def _failures(mod, monkeypatch):
    g = globals()
    monkeypatch.setitem(g, "e4m3_decode", mod.e4m3_decode)
    monkeypatch.setitem(g, "attention_forward_e4m3", mod.attention_forward_e4m3)
    failed = []
    for fn in PINS:
        try:
            fn()
        except Exception:  # noqa: BLE001 -- any failure means the pin caught it
            failed.append(fn.__name__)
    return failed


def test_unmutated_copy_passes_every_pin(monkeypatch):
    assert _failures(_mutant("__all__", "__all__"), monkeypatch) == []


@pytest.mark.parametrize("label,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(label, old, new, monkeypatch):
    assert _failures(_mutant(old, new), monkeypatch), f"no pin caught: {label}"
