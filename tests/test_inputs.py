"""The seeded input generator: determinism, draw order, rounding, shapes."""

import torch

from fa_inputs import WORKLOADS, make_inputs


def test_same_seed_same_tensors_and_draw_order():
    a = make_inputs(1, 2, 16, 8, "bf16", seed=0, backward=True)
    b = make_inputs(1, 2, 16, 8, "bf16", seed=0, backward=True)
    for name in ("q", "k", "v", "do"):
        assert torch.equal(a[name].float(), b[name].float())
    # Q, K, V are drawn in that order from one generator: a run without dO
    # yields the same Q, K, V.
    c = make_inputs(1, 2, 16, 8, "bf16", seed=0)
    for name in ("q", "k", "v"):
        assert torch.equal(a[name].float(), c[name].float())
    g = torch.Generator().manual_seed(0)
    q32 = torch.randn((1, 2, 16, 8), generator=g)
    assert torch.equal(a["q"], q32.to(torch.bfloat16))


def test_input_scale_commutes_with_rounding():
    a = make_inputs(1, 1, 64, 16, "bf16", input_scale=0.5)
    b = make_inputs(1, 1, 64, 16, "bf16")
    assert torch.equal(a["v"].float(), b["v"].float() * 0.5)


def test_workload_table():
    w = WORKLOADS["bf16_n4k_d128"]
    assert (w.B, w.H, w.N, w.d, w.dtype, w.causal, w.input_scale) == (4, 16, 4096, 128,
                                                                     "bf16", False, 0.5)
    assert w.fwd_flops() == 4 * 4 * 16 * 4096**2 * 128
    wc = WORKLOADS["bf16_n16k_d128_causal"]
    assert wc.fwd_flops() == 4 * 16 * 16384**2 * 128 / 2
    assert wc.bwd_flops() == 2.5 * wc.fwd_flops()
    assert WORKLOADS["tiny_f32"].scale == float(torch.tensor(0.125))
    assert abs(WORKLOADS["bf16_n16k_d128"].scale - 128 ** -0.5) < 1e-8
