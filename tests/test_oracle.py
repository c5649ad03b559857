"""Pins for the CPU oracle: checks against facts fixed outside the oracle.

Every check here compares the oracle with something it does not compute
itself: hand-derived worked examples (tests/golden), closed forms, invariants
of softmax attention, pure-Python brute force on tiny inputs, finite
differences, and an independent library routine (torch's CPU float64
attention and autograd). test_oracle_mutations.py plants plausible mistakes in
a copy of the oracle and shows that these pins catch them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (attention_backward, attention_forward, attention_forward_blockwise,
                    attention_probabilities, merge_partials)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# --------------------------------------------------------------- worked examples
def test_golden_forward_hand_example():
    fx = json.load(open(os.path.join(GOLDEN, "hand_forward_n3_d2.json")))
    k, v = np.array(fx["k"]), np.array(fx["v"])
    for case in fx["cases"]:
        o, lse = attention_forward(np.array(case["q"]), k, v, case["scale"], case["causal"])
        np.testing.assert_allclose(o, case["o"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, case["lse"], rtol=0, atol=1e-12)


def test_golden_backward_hand_example():
    fx = json.load(open(os.path.join(GOLDEN, "hand_backward_n2_d1.json")))
    q, k, v, do = (np.array(fx[n]) for n in ("q", "k", "v", "do"))
    for case in fx["cases"]:
        o, lse = attention_forward(q, k, v, fx["scale"], case["causal"])
        np.testing.assert_allclose(o, case["o"], atol=1e-12)
        np.testing.assert_allclose(lse, case["lse"], atol=1e-12)
        dq, dk, dv, _ = attention_backward(q, k, v, do, fx["scale"], case["causal"])
        np.testing.assert_allclose(dq, case["dq"], atol=1e-12)
        np.testing.assert_allclose(dk, case["dk"], atol=1e-12)
        np.testing.assert_allclose(dv, case["dv"], atol=1e-12)


# --------------------------------------------------------------- brute force
def brute_force(q, k, v, scale, causal):
    """Pure-Python loops, no BLAS, no max subtraction (inputs are tiny)."""
    n, d = len(q), len(q[0])
    dv = len(v[0])
    o = [[0.0] * dv for _ in range(n)]
    lse = [0.0] * n
    for i in range(n):
        w = []
        for j in range(len(k)):
            if causal and j > i:
                w.append(0.0)
                continue
            dot = 0.0
            for c in range(d):
                dot += q[i][c] * k[j][c]
            w.append(math.exp(scale * dot))
        z = sum(w)
        lse[i] = math.log(z)
        for c in range(dv):
            o[i][c] = sum(w[j] * v[j][c] for j in range(len(k))) / z
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("n", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("d", [1, 2, 4])
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_tiny(n, d, causal):
    seed = 100 * n + 10 * d + causal
    q, k, v = rand((n, d), seed), rand((n, d), seed + 1), rand((n, d + 1), seed + 2)
    scale = 0.37 + 0.1 * d
    o, lse = attention_forward(q, k, v, scale, causal)
    bo, blse = brute_force(q.tolist(), k.tolist(), v.tolist(), scale, causal)
    np.testing.assert_allclose(o, bo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, blse, rtol=0, atol=1e-12)


def test_rectangular_and_batched_shapes():
    q, k, v = rand((2, 3, 5, 4), 1), rand((2, 3, 7, 4), 2), rand((2, 3, 7, 6), 3)
    o, lse = attention_forward(q, k, v, 0.5, False)
    assert o.shape == (2, 3, 5, 6) and lse.shape == (2, 3, 5)
    for b in range(2):
        for h in range(3):
            bo, blse = brute_force(q[b, h].tolist(), k[b, h].tolist(), v[b, h].tolist(),
                                   0.5, False)
            np.testing.assert_allclose(o[b, h], bo, atol=1e-12)
            np.testing.assert_allclose(lse[b, h], blse, atol=1e-12)


# --------------------------------------------------------------- closed forms
@pytest.mark.parametrize("causal", [False, True])
def test_rows_of_p_sum_to_one(causal):
    p = attention_probabilities(rand((2, 64, 16), 5), rand((2, 64, 16), 6), 0.25, causal)
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-12)
    assert (p >= 0).all()
    if causal:
        assert np.all(np.triu(p[0], 1) == 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_v(causal):
    n, d = 40, 8
    q, v = rand((n, d), 7), rand((n, 3), 8)
    krow = rand((d,), 9)
    k = np.tile(krow, (n, 1))
    scale = 0.3
    o, lse = attention_forward(q, k, v, scale, causal)
    counts = np.arange(1, n + 1) if causal else np.full(n, n)
    mean = np.cumsum(v, 0) / counts[:, None] if causal else np.tile(v.mean(0), (n, 1))
    np.testing.assert_allclose(o, mean, atol=1e-12)
    np.testing.assert_allclose(lse, scale * q @ krow + np.log(counts), atol=1e-12)


def test_causal_row0_returns_v0():
    q, k, v = rand((1, 2, 33, 16), 10), rand((1, 2, 33, 16), 11), rand((1, 2, 33, 16), 12)
    o, lse = attention_forward(q, k, v, 0.25, True)
    np.testing.assert_allclose(o[..., 0, :], v[..., 0, :], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[..., 0], 0.25 * (q[..., 0, :] * k[..., 0, :]).sum(-1),
                               atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_scale_zero_is_uniform_average(causal):
    n = 25
    q, k, v = rand((n, 4), 13), rand((n, 4), 14), rand((n, 5), 15)
    o, lse = attention_forward(q, k, v, 0.0, causal)
    counts = np.arange(1, n + 1) if causal else np.full(n, n)
    ref = np.cumsum(v, 0) / counts[:, None] if causal else np.tile(v.mean(0), (n, 1))
    np.testing.assert_allclose(o, ref, atol=1e-12)
    np.testing.assert_allclose(lse, np.log(counts), atol=1e-12)


def test_single_key():
    q, k, v = rand((3, 1, 1, 6), 16), rand((3, 1, 1, 6), 17), rand((3, 1, 1, 6), 18)
    for causal in (False, True):
        o, lse = attention_forward(q, k, v, 0.7, causal)
        np.testing.assert_allclose(o, v, atol=1e-14)
        np.testing.assert_allclose(lse, 0.7 * (q * k).sum(-1), atol=1e-14)


def test_one_hot_dominant_score_selects_row():
    n = d = 64
    q, k, v = np.eye(n), 30.0 * np.eye(n), rand((n, d), 19)
    o, _ = attention_forward(q, k, v, 1.0, False)
    bound = 2 * (n - 1) * math.exp(-30) * np.abs(v).max()
    assert np.abs(o - v).max() <= bound


# --------------------------------------------------------------- invariants
def test_key_permutation_invariance_and_query_equivariance():
    q, k, v = rand((20, 8), 20), rand((30, 8), 21), rand((30, 5), 22)
    o, lse = attention_forward(q, k, v, 0.4, False)
    pk = np.random.default_rng(0).permutation(30)
    o2, lse2 = attention_forward(q, k[pk], v[pk], 0.4, False)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, atol=1e-12)
    pq = np.random.default_rng(1).permutation(20)
    o3, lse3 = attention_forward(q[pq], k, v, 0.4, False)
    np.testing.assert_allclose(o3, o[pq], atol=1e-12)
    np.testing.assert_allclose(lse3, lse[pq], atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_and_value_affinity(causal):
    """K + 1u^T shifts row i's scores by scale*q_i.u (softmax unchanged);
    O is affine in V: V W + 1c^T -> O W + 1c^T."""
    n, d = 24, 6
    q, k, v = rand((n, d), 23), rand((n, d), 24), rand((n, 4), 25)
    u, w, c = rand((d,), 26), rand((4, 3), 27), rand((3,), 28)
    o, lse = attention_forward(q, k, v, 0.5, causal)
    o2, lse2 = attention_forward(q, k + u, v, 0.5, causal)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(lse2, lse + 0.5 * q @ u, atol=1e-12)
    o3, _ = attention_forward(q, k, v @ w + c, 0.5, causal)
    np.testing.assert_allclose(o3, o @ w + c, atol=1e-12)


def test_sampled_rows_match_full():
    q, k, v = rand((1, 1, 300, 8), 29), rand((1, 1, 300, 8), 30), rand((1, 1, 300, 8), 31)
    o, lse = attention_forward(q, k, v, 0.35, True)
    rows = np.array([0, 1, 77, 150, 299])
    os_, ls_ = attention_forward(q[..., rows, :], k, v, 0.35, True, q_positions=rows)
    np.testing.assert_allclose(os_, o[..., rows, :], atol=1e-13)
    np.testing.assert_allclose(ls_, lse[..., rows], atol=1e-13)


def test_row_chunking_is_invisible(monkeypatch):
    import oracle.attention as oa
    q, k, v = rand((1, 2, 130, 8), 32), rand((1, 2, 130, 8), 33), rand((1, 2, 130, 8), 34)
    do = rand((1, 2, 130, 8), 35)
    ref_f = attention_forward(q, k, v, 0.3, True)
    ref_b = attention_backward(q, k, v, do, 0.3, True)
    monkeypatch.setattr(oa, "ROW_CHUNK", 7)
    for a, b in zip(attention_forward(q, k, v, 0.3, True), ref_f):
        np.testing.assert_allclose(a, b, atol=1e-13)
    for a, b in zip(attention_backward(q, k, v, do, 0.3, True), ref_b):
        np.testing.assert_allclose(a, b, atol=1e-12)


# --------------------------------------------------------------- online recurrence
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bq,bk", [(1, 1), (7, 5), (16, 64), (64, 16), (100, 100), (33, 17)])
def test_blockwise_online_softmax_equals_full(causal, bq, bk):
    q, k, v = rand((2, 97, 12), 40), rand((2, 97, 12), 41), rand((2, 97, 12), 42)
    o, lse = attention_forward(q, k, v, 0.29, causal)
    ob, lseb = attention_forward_blockwise(q, k, v, 0.29, causal, bq, bk)
    np.testing.assert_allclose(ob, o, atol=1e-12)
    np.testing.assert_allclose(lseb, lse, atol=1e-12)


def test_two_shard_merge_equals_full():
    q, k, v = rand((3, 50, 8), 43), rand((3, 90, 8), 44), rand((3, 90, 8), 45)
    o, lse = attention_forward(q, k, v, 0.6, False)
    split = np.random.default_rng(3).permutation(90)
    a, b = split[:31], split[31:]
    oa, la = attention_forward(q, k[:, a], v[:, a], 0.6, False)
    ob, lb = attention_forward(q, k[:, b], v[:, b], 0.6, False)
    om, lm = merge_partials(oa, la, ob, lb)
    np.testing.assert_allclose(om, o, atol=1e-12)
    np.testing.assert_allclose(lm, lse, atol=1e-12)


# --------------------------------------------------------------- gradients
@pytest.mark.parametrize("causal", [False, True])
def test_gradients_match_finite_differences(causal):
    n, d = 6, 3
    q, k, v, do = (rand((n, d), 50 + i) for i in range(4))
    scale = 0.8
    dq, dk, dv, _ = attention_backward(q, k, v, do, scale, causal)

    def loss(qq, kk, vv):
        return float((attention_forward(qq, kk, vv, scale, causal)[0] * do).sum())

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            fd[idx] = (loss(args_p["q"], args_p["k"], args_p["v"])
                       - loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8, err_msg=name)


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_invariants(causal):
    q, k, v, do = (rand((2, 70, 8), 60 + i) for i in range(4))
    o, _ = attention_forward(q, k, v, 0.35, causal)
    dq, dk, dv, dsum = attention_backward(q, k, v, do, 0.35, causal)
    # D_i = sum_j P_ij dP_ij equals rowsum(dO * O) (= dO_i . sum_j P_ij V_j).
    np.testing.assert_allclose(dsum, (do * o).sum(-1), rtol=1e-12, atol=1e-12)
    # Each row of dS sums to zero, so the key gradients sum to zero.
    np.testing.assert_allclose(dk.sum(-2), 0.0, atol=1e-12)
    # Rows of P sum to one, so the value gradients sum to the output gradients.
    np.testing.assert_allclose(dv.sum(-2), do.sum(-2), atol=1e-12)


# --------------------------------------------------------------- library routine
@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_cpu_float64_attention_and_autograd(causal):
    shape = (2, 3, 45, 16)
    q, k, v, do = (rand(shape, 70 + i) for i in range(4))
    scale = 0.21
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                           scale=scale)
    to.backward(torch.tensor(do))
    o, lse = attention_forward(q, k, v, scale, causal)
    np.testing.assert_allclose(o, to.detach().numpy(), atol=1e-12)
    tlse = torch.logsumexp(
        (scale * tq @ tk.transpose(-1, -2)).masked_fill(
            torch.ones(45, 45, dtype=torch.bool).triu(1) if causal
            else torch.zeros(45, 45, dtype=torch.bool), float("-inf")), dim=-1)
    np.testing.assert_allclose(lse, tlse.detach().numpy(), atol=1e-12)
    dq, dk, dv, _ = attention_backward(q, k, v, do, scale, causal)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-11)


# --------------------------------------------------------------- windows and grouped K/V heads
WINDOWS = [(0, 0), (1, 0), (0, 2), (2, 1), (3, -1), (-1, 2)]


def brute_force_general(q, k, v, scale, causal, window):
    """Pure-Python loops over heads, rows and keys with the visibility rule
    spelled out; query head h uses K/V head h // (Hq / Hkv)."""
    hq, hkv = len(q), len(k)
    group = hq // hkv
    o, lse = [], []
    for h in range(hq):
        kh, vh = k[h // group], v[h // group]
        oh, lh = [], []
        for i in range(len(q[h])):
            w = []
            for j in range(len(kh)):
                vis = not (causal and j > i)
                if window[0] >= 0 and j < i - window[0]:
                    vis = False
                if window[1] >= 0 and j > i + window[1]:
                    vis = False
                w.append(math.exp(scale * sum(a * b for a, b in zip(q[h][i], kh[j]))) if vis else 0.0)
            z = sum(w)
            lh.append(math.log(z))
            oh.append([sum(w[j] * vh[j][c] for j in range(len(kh))) / z for c in range(len(vh[0]))])
        o.append(oh)
        lse.append(lh)
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("window", WINDOWS)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("hq,hkv", [(1, 1), (2, 1), (4, 2)])
def test_brute_force_window_and_groups(window, causal, hq, hkv):
    n, d = 7, 3
    seed = 7 * hq + 3 * hkv + 11 * causal + window[0] * 5 + window[1]
    q, k, v = rand((hq, n, d), seed), rand((hkv, n, d), seed + 1), rand((hkv, n, d + 1), seed + 2)
    o, lse = attention_forward(q, k, v, 0.61, causal, window=window)
    bo, blse = brute_force_general(q.tolist(), k.tolist(), v.tolist(), 0.61, causal, window)
    np.testing.assert_allclose(o, bo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, blse, rtol=0, atol=1e-12)


def test_window_closed_forms():
    q, k, v = rand((2, 20, 5), 81), rand((2, 20, 5), 82), rand((2, 20, 3), 83)
    # Each row sees only its own key: O = V, LSE = scale * q_i . k_i.
    o, lse = attention_forward(q, k, v, 0.4, False, window=(0, 0))
    np.testing.assert_allclose(o, v, atol=1e-14)
    np.testing.assert_allclose(lse, 0.4 * (q * k).sum(-1), atol=1e-14)
    # A window covering every key is plain attention; (unbounded, 0) is causal.
    full = attention_forward(q, k, v, 0.4, False)
    for a, b in zip(attention_forward(q, k, v, 0.4, False, window=(19, 25)), full):
        np.testing.assert_allclose(a, b, atol=1e-14)
    causal = attention_forward(q, k, v, 0.4, True)
    for a, b in zip(attention_forward(q, k, v, 0.4, False, window=(-1, 0)), causal):
        np.testing.assert_allclose(a, b, atol=1e-14)


def test_grouped_heads_equal_repeated_heads_and_mqa_closed_form():
    q, k, v = rand((2, 6, 9, 4), 91), rand((2, 3, 9, 4), 92), rand((2, 3, 9, 4), 93)
    o, lse = attention_forward(q, k, v, 0.5, True)
    # Query heads 2g and 2g+1 share K/V head g.
    for h in range(6):
        oh, lh = attention_forward(q[:, h], k[:, h // 2], v[:, h // 2], 0.5, True)
        np.testing.assert_allclose(o[:, h], oh, atol=1e-14)
        np.testing.assert_allclose(lse[:, h], lh, atol=1e-14)
    # One K/V head and identical query heads: identical outputs, and the K/V
    # gradients are the per-head gradients times the number of heads.
    q1 = np.repeat(rand((1, 1, 9, 4), 94), 4, axis=1)
    k1, v1, do1 = rand((1, 1, 9, 4), 95), rand((1, 1, 9, 4), 96), np.repeat(rand((1, 1, 9, 4), 97), 4, axis=1)
    o1, _ = attention_forward(q1, k1, v1, 0.5, False)
    np.testing.assert_allclose(o1, np.repeat(o1[:, :1], 4, axis=1), atol=1e-14)
    _, dk1, dv1, _ = attention_backward(q1, k1, v1, do1, 0.5, False)
    _, dk0, dv0, _ = attention_backward(q1[:, :1], k1, v1, do1[:, :1], 0.5, False)
    np.testing.assert_allclose(dk1, 4 * dk0, atol=1e-12)
    np.testing.assert_allclose(dv1, 4 * dv0, atol=1e-12)


@pytest.mark.parametrize("window", [(2, 1), (4, -1), (-1, 3)])
def test_window_gradients_match_finite_differences(window):
    n, d = 6, 3
    q, k, v, do = (rand((n, d), 150 + i) for i in range(4))
    scale = 0.7
    dq, dk, dv, _ = attention_backward(q, k, v, do, scale, False, window=window)

    def loss(qq, kk, vv):
        return float((attention_forward(qq, kk, vv, scale, False, window=window)[0] * do).sum())

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p[name], args_m[name] = xp, xm
            fd[idx] = (loss(args_p["q"], args_p["k"], args_p["v"])
                       - loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8, err_msg=name)


@pytest.mark.parametrize("window,causal", [((5, 3), False), ((7, -1), True), ((-1, -1), True), ((0, 9), False)])
def test_grouped_window_matches_torch_float64_and_autograd(window, causal):
    b, hq, hkv, n, d = 2, 4, 2, 33, 8
    q, do = rand((b, hq, n, d), 170), rand((b, hq, n, d), 171)
    k, v = rand((b, hkv, n, d), 172), rand((b, hkv, n, d), 173)
    scale = 0.3
    i, j = np.arange(n)[:, None], np.arange(n)[None, :]
    vis = np.ones((n, n), dtype=bool)
    if causal:
        vis &= j <= i
    if window[0] >= 0:
        vis &= j >= i - window[0]
    if window[1] >= 0:
        vis &= j <= i + window[1]
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=torch.tensor(vis), scale=scale, enable_gqa=True)
    to.backward(torch.tensor(do))
    o, _ = attention_forward(q, k, v, scale, causal, window=window)
    np.testing.assert_allclose(o, to.detach().numpy(), atol=1e-12)
    dq, dk, dv, _ = attention_backward(q, k, v, do, scale, causal, window=window)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-11)


# ---------------------------------------------------------- block-sparse masks
def brute_force_blocks(q, k, v, scale, causal, mask, mb):
    """Pure-Python loops for one head with a block mask of mb x mb blocks; a
    row with no visible key gets O = 0 and LSE = -inf."""
    o, lse = [], []
    for i in range(len(q)):
        w = []
        for j in range(len(k)):
            vis = mask[i // mb][j // mb] != 0 and not (causal and j > i)
            w.append(math.exp(scale * sum(a * b for a, b in zip(q[i], k[j]))) if vis else 0.0)
        z = sum(w)
        lse.append(math.log(z) if z > 0 else -math.inf)
        o.append([sum(w[j] * v[j][c] for j in range(len(k))) / z if z > 0 else 0.0
                  for c in range(len(v[0]))])
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,mb", [(7, 2), (9, 3), (12, 4)])
def test_block_mask_brute_force(causal, n, mb):
    nb = -(-n // mb)
    mask = np.random.default_rng(n + mb).integers(0, 2, size=(nb, nb)).astype(np.uint8)
    mask[1, :] = 0  # a block row that sees nothing
    mask[0, 0] = 1
    q, k, v = rand((n, 3), n), rand((n, 3), n + 1), rand((n, 2), n + 2)
    o, lse = attention_forward(q, k, v, 0.7, causal, block_mask=mask, mask_block=mb)
    bo, blse = brute_force_blocks(q.tolist(), k.tolist(), v.tolist(), 0.7, causal, mask.tolist(), mb)
    np.testing.assert_allclose(o, bo, rtol=0, atol=1e-12)
    fin = np.isfinite(blse)
    assert np.array_equal(np.isfinite(lse), fin) and (~fin).any()
    np.testing.assert_allclose(lse[fin], blse[fin], rtol=0, atol=1e-12)
    assert (o[~fin] == 0).all()
    p = attention_probabilities(q, k, 0.7, causal, block_mask=mask, mask_block=mb)
    np.testing.assert_allclose(p.sum(axis=-1), fin.astype(float), rtol=0, atol=1e-12)


def test_all_ones_block_mask_equals_dense():
    q, k, v = rand((2, 3, 70, 8), 1), rand((2, 3, 70, 8), 2), rand((2, 3, 70, 8), 3)
    ones = np.ones((2, 2), dtype=np.uint8)
    for causal in (False, True):
        o0, l0 = attention_forward(q, k, v, 0.3, causal)
        o1, l1 = attention_forward(q, k, v, 0.3, causal, block_mask=ones)
        np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-13)
        np.testing.assert_allclose(l1, l0, rtol=0, atol=1e-13)


def test_block_diagonal_mask_is_attention_within_each_block():
    """Closed form: with only diagonal blocks visible, each block of rows is
    ordinary attention over its own keys."""
    n, mb = 12, 4
    q, k, v = rand((n, 5), 4), rand((n, 5), 5), rand((n, 3), 6)
    mask = np.eye(3, dtype=np.uint8)
    for causal in (False, True):
        o, lse = attention_forward(q, k, v, 0.9, causal, block_mask=mask, mask_block=mb)
        for b in range(3):
            sl = slice(mb * b, mb * b + mb)
            ob, lb = attention_forward(q[sl], k[sl], v[sl], 0.9, causal)
            np.testing.assert_allclose(o[sl], ob, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[sl], lb, rtol=0, atol=1e-12)


def test_hidden_blocks_do_not_matter():
    """Changing K and V inside blocks no row sees changes nothing."""
    n, mb = 16, 4
    q, k, v = rand((n, 4), 7), rand((n, 4), 8), rand((n, 4), 9)
    mask = np.ones((4, 4), dtype=np.uint8)
    mask[:, 2] = 0  # key block 2 hidden from every row
    k2, v2 = k.copy(), v.copy()
    k2[8:12] += 5.0
    v2[8:12] -= 3.0
    o1, l1 = attention_forward(q, k, v, 1.1, False, block_mask=mask, mask_block=mb)
    o2, l2 = attention_forward(q, k2, v2, 1.1, False, block_mask=mask, mask_block=mb)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-13)


def test_block_mask_gradients_match_finite_differences():
    n, mb = 10, 3
    q, k, v, do = rand((n, 3), 21), rand((n, 3), 22), rand((n, 2), 23), rand((n, 2), 24)
    mask = np.array([[1, 0, 1, 0], [1, 1, 0, 0], [0, 1, 1, 0], [1, 0, 0, 1]], dtype=np.uint8)
    mask[1, :] = 0  # rows 3..5 see nothing: zero gradients through them
    dq, dk, dv, _ = attention_backward(q, k, v, do, 0.8, True, block_mask=mask, mask_block=mb)
    assert (dq[3:6] == 0).all()
    h = 1e-6

    def loss(qq, kk, vv):
        o, _ = attention_forward(qq, kk, vv, 0.8, True, block_mask=mask, mask_block=mb)
        return float((o * do).sum())

    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8, err_msg=name)
