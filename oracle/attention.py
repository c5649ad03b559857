"""CPU oracle for exact scaled-dot-product attention -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this module. The product path (the HIP library and its binding) never
calls it, shares no code with it, and fails loudly when its own extension is
missing instead of falling back here.

Everything is computed in float64 with numpy from whatever inputs are passed
(the callers hand in exactly the bf16/fp16/fp32-rounded values the GPU
receives, upcast without loss).

Sources (the pages this restates in code; cited by key below):
  [FA-mem]       "FlashAttention：优化大模型训练的内存与计算效率"
                 (cnnetsun.cn/a/3461300) -- tutorial on the memory hierarchy,
                 safe softmax, causal masking and debugging.
  [FA-principle] "FlashAttention原理：从原始Attention到FlashAttention"
                 (blog.csdn.net/qq_43527718/article/details/142302113) --
                 standard attention, tiling, blockwise softmax, FA2 changes,
                 and an embedded answer "写一个flashattention算子" whose numbered
                 steps give the online-softmax update formulas.

Readings taken where the pages are silent:
  * scale: the scores are multiplied by ``scale`` (1/sqrt(d) in every
    workload, as in the answer's step 3, which divides by sqrt(d)); the
    softmax runs over the scaled scores.
  * causal: key j is hidden from query i when j > i (square self-attention;
    the pages only name an ``is_causal`` switch). Hidden scores are excluded
    exactly (probability 0), not replaced by a large finite number.
  * what is stored for the backward pass: one float per query row,
    LSE_i = m_i + ln(l_i) -- natural log of the sum of exponentials of the
    scaled scores (the pages say "the softmax normalization factor").
  * the backward formulas are not on the pages; they are the derivatives of
    the definition (chain rule through softmax), written out below.
  * in the blockwise recurrence, a row that sees no key inside one block
    contributes nothing from that block (its block max is -inf, its block sum 0).
  * local window (a sliding-window generalization of the causal block
    skipping; the pages only show the causal special case): key j is
    visible to query i when i - left <= j <= i + right, a negative bound
    meaning unbounded on that side; combined with the causal rule when both
    are given. Causal is the window (unbounded, 0).
  * block-sparse attention (named with the window extension among the
    method's sparse variants): a mask of blocks of mask_block query rows x
    mask_block keys, shared by all batches and heads; a hidden block's
    scores are excluded exactly. A row that then sees no key has O = 0 and
    LSE = -inf (the softmax over an empty set has no value; these are its
    limits as a single zero-valued key's score goes to -inf).
  * grouped K/V heads (multi-query / grouped-query attention, named next to
    the method on the pages' overview of later work): with Hq query heads
    and Hkv K/V heads (Hkv divides Hq), query head h attends with K/V head
    h // (Hq / Hkv). The gradient of a K/V head is the sum over the query
    heads that use it.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "attention_forward",
    "attention_probabilities",
    "attention_backward",
    "attention_forward_blockwise",
    "merge_partials",
]

# Rows of S processed at once; bounds the float64 score chunk to
# ROW_CHUNK * N * 8 bytes (16384 keys -> 256 MiB at 2048 rows).
ROW_CHUNK = 2048


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _visible(q_pos: np.ndarray, n_keys: int, causal: bool, window=None,
             block_mask=None, mask_block: int = 64) -> np.ndarray | None:
    """Boolean [rows, n_keys] mask of keys each query may attend to (None = all).

    Causal reading: query at absolute position i sees keys 0..i.
    Window (left, right): query i sees keys i-left .. i+right (negative = unbounded).
    Block mask M (block-sparse attention): query i sees key j only if
    M[i // mask_block, j // mask_block] is nonzero.
    """
    vis = None
    if block_mask is not None:
        bm = np.asarray(block_mask) != 0
        vis = bm[q_pos[:, None] // mask_block, np.arange(n_keys)[None, :] // mask_block]
    if causal:
        c = np.arange(n_keys)[None, :] <= q_pos[:, None]
        vis = c if vis is None else vis & c
    if window is not None:
        left, right = window
        keys = np.arange(n_keys)[None, :]
        if left >= 0:
            lo = keys >= q_pos[:, None] - left
            vis = lo if vis is None else vis & lo
        if right >= 0:
            hi = keys <= q_pos[:, None] + right
            vis = hi if vis is None else vis & hi
    return vis


def _expand_kv(q, k, v):
    """K/V heads repeated so that query head h uses K/V head h // (Hq / Hkv)."""
    if k.ndim < 3 or k.shape[-3] == q.shape[-3]:
        return k, v
    hq, hkv = q.shape[-3], k.shape[-3]
    if hkv < 1 or hq % hkv:
        raise ValueError("the number of K/V heads must divide the number of query heads")
    group = hq // hkv
    return np.repeat(k, group, axis=-3), np.repeat(v, group, axis=-3)


def _reduce_kv_grad(g, hkv):
    """Sum a per-query-head K/V gradient over the query heads of each group."""
    if g.shape[-3] == hkv:
        return g
    group = g.shape[-3] // hkv
    return g.reshape(g.shape[:-3] + (hkv, group) + g.shape[-2:]).sum(axis=-3)


def _scores(qc: np.ndarray, k: np.ndarray, scale: float, vis) -> np.ndarray:
    """S = scale * Q K^T for one chunk of query rows, hidden keys set to -inf.

    [FA-principle §二.2]: the standard pipeline forms S from Q and K^T; the
    answer's step 3 divides the product by sqrt(d) (our ``scale``).
    """
    s = scale * (qc @ k.T)
    if vis is not None:
        s = np.where(vis, s, -np.inf)
    return s


def _softmax_rows(s: np.ndarray):
    """(P, LSE) of the rows of S (hidden entries -inf). A row with no visible
    entry has P = 0 and LSE = -inf (the reading for an empty softmax)."""
    m = s.max(axis=1, keepdims=True)                     # pass 1
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)                     # pass 2
    p = np.where(l > 0, e / np.where(l > 0, l, 1.0), 0.0)  # pass 3
    lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return p, lse[:, 0]


def _head_forward(q, k, v, scale, causal, q_pos, window=None, block_mask=None, mask_block=64):
    """Three-pass safe softmax attention for one head.

    Pass 1: row max m of the scaled scores.     [FA-mem §2.2 safe softmax]
    Pass 2: row sum l of exp(S - m).
    Pass 3: P = exp(S - m) / l, O = P V, LSE = m + ln l.
    This is the plain (unfused) definition of [FA-principle §二.2]: the
    scores and probabilities are formed in full for a chunk of rows.
    """
    n_rows = q.shape[0]
    o = np.empty((n_rows, v.shape[1]), dtype=np.float64)
    lse = np.empty(n_rows, dtype=np.float64)
    for r0 in range(0, n_rows, ROW_CHUNK):
        r1 = min(r0 + ROW_CHUNK, n_rows)
        vis = _visible(q_pos[r0:r1], k.shape[0], causal, window, block_mask, mask_block)
        s = _scores(q[r0:r1], k, scale, vis)
        if block_mask is None:
            m = s.max(axis=1, keepdims=True)             # pass 1
            e = np.exp(s - m)
            l = e.sum(axis=1, keepdims=True)             # pass 2
            p = e / l                                    # pass 3
            lse[r0:r1] = (m + np.log(l))[:, 0]
        else:  # rows may see no key at all
            p, lse[r0:r1] = _softmax_rows(s)
        o[r0:r1] = p @ v
    return o, lse


def _batched(fn, arrays, n_out):
    """Apply a per-head function over all leading (batch, head) dims."""
    lead = arrays[0].shape[:-2]
    flat = [a.reshape((-1,) + a.shape[-2:]) for a in arrays]
    outs = [[] for _ in range(n_out)]
    for i in range(flat[0].shape[0]):
        res = fn(*[a[i] for a in flat])
        for j in range(n_out):
            outs[j].append(res[j])
    return [np.stack(o).reshape(lead + o[0].shape) for o in outs]


def attention_forward(q, k, v, scale: float, causal: bool, q_positions=None, window=None,
                      block_mask=None, mask_block: int = 64):
    """O = softmax(scale * Q K^T [masked]) V and the per-row LSE.

    Shapes: q [..., Hq, Nq, d], k [..., Hkv, Nk, d], v [..., Hkv, Nk, dv]
    (leading dims are batch and heads; Hkv divides Hq, see _expand_kv; plain
    multi-head attention has Hkv = Hq). ``q_positions`` gives the absolute
    position of each query row for the causal and window masks (default
    0..Nq-1), which lets a caller evaluate a sampled subset of rows of a long
    sequence exactly. ``window`` = (left, right) or None. ``block_mask``
    (block-sparse attention): a [ceil(N/mask_block)]^2 array shared by all
    batches and heads; query i sees key j only where
    block_mask[i // mask_block, j // mask_block] is nonzero. With a block
    mask a row may see no key: its O is 0 and its LSE -inf.

    Returns (O [..., Hq, Nq, dv], LSE [..., Hq, Nq]), float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    k, v = _expand_kv(q, k, v)
    pos = np.arange(q.shape[-2]) if q_positions is None else np.asarray(q_positions)
    if pos.shape != (q.shape[-2],):
        raise ValueError("q_positions must have one entry per query row")
    return tuple(_batched(lambda a, b, c: _head_forward(a, b, c, scale, causal, pos, window,
                                                        block_mask, mask_block),
                          [q, k, v], 2))


def attention_probabilities(q, k, scale: float, causal: bool, window=None, q_positions=None,
                            block_mask=None, mask_block: int = 64):
    """P = softmax(scale * Q K^T) materialized ([..., rows, N]; tests only).
    With ``q_positions``, q holds only those rows (their sequence positions)."""
    q, k = _f64(q), _f64(k)
    k, _ = _expand_kv(q, k, k)
    pos = np.arange(q.shape[-2]) if q_positions is None else np.asarray(q_positions)

    def one(a, b):
        s = _scores(a, b, scale, _visible(pos, b.shape[0], causal, window, block_mask, mask_block))
        return (_softmax_rows(s)[0],)

    return _batched(one, [q, k], 1)[0]


def _head_backward(q, k, v, do, scale, causal, window=None, block_mask=None, mask_block=64):
    """Gradients of sum(dO * O) for one head, from the definition.

    Not on the pages (the answer's step 6 only says the scores are recomputed
    instead of stored). With P the softmax of the scaled scores:
      dV = P^T dO
      dP = dO V^T
      D_i = sum_j P_ij dP_ij               (softmax Jacobian-vector term)
      dS = P * (dP - D)                    (gradient w.r.t. the scaled scores)
      dQ = scale * dS K,   dK = scale * dS^T Q
    P is recomputed here from Q and K (three-pass) rather than read back.
    """
    n = q.shape[0]
    pos = np.arange(n)
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dsum = np.empty(n)
    for r0 in range(0, n, ROW_CHUNK):
        r1 = min(r0 + ROW_CHUNK, n)
        s = _scores(q[r0:r1], k, scale,
                    _visible(pos[r0:r1], k.shape[0], causal, window, block_mask, mask_block))
        if block_mask is None:
            e = np.exp(s - s.max(axis=1, keepdims=True))
            p = e / e.sum(axis=1, keepdims=True)
        else:  # rows may see no key at all (P = 0 there)
            p = _softmax_rows(s)[0]
        dv += p.T @ do[r0:r1]
        dp = do[r0:r1] @ v.T
        d_i = (p * dp).sum(axis=1, keepdims=True)
        ds = p * (dp - d_i)
        dq[r0:r1] = scale * (ds @ k)
        dk += scale * (ds.T @ q[r0:r1])
        dsum[r0:r1] = d_i[:, 0]
    return dq, dk, dv, dsum


def attention_backward(q, k, v, do, scale: float, causal: bool, window=None, block_mask=None,
                       mask_block: int = 64):
    """(dQ, dK, dV, D) for the loss sum(dO * O), all float64.

    D is the per-row term sum_j P_ij dP_ij (returned so tests can check that it
    equals rowsum(dO * O)). With grouped K/V heads, dK and dV have the K/V
    head count: each is the sum over the query heads that use that K/V head.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    hkv = k.shape[-3] if k.ndim >= 3 else None
    k, v = _expand_kv(q, k, v)
    dq, dk, dv, dsum = _batched(
        lambda a, b, c, g: _head_backward(a, b, c, g, scale, causal, window, block_mask,
                                          mask_block), [q, k, v, do], 4)
    if hkv is not None:
        dk, dv = _reduce_kv_grad(dk, hkv), _reduce_kv_grad(dv, hkv)
    return dq, dk, dv, dsum


def _head_blockwise(q, k, v, scale, causal, block_q, block_k):
    """Tiled one-pass attention for one head: each query tile's result is
    built up one key tile at a time, never holding more than one tile of
    scores.

    Loop order: query tiles outer, key tiles inner, and tiles that lie wholly
    above the causal diagonal are never visited ([FA-principle] §二.7, the
    FA2 changes). How a key tile is folded in ([FA-principle] §二.5-§二.6,
    tiling with a blockwise softmax; the answer "写一个flashattention算子",
    steps 4-5): the state of a query tile is a pair (acc_o, acc_lse), the
    attention output normalized over the keys folded in so far and the
    log-normalizer of those keys. A key tile yields its own pair
    (tile_o, tile_lse), the softmax restricted to its keys. Two pairs over
    disjoint key sets combine into the pair over their union: the new
    log-normalizer is the log-sum-exp of the two, and each output is weighted
    by exp(own log-normalizer - new one) -- the rescaling by the change of
    the running maximum and sum, carried as logarithms. A row that sees no
    key of a tile has tile_lse = -inf and weight 0 there.
    """
    n, nk, dv = q.shape[0], k.shape[0], v.shape[1]
    o = np.zeros((n, dv))
    lse = np.empty(n)
    for i0 in range(0, n, block_q):
        rows = np.arange(i0, min(i0 + block_q, n))
        acc_o = np.zeros((rows.size, dv))
        acc_lse = np.full(rows.size, -np.inf)
        for j0 in range(0, nk, block_k):
            keys = np.arange(j0, min(j0 + block_k, nk))
            if causal and keys[0] > rows[-1]:
                continue                      # tile wholly above the diagonal
            s = scale * (q[rows] @ k[keys].T)
            if causal:
                s = np.where(keys[None, :] <= rows[:, None], s, -np.inf)
            top = s.max(axis=1)
            sees = np.isfinite(top)           # rows with a visible key in this tile
            shift = np.where(sees, top, 0.0)
            w = np.exp(s - shift[:, None])    # hidden keys: exp(-inf) = 0
            tot = np.where(sees, w.sum(axis=1), 1.0)
            tile_o = (w @ v[keys]) / tot[:, None]
            tile_lse = np.where(sees, shift + np.log(tot), -np.inf)
            new_lse = np.logaddexp(acc_lse, tile_lse)
            live = np.isfinite(new_lse)
            ref = np.where(live, new_lse, 0.0)
            keep_acc = np.where(np.isfinite(acc_lse), np.exp(acc_lse - ref), 0.0)
            keep_tile = np.where(sees, np.exp(tile_lse - ref), 0.0)
            acc_o = keep_acc[:, None] * acc_o + keep_tile[:, None] * tile_o
            acc_lse = new_lse
        o[rows] = acc_o
        lse[rows] = acc_lse
    return o, lse


def attention_forward_blockwise(q, k, v, scale: float, causal: bool,
                                block_q: int = 64, block_k: int = 64):
    """Blockwise (tiled, online-softmax) attention; equals attention_forward."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    return tuple(_batched(lambda a, b, c: _head_blockwise(a, b, c, scale, causal,
                                                          block_q, block_k),
                          [q, k, v], 2))


def merge_partials(o_a, lse_a, o_b, lse_b):
    """Combine attention computed over two disjoint key sets.

    Each part is normalized over its own keys and carries its LSE; the total
    normalizer is the log-sum of both, and each part is reweighted by
    exp(LSE_part - LSE_total): the same fold of two disjoint key sets that
    _head_blockwise applies tile by tile, here to two finished results.
    """
    o_a, lse_a, o_b, lse_b = _f64(o_a), _f64(lse_a), _f64(o_b), _f64(lse_b)
    lse = np.logaddexp(lse_a, lse_b)
    w_a = np.exp(lse_a - lse)[..., None]
    w_b = np.exp(lse_b - lse)[..., None]
    return w_a * o_a + w_b * o_b, lse
