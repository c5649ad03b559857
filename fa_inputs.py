"""Seeded synthetic inputs for IO-aware exact attention.

This module holds no attention arithmetic. It draws the tensors that both
sides of every comparison consume: the HIP path (after a copy to the device)
and the CPU oracle (after an exact upcast to float64). Nothing here imports
either side.

Recipe (the same for every workload):
  * one CPU ``torch.Generator`` seeded with ``seed`` (0 unless stated);
  * float32 standard-normal draws in the fixed order Q, K, V, then dO when a
    backward pass is needed, each of shape [B, H, N, d] (batch, heads,
    sequence, head dim -- the layout in which the tutorial page's code unpacks
    ``q.shape``); with grouped K/V heads, K and V are [B, Hkv, N, d];
  * an optional multiplication by ``input_scale`` (0.5 for the B=4 H=16
    N=4096 workload; a power of two, so it commutes exactly with rounding);
  * a round-to-nearest-even cast to the workload's dtype (torch's cast).

8-bit float inputs (``make_fp8_inputs``) start from the same float32 draws
and store each tensor as OCP E4M3 codes with one per-tensor factor.

Block masks (``make_block_mask``) are byte maps over 64-row x 64-key blocks
in a few structured families (random, banded, banded plus global blocks,
striped, with empty block rows), drawn with a numpy generator of their own.

The named workloads are the five shapes the scope names: a tiny fp32 head, a
causal bf16 head batch at N=1024, a non-causal bf16 batch at N=4096 with
inputs scaled by 0.5, a long-sequence bf16 batch at N=16384 (non-causal and
causal) and a causal fp16 forward+backward batch at N=2048.
"""

from __future__ import annotations

import dataclasses
import math

import torch

_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str  # "f32" | "f16" | "bf16"
    causal: bool
    backward: bool = False
    input_scale: float = 1.0
    seed: int = 0

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(d), rounded to float32 as the kernels receive it."""
        return float(torch.tensor(1.0 / math.sqrt(self.d), dtype=torch.float32))

    @property
    def torch_dtype(self) -> torch.dtype:
        return _DTYPES[self.dtype]

    def fwd_flops(self) -> float:
        """4*B*H*N^2*d, halved when causal (the scope's FLOP convention)."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def bwd_flops(self) -> float:
        return 2.5 * self.fwd_flops()


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 1, 128, 64, "f32", causal=False),
    "causal_bf16_n1k": Workload("causal_bf16_n1k", 2, 8, 1024, 64, "bf16", causal=True),
    "bf16_n4k_d128": Workload("bf16_n4k_d128", 4, 16, 4096, 128, "bf16", causal=False,
                              input_scale=0.5),
    "bf16_n16k_d128": Workload("bf16_n16k_d128", 1, 16, 16384, 128, "bf16", causal=False),
    "bf16_n16k_d128_causal": Workload("bf16_n16k_d128_causal", 1, 16, 16384, 128, "bf16",
                                      causal=True),
    "f16_n2k_fwdbwd_causal": Workload("f16_n2k_fwdbwd_causal", 2, 16, 2048, 64, "f16",
                                      causal=True, backward=True),
}


def make_inputs(B: int, H: int, N: int, d: int, dtype: str, *, seed: int = 0,
                input_scale: float = 1.0, backward: bool = False,
                kv_heads: int | None = None) -> dict:
    """Draw Q, K, V (and dO) on the CPU following the recipe above.

    Returns a dict of contiguous CPU tensors of the requested dtype with keys
    ``q``, ``k``, ``v`` and, when ``backward``, ``do``. ``kv_heads`` (default
    H) is the head count of K and V.
    """
    if dtype not in _DTYPES:
        raise ValueError(f"unknown dtype {dtype!r}")
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    hkv = H if kv_heads is None else kv_heads
    shapes = {"q": (B, H, N, d), "k": (B, hkv, N, d), "v": (B, hkv, N, d), "do": (B, H, N, d)}
    names = ["q", "k", "v"] + (["do"] if backward else [])
    out = {}
    for name in names:
        x = torch.randn(shapes[name], generator=g, dtype=torch.float32)
        if input_scale != 1.0:
            x = x * input_scale
        out[name] = x.to(_DTYPES[dtype]).contiguous()
    return out


E4M3_MAX = 448.0  # largest finite OCP E4M3 value


def make_fp8_inputs(B: int, H: int, N: int, d: int, *, seed: int = 0,
                    kv_heads: int | None = None) -> dict:
    """Q, K, V as OCP E4M3 codes with one dequantization factor per tensor.

    The same float32 draws as ``make_inputs`` (same generator, order and
    shapes); each tensor x is then stored as codes of x / s with
    s = max|x| / 448 (float32), so its largest magnitude maps onto E4M3's
    largest finite value: torch's round-to-nearest-even cast to
    float8_e4m3fn. Returns uint8 CPU tensors ``q8``, ``k8``, ``v8`` and the
    factors ``descale`` = (s_q, s_k, s_v) as Python floats.
    """
    x = make_inputs(B, H, N, d, "f32", seed=seed, kv_heads=kv_heads)
    out, descale = {}, []
    for name in ("q", "k", "v"):
        t = x[name]
        s = torch.tensor(float(t.abs().max()) / E4M3_MAX, dtype=torch.float32)
        codes = (t / s).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
        out[name + "8"] = codes.view(torch.uint8).contiguous()
        descale.append(float(s))
    out["descale"] = tuple(descale)
    return out


MASK_KINDS = ("random", "band", "band_global", "stripes", "empty_rows", "dense", "diagonal")


def make_block_mask(N: int, kind: str, *, seed: int = 0, density: float = 0.5,
                    block: int = 64) -> torch.Tensor:
    """A [ceil(N/block)]^2 uint8 CPU tensor; nonzero = the (query block, key
    block) pair is kept.

    ``random``: each pair kept with probability ``density``, block (0, 0)
    always. ``band``: |i - j| <= 2 blocks. ``band_global``: the band plus
    block row and column 0 plus random pairs at density / 4. ``stripes``:
    key blocks j with j % 3 == i % 3. ``empty_rows``: ``random`` with every
    third block row dropped entirely (those query rows see no key).
    ``dense``: all ones. ``diagonal``: i == j only.
    """
    import numpy as np

    nb = -(-N // block)
    rng = np.random.default_rng(seed)
    i, j = np.meshgrid(np.arange(nb), np.arange(nb), indexing="ij")
    if kind == "random":
        m = rng.random((nb, nb)) < density
        m[0, 0] = True
    elif kind == "band":
        m = np.abs(i - j) <= 2
    elif kind == "band_global":
        m = (np.abs(i - j) <= 2) | (i == 0) | (j == 0) | (rng.random((nb, nb)) < density / 4)
    elif kind == "stripes":
        m = (j % 3) == (i % 3)
    elif kind == "empty_rows":
        m = rng.random((nb, nb)) < density
        m[1::3, :] = False
    elif kind == "dense":
        m = np.ones((nb, nb), dtype=bool)
    elif kind == "diagonal":
        m = i == j
    else:
        raise ValueError(f"unknown mask kind {kind!r}")
    return torch.from_numpy(m.astype(np.uint8)).contiguous()


def workload_inputs(w: Workload) -> dict:
    return make_inputs(w.B, w.H, w.N, w.d, w.dtype, seed=w.seed,
                       input_scale=w.input_scale, backward=w.backward)


def to_f64(t: torch.Tensor):
    """Exact upcast of a (CPU or device) tensor to a float64 numpy array."""
    return t.detach().to("cpu", torch.float64).numpy()
