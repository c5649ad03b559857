"""OCP FP8 E4M3 decoding for the 8-bit forward -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this module; the product path never calls it.

The 8-bit forward takes Q, K and V as E4M3 codes with one dequantization
factor per tensor. What it computes is the attention of the values those
codes stand for, so its oracle decodes the codes here, multiplies by the
factors in float64, and hands the values to ``attention_forward``.

The pages only name FP8 among the data types the method should support next
(section "应用展望" of "FlashAttention与新一代硬件架构融合：解锁大模型训练新高度");
the code
format is the OCP 8-bit floating point specification's E4M3 (the variant
without infinities):
  bit 7 sign; bits 6..3 biased exponent E (bias 7); bits 2..0 mantissa M.
  E = 0      : subnormal, M * 2^-9 (M = 0 gives +-0);
  E = 1..15  : (1 + M/8) * 2^(E - 7), except E = 15, M = 7, which is NaN.
  Largest finite magnitude 448 (E = 15, M = 6); no infinities.
"""

from __future__ import annotations

import numpy as np

from .attention import attention_forward

__all__ = ["e4m3_decode", "attention_forward_e4m3"]


def e4m3_decode(codes) -> np.ndarray:
    """float64 values of E4M3 codes (any integer array of bytes)."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = c >> 7
    e = (c >> 3) & 0xF
    m = c & 0x7
    subnormal = m * 2.0 ** -9
    normal = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    mag = np.where(e == 0, subnormal, normal)
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


def attention_forward_e4m3(q8, k8, v8, descale, scale: float, causal: bool, window=None,
                           q_positions=None):
    """(O, LSE) of attention over Q = s_q * dec(q8), K = s_k * dec(k8),
    V = s_v * dec(v8), with ``descale`` = (s_q, s_k, s_v)."""
    sq, sk, sv = (float(x) for x in descale)
    q = e4m3_decode(q8) * sq
    if q_positions is not None:
        q = q[..., q_positions, :]
    k = e4m3_decode(k8) * sk
    v = e4m3_decode(v8) * sv
    return attention_forward(q, k, v, scale, causal, q_positions=q_positions, window=window)
