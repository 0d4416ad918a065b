"""Symmetric group-wise int4 quantiser of the exit layers (test infrastructure).

Follows the River-LLM explainer, section 4.2 (exit layers hold 4-bit W4A16
copies of every layer) and section 8.1 (``scale = max|w| / 7``, codes are
``round(w / scale)`` clamped to [-8, 7], dequantised as ``code * scale``).
The page quantises a whole tensor with one scale; the workloads here use one
scale per group of G consecutive inputs of each output row (G = 32 or 128), the
reading that keeps the page's formula and applies it per group.

Per row n and group g (columns [gG, (g+1)G)):
    s = bf16(max|W[n, g]| / 7)        (the scale is stored as bf16)
    q = 0                               if s == 0
    q = clamp(rint(W / s), -8, 7)       otherwise, rint = round half to even
    W_hat = q * s                       (exact in float32: |q| <= 8 and s has 8 bits)

The quotient ``W / s`` is formed in float64.  Rounding it to an integer gives
the same code as rounding the real quotient: both operands are bf16, so a
quotient that is not itself a half-integer lies at least 2^-12 (relative) away
from one, far beyond float64 or float32 error.  The scale quotient max/7 has a
period-3 binary expansion, so no intermediate float32 or float64 rounding of
it can land on a bf16 midpoint: bf16(fp32(max/7)) == bf16(max/7).

Pinned by closed-form properties (codes in [-7, 7], |W - W_hat| <= s/2,
W_hat == q*s exactly, the group maximum maps to +-7, zero groups give zero) and
by brute force over all 16 codes for every element.
"""
import numpy as np

from .numerics import bf16_round


def quantize_int4(w: np.ndarray, group: int):
    """Quantise ``w`` [N, K] (bf16 values in float64) group-wise along K.

    Returns ``(q, s)``: int8 codes [N, K] and float64 scales [N, K // group]
    holding bf16 values.
    """
    w = np.asarray(w, dtype=np.float64)
    N, K = w.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    wg = w.reshape(N, K // group, group)
    amax = np.abs(wg).max(axis=2)
    s = bf16_round(amax / 7.0)
    safe = np.where(s == 0.0, 1.0, s)
    q = np.rint(wg / safe[:, :, None])
    q = np.clip(q, -8, 7)
    q = np.where(s[:, :, None] == 0.0, 0.0, q)
    return q.astype(np.int8).reshape(N, K), s


def dequantize_int4(q: np.ndarray, s: np.ndarray, group: int) -> np.ndarray:
    """W_hat = q * s per group, float64 [N, K]."""
    N, K = q.shape
    qg = q.astype(np.float64).reshape(N, K // group, group)
    return (qg * s[:, :, None]).reshape(N, K)
