"""Rounding helpers of the oracle (test infrastructure; see the package header).

bf16 has an 8-bit significand (7 stored bits plus the implicit one), 8
exponent bits and the float32 exponent range.  ``bf16_round`` rounds a float64
value to the nearest bf16 value, ties to even, in one step (no detour through
float32).  Pinned against torch's float32 -> bfloat16 cast on values that
float32 holds exactly, and against hand-made tie cases.
"""
import numpy as np

_BF16_MIN_SUBNORMAL_EXP = -133     # smallest bf16 subnormal is 2^-133
_BF16_MAX = float.fromhex("0x1.fep127")


def bf16_round(x) -> np.ndarray:
    """Round to bf16 (nearest, ties to even); returns float64 holding bf16 values."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                       # x = m * 2^e with 0.5 <= |m| < 1
    # keep 8 significant bits: the unit in the last place is 2^(e-8)
    ulp_exp = np.maximum(e - 8, _BF16_MIN_SUBNORMAL_EXP)
    scaled = np.ldexp(x, -ulp_exp)            # exact: power-of-two scaling
    r = np.ldexp(np.rint(scaled), ulp_exp)    # rint rounds half to even
    r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, x), r)
    return np.where(np.isfinite(x), r, x)


def from_bf16_bits(bits) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float64 exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f32_round(x) -> np.ndarray:
    """Round float64 to float32 (nearest, ties to even) and widen back."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
