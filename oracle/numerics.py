"""Storage rounding used by the oracle (test infrastructure only).

The pages fix no number format. bf16 is IEEE binary32 with the low 16 bits
dropped; rounding to it is round-to-nearest, ties to even, done here on the
fp32 bit pattern.
"""
import numpy as np


def bf16_round(x) -> np.ndarray:
    """Round fp32 values to the nearest bf16 value (ties to even); returns fp32 values."""
    x = np.asarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    keep_lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + keep_lsb) >> 16) << 16
    out = (rounded & 0xFFFFFFFF).astype(np.uint32).view(np.float32).copy()
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.nan
    return out


def round_to(x, dtype: str) -> np.ndarray:
    """Round fp32 values to the storage dtype ("f32" or "bf16"), as fp32 values."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return x.copy()
    if dtype == "bf16":
        return bf16_round(x)
    raise ValueError(dtype)


def round_once(x, dtype: str) -> np.ndarray:
    """Round fp64 values once, to nearest with ties to even, to the storage dtype
    ("f32" or "bf16"); returns fp32 values.

    A bf16 value has 8 significant bits and fp32's exponent range, so the
    spacing of bf16 values around x is 2^(e - 8) for 2^(e-1) <= |x| < 2^e, and
    2^-133 below the smallest normal value 2^-126 (e <= -125). x is divided by
    that spacing (exact: a power of two), rounded to an integer with ties to
    even, and multiplied back; values past the largest bf16 become infinities.
    """
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        with np.errstate(over="ignore"):
            return x.astype(np.float32)
    if dtype != "bf16":
        raise ValueError(dtype)
    _, e = np.frexp(x)
    q = np.ldexp(1.0, np.maximum(e, -125) - 8)
    y = np.rint(x / q) * q
    with np.errstate(over="ignore"):
        return y.astype(np.float32)
