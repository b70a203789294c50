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
