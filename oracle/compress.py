"""Mean-pooled compressed keys (test infrastructure only).

Follows Eq. 2 of the SparDA summary page ("Theoretical Foundation"): entry j is
the mean of keys j*s .. j*s+l-1 with kernel l = 32 and stride s = 16.

Readings where the page is silent:
  * Only complete windows exist: at visible length L there are
    n_c(L) = floor((L - l) / s) + 1 entries (none when L < l).
  * The mean is one fixed fp32 computation: the window's sum is formed as the
    sum of two fp32 partial sums of s consecutive keys each (valid because
    l = 2 s), each partial sum accumulated in ascending token order starting
    from the first key; the total is divided by l (exact: l is a power of two)
    and rounded to the key dtype with round-to-nearest-even. This makes each
    entry one exact value.
"""
import numpy as np

from .numerics import round_to

CMP_KERNEL = 32   # l_{C1} in Eq. 2
CMP_STRIDE = 16   # s_{C1} in Eq. 2
BLOCK = 64        # tokens per KV block


def n_compressed(L: int, l: int = CMP_KERNEL, s: int = CMP_STRIDE) -> int:
    """Number of complete compression windows at visible length L."""
    return 0 if L < l else (L - l) // s + 1


def n_blocks(L: int, block: int = BLOCK) -> int:
    return (L + block - 1) // block


def _partial_sums(K32: np.ndarray, starts, s: int) -> np.ndarray:
    """fp32 sums of K[a], K[a+1], ..., K[a+s-1] for each start a, in token order."""
    acc = K32[starts].copy()
    for i in range(1, s):
        acc = acc + K32[starts + i]          # elementwise fp32 add, one rounding each
    return acc


def compressed_keys(K: np.ndarray, L: int, dtype: str, first: int = 0,
                    l: int = CMP_KERNEL, s: int = CMP_STRIDE) -> np.ndarray:
    """Entries j in [first, n_c(L)) of the compressed keys of one (sequence, KV head).

    K: [T, d] key values (fp32 array holding values of the key dtype), T >= L.
    Returns [n_c(L) - first, d] fp32 values of the key dtype.
    """
    assert l == 2 * s, "the fixed summation order needs l = 2 s"
    K32 = np.asarray(K, dtype=np.float32)
    nc = n_compressed(L, l, s)
    if nc <= first:
        return np.zeros((0, K32.shape[1]), dtype=np.float32)
    j = np.arange(first, nc)
    first_half = _partial_sums(K32, j * s, s)          # keys j*s .. j*s+s-1
    second_half = _partial_sums(K32, j * s + s, s)     # keys j*s+s .. j*s+l-1
    mean = (first_half + second_half) / np.float32(l)
    return round_to(mean, dtype)


def append_compressed_keys(K: np.ndarray, Kc_old: np.ndarray, L_old: int, L_new: int,
                           dtype: str) -> np.ndarray:
    """Compressed keys at length L_new, given those at L_old: only new windows are formed."""
    new = compressed_keys(K, L_new, dtype, first=n_compressed(L_old))
    return np.concatenate([Kc_old[:n_compressed(L_old)], new], axis=0)
