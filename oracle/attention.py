"""Attention over selected blocks and the log-sum-exp merge (test infrastructure only).

Eq. 5 of the SparDA summary page ("Methodology"): the attention query attends
only to the keys and values of the chosen blocks. Reading: a token t of a chosen
block is visible when t < L (and t <= the query position in causal prefill);
the softmax scale is an argument (1.0 for the pre-scaled workloads). All fp64.
"""
import numpy as np

BLOCK = 64


def block_tokens(blocks, L: int, block: int = BLOCK) -> np.ndarray:
    """Token positions of the listed blocks that are < L, in block order."""
    toks = [np.arange(b * block, min((b + 1) * block, L)) for b in blocks]
    return np.concatenate(toks) if toks else np.zeros(0, dtype=np.int64)


def sparse_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, tokens: np.ndarray,
                     scale: float):
    """softmax(scale * q k_t) weighted sum of v_t over the given tokens.

    q: [H, d] query heads sharing these keys; K, V: [T, d].
    Returns (O [H, d], LSE [H]) in fp64; an empty token set gives O = 0, LSE = -inf.
    """
    q64 = np.asarray(q, dtype=np.float64)
    H, d = q64.shape
    if tokens.size == 0:
        return np.zeros((H, d)), np.full(H, -np.inf)
    k64 = np.asarray(K, dtype=np.float64)[tokens]
    v64 = np.asarray(V, dtype=np.float64)[tokens]
    z = scale * (q64 @ k64.T)                         # [H, n]
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    l = e.sum(axis=1, keepdims=True)
    O = (e @ v64) / l
    LSE = m[:, 0] + np.log(l[:, 0])
    return O, LSE


def split_attention_partials(q, K, V, token_parts, scale):
    """Unnormalised partials (m, l, acc) of attention over each token subset."""
    parts = []
    q64 = np.asarray(q, dtype=np.float64)
    for toks in token_parts:
        if len(toks) == 0:
            parts.append((np.full(q64.shape[0], -np.inf), np.zeros(q64.shape[0]),
                          np.zeros_like(q64)))
            continue
        z = scale * (q64 @ np.asarray(K, dtype=np.float64)[toks].T)
        m = z.max(axis=1)
        e = np.exp(z - m[:, None])
        parts.append((m, e.sum(axis=1), e @ np.asarray(V, dtype=np.float64)[toks]))
    return parts


def lse_merge(parts):
    """Merge partials (m_s, l_s, acc_s) into (O, LSE) by rescaling to the global max."""
    ms = np.stack([p[0] for p in parts])              # [S, H]
    M = ms.max(axis=0)
    Msafe = np.where(np.isfinite(M), M, 0.0)
    w = np.where(np.isfinite(ms), np.exp(ms - Msafe), 0.0)
    l = sum(w[i] * parts[i][1] for i in range(len(parts)))
    acc = sum(w[i][:, None] * parts[i][2] for i in range(len(parts)))
    with np.errstate(divide="ignore", invalid="ignore"):
        O = np.where(l[:, None] > 0, acc / np.where(l > 0, l, 1.0)[:, None], 0.0)
        LSE = np.where(l > 0, M + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return O, LSE
