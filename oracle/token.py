"""Token-level selection with one index shared by several layers (test infrastructure only).

Follows two passages of the pages:
  * the CLSA abstract on the page "HySparse2: Hybrid Sparse Attention with
    Two-Level KV Sharing": one indexer computes a top-k over individual tokens
    once, and every layer that shares the KV cache reuses that index;
  * the JSSA item on the "Sparse Attention" topic page: candidate tokens are
    scored in a shared low-dimensional query-key space, and each KV head keeps
    its own selected token set.

Readings where the pages are silent (each one stated where it is used):
  * a token's score is the raw score of Eq. 4 on the SparDA summary page
    ("Methodology"; one vector per group, no softmax, as in its "Compact
    Forecast Indexer") taken against that token's index key instead of a
    compressed entry: s_t = sum over the group's selector vectors of sel . Ki_t.
    Ki is the index-key cache, either the keys themselves (index dimension =
    head dimension) or a lower-dimensional projection of them (the JSSA
    subspace); the projections are model weights and not part of this path;
  * the first n_init and the last n_local visible tokens are always kept (the
    token counterpart of Eq. 1's initial and local sets); the top_k among the
    other visible tokens are chosen by score, ties to the lower token index;
  * attention over the selected tokens is Eq. 5 with that token set
    (oracle.attention.sparse_attention), and with a shared index every layer
    attends, with its own query, keys and values, over the anchor's tokens.
All arithmetic fp64.
"""
import numpy as np

from .attention import sparse_attention


def token_candidates(L: int, n_init: int, n_local: int):
    """(kept initial tokens, kept local tokens, top-k candidates) at visible length L."""
    init_hi = max(0, min(n_init, L))
    local_lo = max(init_hi, L - max(0, n_local))
    init = list(range(0, init_hi))
    local = list(range(local_lo, L))
    cand = list(range(init_hi, local_lo))
    return init, local, cand


def token_scores(sel: np.ndarray, Ki: np.ndarray, L: int) -> np.ndarray:
    """Raw scores of the visible tokens for one group.

    sel: [G, d_i] selector vectors of the group (the G query heads' index
    queries, or one Forecast); Ki: [>= L, d_i] index keys. Returns s [L] fp64:
    s_t = sum_g sel_g . Ki_t.
    """
    s64 = np.asarray(sel, dtype=np.float64)
    k64 = np.asarray(Ki, dtype=np.float64)[:L]
    if L == 0:
        return np.zeros(0)
    return (s64 @ k64.T).sum(axis=0)


def top_k_tokens(s: np.ndarray, cand, k: int):
    """The k candidates with the largest score; ties go to the lower token index."""
    cand = np.asarray(cand, dtype=np.int64)
    if cand.size == 0 or k <= 0:
        return []
    order = np.lexsort((cand, -s[cand]))          # primary key -score, then token index
    return cand[order[:min(k, cand.size)]].tolist()


def select_tokens(sel: np.ndarray, Ki: np.ndarray, L: int, top_k: int, n_init: int,
                  n_local: int, return_scores: bool = False):
    """Kept initial and local tokens united with the top_k scored candidates,
    ascending (and the scores if asked)."""
    s = token_scores(sel, Ki, L)
    init, local, cand = token_candidates(L, n_init, n_local)
    toks = sorted(set(init) | set(local) | set(top_k_tokens(s, cand, top_k)))
    return (toks, s) if return_scores else toks


def token_decode_unit(q_group: np.ndarray, K: np.ndarray, V: np.ndarray, tokens, scale: float):
    """Attention of one KV head's query heads over the selected tokens (Eq. 5)."""
    return sparse_attention(q_group, K, V, np.asarray(tokens, dtype=np.int64), scale)


def token_crosslayer_step(layers, sel, Ki, seq_lens, top_k: int, n_init: int, n_local: int,
                          scale: float, units=None):
    """One decode step in which the anchor's token index serves every layer.

    layers: list of dicts with Q [B, Hq, d], K, V [B, Hkv, T, d]; sel [B, H_sel, d_i]
    the anchor's selector (H_sel = Hkv: one Forecast per group; H_sel = Hq:
    the group's query heads, summed); Ki [B, Hkv, T, d_i] the anchor's index keys.
    Returns ({(b, kvh): tokens}, [O per layer], [LSE per layer]) with O
    [B, Hq, d] and LSE [B, Hq] (zeros / -inf outside the listed units).
    """
    B, Hkv = Ki.shape[:2]
    Hq = layers[0]["Q"].shape[1]
    G, Gs = Hq // Hkv, sel.shape[1] // Hkv
    units = units if units is not None else [(b, h) for b in range(B) for h in range(Hkv)]
    tokens = {}
    for (b, h) in units:
        tokens[(b, h)] = select_tokens(sel[b, h * Gs:(h + 1) * Gs], Ki[b, h], int(seq_lens[b]),
                                       top_k, n_init, n_local)
    outs, lses = [], []
    for lay in layers:
        d = lay["Q"].shape[2]
        O = np.zeros((B, Hq, d))
        LSE = np.full((B, Hq), -np.inf)
        for (b, h), toks in tokens.items():
            o, l = token_decode_unit(lay["Q"][b, h * G:(h + 1) * G], lay["K"][b, h],
                                     lay["V"][b, h], toks, scale)
            O[b, h * G:(h + 1) * G] = o
            LSE[b, h * G:(h + 1) * G] = l
        outs.append(O)
        lses.append(LSE)
    return tokens, outs, lses
