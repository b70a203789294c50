"""One decode step, per (sequence, KV head) unit (test infrastructure only).

Chains the SparDA summary page's steps for a single new token: Eq. 2
compressed keys (given), Eq. 4 / Eq. 6 scoring and top-k, Eq. 1 union, Eq. 5
attention with the real query. Reading: the decode query sits at position L-1
(its own key and value are already in the cache) and the G query heads of a KV
head (heads kvh*G .. kvh*G+G-1) all use that KV head's block set.
"""
import numpy as np

from .select import select_blocks, SelectParams
from .attention import sparse_attention, block_tokens


def decode_unit(q_group, sel_group, K, V, Kc, L, p: SelectParams, scale: float):
    """Returns (blocks, O [G, d], LSE [G], block scores) for one unit."""
    blocks, BS = select_blocks(sel_group, Kc, L, p, return_scores=True)
    O, LSE = sparse_attention(q_group, K, V, block_tokens(blocks, L), scale)
    return blocks, O, LSE, BS


def decode_step(Q, sel, K, V, Kc, seq_lens, p: SelectParams, scale: float, units=None,
                blocks_override=None):
    """Decode step over all (or the listed) units.

    Q [B, Hq, d]; sel [B, H_sel, d] with H_sel = Hq (query selector) or Hkv
    (one Forecast per group); K, V [B, Hkv, T, d]; Kc [B, Hkv, NC, d].
    blocks_override[(b, kvh)] replaces the selection (attention on a given set).
    Returns dict: blocks {(b,kvh): list}, scores {(b,kvh): BS}, O and LSE arrays
    (NaN where a unit was not computed).
    """
    B, Hq, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    Gs = sel.shape[1] // Hkv
    if units is None:
        units = [(b, h) for b in range(B) for h in range(Hkv)]
    O = np.full((B, Hq, d), np.nan)
    LSE = np.full((B, Hq), np.nan)
    blocks, scores = {}, {}
    for (b, h) in units:
        L = int(seq_lens[b])
        qg = Q[b, h * G:(h + 1) * G]
        sg = sel[b, h * Gs:(h + 1) * Gs]
        if blocks_override is not None:
            blk = blocks_override[(b, h)]
            o, lse = sparse_attention(qg, K[b, h], V[b, h], block_tokens(blk, L), scale)
            bs = None
        else:
            blk, o, lse, bs = decode_unit(qg, sg, K[b, h], V[b, h], Kc[b, h], L, p, scale)
        blocks[(b, h)] = blk
        scores[(b, h)] = bs
        O[b, h * G:(h + 1) * G] = o
        LSE[b, h * G:(h + 1) * G] = lse
    return dict(blocks=blocks, scores=scores, O=O, LSE=LSE)
