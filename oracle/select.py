"""Block scoring, top-k and the block union (test infrastructure only).

Follows the SparDA summary page:
  * Eq. 1 ("Theoretical Foundation"): the attended set is the union of the
    initial blocks, the local (most recent) blocks and the top-k blocks.
  * Eq. 4 ("Methodology"): the top-k is taken over scores of a selector vector
    against the compressed keys; with the Forecast, one vector per GQA group
    scores raw dot products with no softmax ("Compact Forecast Indexer").
  * Eq. 6 (target form): the query-driven selector sums, over the G query heads
    of a group, each head's softmax over the compressed entries.

Readings where the page is silent:
  * softmax temperature is 1 (queries arrive pre-scaled by 1/sqrt(d)); each
    head's softmax runs over every complete entry j < n_c(L);
  * RAW_SUM scores an entry by the sum over the group of the raw dot products
    (with one Forecast vector per group that is its dot product);
  * a block's score is the max over the compressed entries whose whole window
    lies inside the block (for 64-token blocks, kernel 32, stride 16: entries
    4b, 4b+1, 4b+2). Parity unpinned by the pages for this membership choice:
    it is pinned only by brute force over this definition;
  * top-k competes only among blocks that are neither initial nor local, ties
    go to the lower block index, and the union is returned in ascending order.
"""
from dataclasses import dataclass

import numpy as np

from .compress import n_compressed, n_blocks, CMP_KERNEL, CMP_STRIDE, BLOCK

SOFTMAX_SUM = "softmax_sum"
RAW_SUM = "raw_sum"


@dataclass(frozen=True)
class SelectParams:
    top_k: int
    n_init: int = 1
    n_local: int = 2
    score_mode: str = SOFTMAX_SUM


def entry_scores(sel: np.ndarray, Kc: np.ndarray, mode: str) -> np.ndarray:
    """Score every compressed entry for one group.

    sel: [G, d] selector vectors of the group (G query heads, or 1 Forecast).
    Kc:  [n_c, d] compressed keys visible at this step.
    Returns S [n_c] in fp64.
    """
    sel64 = np.asarray(sel, dtype=np.float64)
    K64 = np.asarray(Kc, dtype=np.float64)
    logits = sel64 @ K64.T                                   # [G, n_c]
    if K64.shape[0] == 0:
        return np.zeros(0)
    if mode == RAW_SUM:
        return logits.sum(axis=0)
    if mode == SOFTMAX_SUM:
        m = logits.max(axis=1, keepdims=True)
        e = np.exp(logits - m)
        p = e / e.sum(axis=1, keepdims=True)
        return p.sum(axis=0)
    raise ValueError(mode)


def block_entries(b: int, n_c: int, block: int = BLOCK, l: int = CMP_KERNEL,
                  s: int = CMP_STRIDE):
    """Compressed entries whose window [j*s, j*s+l) lies wholly inside block b.

    j*s >= b*block  <=>  j >= ceil(b*block / s);  j*s + l <= (b+1)*block  <=>
    j <= floor(((b+1)*block - l) / s).
    """
    lo = -(-(b * block) // s)
    hi = ((b + 1) * block - l) // s
    return list(range(max(lo, 0), min(hi, n_c - 1) + 1))


def block_scores(S: np.ndarray, nb: int) -> np.ndarray:
    """Block score = max over its inside entries (-inf for a block with none)."""
    n_c = S.shape[0]
    out = np.full(nb, -np.inf)
    for b in range(nb):
        js = block_entries(b, n_c)
        if js:
            out[b] = S[js].max()
    return out


def candidate_sets(nb: int, n_init: int, n_local: int):
    """(initial blocks, local blocks, top-k candidates) for nb visible blocks."""
    init = list(range(0, min(n_init, nb)))
    local = list(range(max(0, nb - n_local), nb))
    taken = set(init) | set(local)
    cand = [b for b in range(nb) if b not in taken]
    return init, local, cand


def top_k_blocks(BS: np.ndarray, cand, k: int):
    """The k candidates with the largest block score; ties go to the lower index."""
    cand = np.asarray(cand, dtype=np.int64)
    if cand.size == 0 or k <= 0:
        return []
    order = np.lexsort((cand, -BS[cand]))       # primary key -score, then block index
    return cand[order[:min(k, cand.size)]].tolist()


def select_blocks(sel: np.ndarray, Kc: np.ndarray, L: int, p: SelectParams,
                  return_scores: bool = False):
    """Eq. 1 / Eq. 4: union of init, local and top-k blocks at visible length L.

    Kc may hold more entries than are visible; only j < n_c(L) are scored.
    Returns the sorted block list (and the fp64 block scores if asked).
    """
    nc = n_compressed(L)
    nb = n_blocks(L)
    S = entry_scores(sel, np.asarray(Kc)[:nc], p.score_mode)
    BS = block_scores(S, nb)
    init, local, cand = candidate_sets(nb, p.n_init, p.n_local)
    top = top_k_blocks(BS, cand, p.top_k)
    union = sorted(set(init) | set(local) | set(top))
    if return_scores:
        return union, BS
    return union
