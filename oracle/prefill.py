"""Chunked causal prefill with tile-shared block sets (test infrastructure only).

Attention over chosen blocks is Eq. 5 of the SparDA summary page; the
selection per query is Eq. 4 / Eq. 6 with the Eq. 1 union. Tile-level sharing
of one selection across neighbouring queries follows the Kascade abstract
(page "CoSA ...", second paper: "tile-level operations" for prefill).

Readings:
  * a chunk starts at a multiple of 64; tile t holds queries q_start+64t ..
    q_start+64t+63 (the last tile may be shorter), i.e. they all lie in one
    64-token block bt;
  * query p selects at visible length L = p + 1: each of its G heads takes a
    softmax over the entries j < n_c(p + 1), summed over the group (or raw sums);
    its top-k competes over blocks that are neither initial nor in the local
    window of n_local blocks ending at block bt;
  * the tile's set is the union of its queries' top-k sets, the initial blocks
    and that local window; every query of the tile attends to this set,
    causally (token t visible to query p when t <= p).
"""
import numpy as np

from .compress import n_compressed, n_blocks
from .select import entry_scores, block_scores, candidate_sets, top_k_blocks, SelectParams
from .attention import sparse_attention, block_tokens

TILE = 64


def prefill_tile_select(q_tile, Kc, positions, p: SelectParams, return_per_query=False):
    """Tile union for one KV head.

    q_tile: [n_q, G, d] the group's query heads for the tile's queries.
    positions: [n_q] absolute positions (all in one 64-token block).
    """
    nb = n_blocks(int(positions[-1]) + 1)
    assert all(n_blocks(int(x) + 1) == nb for x in positions)
    init, local, cand = candidate_sets(nb, p.n_init, p.n_local)
    union = set(init) | set(local)
    per_query = []
    for i, pos in enumerate(positions):
        L = int(pos) + 1
        S = entry_scores(q_tile[i], np.asarray(Kc)[:n_compressed(L)], p.score_mode)
        BS = block_scores(S, nb)
        top = top_k_blocks(BS, cand, p.top_k)
        per_query.append((top, BS))
        union |= set(top)
    union = sorted(union)
    if return_per_query:
        return union, per_query
    return union


def tile_attention(q_tile, K, V, blocks, positions, scale: float):
    """Eq. 5 for every query of one tile over the tile's block set, causally.

    q_tile: [n_q, G, d] the group's heads of the tile's queries; K, V: [T, d];
    positions: [n_q] absolute query positions. Query p attends to the tokens
    t <= p of the listed blocks: one score matrix over the set's tokens with
    the invisible ones at -inf, the same softmax and weighted sum as
    attention.sparse_attention per query. Returns (O [n_q, G, d], LSE [n_q, G]).
    """
    q64 = np.asarray(q_tile, dtype=np.float64)
    n_q, G, d = q64.shape
    toks = block_tokens(blocks, int(positions[-1]) + 1)
    if toks.size == 0:
        return np.zeros((n_q, G, d)), np.full((n_q, G), -np.inf)
    k64 = np.asarray(K, dtype=np.float64)[toks]
    v64 = np.asarray(V, dtype=np.float64)[toks]
    z = scale * (q64.reshape(n_q * G, d) @ k64.T).reshape(n_q, G, -1)
    visible = toks[None, :] <= np.asarray(positions)[:, None]          # [n_q, n]
    z = np.where(visible[:, None, :], z, -np.inf)
    m = z.max(axis=2, keepdims=True)
    e = np.exp(z - m)
    l = e.sum(axis=2, keepdims=True)
    O = (e.reshape(n_q * G, -1) @ v64).reshape(n_q, G, d) / l
    return O, m[:, :, 0] + np.log(l[:, :, 0])


def prefill_attention(Q, K, V, tile_blocks, q_start: int, scale: float, tiles=None):
    """Causal attention of each chunk query over its tile's block set.

    Q [Tq, Hq, d]; K, V [Hkv, T, d]; tile_blocks[(t, kvh)] sorted block list.
    Returns (O [Tq, Hq, d], LSE [Tq, Hq]); NaN for tiles not computed.
    """
    Tq, Hq, d = Q.shape
    Hkv = K.shape[0]
    G = Hq // Hkv
    n_tiles = (Tq + TILE - 1) // TILE
    O = np.full((Tq, Hq, d), np.nan)
    LSE = np.full((Tq, Hq), np.nan)
    todo = tiles if tiles is not None else [(t, h) for t in range(n_tiles) for h in range(Hkv)]
    for (t, h) in todo:
        blocks = tile_blocks[(t, h)]
        for i in range(t * TILE, min((t + 1) * TILE, Tq)):
            pos = q_start + i
            toks = block_tokens(blocks, pos + 1)          # causal: t <= pos
            o, lse = sparse_attention(Q[i, h * G:(h + 1) * G], K[h], V[h], toks, scale)
            O[i, h * G:(h + 1) * G] = o
            LSE[i, h * G:(h + 1) * G] = lse
    return O, LSE


def prefill_chunk(Q, K, V, Kc, q_start: int, p: SelectParams, scale: float, tiles=None):
    """Selection and attention for a chunk (one sequence).

    Kc [Hkv, NC, d] compressed keys covering the whole context.
    tiles: optional list of (tile, kvh) to compute (others are skipped).
    """
    assert q_start % TILE == 0
    Tq, Hq, d = Q.shape
    Hkv = K.shape[0]
    G = Hq // Hkv
    n_tiles = (Tq + TILE - 1) // TILE
    todo = tiles if tiles is not None else [(t, h) for t in range(n_tiles) for h in range(Hkv)]
    unions = {}
    for (t, h) in todo:
        lo, hi = t * TILE, min((t + 1) * TILE, Tq)
        qt = Q[lo:hi, h * G:(h + 1) * G]
        unions[(t, h)] = prefill_tile_select(qt, Kc[h], np.arange(q_start + lo, q_start + hi), p)
    O, LSE = prefill_attention(Q, K, V, unions, q_start, scale, tiles=todo)
    return dict(blocks=unions, O=O, LSE=LSE)
