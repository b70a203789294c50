"""Pins of the token-level oracle (oracle.token) against a hand-worked example,
brute force, the block-level oracle, closed forms and dense attention."""
import itertools
import json
import pathlib

import numpy as np
import pytest
import torch

import oracle
from oracle import SelectParams

GOLDEN = pathlib.Path(__file__).parent / "golden"


def test_worked_example_token_topk():
    g = json.loads((GOLDEN / "token_topk_worked.json").read_text())
    c = np.array(g["c"], dtype=np.float64)
    L = c.size
    Ki = c[:, None]
    for k, want in g["union_plus"].items():
        assert oracle.select_tokens(np.ones((1, 1)), Ki, L, int(k), g["n_init"], g["n_local"]) == want
    assert oracle.select_tokens(-np.ones((1, 1)), Ki, L, 2, g["n_init"], g["n_local"]) == \
        g["union_minus_k2"]
    two = np.array([[1.0], [2.0]])                        # raw sum over a group of two selectors
    assert oracle.select_tokens(two, Ki, L, 3, g["n_init"], g["n_local"]) == g["union_plus"]["3"]


def _dominates(chosen, s, cand):
    """Every chosen candidate outranks every unchosen one (score, then lower index)."""
    rest = [u for u in cand if u not in chosen]
    return all(s[t] > s[u] or (s[t] == s[u] and t < u) for t in chosen for u in rest)


@pytest.mark.parametrize("seed", range(6))
def test_top_k_tokens_brute_force(seed):
    rng = np.random.default_rng(seed)
    L = 11
    s = rng.integers(0, 4, L).astype(np.float64)          # many exact ties
    for n_init, n_local in ((0, 0), (1, 2), (3, 1)):
        _, _, cand = oracle.token_candidates(L, n_init, n_local)
        for k in range(0, len(cand) + 2):
            got = oracle.top_k_tokens(s, cand, k)
            kk = min(k, len(cand))
            winners = [set(c) for c in itertools.combinations(cand, kk) if _dominates(set(c), s, cand)]
            assert len(winners) == 1 and set(got) == winners[0], (seed, n_init, n_local, k)
            assert len(got) == kk


def test_candidate_windows_and_union_sizes():
    rng = np.random.default_rng(3)
    for L in range(0, 40):
        for n_init, n_local in ((0, 0), (2, 3), (5, 0), (0, 7), (64, 128)):
            init, local, cand = oracle.token_candidates(L, n_init, n_local)
            assert init + cand + local == list(range(L))     # a partition of the visible tokens
            assert len(init) == min(n_init, L)
            assert len(local) == min(n_local, L - len(init))
            Ki = rng.standard_normal((max(L, 1), 4))
            sel = rng.standard_normal((1, 4))
            for k in (0, 1, 5, 100):
                toks = oracle.select_tokens(sel, Ki, L, k, n_init, n_local)
                assert toks == sorted(set(toks)) and all(0 <= t < L for t in toks)
                assert len(toks) == min(L, len(init) + len(local) + k)


def test_token_scores_closed_form_one_hot_keys():
    """Ki_t = c_t e_(t mod 8) and selector w: s_t = w[t mod 8] c_t."""
    rng = np.random.default_rng(4)
    L, d = 50, 8
    c = rng.standard_normal(L)
    Ki = np.zeros((L, d))
    Ki[np.arange(L), np.arange(L) % d] = c
    w = rng.standard_normal(d)
    s = oracle.token_scores(w[None], Ki, L)
    assert np.allclose(s, w[np.arange(L) % d] * c, rtol=0, atol=1e-15)
    # a group of selectors scores with the sum of their dot products
    w2 = rng.standard_normal(d)
    s2 = oracle.token_scores(np.stack([w, w2]), Ki, L)
    assert np.allclose(s2, (w + w2)[np.arange(L) % d] * c, rtol=0, atol=1e-14)
    # only the first L index keys are read
    Ki_long = np.concatenate([Ki, np.full((5, d), np.nan)])
    assert np.array_equal(oracle.token_scores(w[None], Ki_long, L), s)


@pytest.mark.parametrize("seed", range(3))
def test_block_constant_keys_reduce_to_the_block_selection(seed):
    """When every key of a 64-token block is the same vector, each block's
    score (Eq. 4 raw form over its inside compressed entries) equals each of
    its tokens' scores, so a token top-k of 64 * k tokens with 64 * n_init
    initial and 64 * n_local local tokens takes exactly the tokens of the
    block top-k (ties between blocks also go to the lower index)."""
    rng = np.random.default_rng(seed)
    nb, d = 30, 16
    L = 64 * nb
    w = rng.integers(-3, 4, (nb, d)).astype(np.float32)   # small integers: exact means, some ties
    K = np.repeat(w, 64, axis=0)
    sel = rng.integers(-2, 3, (1, d)).astype(np.float32)
    Kc = oracle.compressed_keys(K, L, "f32")
    for k in (1, 4, 9, 27, 40):
        p = SelectParams(top_k=k, n_init=1, n_local=2, score_mode=oracle.RAW_SUM)
        blocks = oracle.select_blocks(sel, Kc, L, p)
        toks = oracle.select_tokens(sel, K, L, 64 * k, 64, 128)
        want = oracle.attention.block_tokens(blocks, L).tolist()
        assert toks == want, (seed, k)


@pytest.mark.parametrize("L", [1, 37, 200])
def test_all_tokens_selected_is_dense_attention(L):
    rng = np.random.default_rng(L)
    d, G = 32, 4
    q = rng.standard_normal((G, d)) / np.sqrt(d)
    K = rng.standard_normal((L + 5, d))
    V = rng.standard_normal((L + 5, d))
    Ki = rng.standard_normal((L + 5, 8))
    toks = oracle.select_tokens(rng.standard_normal((1, 8)), Ki, L, L, 2, 3)
    assert toks == list(range(L))
    O, lse = oracle.token_decode_unit(q, K, V, toks, 1.0)
    qt = torch.from_numpy(q)[:, None]                      # [G, 1, d]
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt, torch.from_numpy(K[:L])[None].expand(G, L, d),
        torch.from_numpy(V[:L])[None].expand(G, L, d), scale=1.0)[:, 0]
    assert np.allclose(O, ref.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(lse, torch.logsumexp(qt[:, 0] @ torch.from_numpy(K[:L]).T, dim=1).numpy(),
                       rtol=1e-12, atol=1e-12)


def test_crosslayer_uses_the_anchor_index():
    rng = np.random.default_rng(9)
    B, Hq, Hkv, d, di, T = 2, 8, 2, 16, 8, 300
    lens = [300, 123]
    layers = [dict(Q=rng.standard_normal((B, Hq, d)), K=rng.standard_normal((B, Hkv, T, d)),
                   V=rng.standard_normal((B, Hkv, T, d))) for _ in range(3)]
    Ki = rng.standard_normal((B, Hkv, T, di))
    sel = rng.standard_normal((B, Hkv, di))
    toks, outs, lses = oracle.token_crosslayer_step(layers, sel, Ki, lens, 20, 4, 8, 1.0)
    for (b, h), t in toks.items():
        assert t == oracle.select_tokens(sel[b, h:h + 1], Ki[b, h], lens[b], 20, 4, 8)
        assert len(t) == 32
    # identical layers give identical outputs; a layer attends over the shared
    # tokens, not over a selection of its own
    same = oracle.token_crosslayer_step([layers[0], layers[0]], sel, Ki, lens, 20, 4, 8, 1.0)
    assert np.array_equal(same[1][0], same[1][1])
    other_sel = rng.standard_normal((B, Hkv, di))
    b, h = 0, 1
    own = oracle.select_tokens(other_sel[b, h:h + 1], Ki[b, h], lens[b], 20, 4, 8)
    assert own != toks[(b, h)]
    o_own, _ = oracle.token_decode_unit(layers[2]["Q"][b, 4 * h:4 * h + 4], layers[2]["K"][b, h],
                                        layers[2]["V"][b, h], own, 1.0)
    assert not np.allclose(outs[2][b, 4 * h:4 * h + 4], o_own)
    # a group of query-head selectors (H_sel = Hq) scores with their sum
    selq = rng.standard_normal((B, Hq, di))
    tq, _, _ = oracle.token_crosslayer_step(layers[:1], selq, Ki, lens, 20, 4, 8, 1.0)
    summed = selq.reshape(B, Hkv, 4, di).sum(axis=2)
    ts, _, _ = oracle.token_crosslayer_step(layers[:1], summed, Ki, lens, 20, 4, 8, 1.0)
    assert tq == ts
