"""Pins for the oracle's attention over chosen blocks (Eq. 5), decode, prefill and reuse.

CPU only. Special cases that reduce to torch's scaled_dot_product_attention
(every block chosen), closed forms (constant values, zero query), the gather
vs. masked-dense identity, log-sum-exp merges of random partitions, per-query
brute force for tile selection, and the cross-layer identities.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import oracle
import synth
from oracle import SelectParams, SOFTMAX_SUM, RAW_SUM
from oracle.attention import block_tokens


def _sdpa(q, K, V, mask=None, scale=1.0):
    """torch reference on CPU in fp64: q [H, d], K/V [n, d], mask [n] bool (True = keep)."""
    qt = torch.from_numpy(np.asarray(q, np.float64))[None, :, None, :]
    kt = torch.from_numpy(np.asarray(K, np.float64))[None, None].expand(1, q.shape[0], -1, -1)
    vt = torch.from_numpy(np.asarray(V, np.float64))[None, None].expand(1, q.shape[0], -1, -1)
    am = None if mask is None else torch.from_numpy(mask)[None, None, None, :]
    return Fn.scaled_dot_product_attention(qt, kt, vt, attn_mask=am, scale=scale)[0, :, 0].numpy()


@pytest.mark.parametrize("L", [64, 100, 1000, 2049])
def test_all_blocks_chosen_equals_dense_sdpa(L):
    rng = np.random.default_rng(L)
    d = 32
    K = rng.standard_normal((L + 10, d))
    V = rng.standard_normal((L + 10, d))
    q = rng.standard_normal((4, d)) / np.sqrt(d)
    Kc = oracle.compressed_keys(K.astype(np.float32), L, "f32")
    p = SelectParams(top_k=10 ** 6)
    blocks = oracle.select_blocks(q, Kc, L, p)
    assert blocks == list(range(oracle.n_blocks(L)))
    O, LSE = oracle.sparse_attention(q, K, V, block_tokens(blocks, L), scale=0.7)
    ref = _sdpa(q, K[:L], V[:L], scale=0.7)
    assert np.allclose(O, ref, rtol=1e-12, atol=1e-12)
    lse_ref = torch.logsumexp(0.7 * torch.from_numpy(q) @ torch.from_numpy(K[:L]).T, -1).numpy()
    assert np.allclose(LSE, lse_ref, rtol=1e-13, atol=1e-13)


def test_gather_equals_masked_dense():
    rng = np.random.default_rng(1)
    L, d = 1000, 16
    K = rng.standard_normal((L, d))
    V = rng.standard_normal((L, d))
    q = rng.standard_normal((3, d))
    blocks = [0, 3, 7, 14, 15]                     # block 15 is partial: tokens 960..999
    O, _ = oracle.sparse_attention(q, K, V, block_tokens(blocks, L), scale=0.25)
    mask = np.zeros(L, dtype=bool)
    for b in blocks:
        mask[64 * b:64 * b + 64] = True
    ref = _sdpa(q, K, V, mask=mask, scale=0.25)
    assert np.allclose(O, ref, rtol=1e-12, atol=1e-12)
    assert block_tokens([15], L).tolist() == list(range(960, 1000))


def test_closed_forms_constant_values_and_zero_query():
    rng = np.random.default_rng(2)
    L, d = 700, 8
    K = rng.standard_normal((L, d))
    toks = block_tokens([0, 4, 10], L)
    Vc = np.tile(np.arange(d, dtype=np.float64), (L, 1))
    O, _ = oracle.sparse_attention(rng.standard_normal((2, d)), K, Vc, toks, 1.0)
    assert np.allclose(O, np.arange(d)[None].repeat(2, 0), rtol=0, atol=1e-13)
    V = rng.standard_normal((L, d))
    O0, LSE0 = oracle.sparse_attention(np.zeros((2, d)), K, V, toks, 1.0)
    sel = np.zeros(L, dtype=bool)
    sel[0:64] = sel[256:320] = sel[640:700] = True
    assert np.allclose(O0, V[sel].mean(0)[None].repeat(2, 0), atol=1e-13)
    assert np.allclose(LSE0, np.log(sel.sum()))


def test_lse_merge_of_random_partitions_equals_unsplit():
    rng = np.random.default_rng(3)
    L, d = 1500, 16
    K, V = rng.standard_normal((L, d)), rng.standard_normal((L, d))
    q = rng.standard_normal((4, d))
    toks = block_tokens([0, 2, 5, 9, 11, 20, 23], L)
    O, LSE = oracle.sparse_attention(q, K, V, toks, 0.5)
    for trial in range(5):
        cuts = np.sort(rng.choice(np.arange(1, toks.size), size=trial + 1, replace=False))
        parts = np.split(toks, cuts)
        parts.append(np.zeros(0, dtype=np.int64))        # an empty split is harmless
        O2, LSE2 = oracle.lse_merge(oracle.split_attention_partials(q, K, V, parts, 0.5))
        assert np.allclose(O2, O, rtol=1e-12, atol=1e-13)
        assert np.allclose(LSE2, LSE, rtol=1e-13, atol=1e-13)


def test_decode_step_query_and_forecast_agree_with_per_unit_pieces():
    w = synth.scaled(synth.WORKLOADS["decode_forecast_bf16_128k"], B=2, Hq=8, Hkv=2, T=3000)
    inp = synth.make_decode_inputs(w, seq_lens=[3000, 2111])
    Q, F = inp["Q"].float().numpy(), inp["F"].float().numpy()
    K, V = inp["K"].float().numpy(), inp["V"].float().numpy()
    lens = inp["seq_lens"].numpy()
    Kc = np.zeros((2, 2, oracle.n_compressed(3000), 128), np.float32)
    for b in range(2):
        for h in range(2):
            c = oracle.compressed_keys(K[b, h], int(lens[b]), "bf16")
            Kc[b, h, :c.shape[0]] = c
    p = SelectParams(top_k=w.top_k, n_init=1, n_local=2, score_mode=RAW_SUM)
    r = oracle.decode_step(Q, F, K, V, Kc, lens, p, 1.0)
    for (b, h), blk in r["blocks"].items():
        L = int(lens[b])
        assert len(blk) == min(oracle.n_blocks(L), w.top_k + 3)
        ref = _sdpa(Q[b, 4 * h:4 * h + 4], K[b, h], V[b, h],
                    mask=np.isin(np.arange(K.shape[2]) // 64, blk) & (np.arange(K.shape[2]) < L))
        assert np.allclose(r["O"][b, 4 * h:4 * h + 4], ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- prefill

def _prefill_case(T=2560, q_start=2048, Hq=8, Hkv=2, d=32, seed=0):
    rng = np.random.default_rng(seed)
    Q = oracle.bf16_round((rng.standard_normal((T - q_start, Hq, d)) / np.sqrt(d)).astype(np.float32))
    K = oracle.bf16_round(rng.standard_normal((Hkv, T, d)).astype(np.float32))
    V = oracle.bf16_round(rng.standard_normal((Hkv, T, d)).astype(np.float32))
    Kc = np.stack([oracle.compressed_keys(K[h], T, "bf16") for h in range(Hkv)])
    return Q, K, V, Kc


def test_prefill_tile_union_is_union_of_per_query_decode_selections():
    Q, K, V, Kc = _prefill_case()
    p = SelectParams(top_k=5, n_init=1, n_local=4, score_mode=SOFTMAX_SUM)
    q_start, G = 2048, 4
    for t in (0, 3, 7):
        for h in range(2):
            pos = np.arange(q_start + 64 * t, q_start + 64 * t + 64)
            qt = Q[64 * t:64 * t + 64, G * h:G * h + G]
            union = oracle.prefill_tile_select(qt, Kc[h], pos, p)
            # brute force: each query selects exactly as a decode step at L = p + 1 would
            acc = set()
            for i, x in enumerate(pos):
                acc |= set(oracle.select_blocks(qt[i], Kc[h], int(x) + 1, p))
            assert union == sorted(acc)
            bt = pos[0] // 64
            assert set(range(bt - 3, bt + 1)) <= set(union) and 0 in union
            assert max(union) == bt


def test_prefill_one_query_tile_equals_decode():
    Q, K, V, Kc = _prefill_case(T=2049, q_start=2048)
    p = SelectParams(top_k=6, n_init=1, n_local=4)
    r = oracle.prefill_chunk(Q, K, V, Kc, 2048, p, 1.0)
    for h in range(2):
        blk = oracle.select_blocks(Q[0, 4 * h:4 * h + 4], Kc[h], 2049, p)
        assert r["blocks"][(0, h)] == blk
        o, lse = oracle.sparse_attention(Q[0, 4 * h:4 * h + 4], K[h], V[h], block_tokens(blk, 2049), 1.0)
        assert np.allclose(r["O"][0, 4 * h:4 * h + 4], o, rtol=1e-14, atol=1e-14)


def test_prefill_all_blocks_equals_causal_sdpa():
    T, q_start = 1200, 1024
    Q, K, V, Kc = _prefill_case(T=T, q_start=q_start)
    p = SelectParams(top_k=10 ** 6, n_init=1, n_local=4)
    r = oracle.prefill_chunk(Q, K, V, Kc, q_start, p, 1.0)
    Hq, G = Q.shape[1], 4
    qt = torch.from_numpy(Q.astype(np.float64)).permute(1, 0, 2)[None]          # [1,Hq,Tq,d]
    kt = torch.from_numpy(K.astype(np.float64)).repeat_interleave(G, 0)[None]    # [1,Hq,T,d]
    vt = torch.from_numpy(V.astype(np.float64)).repeat_interleave(G, 0)[None]
    causal = torch.arange(T)[None, :] <= (q_start + torch.arange(T - q_start))[:, None]
    ref = Fn.scaled_dot_product_attention(qt, kt, vt, attn_mask=causal, scale=1.0)[0].permute(1, 0, 2).numpy()
    assert np.allclose(r["O"], ref, rtol=1e-11, atol=1e-12)


def test_prefill_tile_attention_equals_per_query_attention_and_causal_sdpa():
    """oracle.tile_attention (all queries of a tile at once, causal mask) is
    the per-query Eq. 5 of sparse_attention over each query's visible tokens,
    and with every block chosen it is causal dense attention (SDPA)."""
    T, q_start = 1300, 1216                               # a full tile and a partial one
    Q, K, V, Kc = _prefill_case(T=T, q_start=q_start)
    G = 4
    rng = np.random.default_rng(5)
    for t, n_q in ((0, 64), (1, T - q_start - 64)):
        lo = 64 * t
        pos = np.arange(q_start + lo, q_start + lo + n_q)
        nb = oracle.n_blocks(int(pos[-1]) + 1)
        for h in range(K.shape[0]):
            blocks = sorted(set(rng.choice(nb, size=min(nb, 7), replace=False).tolist()) | {nb - 1})
            O, L = oracle.tile_attention(Q[lo:lo + n_q, G * h:G * h + G], K[h], V[h], blocks, pos, 1.0)
            for i, p_ in enumerate(pos):
                o, l = oracle.sparse_attention(Q[lo + i, G * h:G * h + G], K[h], V[h],
                                               block_tokens(blocks, int(p_) + 1), 1.0)
                assert np.allclose(O[i], o, rtol=1e-12, atol=1e-13)
                assert np.allclose(L[i], l, rtol=1e-12, atol=1e-13)
            O, L = oracle.tile_attention(Q[lo:lo + n_q, G * h:G * h + G], K[h], V[h],
                                         list(range(nb)), pos, 1.0)
            qt = torch.from_numpy(Q[lo:lo + n_q, G * h:G * h + G].astype(np.float64)).permute(1, 0, 2)
            kt = torch.from_numpy(K[h, :int(pos[-1]) + 1].astype(np.float64))[None].expand(G, -1, -1)
            vt = torch.from_numpy(V[h, :int(pos[-1]) + 1].astype(np.float64))[None].expand(G, -1, -1)
            mask = torch.arange(int(pos[-1]) + 1)[None, :] <= torch.from_numpy(pos)[:, None]
            ref = Fn.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=1.0)
            assert np.allclose(O, ref.permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- cross-layer reuse

def test_crosslayer_step_shares_anchor_selection_and_grows_keys():
    w = synth.scaled(synth.WORKLOADS["crosslayer_bf16_64k"], B=2, Hq=8, Hkv=2, T=1500)
    T0, steps = 1500, 20
    layers = []
    for l in range(3):
        inp = synth.make_decode_inputs(w, T_cap=T0 + steps, layer=l)
        layers.append(dict(K=inp["K"].float().numpy(), V=inp["V"].float().numpy()))
    qs = [[q.float().numpy() for q in synth.make_decode_queries(w, steps, seed_offset=100 + l)]
          for l in range(3)]
    p = SelectParams(top_k=7)
    Kc = np.zeros((2, 2, oracle.n_compressed(T0 + steps), 128), np.float32)
    for b in range(2):
        for h in range(2):
            c = oracle.compressed_keys(layers[0]["K"][b, h], T0, "bf16")
            Kc[b, h, :c.shape[0]] = c
    lens = np.array([T0, T0])
    for s in range(steps):
        new = lens + 1
        for l in range(3):
            layers[l]["Q"] = qs[l][s]
        Kc, blocks, outs, _ = oracle.crosslayer_step(layers, Kc, lens, new, p, 1.0, "bf16")
        for (b, h), blk in blocks.items():
            for l in range(3):
                o, _ = oracle.sparse_attention(layers[l]["Q"][b, 4 * h:4 * h + 4], layers[l]["K"][b, h],
                                               layers[l]["V"][b, h], block_tokens(blk, int(new[b])), 1.0)
                assert np.allclose(outs[l][b, 4 * h:4 * h + 4], o, rtol=1e-14, atol=1e-14)
        lens = new
    for b in range(2):
        for h in range(2):
            bulk = oracle.compressed_keys(layers[0]["K"][b, h], int(lens[b]), "bf16")
            assert np.array_equal(Kc[b, h, :bulk.shape[0]], bulk)
