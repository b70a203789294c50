"""Pins for the oracle's scoring, block aggregation, top-k and union.

CPU only. Eq. 1 (union), Eq. 4 (raw Forecast top-k) and the Eq. 6 form of the
group-summed softmax selector on the SparDA summary page. Checks use invariants,
library routines (torch softmax), brute force over all k-subsets, one-hot
spikes and a hand-worked fixture.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import SelectParams, SOFTMAX_SUM, RAW_SUM

HERE = os.path.dirname(os.path.abspath(__file__))


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_softmax_sum_sums_to_group_size_and_matches_torch_softmax():
    sel = _rand((4, 16), 1) / 4
    Kc = _rand((300, 16), 2)
    S = oracle.entry_scores(sel, Kc, SOFTMAX_SUM)
    assert abs(S.sum() - 4.0) < 1e-12
    ref = torch.softmax(torch.from_numpy(sel) @ torch.from_numpy(Kc).T, dim=-1).sum(0).numpy()
    assert np.allclose(S, ref, rtol=1e-13, atol=0)


def test_raw_sum_is_dot_with_group_sum_and_linear():
    sel = _rand((4, 16), 3)
    Kc = _rand((50, 16), 4)
    S = oracle.entry_scores(sel, Kc, RAW_SUM)
    assert np.allclose(S, torch.mv(torch.from_numpy(Kc), torch.from_numpy(sel).sum(0)).numpy())
    # linear in the compressed keys
    Kc2 = _rand((50, 16), 5)
    S2 = oracle.entry_scores(sel, Kc2, RAW_SUM)
    S3 = oracle.entry_scores(sel, 2.0 * Kc - 3.0 * Kc2, RAW_SUM)
    assert np.allclose(S3, 2.0 * S - 3.0 * S2)


def test_head_permutation_invariance():
    sel = _rand((4, 16), 6)
    Kc = _rand((77, 16), 7)
    for mode in (SOFTMAX_SUM, RAW_SUM):
        a = oracle.entry_scores(sel, Kc, mode)
        b = oracle.entry_scores(sel[[2, 0, 3, 1]], Kc, mode)
        assert np.allclose(a, b, rtol=1e-14, atol=1e-300)


def test_single_head_softmax_and_raw_rank_alike():
    sel = _rand((1, 16), 8)
    Kc = _rand((600, 16), 9)
    a = oracle.entry_scores(sel, Kc, SOFTMAX_SUM)
    b = oracle.entry_scores(sel, Kc, RAW_SUM)
    assert np.array_equal(np.argsort(-a, kind="stable"), np.argsort(-b, kind="stable"))
    for L in (600 * 16 + 16, 3000, 1111):
        pa = SelectParams(top_k=7, score_mode=SOFTMAX_SUM)
        pb = SelectParams(top_k=7, score_mode=RAW_SUM)
        assert oracle.select_blocks(sel, Kc, L, pa) == oracle.select_blocks(sel, Kc, L, pb)


def test_block_membership_by_one_hot_spike():
    """A spike in entry j raises block j // 4 when its window lies inside (j % 4 != 3), else none."""
    n_c = 4 * 12 + 3
    sel = np.zeros((1, 4))
    sel[0, 0] = 1.0
    for j in range(n_c):
        Kc = np.zeros((n_c, 4))
        Kc[j, 0] = 5.0
        BS = oracle.block_scores(oracle.entry_scores(sel, Kc, RAW_SUM), 13)
        raised = [b for b in range(13) if BS[b] > 0]
        want = [j // 4] if (j % 4 != 3 and j // 4 < 13) else []
        assert raised == want, (j, raised)
        # the window [16j, 16j+32) really lies inside the raised block's 64 tokens
        for b in raised:
            assert 64 * b <= 16 * j and 16 * j + 32 <= 64 * b + 64


def _brute_top_k(BS, cand, k):
    """Best k-subset by total score; among equal totals the lexicographically smallest ids."""
    best, best_key = None, None
    for sub in itertools.combinations(sorted(cand), min(k, len(cand))):
        key = (-sum(BS[b] for b in sub), sub)
        if best_key is None or key < best_key:
            best, best_key = list(sub), key
    return best


@pytest.mark.parametrize("seed", range(6))
def test_top_k_brute_force_tiny(seed):
    rng = np.random.default_rng(seed)
    nb = int(rng.integers(4, 11))
    BS = rng.standard_normal(nb)
    for k in range(0, nb + 1):
        init, local, cand = oracle.candidate_sets(nb, 1, 2)
        got = sorted(oracle.top_k_blocks(BS, cand, k))
        assert got == _brute_top_k(BS, cand, k)


def test_ties_go_to_lower_index():
    BS = np.array([9.0, 1.0, 3.0, 3.0, 2.0, 3.0, 0.5, 7.0, 8.0])
    _, _, cand = oracle.candidate_sets(9, 1, 2)           # candidates 1..6
    assert oracle.top_k_blocks(BS, cand, 2) == [2, 3]
    assert oracle.top_k_blocks(BS, cand, 3) == [2, 3, 5]
    assert sorted(oracle.top_k_blocks(BS, cand, 4)) == [2, 3, 4, 5]


def test_duplicated_blocks_resolve_to_lower_id():
    """Two blocks with bit-identical keys tie exactly; the lower block id wins."""
    rng = np.random.default_rng(12)
    L = 64 * 20
    K = oracle.bf16_round(rng.standard_normal((L, 32)).astype(np.float32))
    K[64 * 13:64 * 14] = K[64 * 6:64 * 7] + 0    # block 13 duplicates block 6
    sel = np.ones((1, 32), dtype=np.float32) * 0.0
    sel[0] = K[64 * 6:64 * 7].mean(0) * 3        # make block 6 (and 13) score highest
    Kc = oracle.compressed_keys(K, L, "bf16")
    _, BS = oracle.select_blocks(sel, Kc, L, SelectParams(top_k=1, score_mode=RAW_SUM), True)
    assert BS[6] == BS[13] and np.argmax(BS[1:18]) + 1 in (6, 13)
    assert oracle.select_blocks(sel, Kc, L, SelectParams(top_k=1, score_mode=RAW_SUM)) == \
        [0, 6, 18, 19]


@pytest.mark.parametrize("L", [1, 31, 64, 65, 128, 191, 192, 193, 640, 1000, 4097])
@pytest.mark.parametrize("k,n_init,n_local", [(0, 1, 2), (3, 1, 2), (16, 1, 2), (2, 2, 4),
                                                (100, 1, 2)])
def test_union_size_and_contents(L, k, n_init, n_local):
    rng = np.random.default_rng(L + 17 * k)
    Kc = rng.standard_normal((oracle.n_compressed(L) + 3, 8))
    sel = rng.standard_normal((2, 8))
    p = SelectParams(top_k=k, n_init=n_init, n_local=n_local)
    B = oracle.select_blocks(sel, Kc, L, p)
    nb = oracle.n_blocks(L)
    assert B == sorted(set(B))
    assert len(B) == min(nb, k + n_init + n_local)
    assert set(range(min(n_init, nb))) <= set(B)
    assert set(range(max(0, nb - n_local), nb)) <= set(B)
    assert all(0 <= b < nb for b in B)


def test_hand_worked_fixture():
    g = json.load(open(os.path.join(HERE, "golden", "eq2_ramp.json")))
    K = np.arange(g["L"], dtype=np.float32)[:, None]
    Kc = oracle.compressed_keys(K, g["L"], "f32")
    S = oracle.entry_scores(np.ones((1, 1)), Kc, RAW_SUM)
    BS = oracle.block_scores(S, 4)
    assert np.array_equal(BS[:3], g["block_scores_raw_plus1"]) and BS[3] == -np.inf
    p = SelectParams(top_k=1, n_init=1, n_local=2, score_mode=RAW_SUM)
    assert oracle.select_blocks(np.ones((1, 1)), Kc, g["L"], p) == g["union_k1"]
    K2 = np.arange(g["L2"], dtype=np.float32)[:, None]
    Kc2 = oracle.compressed_keys(K2, g["L2"], "f32")
    p3 = SelectParams(top_k=3, n_init=1, n_local=2, score_mode=RAW_SUM)
    assert oracle.select_blocks(np.ones((1, 1)), Kc2, g["L2"], p3) == g["union2_plus_k3"]
    assert oracle.select_blocks(-np.ones((1, 1)), Kc2, g["L2"], p3) == g["union2_minus_k3"]


@pytest.mark.parametrize("name", ["decode_tiny_f32_8k"])
def test_planted_blocks_are_recalled(name):
    w = synth.WORKLOADS[name]
    inp = synth.make_decode_inputs(w)
    Q = inp["Q"].float().numpy()
    K = inp["K"].float().numpy()
    p = SelectParams(top_k=w.top_k, n_init=w.n_init, n_local=w.n_local, score_mode=w.score_mode)
    for h in range(w.Hkv):
        Kc = oracle.compressed_keys(K[0, h], w.T, w.dtype)
        B = oracle.select_blocks(Q[0, h * w.G:(h + 1) * w.G], Kc, w.T, p)
        assert set(inp["planted"][0][h]) <= set(B)
        assert len(B) == w.top_k + w.n_init + w.n_local


def test_planted_recall_forecast_and_gqa_small():
    for name, mode in (("decode_forecast_bf16_128k", RAW_SUM), ("decode_gqa_bf16_32k", SOFTMAX_SUM)):
        w = synth.scaled(synth.WORKLOADS[name], B=2, T=16384)
        inp = synth.make_decode_inputs(w)
        K = inp["K"].float().numpy()
        sel = (inp["F"] if w.selector == "forecast" else inp["Q"]).float().numpy()
        Gs = sel.shape[1] // w.Hkv
        p = SelectParams(top_k=w.top_k, n_init=w.n_init, n_local=w.n_local, score_mode=mode)
        for b in range(w.B):
            for h in range(w.Hkv):
                Kc = oracle.compressed_keys(K[b, h], w.T, w.dtype)
                B = oracle.select_blocks(sel[b, h * Gs:(h + 1) * Gs], Kc, w.T, p)
                assert set(inp["planted"][b][h]) <= set(B)
