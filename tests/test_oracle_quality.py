"""Pins of the oracle's selection-quality measures (block attention mass, recall,
rest bucket, mass-optimal set) against a library routine, closed forms and brute
force."""
import itertools

import numpy as np
import torch

import oracle


def _rand(seed, L, d=16):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(d), rng.standard_normal((L, d))


def test_block_mass_equals_sdpa_with_block_indicator_values():
    """SDPA with V = one-hot block membership returns exactly the block masses."""
    for L in (1, 63, 64, 65, 700):
        q, K = _rand(L, L)
        scale = 0.3
        nb = oracle.n_blocks(L)
        V = np.zeros((L, nb))
        V[np.arange(L), np.arange(L) // 64] = 1.0
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(q)[None, None, None], torch.tensor(K)[None, None], torch.tensor(V)[None, None],
            scale=scale)[0, 0, 0].numpy()
        assert np.allclose(oracle.block_mass(q, K, L, scale), ref, rtol=1e-12, atol=1e-15)


def test_mass_closed_forms():
    # constant keys: uniform attention, a block's mass is its token count / L
    L = 200
    K = np.ones((L, 8))
    m = oracle.block_mass(np.ones(8), K, L, 1.0)
    assert np.allclose(m, [64 / L, 64 / L, 64 / L, 8 / L])
    # one key far above the rest takes (nearly) all the mass
    q, K = _rand(1, 500)
    K[300] = 60.0 * q
    m = oracle.block_mass(q, K, 500, 1.0)
    assert m[300 // 64] > 1 - 1e-12
    # only the first L keys count
    q, K = _rand(2, 400)
    K2 = K.copy()
    K2[250:] = 1e3
    assert np.allclose(oracle.block_mass(q, K, 250, 0.5), oracle.block_mass(q, K2, 250, 0.5))


def test_recall_and_rest_bucket():
    q, K = _rand(3, 640)
    m = oracle.block_mass(q, K, 640, 0.7)
    assert abs(m.sum() - 1) < 1e-12
    assert abs(oracle.recall(m, range(10)) - 1) < 1e-12
    assert oracle.recall(m, []) == 0.0
    dist = oracle.rest_bucket_distribution(m, [0, 3, 9])
    assert np.allclose(dist[:3], m[[0, 3, 9]]) and abs(dist.sum() - 1) < 1e-12
    assert abs(dist[-1] - (1 - oracle.recall(m, [0, 3, 9]))) < 1e-15


def test_mass_optimal_set_is_optimal_by_brute_force():
    for seed in range(5):
        q, K = _rand(10 + seed, 64 * 9 - 5)
        m = oracle.block_mass(q, K, K.shape[0], 1.0)
        nb = len(m)
        for k in (0, 1, 3, 6, 20):
            best = oracle.mass_optimal_blocks(m, k, 1, 2)
            fixed = {0, nb - 2, nb - 1}
            cand = [b for b in range(nb) if b not in fixed]
            kk = min(k, len(cand))
            brute = max(oracle.recall(m, sorted(fixed | set(c))) for c in itertools.combinations(cand, kk))
            assert abs(oracle.recall(m, best) - brute) < 1e-12
            assert len(best) == len(fixed) + kk
