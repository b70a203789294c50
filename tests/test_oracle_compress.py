"""Pins for the oracle's compressed keys (Eq. 2 of the SparDA summary page).

CPU only. Each test checks the oracle against something other than itself:
a library routine (torch avg_pool1d, torch's bf16 cast), closed forms, a
hand-worked fixture, or the bulk/incremental identity.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def test_entry_count_closed_form():
    assert [oracle.n_compressed(L) for L in (0, 1, 31, 32, 47, 48, 63, 64, 65, 8192)] == \
        [0, 0, 0, 1, 1, 2, 2, 3, 3, 511]
    # torch's pooling produces the same number of complete windows
    for L in (32, 47, 48, 200, 1000, 4097):
        x = torch.zeros(1, 1, L, dtype=torch.float64)
        n = torch.nn.functional.avg_pool1d(x, 32, 16).shape[-1]
        assert n == oracle.n_compressed(L)


@pytest.mark.parametrize("L", [32, 100, 1000, 4133])
def test_matches_avg_pool1d(L):
    rng = np.random.default_rng(L)
    K = rng.standard_normal((L + 7, 16)).astype(np.float32)
    got = oracle.compressed_keys(K, L, "f32")
    ref = torch.nn.functional.avg_pool1d(
        torch.from_numpy(K[:L].astype(np.float64)).T[None], 32, 16)[0].T.numpy()
    assert got.shape == ref.shape
    # fp32 summation error bound: each 16-term partial sum errs by at most 15 u sum|k|
    absmean = torch.nn.functional.avg_pool1d(
        torch.from_numpy(np.abs(K[:L]).astype(np.float64)).T[None], 32, 16)[0].T.numpy()
    bound = 17 * 2.0 ** -24 * absmean + 1e-30
    assert np.all(np.abs(got - ref) <= bound)


def test_constant_keys_give_the_constant_exactly():
    # constants with few mantissa bits: every partial sum is exact, so the mean is the constant
    for dt, c in (("f32", 0.3125), ("bf16", -1.703125), ("f32", -7.75), ("bf16", 0.0)):
        K = np.full((300, 8), c, dtype=np.float32)
        got = oracle.compressed_keys(K, 300, dt)
        assert got.shape == (oracle.n_compressed(300), 8)
        assert np.all(got == np.float32(c))


def test_ramp_is_window_midpoint_and_golden_fixture():
    g = json.load(open(os.path.join(HERE, "golden", "eq2_ramp.json")))
    L = g["L"]
    K = np.arange(L, dtype=np.float32)[:, None]
    got = oracle.compressed_keys(K, L, "f32")[:, 0]
    assert got.shape[0] == g["n_c"]
    assert np.array_equal(got, np.array(g["entries"], dtype=np.float32))
    L2 = g["L2"]
    K2 = np.arange(L2, dtype=np.float32)[:, None]
    got2 = oracle.compressed_keys(K2, L2, "f32")[:, 0]
    assert got2.shape[0] == g["n_c2"]
    assert np.array_equal(got2, 16 * np.arange(g["n_c2"], dtype=np.float32) + 15.5)


def test_bf16_rounding_matches_torch_cast():
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 65504.0, 3.3895e38, 1e-40, 0.0,
                  -0.0, np.inf, -np.inf], dtype=np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    got = oracle.bf16_round(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    # halfway cases go to the even mantissa
    assert oracle.bf16_round(np.float32(1 + 2 ** -8)) == np.float32(1.0)
    assert oracle.bf16_round(np.float32(1 + 3 * 2 ** -8)) == np.float32(1 + 2 ** -6)


def test_bf16_entries_are_rounded_fp32_means():
    rng = np.random.default_rng(7)
    Kf = rng.standard_normal((640, 32)).astype(np.float32)
    Kb = oracle.bf16_round(Kf)
    got = oracle.compressed_keys(Kb, 640, "bf16")
    mean32 = oracle.compressed_keys(Kb, 640, "f32")
    ref = torch.from_numpy(mean32).to(torch.bfloat16).float().numpy()
    assert np.array_equal(got, ref)
    # and within one bf16 rounding of the exact mean
    exact = torch.nn.functional.avg_pool1d(
        torch.from_numpy(Kb.astype(np.float64)).T[None], 32, 16)[0].T.numpy()
    assert np.all(np.abs(got - exact) <= 2.0 ** -8 * np.abs(exact) + 1e-6)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_incremental_equals_bulk(dt):
    rng = np.random.default_rng(11)
    K = oracle.round_to(rng.standard_normal((700, 16)).astype(np.float32), dt)
    bulk = oracle.compressed_keys(K, 700, dt)
    Kc = np.zeros((0, 16), dtype=np.float32)
    L_old = 0
    for L in list(range(1, 130)) + [131, 200, 263, 400, 555, 700]:
        Kc = oracle.append_compressed_keys(K, Kc, L_old, L, dt)
        assert Kc.shape[0] == oracle.n_compressed(L)
        L_old = L
    assert np.array_equal(Kc, bulk)


def test_future_tokens_are_not_read():
    rng = np.random.default_rng(3)
    K = rng.standard_normal((500, 8)).astype(np.float32)
    a = oracle.compressed_keys(K, 333, "f32")
    K2 = K.copy()
    K2[333:] = np.nan
    b = oracle.compressed_keys(K2, 333, "f32")
    assert np.array_equal(a, b)
