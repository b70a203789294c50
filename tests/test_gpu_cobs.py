"""GPU parity of the second-order block statistic path against oracle.cobs.

Block statistics: within one unit in the last place of the key dtype of the
oracle's fp64 mean and variance rounded once (identical in practice).
Block scores: elementwise tolerance. Block sets:
exact (lower index on ties) except for near ties (parity.selection_ok). The
reading of the statistic itself is not fixed by the pages (oracle.cobs).
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_12_amd as sa
import oracle
from oracle import SelectParams
from oracle.attention import block_tokens
from parity import selection_ok, gpu_rows, assert_close, to_np, ulp_distance

pytestmark = pytest.mark.gpu
DEV = "cuda"
TD = {"f32": torch.float32, "bf16": torch.bfloat16}
BITS = {"f32": torch.int32, "bf16": torch.int16}


def rand(shape, dt, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g) * scale).to(TD[dt])


def lens_t(lens):
    return torch.tensor(lens, dtype=torch.int32, device=DEV)


def assert_within_one_ulp(got, ref, dt, what):
    d = ulp_distance(got.float().numpy(), ref.float().numpy(), dt)
    assert d.max(initial=0) <= 1, (what, int(d.max()), int((d > 0).sum()))
    return int((d > 0).sum())


def _stats_gpu(K, lens, nb_cap=None, fill=1024.0):
    B, Hkv, T, d = K.shape
    nb_cap = nb_cap if nb_cap is not None else (T + 63) // 64
    S = torch.full((B, Hkv, nb_cap, 2, d), fill, dtype=K.dtype, device=DEV)
    sa.cobs_stats(K.to(DEV), S, lens_t([0] * B), lens_t(lens))
    return S


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_cobs_stats_bulk_and_incremental_within_one_ulp(dt):
    B, Hkv, T = 3, 2, 1000
    lens = [1000, 640, 63]
    K = rand((B, Hkv, T, 128), dt, 1, scale=2.0) + 0.5
    S = _stats_gpu(K, lens)
    got = S.cpu()
    for b in range(B):
        for h in range(Hkv):
            mu, var = oracle.block_stats(K[b, h].float().numpy(), lens[b], dt)
            n = mu.shape[0]
            ref = torch.from_numpy(np.stack([mu, var], axis=1)).to(TD[dt])
            assert_within_one_ulp(got[b, h, :n], ref, dt, (b, h))
            assert torch.all(got[b, h, n:] == 1024.0), "rows of incomplete blocks stay untouched"
    # incremental: one token at a time across a block edge, then a jump
    Kd = K.to(DEV)
    S2 = torch.full_like(S, 1024.0)
    steps = [[0, 0, 0], [63, 63, 63], [64, 64, 63], [65, 127, 63], [128, 640, 63], [1000, 640, 63]]
    for i in range(1, len(steps)):
        sa.cobs_stats(Kd, S2, lens_t(steps[i - 1]), lens_t(steps[i]), max_new_blocks=16)
    assert torch.equal(S2.cpu().view(BITS[dt]), got.view(BITS[dt]))


def _check_cobs_select(sel, K, lens, T_cap, k, n_init, n_local, mode, dt, order, exact=False):
    S = _stats_gpu(K, lens)
    idx, cnt, bs = sa.cobs_select(sel.to(DEV), S, lens_t(lens), T_cap, k, n_init, n_local, mode,
                                  order, block_scores=True)
    rows = gpu_rows(idx, cnt)
    bs = bs.cpu().numpy().astype(np.float64)
    Sel = to_np(sel)
    B, Hkv = K.shape[:2]
    Gs = Sel.shape[1] // Hkv
    p = SelectParams(top_k=k, n_init=n_init, n_local=n_local, score_mode=mode)
    kinds = []
    for b in range(B):
        for h in range(Hkv):
            L = lens[b]
            mu, var = oracle.block_stats(K[b, h].float().numpy(), L, dt)
            nbc = mu.shape[0]
            assert_within_one_ulp(S[b, h, :nbc].cpu(),
                                  torch.from_numpy(np.stack([mu, var], axis=1)).to(TD[dt]), dt, (b, h))
            ref, BS = oracle.select_blocks_cobs(Sel[b, h * Gs:(h + 1) * Gs], mu, var, L, p, order,
                                                return_scores=True)
            nb = oracle.n_blocks(L)
            fin = np.isfinite(BS)
            assert np.array_equal(np.isfinite(bs[b, h, :nb]), fin), (b, h)
            if fin.any():
                scale = np.abs(BS[fin]).max()
                assert np.allclose(bs[b, h, :nb][fin], BS[fin], rtol=2e-5, atol=2e-6 * scale), (b, h)
            assert np.all(np.isneginf(bs[b, h, nb:]))
            if exact:
                assert rows[(b, h)] == ref, (b, h, rows[(b, h)], ref)
                kinds.append("exact")
            else:
                ok, why = selection_ok(rows[(b, h)], ref, BS, nb, k, n_init, n_local)
                assert ok, ((b, h), why, rows[(b, h)], ref)
                kinds.append(why)
    return kinds, idx, cnt


@pytest.mark.parametrize("mode,G,dt", [("softmax_sum", 4, "bf16"), ("softmax_sum", 4, "f32"),
                                       ("raw_sum", 1, "bf16"), ("raw_sum", 1, "f32"),
                                       ("softmax_sum", 1, "bf16"), ("raw_sum", 4, "bf16"),
                                       ("softmax_sum", 8, "bf16"), ("softmax_sum", 2, "f32")])
@pytest.mark.parametrize("order", [1, 2])
def test_cobs_select_parity(mode, G, dt, order):
    B, Hkv, T = 3, 2, 20000                           # 313 blocks: two scoring chunks
    lens = [20000, 9000, 700]
    K = rand((B, Hkv, T, 128), dt, 2)
    sel = rand((B, Hkv * G, 128), dt, 3, scale=128 ** -0.5)
    kinds, _, _ = _check_cobs_select(sel, K, lens, T, 24, 1, 2, mode, dt, order)
    assert kinds.count("exact") >= len(kinds) - 1


@pytest.mark.parametrize("L", [0, 10, 63, 64, 65, 127, 128, 129, 192, 260, 16384])
def test_cobs_select_short_lengths_and_edges(L):
    dt = "bf16"
    T = 16384
    K = rand((1, 2, T, 128), dt, 4)
    sel = rand((1, 8, 128), dt, 5, scale=128 ** -0.5)
    for k in (0, 1, 3, 300):
        _check_cobs_select(sel, K, [L], T, k, 1, 2, "softmax_sum", dt, 2)
    # no local blocks: the partial last block is a candidate without statistics
    _check_cobs_select(sel, K, [L], T, 2, 1, 0, "raw_sum", dt, 2)


def _hadamard64():
    H = np.array([[1.0]])
    while H.shape[0] < 64:
        H = np.block([[H, H], [H, -H]])
    return H


def test_cobs_second_order_finds_spread_blocks_and_decode_runs_on_them():
    """Blocks whose keys spread in the query's strongest channels (zero-mean,
    mutually orthogonal sign patterns, so the block mean and the off-diagonal
    covariance are unchanged) carry far more attention mass: the second-order
    selection includes them, the first order does not, and decode attention
    over the second-order set matches the oracle and captures more of the
    exact mass."""
    dt = "bf16"
    B, Hq, Hkv, T = 1, 8, 2, 64 * 128
    g = torch.Generator().manual_seed(6)
    K = torch.randn((B, Hkv, T, 128), generator=g) * 0.5
    V = torch.randn((B, Hkv, T, 128), generator=g)
    Q = torch.randn((B, Hq, 128), generator=g) * 0.05
    Q[..., :4] = 1.0                                   # the strongest channels of every head
    H = torch.from_numpy(_hadamard64()[1:5].T.copy()).float()   # [64 tokens, 4 channels]
    spread = [11, 40, 77, 100]
    for h in range(Hkv):
        for blk in spread:
            K[0, h, 64 * blk:64 * (blk + 1), :4] += 2.0 * H
    K, V, Q = K.to(TD[dt]), V.to(TD[dt]), Q.to(TD[dt])
    lens = [T]
    k = 8
    _, idx1, cnt1 = _check_cobs_select(Q, K, lens, T, k, 1, 2, "softmax_sum", dt, 1)
    _, idx2, cnt2 = _check_cobs_select(Q, K, lens, T, k, 1, 2, "softmax_sum", dt, 2)
    r1, r2 = gpu_rows(idx1, cnt1), gpu_rows(idx2, cnt2)
    for h in range(Hkv):
        assert set(spread) <= set(r2[(0, h)])
        assert not set(spread) <= set(r1[(0, h)])
    O, lse = sa.decode(Q.to(DEV), K.to(DEV), V.to(DEV), lens_t(lens), idx2, cnt2, 1.0)
    Qn, Kn, Vn = to_np(Q), to_np(K), to_np(V)
    for h in range(Hkv):
        o, l = oracle.sparse_attention(Qn[0, 4 * h:4 * h + 4], Kn[0, h], Vn[0, h],
                                       block_tokens(r2[(0, h)], T), 1.0)
        assert_close(to_np(O)[0, 4 * h:4 * h + 4], o, dt, f"O head group {h}")
        for g4 in range(4):
            mass = oracle.block_mass(Qn[0, 4 * h + g4], Kn[0, h], T, 1.0)
            assert oracle.recall(mass, r2[(0, h)]) > oracle.recall(mass, r1[(0, h)]) + 0.2


# ------------------------------------------------------------------ one-call step

@pytest.mark.parametrize("mode,G,dt,order", [("softmax_sum", 4, "bf16", 2), ("softmax_sum", 4, "f32", 1),
                                              ("softmax_sum", 1, "bf16", 2), ("softmax_sum", 2, "bf16", 1),
                                              ("softmax_sum", 8, "bf16", 2), ("raw_sum", 1, "bf16", 2),
                                              ("raw_sum", 4, "f32", 2)])
def test_cobs_decode_step_equals_separate_calls(mode, G, dt, order):
    """sparse_attn_cobs_decode_step (statistics append + selection + attention,
    with the top-k inside the attention workgroups where it applies) gives the
    three calls' statistics, block sets and outputs bit for bit, over steps
    whose new tokens complete blocks, cross several blocks, or complete none."""
    B, Hkv, T = 3, 2, 9000
    Hq = 4 * Hkv
    K = rand((B, Hkv, T, 128), dt, 40).to(DEV)
    V = rand((B, Hkv, T, 128), dt, 41).to(DEV)
    nb = (T + 63) // 64
    steps = [([4000, 700, 64], [4001, 704, 65]), ([4001, 704, 65], [4096, 705, 128]),
             ([4096, 705, 128], [5000, 1300, 129]), ([5000, 1300, 129], [9000, 1301, 190])]
    S_a = torch.full((B, Hkv, nb, 2, 128), 7.0, dtype=TD[dt], device=DEV)
    sa.cobs_stats(K, S_a, lens_t([0] * B), lens_t(steps[0][0]))
    S_b = S_a.clone()
    k = 20
    for i, (lp, ln) in enumerate(steps):
        Q = rand((B, Hq, 128), dt, 50 + i, scale=128 ** -0.5).to(DEV)
        sel = Q if G == 4 else rand((B, Hkv * G, 128), dt, 60 + i, scale=128 ** -0.5).to(DEV)
        Lp, Ln = lens_t(lp), lens_t(ln)
        mxb = max(b // 64 - a // 64 for a, b in zip(lp, ln)) + 1
        O1, lse1, idx1, cnt1 = sa.cobs_decode_step(Q, sel, K, V, S_a, Lp, Ln, k, 1, 2, mode, order,
                                                   max_new_blocks=mxb)
        sa.cobs_stats(K, S_b, Lp, Ln, max_new_blocks=mxb)
        idx2, cnt2, _ = sa.cobs_select(sel, S_b, Ln, T, k, 1, 2, mode, order)
        O2, lse2 = sa.decode(Q, K, V, Ln, idx2, cnt2, 1.0)
        torch.cuda.synchronize()
        assert torch.equal(S_a.view(BITS[dt]), S_b.view(BITS[dt])), (i, "statistics")
        assert torch.equal(idx1, idx2) and torch.equal(cnt1, cnt2), (i, mode)
        assert torch.equal(O1, O2) and torch.equal(lse1, lse2), (i, mode)


def test_cobs_decode_step_at_and_past_the_fused_limits():
    """2048 blocks (top-k inside the attention workgroups) and 2049 blocks
    (separate top-k launch), softmax mode, against the separate calls and the
    oracle's selection."""
    for T in (64 * 2048, 64 * 2048 + 64):
        B, Hkv, G = 1, 2, 4
        K = rand((B, Hkv, T, 128), "bf16", 70).to(DEV)
        V = rand((B, Hkv, T, 128), "bf16", 71).to(DEV)
        Q = rand((B, 4 * Hkv, 128), "bf16", 72, scale=128 ** -0.5).to(DEV)
        nb = (T + 63) // 64
        S = _stats_gpu(K.cpu(), [T - 1], nb_cap=nb)
        S2 = S.clone()
        Lp, Ln = lens_t([T - 1]), lens_t([T])
        O1, lse1, idx1, cnt1 = sa.cobs_decode_step(Q, Q, K, V, S, Lp, Ln, 60, 1, 2, "softmax_sum", 2)
        sa.cobs_stats(K, S2, Lp, Ln)
        idx2, cnt2, bs = sa.cobs_select(Q, S2, Ln, T, 60, 1, 2, "softmax_sum", 2, block_scores=True)
        O2, lse2 = sa.decode(Q, K, V, Ln, idx2, cnt2, 1.0)
        torch.cuda.synchronize()
        assert torch.equal(idx1, idx2) and torch.equal(cnt1, cnt2), T
        assert torch.equal(O1, O2) and torch.equal(lse1, lse2), T
        Kn = K.float().cpu().numpy()
        p = SelectParams(top_k=60, n_init=1, n_local=2, score_mode="softmax_sum")
        rows = gpu_rows(idx1, cnt1)
        bsn = bs.cpu().numpy().astype(np.float64)
        for h in range(Hkv):
            mu, var = oracle.block_stats(Kn[0, h], T, "bf16")
            ref, BS = oracle.select_blocks_cobs(to_np(Q)[0, h * G:(h + 1) * G], mu, var, T, p, 2,
                                                return_scores=True)
            ok, why = selection_ok(rows[(0, h)], ref, BS, oracle.n_blocks(T), 60, 1, 2)
            assert ok, (T, h, why)
            fin = np.isfinite(BS)
            assert np.allclose(bsn[0, h, :nb][fin], BS[fin], rtol=2e-5,
                               atol=2e-6 * np.abs(BS[fin]).max())
