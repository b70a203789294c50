"""GPU parity of each entry point against the CPU oracle on small seeded inputs
that span several workgroups, ragged lengths and the degenerate cases.

Compressed keys: bit-exact. Block sets: exact (lower index on ties) except for
near ties. Attention: elementwise tolerance, checked on the GPU's own block sets.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_12_amd as sa
import oracle
from oracle import SelectParams
from oracle.attention import block_tokens
from parity import (selection_ok, gpu_rows, assert_close, to_np, oracle_kc, TOL)

pytestmark = pytest.mark.gpu
DEV = "cuda"
TD = {"f32": torch.float32, "bf16": torch.bfloat16}
BITS = {"f32": torch.int32, "bf16": torch.int16}


def rand(shape, dt, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g) * scale).to(TD[dt])


def lens_t(lens):
    return torch.tensor(lens, dtype=torch.int32, device=DEV)


# ------------------------------------------------------------------ compress

@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_compress_bulk_bit_exact(dt):
    B, Hkv, T = 3, 2, 1000
    lens = [1000, 517, 31]
    K = rand((B, Hkv, T, 128), dt, 1)
    nc_cap = oracle.n_compressed(T)
    Kc = torch.full((B, Hkv, nc_cap, 128), 1024.0, dtype=TD[dt], device=DEV)
    sa.compress(K.to(DEV), Kc, lens_t([0] * B), lens_t(lens))
    ref = torch.from_numpy(oracle_kc(K.float().numpy(), lens, dt, nc_cap)).to(TD[dt])
    got = Kc.cpu()
    for b in range(B):
        n = oracle.n_compressed(lens[b])
        assert torch.equal(got[b, :, :n].view(BITS[dt]), ref[b, :, :n].view(BITS[dt])), b
        assert torch.all(got[b, :, n:] == 1024.0), "entries past n_c(L) must stay untouched"


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_compress_incremental_equals_bulk(dt):
    B, Hkv, T = 2, 3, 700
    K = rand((B, Hkv, T, 128), dt, 2)
    Kd = K.to(DEV)
    nc_cap = oracle.n_compressed(T)
    Kc = torch.zeros((B, Hkv, nc_cap, 128), dtype=TD[dt], device=DEV)
    schedule = [[0, 0], [31, 5], [32, 40], [47, 47], [48, 48], [49, 64], [100, 99], [101, 100],
                [355, 240], [356, 512], [700, 600]]
    for step in range(1, len(schedule)):
        sa.compress(Kd, Kc, lens_t(schedule[step - 1]), lens_t(schedule[step]), max_new_entries=2)
    final = schedule[-1]
    ref = torch.from_numpy(oracle_kc(K.float().numpy(), final, dt, nc_cap)).to(TD[dt])
    got = Kc.cpu()
    for b in range(B):
        n = oracle.n_compressed(final[b])
        assert torch.equal(got[b, :, :n].view(BITS[dt]), ref[b, :, :n].view(BITS[dt]))


# ------------------------------------------------------------------ select

def _kc_for(K, lens, dt):
    """Compressed keys built by the HIP path (bit-exactness is checked above)."""
    B, Hkv, T, d = K.shape
    Kc = torch.zeros((B, Hkv, oracle.n_compressed(T), d), dtype=K.dtype, device=DEV)
    sa.compress(K, Kc, lens_t([0] * B), lens_t(lens))
    return Kc


def _check_select(sel, K, lens, T_cap, k, n_init, n_local, mode, dt, exact=False):
    Kd = K.to(DEV)
    Kc = _kc_for(Kd, lens, dt)
    idx, cnt, bs = sa.select(sel.to(DEV), Kc, lens_t(lens), T_cap, k, n_init, n_local, mode,
                             block_scores=True)
    rows = gpu_rows(idx, cnt)
    bs = bs.cpu().numpy().astype(np.float64)
    Kc_ref = oracle_kc(K.float().numpy(), lens, dt, Kc.shape[2])
    S = to_np(sel)
    B, Hkv = K.shape[:2]
    Gs = S.shape[1] // Hkv
    p = SelectParams(top_k=k, n_init=n_init, n_local=n_local, score_mode=mode)
    kinds = []
    for b in range(B):
        for h in range(Hkv):
            L = lens[b]
            ref, BS = oracle.select_blocks(S[b, h * Gs:(h + 1) * Gs], Kc_ref[b, h], L, p, True)
            nb = oracle.n_blocks(L)
            if exact:
                assert rows[(b, h)] == ref, (b, h, rows[(b, h)], ref)
                kinds.append("exact")
            else:
                ok, why = selection_ok(rows[(b, h)], ref, BS, nb, k, n_init, n_local)
                assert ok, ((b, h), why, rows[(b, h)], ref)
                kinds.append(why)
            fin = np.isfinite(BS)
            assert np.array_equal(np.isfinite(bs[b, h, :nb]), fin)
            if fin.any():
                scale = np.abs(BS[fin]).max()
                assert np.allclose(bs[b, h, :nb][fin], BS[fin], rtol=2e-5, atol=2e-6 * scale)
            assert np.all(np.isneginf(bs[b, h, nb:]))
    return kinds


@pytest.mark.parametrize("mode,G,dt", [("softmax_sum", 4, "f32"), ("softmax_sum", 4, "bf16"),
                                       ("raw_sum", 4, "bf16"), ("raw_sum", 1, "bf16"),
                                       ("raw_sum", 1, "f32"), ("softmax_sum", 1, "bf16"),
                                       ("softmax_sum", 2, "f32"), ("softmax_sum", 8, "bf16")])
def test_select_parity(mode, G, dt):
    B, Hkv, T = 3, 2, 5000
    lens = [5000, 3333, 700]
    K = rand((B, Hkv, T, 128), dt, 3)
    sel = rand((B, G * Hkv, 128), dt, 4, scale=128 ** -0.5)
    kinds = _check_select(sel, K, lens, T, 16, 1, 2, mode, dt)
    assert kinds.count("exact") >= len(kinds) - 1


@pytest.mark.parametrize("L", [0, 10, 31, 32, 64, 100, 191, 192, 193, 260, 4097])
def test_select_short_and_degenerate_lengths(L):
    dt = "bf16"
    K = rand((2, 2, 4100, 128), dt, 5)
    sel = rand((2, 8, 128), dt, 6, scale=128 ** -0.5)
    lens = [L, min(4100, L + 37)]
    for k in (0, 3, 1000):
        _check_select(sel, K, lens, 4100, k, 1, 2, "softmax_sum", dt)
        _check_select(sel[:, ::4].contiguous(), K, lens, 4100, k, 2, 3, "raw_sum", dt)


def test_select_exact_ties_go_to_lower_index():
    dt = "bf16"
    T = 64 * 40
    K = rand((1, 2, T, 128), dt, 7)
    for h in range(2):
        K[0, h, 64 * 27:64 * 28] = K[0, h, 64 * 9:64 * 10]      # block 27 duplicates block 9
        K[0, h, 64 * 30:64 * 31] = K[0, h, 64 * 9:64 * 10]      # and block 30 too
    mean9 = K[0, :, 64 * 9:64 * 10].float().mean(1)            # [2, 128]
    sel = (mean9 * 0.5).to(TD[dt])[None]                       # one Forecast per KV head
    for k in (1, 2, 3):
        _check_select(sel, K, [T], T, k, 1, 2, "raw_sum", dt, exact=True)
    selq = mean9.repeat_interleave(4, 0)[None].to(TD[dt]) * 0.3
    for k in (1, 2):
        _check_select(selq, K, [T], T, k, 1, 2, "softmax_sum", dt, exact=True)


@pytest.mark.parametrize("mode", ["raw_sum", "softmax_sum"])
@pytest.mark.parametrize("outlier", [False, True])
def test_select_many_exact_ties_at_the_threshold(mode, outlier):
    """Block scores that take four values only (every key of block b is
    v_b * e_0), so the k-th largest sits in a run of ~150 exactly equal
    scores: ties must go to the lower block ids. With one outlier block far
    above the rest, every other score lands in the lowest value bucket and the
    top-k falls back to the exact radix select; without it, the boundary
    bucket is ranked directly."""
    dt = "bf16"
    nb = 600
    T = 64 * nb
    g = torch.Generator().manual_seed(21)
    v = (torch.randint(0, 4, (2, nb), generator=g).float() * 0.25)
    if outlier:
        # far above the rest, yet small enough that the others' softmax terms
        # stay normal fp32 numbers (no underflow to equal zeros)
        v[:, 300] = 1000.0 if mode == "raw_sum" else 40.0
    K = torch.zeros((1, 2, T, 128))
    K[0, :, :, 0] = v.repeat_interleave(64, dim=1)
    K = K.to(TD[dt])
    if mode == "raw_sum":
        sel = torch.zeros((1, 2, 128))
        sel[..., 0] = 1.0
    else:
        sel = torch.zeros((1, 8, 128))
        sel[..., 0] = 0.5
    for k in (1, 100, 300):
        _check_select(sel.to(TD[dt]), K, [T], T, k, 1, 2, mode, dt, exact=True)


@pytest.mark.parametrize("mode", ["raw_sum", "softmax_sum"])
@pytest.mark.parametrize("pattern", ["four_values", "outlier", "all_equal"])
def test_select_ties_on_a_grid_of_many_units(mode, pattern):
    """1024 (sequence, KV head) units, the grid size from which the top-k
    buckets candidates by value before ranking: exact ties at the threshold
    (four score values), one far outlier, and all scores equal (a range that
    does not bucket, handled by the radix select). Sampled units are compared
    with the oracle exactly; every unit's count is checked."""
    dt = "bf16"
    B, Hkv, nb = 512, 2, 40
    T = 64 * nb
    g = torch.Generator().manual_seed(22)
    if pattern == "all_equal":
        v = torch.full((B, Hkv, nb), 0.5)
    else:
        v = torch.randint(0, 4, (B, Hkv, nb), generator=g).float() * 0.25
        if pattern == "outlier":
            v[:, :, 17] = 1000.0 if mode == "raw_sum" else 40.0
    K = torch.zeros((B, Hkv, T, 128), dtype=TD[dt])
    K[..., 0] = v.repeat_interleave(64, dim=2).to(TD[dt])
    G = 1 if mode == "raw_sum" else 4
    sel = torch.zeros((B, Hkv * G, 128))
    sel[..., 0] = 1.0 if mode == "raw_sum" else 0.5
    sel = sel.to(TD[dt])
    Kd = K.to(DEV)
    Kc = _kc_for(Kd, [T] * B, dt)
    S = to_np(sel)
    sampled = list(range(0, B, 37))
    Kc_ref = {b: oracle_kc(K[b:b + 1].float().numpy(), [T], dt, Kc.shape[2])[0] for b in sampled}
    for k in (1, 10, 20):
        idx, cnt, _ = sa.select(sel.to(DEV), Kc, lens_t([T] * B), T, k, 1, 2, mode)
        assert torch.all(cnt.cpu() == k + 3)
        rows = gpu_rows(idx, cnt)
        p = SelectParams(top_k=k, n_init=1, n_local=2, score_mode=mode)
        for b in sampled:
            for h in range(Hkv):
                ref = oracle.select_blocks(S[b, h * G:(h + 1) * G], Kc_ref[b][h], T, p)
                assert rows[(b, h)] == ref, (pattern, k, b, h, rows[(b, h)], ref)


# ------------------------------------------------------------------ decode

def _decode_case(dt, lens, T_cap, blocks_of, n_split, out=torch.float32, seed=10, G=4):
    B, Hkv = len(lens), 2
    Hq = G * Hkv
    Q = rand((B, Hq, 128), dt, seed, scale=128 ** -0.5)
    K = rand((B, Hkv, T_cap, 128), dt, seed + 1)
    V = rand((B, Hkv, T_cap, 128), dt, seed + 2)
    cap = max(1, max(len(v) for v in blocks_of.values()))
    idx = torch.full((B, Hkv, cap), -1, dtype=torch.int32)
    cnt = torch.zeros((B, Hkv), dtype=torch.int32)
    for (b, h), blk in blocks_of.items():
        idx[b, h, :len(blk)] = torch.tensor(blk, dtype=torch.int32)
        cnt[b, h] = len(blk)
    O, lse = sa.decode(Q.to(DEV), K.to(DEV), V.to(DEV), lens_t(lens), idx.to(DEV), cnt.to(DEV),
                       1.0, out_dtype=out, n_split=n_split)
    Qn, Kn, Vn = to_np(Q), to_np(K), to_np(V)
    On, Ln = to_np(O), lse.cpu().numpy()
    for (b, h), blk in blocks_of.items():
        rows = slice(G * h, G * h + G)
        o, l = oracle.sparse_attention(Qn[b, rows], Kn[b, h], Vn[b, h],
                                       block_tokens(blk, lens[b]), 1.0)
        if len(blk) == 0 or block_tokens(blk, lens[b]).size == 0:
            assert np.all(On[b, rows] == 0) and np.all(np.isneginf(Ln[b, rows]))
            continue
        if out == torch.float32:
            assert_close(On[b, rows], o, dt, f"O unit {(b, h)}")
        else:
            assert np.allclose(On[b, rows], o, atol=TOL[dt][0] + 2e-2, rtol=1e-2)
        assert_close(Ln[b, rows], l, dt, f"LSE unit {(b, h)}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n_split", [1, 3, 0, 40])
def test_decode_parity(dt, n_split):
    lens = [5000, 3333, 70]
    rng = np.random.default_rng(11)
    blocks_of = {}
    for b, L in enumerate(lens):
        nb = oracle.n_blocks(L)
        for h in range(2):
            n = min(nb, 19)
            pick = sorted(rng.choice(nb, size=n, replace=False).tolist())
            if nb - 1 not in pick:
                pick[-1] = nb - 1                  # the partial last block is always attended
                pick = sorted(set(pick))
            blocks_of[(b, h)] = pick
    blocks_of[(2, 1)] = []                          # a unit with nothing selected
    _decode_case(dt, lens, 5000, blocks_of, n_split)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("G", [1, 2, 8])
@pytest.mark.parametrize("n_split", [1, 0, 5])
def test_decode_parity_other_gqa_ratios(dt, G, n_split):
    """G query heads per KV head (Eq. 5 with the group's heads sharing the KV
    head's blocks), for G = 1, 2 and 8."""
    lens = [5000, 3333, 70]
    rng = np.random.default_rng(12 + G)
    blocks_of = {}
    for b, L in enumerate(lens):
        nb = oracle.n_blocks(L)
        for h in range(2):
            pick = sorted(set(rng.choice(nb, size=min(nb, 23), replace=False).tolist()) | {nb - 1})
            blocks_of[(b, h)] = pick
    blocks_of[(2, 1)] = []
    _decode_case(dt, lens, 5000, blocks_of, n_split, G=G, seed=40 + G)
    if dt == "bf16":
        _decode_case(dt, lens, 5000, blocks_of, n_split, out=torch.bfloat16, G=G, seed=50 + G)


def test_decode_unsorted_blocks_and_bf16_output():
    lens = [4096, 1000]
    blocks_of = {(0, 0): [63, 0, 17, 5], (0, 1): [1, 2, 3], (1, 0): [15, 2, 0], (1, 1): [0]}
    _decode_case("bf16", lens, 4096, blocks_of, 2)
    _decode_case("bf16", lens, 4096, blocks_of, 0, out=torch.bfloat16)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_select_then_decode_dense_limit_equals_dense_attention(dt):
    """With top-k covering every block the path is dense attention (torch SDPA on CPU, fp64)."""
    B, Hq, Hkv, T = 2, 8, 2, 2000
    lens = [2000, 1234]
    Q = rand((B, Hq, 128), dt, 20, scale=128 ** -0.5)
    K = rand((B, Hkv, T, 128), dt, 21)
    V = rand((B, Hkv, T, 128), dt, 22)
    Kd = K.to(DEV)
    Kc = _kc_for(Kd, lens, dt)
    k = oracle.n_blocks(T)
    idx, cnt, _ = sa.select(Q.to(DEV), Kc, lens_t(lens), T, k, 1, 2, "softmax_sum")
    O, _ = sa.decode(Q.to(DEV), Kd, V.to(DEV), lens_t(lens), idx, cnt, 1.0)
    for b in range(B):
        L = lens[b]
        assert cnt[b].tolist() == [oracle.n_blocks(L)] * Hkv
        for h in range(Hkv):
            q = Q[b, 4 * h:4 * h + 4].double()[None, :, None]
            kk = K[b, h, :L].double()[None, None].expand(1, 4, -1, -1)
            vv = V[b, h, :L].double()[None, None].expand(1, 4, -1, -1)
            ref = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, scale=1.0)[0, :, 0]
            assert_close(to_np(O[b, 4 * h:4 * h + 4]), ref.numpy(), dt, "dense limit")


# ------------------------------------------------------------------ graph replay

def test_graph_replay_matches_eager_step():
    """A captured decode step replays to the same bits as the eager step, replay after
    replay, with eager work and synchronisations in between."""
    import synth
    from block_sparse_attention_12_amd.pipeline import SparseDecoder
    w = synth.scaled(synth.WORKLOADS["decode_forecast_bf16_128k"], B=2, T=8192)
    inp = synth.make_decode_inputs(w, device=DEV)
    lens = inp["seq_lens"]
    prev = lens - 1
    dec = SparseDecoder(w.B, w.Hq, w.Hkv, w.T, w.top_k, w.n_init, w.n_local, w.selector,
                        w.score_mode)
    Kc = dec.new_kc(inp["K"].dtype)
    dec.build(inp["K"], Kc, prev)
    dec.step(inp["Q"], inp["F"], inp["K"], inp["V"], Kc, prev, lens)
    torch.cuda.synchronize()
    ref_O, ref_idx, ref_kc = dec.O.clone(), dec.idx.clone(), Kc.clone()
    g = dec.capture(lambda: dec.step(inp["Q"], inp["F"], inp["K"], inp["V"], Kc, prev, lens))
    for r in range(4):
        dec.O.zero_()
        dec.idx.fill_(-7)
        Kc[:, :, -1].zero_()                   # the appended entry is rewritten by each replay
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dec.idx, ref_idx), r
        assert torch.equal(dec.O, ref_O), r
        assert torch.equal(Kc, ref_kc), r
        _ = (inp["Q"].float() * 2).sum().item()  # unrelated eager work between replays


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (1 << 24) + 16 * 777])
def test_stream_read_xor_matches_host(nbytes):
    """The stream-read measurement kernel reads every word exactly once: the XOR
    of its per-workgroup words equals the XOR of the buffer."""
    g = torch.Generator().manual_seed(nbytes)
    host = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), generator=g, dtype=torch.int32)
    out = sa.stream_read(host.to("cuda"))
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert got == want


@pytest.mark.parametrize("mode,G", [("softmax_sum", 4), ("raw_sum", 1)])
def test_select_and_decode_at_the_largest_block_count(mode, G):
    """2^21 tokens: 32768 blocks, the largest block count the selection takes
    (1024 threads x 32 blocks per top-k workgroup), one (sequence, KV head)."""
    dt = "bf16"
    T = 64 * 32768
    g = torch.Generator(device=DEV).manual_seed(31)
    K = torch.randn((1, 1, T, 128), generator=g, device=DEV).to(torch.bfloat16)
    V = torch.randn((1, 1, T, 128), generator=g, device=DEV).to(torch.bfloat16)
    Q = (torch.randn((1, 4, 128), generator=g, device=DEV) * 128 ** -0.5).to(torch.bfloat16)
    sel = Q if G == 4 else (torch.randn((1, 1, 128), generator=g, device=DEV) * 128 ** -0.5).to(torch.bfloat16)
    L = T - 37
    Kc = torch.zeros((1, 1, oracle.n_compressed(T), 128), dtype=torch.bfloat16, device=DEV)
    sa.compress(K, Kc, lens_t([0]), lens_t([L]))
    k = 64
    idx, cnt, bs = sa.select(sel, Kc, lens_t([L]), T, k, 1, 2, mode, block_scores=True)
    O, lse = sa.decode(Q, K, V, lens_t([L]), idx, cnt, 1.0)
    rows = gpu_rows(idx, cnt)
    Kn = K[0, 0].float().cpu().numpy()
    Kc_ref = oracle.compressed_keys(Kn, L, dt)
    assert np.array_equal(Kc[0, 0, :Kc_ref.shape[0]].float().cpu().numpy(), Kc_ref)
    p = SelectParams(top_k=k, n_init=1, n_local=2, score_mode=mode)
    ref, BS = oracle.select_blocks(to_np(sel)[0], Kc_ref, L, p, True)
    nb = oracle.n_blocks(L)
    ok, why = selection_ok(rows[(0, 0)], ref, BS, nb, k, 1, 2)
    assert ok, (why, rows[(0, 0)][:10], ref[:10])
    got_bs = bs[0, 0, :nb].cpu().numpy().astype(np.float64)
    fin = np.isfinite(BS)
    assert np.array_equal(np.isfinite(got_bs), fin)
    scale = np.abs(BS[fin]).max()
    assert np.allclose(got_bs[fin], BS[fin], rtol=2e-5, atol=2e-6 * scale)
    o, l = oracle.sparse_attention(to_np(Q)[0], Kn, V[0, 0].float().cpu().numpy(),
                                   block_tokens(rows[(0, 0)], L), 1.0)
    assert_close(to_np(O)[0], o, dt, "O")
    assert_close(lse.cpu().numpy()[0], l, dt, "LSE")
