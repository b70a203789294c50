"""GPU parity of the token-level index (sparse_attn_token_select) and of
attention over token lists (sparse_attn_token_decode) against oracle.token.

Token scores: within a bound of the fp32 rounding of each score. Token sets:
exact (ties to the lower token), except inside that rounding band around the
k-th score. Attention: elementwise tolerance on the GPU's own token sets.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_12_amd as sa
import oracle
from parity import assert_close, to_np, token_selection_ok, gpu_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"
TD = {"f32": torch.float32, "bf16": torch.bfloat16}


def rand(shape, dt, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g) * scale).to(TD[dt])


def lens_t(lens):
    return torch.tensor(lens, dtype=torch.int32, device=DEV)


def _score_bound(sel_sum, Ki_unit, L):
    """fp32 rounding bound of each token's score: 2e-6 * sum_c |sel_c * Ki_tc|."""
    return 2e-6 * (np.abs(Ki_unit[:L].astype(np.float64)) @ np.abs(sel_sum.astype(np.float64))) + 1e-30


def _check_token_select(sel, Ki, lens, k, n_init, n_local, exact=False, units=None):
    B, Hkv, T_cap, di = Ki.shape
    Gs = sel.shape[1] // Hkv
    idx, cnt, sc = sa.token_select(sel.to(DEV), Ki.to(DEV), lens_t(lens), k, n_init, n_local,
                                   scores=True)
    rows = gpu_rows(idx, cnt)
    S = to_np(sel)
    Kn = to_np(Ki)
    scn = sc.cpu().numpy().astype(np.float64)
    units = units if units is not None else [(b, h) for b in range(B) for h in range(Hkv)]
    kinds = []
    for (b, h) in units:
        L = lens[b]
        ref, s = oracle.select_tokens(S[b, h * Gs:(h + 1) * Gs], Kn[b, h], L, k, n_init, n_local,
                                      return_scores=True)
        bound = _score_bound(S[b, h * Gs:(h + 1) * Gs].sum(0), Kn[b, h], L)
        assert np.all(np.abs(scn[b, h, :L] - s) <= bound), (b, h, np.abs(scn[b, h, :L] - s).max())
        assert np.all(np.isneginf(scn[b, h, L:]))
        if exact:
            assert rows[(b, h)] == ref, (b, h, rows[(b, h)][:20], ref[:20])
            kinds.append("exact")
        else:
            _, _, cand = oracle.token_candidates(L, n_init, n_local)
            ok, why = token_selection_ok(rows[(b, h)], ref, s, bound, k, cand)
            assert ok, ((b, h), why)
            kinds.append(why)
    return kinds, idx, cnt


@pytest.mark.parametrize("dt,di,Gs", [("bf16", 64, 1), ("bf16", 128, 1), ("bf16", 128, 4),
                                      ("f32", 64, 1), ("f32", 128, 4)])
def test_token_select_parity(dt, di, Gs):
    B, Hkv, T = 3, 2, 10000
    lens = [10000, 4097, 300]
    Ki = rand((B, Hkv, T, di), dt, 1)
    sel = rand((B, Hkv * Gs, di), dt, 2, scale=di ** -0.5)
    kinds, _, _ = _check_token_select(sel, Ki, lens, 500, 64, 128)
    assert kinds.count("exact") >= len(kinds) - 1


@pytest.mark.parametrize("k", [0, 1, 37, 4095, 4096, 20000])
def test_token_select_lengths_at_chunk_edges(k):
    """Lengths on and around the 4096-token chunk edges, tiny and empty
    lengths, k = 0 and k covering every candidate."""
    dt, di = "bf16", 64
    lens = [0, 1, 100, 192, 193, 4096, 4097, 8192, 8191, 12289]
    B, Hkv = len(lens), 2
    T = 12289
    Ki = rand((B, Hkv, T, di), dt, 3)
    sel = rand((B, Hkv, di), dt, 4, scale=0.125)
    _check_token_select(sel, Ki, lens, k, 64, 128)


def test_token_select_exact_ties_and_integer_scores():
    """Index keys and selectors of small integers: every score is an exact
    integer in fp32, with many equal scores, so the sets must match the
    oracle exactly (ties to the lower token index), also across chunks."""
    B, Hkv, T, di = 2, 2, 9000, 64
    g = torch.Generator().manual_seed(5)
    Ki = torch.randint(-2, 3, (B, Hkv, T, di), generator=g).to(torch.bfloat16)
    sel = torch.randint(-1, 2, (B, Hkv, di), generator=g).to(torch.bfloat16)
    for k in (1, 50, 700, 3000):
        _check_token_select(sel, Ki, [9000, 5000], k, 16, 32, exact=True)
    # a group of 4 query-head selectors (summed)
    selq = torch.randint(-1, 2, (B, Hkv * 4, di), generator=g).to(torch.bfloat16)
    _check_token_select(selq, Ki, [8999, 4096], 333, 0, 0, exact=True)


def test_token_select_one_value_everywhere():
    """All candidate scores equal: the top-k is the lowest candidate ids."""
    B, Hkv, T, di = 1, 2, 5000, 64
    Ki = torch.ones((B, Hkv, T, di), dtype=torch.bfloat16)
    sel = torch.ones((B, Hkv, di), dtype=torch.bfloat16)
    kinds, idx, cnt = _check_token_select(sel, Ki, [5000], 100, 10, 20, exact=True)
    rows = gpu_rows(idx, cnt)
    assert rows[(0, 0)] == list(range(0, 110)) + list(range(4980, 5000))


def test_token_select_many_units_sampled():
    B, Hkv, T, di = 64, 8, 6000, 64
    lens = [6000 - 37 * b for b in range(B)]
    Ki = rand((B, Hkv, T, di), "bf16", 6)
    sel = rand((B, Hkv, di), "bf16", 7, scale=0.125)
    units = [(b, h) for b in range(0, B, 9) for h in (0, 5)]
    kinds, _, _ = _check_token_select(sel, Ki, lens, 256, 64, 128, units=units)
    assert kinds.count("exact") >= len(kinds) - 1


# ------------------------------------------------------------------ attention over token lists

def _token_decode_case(dt, lens, T_cap, lists, n_split, out=torch.float32, seed=20, G=4):
    B, Hkv = len(lens), 2
    Hq = G * Hkv
    Q = rand((B, Hq, 128), dt, seed, scale=128 ** -0.5)
    K = rand((B, Hkv, T_cap, 128), dt, seed + 1)
    V = rand((B, Hkv, T_cap, 128), dt, seed + 2)
    cap = max(1, max(len(v) for v in lists.values()))
    idx = torch.full((B, Hkv, cap), -1, dtype=torch.int32)
    cnt = torch.zeros((B, Hkv), dtype=torch.int32)
    for (b, h), toks in lists.items():
        idx[b, h, :len(toks)] = torch.tensor(toks, dtype=torch.int32)
        cnt[b, h] = len(toks)
    O, lse = sa.token_decode(Q.to(DEV), K.to(DEV), V.to(DEV), lens_t(lens), idx.to(DEV), cnt.to(DEV),
                             1.0, out_dtype=out, n_split=n_split)
    Qn, Kn, Vn = to_np(Q), to_np(K), to_np(V)
    On, Ln = to_np(O), lse.cpu().numpy()
    for (b, h), toks in lists.items():
        valid = [t for t in toks if 0 <= t < lens[b]]
        rows = slice(G * h, G * h + G)
        o, l = oracle.token_decode_unit(Qn[b, rows], Kn[b, h], Vn[b, h], valid, 1.0)
        if not valid:
            assert np.all(On[b, rows] == 0) and np.all(np.isneginf(Ln[b, rows]))
            continue
        assert_close(On[b, rows], o, dt if out == torch.float32 else "bf16", f"O unit {(b, h)}")
        assert_close(Ln[b, rows], l, dt, f"LSE unit {(b, h)}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n_split", [0, 1, 3, 8])
def test_token_decode_parity(dt, n_split):
    rng = np.random.default_rng(30)
    lens = [3000, 1234, 70]
    T_cap = 3000
    lists = {}
    for b, L in enumerate(lens):
        for h in range(2):
            n = [700, 130, 64][b] if h == 0 else [1, 65, 70][b]
            toks = rng.choice(L, size=min(n, L), replace=False).tolist()
            lists[(b, h)] = toks                                    # unsorted on purpose
    _token_decode_case(dt, lens, T_cap, lists, n_split)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("G", [1, 2, 8])
def test_token_decode_other_gqa_ratios(dt, G):
    rng = np.random.default_rng(31 + G)
    lens = [3000, 1234, 70]
    lists = {}
    for b, L in enumerate(lens):
        for h in range(2):
            n = [700, 130, 64][b] if h == 0 else [1, 65, 70][b]
            lists[(b, h)] = rng.choice(L, size=min(n, L), replace=False).tolist()
    _token_decode_case(dt, lens, 3000, lists, 0, G=G, seed=60 + G)
    _token_decode_case(dt, lens, 3000, lists, 3, G=G, seed=70 + G)


def test_token_decode_ignores_out_of_range_and_empty_lists():
    lens = [500, 200]
    lists = {(0, 0): [5, 499, 500, 10_000, -1, 7], (0, 1): [], (1, 0): [199, 0, 250],
             (1, 1): [300, 400]}
    _token_decode_case("bf16", lens, 600, lists, 0, out=torch.bfloat16)


def test_token_select_then_decode_shared_by_layers():
    """One index from the anchor's selector serves three layers (CLSA)."""
    B, Hq, Hkv, T, di = 2, 8, 2, 7000, 64
    lens = [7000, 5000]
    dt = "bf16"
    Ki = rand((B, Hkv, T, di), dt, 40)
    sel = rand((B, Hkv, di), dt, 41, scale=0.125)
    layers = [dict(Q=rand((B, Hq, 128), dt, 50 + l, scale=128 ** -0.5),
                   K=rand((B, Hkv, T, 128), dt, 60 + l), V=rand((B, Hkv, T, 128), dt, 70 + l))
              for l in range(3)]
    idx, cnt, _ = sa.token_select(sel.to(DEV), Ki.to(DEV), lens_t(lens), 600, 64, 128)
    rows = gpu_rows(idx, cnt)
    nl = [{k: to_np(v) for k, v in lay.items()} for lay in layers]
    toks_ref, outs, lses = oracle.token_crosslayer_step(nl, to_np(sel), to_np(Ki), lens, 600, 64,
                                                        128, 1.0)
    for u in rows:
        ok, why = token_selection_ok(rows[u], toks_ref[u], oracle.token_scores(
            to_np(sel)[u[0], u[1]:u[1] + 1], to_np(Ki)[u[0], u[1]], lens[u[0]]),
            _score_bound(to_np(sel)[u[0], u[1]], to_np(Ki)[u[0], u[1]], lens[u[0]]), 600,
            oracle.token_candidates(lens[u[0]], 64, 128)[2])
        assert ok, (u, why)
    for l, lay in enumerate(layers):
        O, lse = sa.token_decode(lay["Q"].to(DEV), lay["K"].to(DEV), lay["V"].to(DEV), lens_t(lens),
                                 idx, cnt, 1.0)
        On = to_np(O)
        for (b, h), toks in rows.items():
            o, _ = oracle.token_decode_unit(nl[l]["Q"][b, 4 * h:4 * h + 4], nl[l]["K"][b, h],
                                            nl[l]["V"][b, h], toks, 1.0)
            assert_close(On[b, 4 * h:4 * h + 4], o, dt, f"layer {l} unit {(b, h)}")
