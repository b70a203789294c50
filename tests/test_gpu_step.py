"""sparse_attn_decode_step (append + select + attend in one call) against the
three separate calls it stands for: identical block sets, identical outputs,
identical compressed keys afterwards. Covers the raw-sum path, where the
append shares the scoring launch and the scorer forms new entries from the
keys, with jumps that put new entries inside candidate blocks."""
import pytest
import torch

import block_sparse_attention_12_amd as sa
from parity import gpu_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"
TD = {"f32": torch.float32, "bf16": torch.bfloat16}
BITS = {"f32": torch.int32, "bf16": torch.int16}


def rand(shape, dt, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g) * scale).to(TD[dt]).to(DEV)


def lens_t(lens):
    return torch.tensor(lens, dtype=torch.int32, device=DEV)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("mode,G", [("raw_sum", 1), ("raw_sum", 4), ("softmax_sum", 4)])
@pytest.mark.parametrize("n_local", [2, 1, 0])
def test_decode_step_equals_separate_calls(dt, mode, G, n_local):
    B, Hq, Hkv, T = 3, 8, 2, 6000
    K = rand((B, Hkv, T, 128), dt, 1)
    V = rand((B, Hkv, T, 128), dt, 2)
    nc_cap = sa.n_compressed(T)
    # (lens_prev, lens_now) per step: single tokens across window / block edges,
    # and jumps whose new entries land inside candidate blocks
    steps = [([2000, 511, 64], [2001, 512, 65]), ([2001, 512, 65], [2016, 528, 96]),
             ([2016, 528, 96], [2600, 1500, 97]), ([2600, 1500, 97], [6000, 1501, 700])]
    Kc_a = torch.zeros((B, Hkv, nc_cap, 128), dtype=TD[dt], device=DEV)
    Kc_b = torch.zeros_like(Kc_a)
    first = lens_t(steps[0][0])
    sa.compress(K, Kc_a, lens_t([0] * B), first)
    sa.compress(K, Kc_b, lens_t([0] * B), first)
    k = 24
    for i, (lp, ln) in enumerate(steps):
        Q = rand((B, Hq, 128), dt, 10 + i, scale=128 ** -0.5)
        sel = Q if G == 4 else rand((B, Hkv, 128), dt, 20 + i, scale=128 ** -0.5)
        Lp, Ln = lens_t(lp), lens_t(ln)
        mx = max(b - a for a, b in zip(lp, ln))
        O1, lse1, idx1, cnt1 = sa.decode_step(Q, sel, K, V, Kc_a, Lp, Ln, k, 1, n_local, mode,
                                              max_new_tokens=mx)
        sa.compress(K, Kc_b, Lp, Ln, max_new_entries=mx // 16 + 2)
        idx2, cnt2, _ = sa.select(sel, Kc_b, Ln, T, k, 1, n_local, mode)
        O2, lse2 = sa.decode(Q, K, V, Ln, idx2, cnt2, 1.0)
        torch.cuda.synchronize()
        assert gpu_rows(idx1, cnt1) == gpu_rows(idx2, cnt2), (i, mode)
        assert torch.equal(O1, O2) and torch.equal(lse1, lse2), (i, mode)
        assert torch.equal(Kc_a.view(BITS[dt]), Kc_b.view(BITS[dt])), (i, "compressed keys")


def test_decode_step_validation_and_workspace():
    p = sa.make_params(16, 1, 2, "raw_sum")
    need = sa.decode_step_workspace_size(2, 8, 2, 2, 4096, p, 19, 4)
    assert need >= sa.select_workspace_size(2, 2, 2, 4096, p) + sa.decode_workspace_size(2, 8, 2, 19, 4)
    Q = torch.zeros((2, 8, 128), dtype=torch.bfloat16, device=DEV)
    K = torch.zeros((2, 2, 4096, 128), dtype=torch.bfloat16, device=DEV)
    Kc = torch.zeros((2, 2, sa.n_compressed(4096), 128), dtype=torch.bfloat16, device=DEV)
    L = lens_t([4096, 100])
    with pytest.raises(sa.SparseAttnError):
        sa.decode_step(Q, Q[:, :3].contiguous(), K, K, Kc, L, L, 16, 1, 2, "raw_sum")   # H_sel 3
    with pytest.raises(sa.SparseAttnError):
        sa.decode_step(Q, Q, K, K, Kc, L, L, 16, 1, 2, "raw_sum",
                       workspace=torch.empty(16, dtype=torch.uint8, device=DEV))


# Up to 2048 blocks and 1024 list entries, the attention workgroups take their
# unit's top-k themselves from the block scores; past either limit, and for 8
# selector heads a group in the softmax-sum form, a separate top-k launch does.
# Both sides must give the separate calls' sets and outputs bit for bit.
@pytest.mark.parametrize("case", [
    dict(mode="raw_sum", G=1, B=1, Hkv=2, T=64 * 2048, lens=[64 * 2048], k=1000, n_split=0),
    dict(mode="softmax_sum", G=4, B=2, Hkv=2, T=64 * 2048, lens=[64 * 2048 - 5, 3000], k=1021,
         n_split=7),
    dict(mode="raw_sum", G=1, B=1, Hkv=2, T=64 * 2048 + 1, lens=[64 * 2048 + 1], k=100, n_split=0),
    dict(mode="softmax_sum", G=4, B=1, Hkv=2, T=70000, lens=[70000], k=1022, n_split=3),
    dict(mode="softmax_sum", G=8, B=2, Hkv=2, T=6000, lens=[6000, 777], k=40, n_split=0),
    dict(mode="softmax_sum", G=2, B=2, Hkv=2, T=6000, lens=[6000, 0], k=40, n_split=1),
    dict(mode="softmax_sum", G=1, B=3, Hkv=2, T=9000, lens=[9000, 4100, 70], k=30, n_split=0),
    dict(mode="raw_sum", G=4, B=2, Hkv=2, T=9000, lens=[8999, 64], k=30, n_split=5, dt="f32"),
    dict(mode="raw_sum", G=1, B=128, Hkv=8, T=2000, lens=None, k=12, n_split=0),
    dict(mode="softmax_sum", G=4, B=128, Hkv=8, T=2000, lens=None, k=12, n_split=2),
], ids=["raw-2048blk-k1000", "soft-2048blk-cap1024", "raw-2049blk", "soft-cap1025",
        "soft-G8", "soft-G2-empty", "soft-G1", "raw-G4-f32", "raw-1024units", "soft-1024units"])
def test_decode_step_fused_and_separate_topk(case):
    dt = case.get("dt", "bf16")
    B, Hkv, T, G, k = case["B"], case["Hkv"], case["T"], case["G"], case["k"]
    Hq = 4 * Hkv
    lens = case["lens"] or [T - 13 * b for b in range(B)]
    K = rand((B, Hkv, T, 128), dt, 31)
    V = rand((B, Hkv, T, 128), dt, 32)
    Q = rand((B, Hq, 128), dt, 33, scale=128 ** -0.5)
    sel = Q if G == 4 else rand((B, Hkv * G, 128), dt, 34, scale=128 ** -0.5)
    nc_cap = sa.n_compressed(T)
    lp = [max(0, L - 1) for L in lens]
    Kc_a = torch.zeros((B, Hkv, nc_cap, 128), dtype=TD[dt], device=DEV)
    sa.compress(K, Kc_a, lens_t([0] * B), lens_t(lp))
    Kc_b = Kc_a.clone()
    Lp, Ln = lens_t(lp), lens_t(lens)
    O1, lse1, idx1, cnt1 = sa.decode_step(Q, sel, K, V, Kc_a, Lp, Ln, k, 1, 2, case["mode"],
                                          n_split=case["n_split"])
    sa.compress(K, Kc_b, Lp, Ln)
    idx2, cnt2, _ = sa.select(sel, Kc_b, Ln, T, k, 1, 2, case["mode"])
    O2, lse2 = sa.decode(Q, K, V, Ln, idx2, cnt2, 1.0, n_split=case["n_split"])
    torch.cuda.synchronize()
    assert torch.equal(idx1, idx2) and torch.equal(cnt1, cnt2)
    assert torch.equal(O1, O2) and torch.equal(lse1, lse2)
    assert torch.equal(Kc_a.view(BITS[dt]), Kc_b.view(BITS[dt]))


def test_decode_step_random_configurations():
    """Seeded random shapes, lengths, budgets and modes: the one-call step and
    the three separate calls agree bit for bit (sets, outputs, compressed keys)."""
    import random
    rng = random.Random(2024)
    for trial in range(12):
        dt = rng.choice(["bf16", "bf16", "f32"])
        mode, G = rng.choice([("raw_sum", 1), ("raw_sum", 4), ("softmax_sum", 4), ("softmax_sum", 1),
                              ("softmax_sum", 2), ("softmax_sum", 8)])
        B, Hkv = rng.randint(1, 4), rng.choice([1, 2, 4])
        T = rng.choice([700, 3000, 9000, 20000, 64 * 2048])
        n_init, n_local = rng.randint(0, 3), rng.randint(0, 4)
        k = rng.choice([0, 1, 7, 30, 200])
        if k + n_init + n_local == 0:
            n_local = 1                                  # a set of capacity 0 is not a call
        n_split = rng.choice([0, 0, 1, 3])
        new = rng.choice([1, 1, 5, 40])
        lens = [rng.randint(0, T) for _ in range(B)]
        lp = [max(0, L - rng.randint(0, new)) for L in lens]
        K = rand((B, Hkv, T, 128), dt, 100 + trial)
        V = rand((B, Hkv, T, 128), dt, 200 + trial)
        Q = rand((B, 4 * Hkv, 128), dt, 300 + trial, scale=128 ** -0.5)
        sel = Q if G == 4 else rand((B, Hkv * G, 128), dt, 400 + trial, scale=128 ** -0.5)
        nc_cap = sa.n_compressed(T)
        Kc_a = torch.zeros((B, Hkv, nc_cap, 128), dtype=TD[dt], device=DEV)
        sa.compress(K, Kc_a, lens_t([0] * B), lens_t(lp))
        Kc_b = Kc_a.clone()
        Lp, Ln = lens_t(lp), lens_t(lens)
        mx = max(b - a for a, b in zip(lp, lens))
        case = (trial, dt, mode, G, B, Hkv, T, n_init, n_local, k, n_split, lens, lp)
        print("case", case, flush=True)
        O1, lse1, idx1, cnt1 = sa.decode_step(Q, sel, K, V, Kc_a, Lp, Ln, k, n_init, n_local, mode,
                                              max_new_tokens=mx, n_split=n_split)
        sa.compress(K, Kc_b, Lp, Ln, max_new_entries=mx // 16 + 2)
        idx2, cnt2, _ = sa.select(sel, Kc_b, Ln, T, k, n_init, n_local, mode)
        O2, lse2 = sa.decode(Q, K, V, Ln, idx2, cnt2, 1.0, n_split=n_split)
        torch.cuda.synchronize()
        assert torch.equal(idx1, idx2) and torch.equal(cnt1, cnt2), case
        assert torch.equal(O1, O2) and torch.equal(lse1, lse2), case
        assert torch.equal(Kc_a.view(BITS[dt]), Kc_b.view(BITS[dt])), case
