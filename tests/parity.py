"""Comparison rules shared by the GPU parity tests (HIP path vs. the CPU oracle).

Selected blocks must match the oracle exactly (ties toward the lower block
index), except when the oracle's k-th and (k+1)-th candidate scores differ by
less than 1e-5 relative: then any set is accepted whose differing blocks all
score within 1e-5 relative of the k-th. Attention outputs are checked against
the oracle's attention over the GPU's own block sets, elementwise as
|gpu - oracle| <= atol + rtol * |oracle|, with (atol, rtol) = (2e-3, 1e-2) for
bf16 inputs and (1e-5, 1e-5) for fp32 inputs.
"""
import numpy as np
import torch

import oracle

TOL = {"bf16": (2e-3, 1e-2), "f32": (1e-5, 1e-5)}
NEAR_TIE = 1e-5


def rel_close(a, b, tol=NEAR_TIE):
    return abs(a - b) <= tol * max(abs(a), abs(b))


def selection_ok(gpu_blocks, ref_blocks, BS, nb, k, n_init, n_local):
    """True if the GPU's block set is acceptable under the exact/near-tie rule."""
    gpu_blocks = list(gpu_blocks)
    if gpu_blocks == list(ref_blocks):
        return True, "exact"
    _, _, cand = oracle.candidate_sets(nb, n_init, n_local)
    if len(cand) <= k or k <= 0:
        return False, "mismatch with no tie possible"
    order = oracle.top_k_blocks(BS, cand, len(cand))
    s_k, s_k1 = BS[order[k - 1]], BS[order[k]]
    if not rel_close(s_k, s_k1):
        return False, f"mismatch, k-th/(k+1)-th gap not a near tie ({s_k} vs {s_k1})"
    if len(gpu_blocks) != len(ref_blocks) or gpu_blocks != sorted(set(gpu_blocks)):
        return False, "near tie but wrong size or order"
    diff = set(gpu_blocks) ^ set(ref_blocks)
    if all(rel_close(BS[b], s_k) for b in diff):
        return True, "near tie"
    return False, "near tie but a differing block is outside the band"


def gpu_rows(idx: torch.Tensor, cnt: torch.Tensor):
    """{(b, kvh): list of blocks} from device idx/cnt, checking the -1 padding."""
    I = idx.cpu().numpy()
    C = cnt.cpu().numpy()
    out = {}
    for b in range(I.shape[0]):
        for h in range(I.shape[1]):
            n = int(C[b, h])
            row = I[b, h]
            assert np.all(row[n:] == -1), f"padding of ({b},{h}) not -1"
            out[(b, h)] = row[:n].tolist()
    return out


def assert_close(gpu, ref, dtype, what=""):
    atol, rtol = TOL[dtype]
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(gpu - ref)
    bad = err > atol + rtol * np.abs(ref)
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside tolerance; max abs err "
                           f"{err.max():.3e} at {np.unravel_index(err.argmax(), err.shape)}")
    return float(err.max()) if err.size else 0.0


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def oracle_kc(K: np.ndarray, lens, dtype, nc_cap):
    """Oracle compressed keys for every unit: [B, Hkv, nc_cap, d] (zeros past n_c(L))."""
    B, Hkv, _, d = K.shape
    out = np.zeros((B, Hkv, nc_cap, d), dtype=np.float32)
    for b in range(B):
        for h in range(Hkv):
            c = oracle.compressed_keys(K[b, h], int(lens[b]), dtype)
            out[b, h, :c.shape[0]] = c
    return out


def tile_union_ok(gpu_union, ref_union, per_query, k, cand):
    """Tile block sets: exact, or every differing block is inside some query's
    near-tie band (the query's k-th and (k+1)-th candidate scores differ by
    less than 1e-5 relative and the block scores within 1e-5 of the k-th)."""
    gpu_union = list(gpu_union)
    if gpu_union == list(ref_union):
        return True, "exact"
    if gpu_union != sorted(set(gpu_union)):
        return False, "not ascending / duplicates"
    diff = set(gpu_union) ^ set(ref_union)
    for b in diff:
        explained = False
        for top, BS in per_query:
            if len(cand) <= k or k <= 0:
                continue
            order = oracle.top_k_blocks(BS, cand, len(cand))
            s_k, s_k1 = BS[order[k - 1]], BS[order[k]]
            if rel_close(s_k, s_k1) and rel_close(BS[b], s_k):
                explained = True
                break
        if not explained:
            return False, f"block {b} differs outside any near-tie band"
    return True, "near tie"


def token_selection_ok(gpu_tokens, ref_tokens, s, bound, k, cand):
    """Token sets: exact, or of the same size and ascending with every token
    in which they differ scoring (oracle, fp64) within the fp32 rounding band
    of the k-th candidate score: |s_t - s_k| <= bound_t + bound_k, where
    bound_t bounds the fp32 error of token t's score."""
    gpu_tokens = list(gpu_tokens)
    if gpu_tokens == list(ref_tokens):
        return True, "exact"
    if len(gpu_tokens) != len(ref_tokens) or gpu_tokens != sorted(set(gpu_tokens)):
        return False, "wrong size, order or duplicates"
    cand = np.asarray(cand, dtype=np.int64)
    if k <= 0 or cand.size <= k:
        return False, "mismatch with no tie possible"
    order = oracle.top_k_tokens(s, cand, k)
    kth = order[-1]
    diff = set(gpu_tokens) ^ set(ref_tokens)
    if all(abs(s[t] - s[kth]) <= bound[t] + bound[kth] for t in diff):
        return True, "near tie"
    return False, "a differing token is outside the rounding band of the k-th score"


def ulp_distance(got: np.ndarray, ref: np.ndarray, dtype: str) -> np.ndarray:
    """Number of representable values of dtype ("f32" or "bf16") between two
    arrays of that dtype's values (given as fp32 numbers)."""
    def ordered(x):
        bits = np.asarray(x, dtype=np.float32).view(np.int32).astype(np.int64)
        if dtype == "bf16":
            assert np.all(bits & 0xFFFF == 0), "not bf16 values"
            bits = bits >> 16
            top = 2 ** 15
        else:
            top = 2 ** 31
        return np.where(bits < 0, -(bits & (top - 1)), bits)
    return np.abs(ordered(got) - ordered(ref))


def assert_same_attention(O1, O2, lse1, lse2, what=""):
    """Two GPU computations of the same attention over the same block sets that
    may split and sum the blocks in different orders (the one-call decode step
    against the separate calls): equal up to fp32 summation order."""
    a, b = O1.float().cpu(), O2.float().cpu()
    assert torch.allclose(a, b, rtol=1e-5, atol=1e-6), (what, float((a - b).abs().max()))
    la, lb = lse1.float().cpu(), lse2.float().cpu()
    assert torch.equal(torch.isinf(la), torch.isinf(lb)), what
    fin = torch.isfinite(la)
    assert torch.allclose(la[fin], lb[fin], rtol=1e-5, atol=1e-6), (what, "lse")
