"""Seeded synthetic inputs for block-sparse attention workloads.

This module is shared by the GPU path's tests and benchmark and by the CPU
oracle's tests. It only draws random tensors and shapes them; it holds none of
the method's arithmetic (no pooling, scoring, selection or attention).

Recipe (the same for every workload):
  * Q, K, V (and the Forecast vectors F when a workload scores with them) are
    fp32 draws from N(0, 1) made by one ``torch.Generator`` seeded per workload.
  * Q and F are scaled by 1/sqrt(head_dim), so attention and scoring use a
    softmax scale of 1.0.
  * Planted blocks: in each (sequence, KV head) ``planted`` distinct 64-token
    blocks are drawn uniformly from the blocks that can be chosen by top-k (not
    the initial block, not the local window). Every key of those blocks gets
    ``+2 * u`` added, where u is the unit vector of the group-summed query
    (query-scored workloads) or of the Forecast vector (Forecast-scored ones),
    taken in fp32 before the cast.
  * Spread blocks (workloads with ``spread`` > 0): ``spread`` further distinct
    choosable blocks per (sequence, KV head) get, in the 4 channels where the
    group-summed query is largest in magnitude, 8 * P[t, c] added, P being
    zero-mean, mutually orthogonal +-1 patterns over the block's 64 tokens:
    the block mean is unchanged and only those channels' variance grows.
  * Finally every tensor is cast to the workload dtype (fp32 or bf16).
Lengths may be ragged: positions at or beyond a sequence's length hold random
values that no step may read. Token-index workloads (``make_token_inputs``)
follow the same recipe with index keys and index vectors of their own
dimension, planted tokens instead of planted blocks.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace, field
from typing import Optional, Sequence

import torch

BLOCK = 64  # tokens per KV block


@dataclass(frozen=True)
class DecodeWorkload:
    """One decode step of one attention layer (or several layers sharing a selection)."""
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    T: int                  # context length of every sequence (L at the decode step)
    dtype: str              # "f32" or "bf16"
    top_k: int
    n_init: int
    n_local: int
    selector: str           # "query" (group-summed query heads) or "forecast"
    score_mode: str         # "softmax_sum" or "raw_sum"
    planted: int            # planted blocks per (sequence, KV head)
    seed: int
    layers: int = 1         # layers sharing one selection (cross-layer reuse), or decoded per step
    steps: int = 0          # appended decode steps (cross-layer workload only)
    lookahead: bool = False # each layer selects with its own Forecast; layer l+1's selection
                            # runs while layer l attends
    spread: int = 0         # planted high-variance blocks per (sequence, KV head)
    cobs: bool = False      # selection by block statistics (first / second order)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


@dataclass(frozen=True)
class PrefillWorkload:
    """One chunk of causal prefill for a single sequence."""
    name: str
    Hq: int
    Hkv: int
    d: int
    T: int                  # total context length after the chunk
    q_start: int            # first query position of the chunk (multiple of 64)
    dtype: str
    top_k: int
    n_init: int
    n_local: int
    seed: int

    @property
    def Tq(self) -> int:
        return self.T - self.q_start

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


@dataclass(frozen=True)
class TokenWorkload:
    """One decode step through several layers that share one token-level index."""
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    d_i: int                # index-key dimension
    T: int
    dtype: str
    top_k: int              # tokens chosen by score
    n_init: int             # first tokens always kept
    n_local: int            # last tokens always kept
    planted: int            # planted tokens per (sequence, KV head)
    layers: int             # layers attending with the shared index
    seed: int

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


TOKEN_WORKLOADS = {
    # the 128K Forecast decode shape with a 64-dimensional token index: one
    # index per step (4096 + 64 + 128 tokens per KV head, the token budget of
    # 64 + 1 + 2 blocks) shared by 4 layers
    "tokenindex_forecast_bf16_128k": TokenWorkload(
        "tokenindex_forecast_bf16_128k", B=8, Hq=32, Hkv=8, d=128, d_i=64, T=131072, dtype="bf16",
        top_k=4096, n_init=64, n_local=128, planted=512, layers=4, seed=6),
}

WORKLOADS = {
    # tiny single-layer decode, fp32, 4 planted blocks per KV head
    "decode_tiny_f32_8k": DecodeWorkload(
        "decode_tiny_f32_8k", B=1, Hq=8, Hkv=2, d=128, T=8192, dtype="f32",
        top_k=16, n_init=1, n_local=2, selector="query", score_mode="softmax_sum",
        planted=4, seed=1),
    # 8B-style GQA decode layer at 32K
    "decode_gqa_bf16_32k": DecodeWorkload(
        "decode_gqa_bf16_32k", B=16, Hq=32, Hkv=8, d=128, T=32768, dtype="bf16",
        top_k=64, n_init=1, n_local=2, selector="query", score_mode="softmax_sum",
        planted=8, seed=2),
    # Forecast-scored long decode at 128K
    "decode_forecast_bf16_128k": DecodeWorkload(
        "decode_forecast_bf16_128k", B=8, Hq=32, Hkv=8, d=128, T=131072, dtype="bf16",
        top_k=64, n_init=1, n_local=2, selector="forecast", score_mode="raw_sum",
        planted=8, seed=3),
    # the 128K Forecast decode through 4 layers, each with its own selection,
    # layer l+1's selection overlapped with layer l's attention
    "lookahead_forecast_bf16_128k": DecodeWorkload(
        "lookahead_forecast_bf16_128k", B=8, Hq=32, Hkv=8, d=128, T=131072, dtype="bf16",
        top_k=64, n_init=1, n_local=2, selector="forecast", score_mode="raw_sum",
        planted=8, seed=3, layers=4, lookahead=True),
    # the 128K GQA decode shape selected by block mean and variance (second
    # order), with 8 mean-shifted and 8 high-variance planted blocks per KV head
    "decode_cobs_gqa_bf16_128k": DecodeWorkload(
        "decode_cobs_gqa_bf16_128k", B=8, Hq=32, Hkv=8, d=128, T=131072, dtype="bf16",
        top_k=64, n_init=1, n_local=2, selector="query", score_mode="softmax_sum",
        planted=8, seed=7, spread=8, cobs=True),
    # cross-layer reuse: 4 layers share layer 0's selection, 16 appended steps
    "crosslayer_bf16_64k": DecodeWorkload(
        "crosslayer_bf16_64k", B=32, Hq=32, Hkv=8, d=128, T=65536, dtype="bf16",
        top_k=64, n_init=1, n_local=2, selector="query", score_mode="softmax_sum",
        planted=0, seed=5000, layers=4, steps=16),
}

PREFILL_WORKLOADS = {
    "prefill_chunk_bf16_128k": PrefillWorkload(
        "prefill_chunk_bf16_128k", Hq=32, Hkv=8, d=128, T=131072, q_start=129024,
        dtype="bf16", top_k=32, n_init=1, n_local=4, seed=4),
}


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, g, device):
    return torch.randn(*shape, generator=g, device=device, dtype=torch.float32)


def choosable_blocks(L: int, n_init: int, n_local: int):
    """Blocks top-k may pick at length L (not initial, not in the local window)."""
    nb = (L + BLOCK - 1) // BLOCK
    return list(range(min(n_init, nb), max(min(n_init, nb), nb - n_local)))


def _plant(Kb: torch.Tensor, u: torch.Tensor, blocks: Sequence[int]):
    """Add 2*u to every key of the listed 64-token blocks (Kb: [T, d] fp32, in place)."""
    for blk in blocks:
        Kb[blk * BLOCK:(blk + 1) * BLOCK] += 2.0 * u
    return None


def _sign_patterns(n: int, device) -> torch.Tensor:
    """n mutually orthogonal, zero-mean +-1 patterns over the 64 tokens of a
    block (rows 1..n of the Sylvester Hadamard matrix), as [64, n]."""
    H = torch.ones((1, 1))
    while H.shape[0] < BLOCK:
        H = torch.cat([torch.cat([H, H], 1), torch.cat([H, -H], 1)], 0)
    return H[1:n + 1].T.contiguous().to(device)


def _plant_spread(Kb: torch.Tensor, dirv: torch.Tensor, blocks: Sequence[int], amp: float = 8.0):
    """Spread the keys of the listed blocks along the 4 channels where dirv is
    largest in magnitude: channel c of token t gets amp * P[t, c] added, with
    P zero-mean orthogonal sign patterns, so the block mean and the
    cross-channel covariance stay as they were and only the per-channel
    variance of those channels grows (by amp^2)."""
    ch = torch.topk(dirv.abs(), 4).indices
    P = _sign_patterns(4, Kb.device)
    for blk in blocks:
        Kb[blk * BLOCK:(blk + 1) * BLOCK, ch] += amp * P


def make_decode_inputs(w: DecodeWorkload, device="cpu", seq_lens: Optional[Sequence[int]] = None,
                       T_cap: Optional[int] = None, layer: int = 0, replicas: int = 1):
    """Draw one layer's decode inputs.

    Returns a dict with
      Q [B, Hq, d], F [B, Hkv, d] (forecast workloads only), K, V [B, Hkv, T_cap, d]
      in the workload dtype, seq_lens (int32 [B], same device), planted and
      spread (lists per sequence of lists per KV head of block ids; spread is
      empty without spread blocks) and the scale (1.0).
    """
    device = torch.device(device)
    lens = list(seq_lens) if seq_lens is not None else [w.T] * w.B
    assert len(lens) == w.B
    cap = T_cap if T_cap is not None else max(lens)
    assert cap >= max(lens)
    g = _generator(w.seed + layer, device)
    dt = torch_dtype(w.dtype)
    inv = 1.0 / math.sqrt(w.d)
    Q = _randn((w.B, w.Hq, w.d), g, device) * inv
    F = _randn((w.B, w.Hkv, w.d), g, device) * inv if w.selector == "forecast" else None
    K = torch.empty((w.B, w.Hkv, cap, w.d), dtype=dt, device=device)
    V = torch.empty((w.B, w.Hkv, cap, w.d), dtype=dt, device=device)
    planted, spread = [], []
    for b in range(w.B):
        Kb = _randn((w.Hkv, cap, w.d), g, device)
        Vb = _randn((w.Hkv, cap, w.d), g, device)
        pl_b, sp_b = [], []
        for h in range(w.Hkv):
            blocks = []
            if w.planted > 0:
                cand = choosable_blocks(lens[b], w.n_init, w.n_local)
                n = min(w.planted, len(cand))
                perm = torch.randperm(len(cand), generator=g, device=device)[:n].tolist()
                blocks = sorted(cand[i] for i in perm)
                if w.selector == "forecast":
                    dirv = F[b, h]
                else:
                    dirv = Q[b, h * w.G:(h + 1) * w.G].sum(0)
                u = dirv / dirv.norm()
                _plant(Kb[h], u, blocks)
                if w.spread > 0:
                    rest = [c for c in cand if c not in blocks]
                    pick = torch.randperm(len(rest), generator=g, device=device)[:w.spread].tolist()
                    sp = sorted(rest[i] for i in pick)
                    _plant_spread(Kb[h], dirv, sp)
                    sp_b.append(sp)
            pl_b.append(blocks)
        planted.append(pl_b)
        spread.append(sp_b)
        K[b].copy_(Kb)
        V[b].copy_(Vb)
        del Kb, Vb
    out = dict(Q=Q.to(dt), K=K, V=V, scale=1.0, planted=planted, spread=spread,
               seq_lens=torch.tensor(lens, dtype=torch.int32, device=device))
    if F is not None:
        out["F"] = F.to(dt)
    return out


def make_decode_queries(w: DecodeWorkload, n: int, device="cpu", seed_offset: int = 100):
    """Extra decode queries (one [B, Hq, d] tensor per appended step)."""
    device = torch.device(device)
    g = _generator(w.seed + seed_offset, device)
    inv = 1.0 / math.sqrt(w.d)
    return [(_randn((w.B, w.Hq, w.d), g, device) * inv).to(torch_dtype(w.dtype)) for _ in range(n)]


def make_prefill_inputs(w: PrefillWorkload, device="cpu"):
    """Draw one sequence's prefill-chunk inputs.

    Returns Q [Tq, Hq, d] for positions q_start..T-1 and K, V [1, Hkv, T, d] (the
    whole context including the chunk's own keys), plus q_start and scale 1.0.
    """
    device = torch.device(device)
    g = _generator(w.seed, device)
    dt = torch_dtype(w.dtype)
    inv = 1.0 / math.sqrt(w.d)
    Q = (_randn((w.Tq, w.Hq, w.d), g, device) * inv).to(dt)
    K = torch.empty((1, w.Hkv, w.T, w.d), dtype=dt, device=device)
    V = torch.empty((1, w.Hkv, w.T, w.d), dtype=dt, device=device)
    for h in range(w.Hkv):
        K[0, h].copy_(_randn((w.T, w.d), g, device))
    for h in range(w.Hkv):
        V[0, h].copy_(_randn((w.T, w.d), g, device))
    return dict(Q=Q, K=K, V=V, q_start=w.q_start, scale=1.0)


def make_token_inputs(w: TokenWorkload, device="cpu", seq_lens: Optional[Sequence[int]] = None,
                      T_cap: Optional[int] = None, layers: Optional[int] = None):
    """Draw a token-index decode step's inputs.

    Index side: Ki [B, Hkv, T_cap, d_i] index keys and one Forecast-style
    index vector per group Fi [B, Hkv, d_i] (scaled by 1/sqrt(d_i)); in each
    (sequence, KV head) ``planted`` distinct tokens outside the kept initial /
    local windows get +2 * u added to their index key, u the unit vector of
    that group's Fi (fp32, before the cast). Attention side, per layer: Q
    [B, Hq, d] (scaled by 1/sqrt(d)), K, V [B, Hkv, T_cap, d]. Returns a dict
    with Ki, Fi, seq_lens, planted, layers (list of dicts) and scale 1.0.
    """
    device = torch.device(device)
    lens = list(seq_lens) if seq_lens is not None else [w.T] * w.B
    cap = T_cap if T_cap is not None else max(lens)
    n_layers = w.layers if layers is None else layers
    g = _generator(w.seed, device)
    dt = torch_dtype(w.dtype)
    Fi = _randn((w.B, w.Hkv, w.d_i), g, device) / math.sqrt(w.d_i)
    Ki = torch.empty((w.B, w.Hkv, cap, w.d_i), dtype=dt, device=device)
    planted = []
    for b in range(w.B):
        Kb = _randn((w.Hkv, cap, w.d_i), g, device)
        pl_b = []
        lo, hi = min(w.n_init, lens[b]), max(min(w.n_init, lens[b]), lens[b] - w.n_local)
        for h in range(w.Hkv):
            toks = []
            if w.planted > 0 and hi > lo:
                n = min(w.planted, hi - lo)
                toks = sorted((lo + torch.randperm(hi - lo, generator=g, device=device)[:n]).tolist())
                u = Fi[b, h] / Fi[b, h].norm()
                Kb[h, toks] += 2.0 * u
            pl_b.append(toks)
        planted.append(pl_b)
        Ki[b].copy_(Kb)
        del Kb
    inv = 1.0 / math.sqrt(w.d)
    lay = []
    for l in range(n_layers):
        gl = _generator(w.seed + 1 + l, device)
        Q = (_randn((w.B, w.Hq, w.d), gl, device) * inv).to(dt)
        K = torch.empty((w.B, w.Hkv, cap, w.d), dtype=dt, device=device)
        V = torch.empty((w.B, w.Hkv, cap, w.d), dtype=dt, device=device)
        for b in range(w.B):
            K[b].copy_(_randn((w.Hkv, cap, w.d), gl, device))
            V[b].copy_(_randn((w.Hkv, cap, w.d), gl, device))
        lay.append(dict(Q=Q, K=K, V=V))
    return dict(Ki=Ki, Fi=Fi.to(dt), seq_lens=torch.tensor(lens, dtype=torch.int32, device=device),
                planted=planted, layers=lay, scale=1.0)


def scaled(w, **kw):
    """A copy of a workload with some fields replaced (smaller test sizes)."""
    return replace(w, **kw)
