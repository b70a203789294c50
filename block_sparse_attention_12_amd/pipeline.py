"""Decode-step and prefill drivers over the C ABI (no arithmetic of their own).

A decode step of one layer is: append the compressed-key entries completed by
the new token (Eq. 2), select blocks with the query or Forecast (Eq. 4 / Eq. 6
and the Eq. 1 union), and attend over them (Eq. 5). With cross-layer reuse one
selection from the anchor layer serves several layers. Outputs, index buffers
and workspaces are allocated once here so a step enqueues kernels only.
"""
from __future__ import annotations

from typing import Optional, Sequence

import torch

from . import (compress, select, decode, prefill_chunk, prefill_attend, make_params,
               select_workspace_size, token_select, token_decode, token_select_workspace_size,
               token_decode_workspace_size, cobs_stats, cobs_select, cobs_select_workspace_size,
               n_blocks, decode_step, decode_step_workspace_size, decode_step_splits,
               cobs_decode_step,
               cobs_decode_step_workspace_size,
               decode_workspace_size, prefill_workspace_size, prefill_tile_cap, n_compressed)


class SparseDecoder:
    """Buffers and calls for one decode configuration (fixed B, heads, capacity)."""

    def __init__(self, B: int, Hq: int, Hkv: int, T_cap: int, top_k: int, n_init: int = 1,
                 n_local: int = 2, selector: str = "query", score_mode: str = "softmax_sum",
                 device="cuda", n_split: int = 0, out_dtype=torch.float32, want_lse: bool = True):
        self.B, self.Hq, self.Hkv, self.T_cap = B, Hq, Hkv, T_cap
        self.top_k, self.n_init, self.n_local = top_k, n_init, n_local
        self.selector, self.score_mode, self.n_split = selector, score_mode, n_split
        self.H_sel = Hq if selector == "query" else Hkv
        self.cap = top_k + n_init + n_local
        self.nc_cap = n_compressed(T_cap)
        dev = torch.device(device)
        self.device = dev
        p = make_params(top_k, n_init, n_local, score_mode)
        self.idx = torch.empty((B, Hkv, self.cap), dtype=torch.int32, device=dev)
        self.cnt = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
        sws = select_workspace_size(B, Hkv, self.H_sel, T_cap, p)
        self.sel_ws = torch.empty(max(sws, 1), dtype=torch.uint8, device=dev)
        dws = decode_workspace_size(B, Hq, Hkv, self.cap, n_split)
        self.dec_ws = torch.empty(max(dws, 1), dtype=torch.uint8, device=dev)
        self.O = torch.empty((B, Hq, 128), dtype=out_dtype, device=dev)
        self.lse = torch.empty((B, Hq), dtype=torch.float32, device=dev) if want_lse else None

    def new_kc(self, dtype) -> torch.Tensor:
        return torch.empty((self.B, self.Hkv, self.nc_cap, 128), dtype=dtype, device=self.device)

    def build(self, K, Kc, seq_lens):
        zeros = torch.zeros_like(seq_lens)
        compress(K, Kc, zeros, seq_lens, max_new_entries=self.nc_cap)

    def append(self, K, Kc, lens_prev, lens_now, max_new_entries: int = 1):
        compress(K, Kc, lens_prev, lens_now, max_new_entries=max_new_entries)

    def select(self, sel, Kc, seq_lens, block_scores=None):
        return select(sel, Kc, seq_lens, self.T_cap, self.top_k, self.n_init, self.n_local,
                      self.score_mode, idx=self.idx, cnt=self.cnt, block_scores=block_scores,
                      workspace=self.sel_ws)

    def attn_splits(self, dtype) -> int:
        """Split-K workgroups per (b, kvh) of the decode step (fused_step) for
        keys of this dtype; attend uses the same, so step and fused_step agree
        up to fp32 summation order."""
        p = make_params(self.top_k, self.n_init, self.n_local, self.score_mode)
        return decode_step_splits(dtype, self.B, self.Hkv, self.T_cap, p, self.cap, 1, self.n_split)

    def attend(self, Q, K, V, seq_lens, O: Optional[torch.Tensor] = None, lse=None, scale=1.0):
        O = self.O if O is None else O
        lse = self.lse if lse is None else lse
        ns = self.attn_splits(K.dtype)
        need = decode_workspace_size(self.B, self.Hq, self.Hkv, self.cap, ns)
        if self.dec_ws.numel() < need:
            self.dec_ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return decode(Q, K, V, seq_lens, self.idx, self.cnt, scale, O=O, lse=lse,
                      want_lse=lse is not None, n_split=ns, workspace=self.dec_ws)

    def step(self, Q, sel, K, V, Kc, lens_prev, lens_now, scale=1.0):
        """One single-layer decode step: append, select, attend (three calls)."""
        self.append(K, Kc, lens_prev, lens_now)
        self.select(sel, Kc, lens_now)
        return self.attend(Q, K, V, lens_now, scale=scale)

    def fused_step(self, Q, sel, K, V, Kc, lens_prev, lens_now, scale=1.0, max_new_tokens=1,
                   O=None, lse=None):
        """The same step through sparse_attn_decode_step (one call; in raw-sum
        mode the append shares the scoring launch). O / lse: output buffers
        other than the decoder's own."""
        if getattr(self, "step_ws", None) is None:
            p = make_params(self.top_k, self.n_init, self.n_local, self.score_mode)
            need = decode_step_workspace_size(self.B, self.Hq, self.Hkv, self.H_sel, self.T_cap, p,
                                              self.cap, self.n_split)
            self.step_ws = torch.empty(max(need, 1), dtype=torch.uint8, device=self.device)
        O, lse, _, _ = decode_step(Q, sel, K, V, Kc, lens_prev, lens_now, self.top_k, self.n_init,
                                   self.n_local, self.score_mode, scale, max_new_tokens,
                                   idx=self.idx, cnt=self.cnt, O=self.O if O is None else O,
                                   lse=self.lse if lse is None else lse,
                                   want_lse=self.lse is not None or lse is not None,
                                   n_split=self.n_split, workspace=self.step_ws)
        return O, lse

    def capture(self, fn, warmup: int = 2):
        """Capture fn() (a sequence of the calls above on fixed buffers) into a
        HIP graph; returns the torch.cuda.CUDAGraph to replay. Every call only
        enqueues kernels on the current stream (no allocation, no memset), so
        the captured graph is the same kernel sequence with its launch gaps
        removed."""
        s = torch.cuda.Stream(device=self.device)
        s.wait_stream(torch.cuda.current_stream(self.device))
        with torch.cuda.stream(s):
            for _ in range(warmup):
                fn()
        torch.cuda.current_stream(self.device).wait_stream(s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return g

    def crosslayer_step(self, layers: Sequence[dict], Kc, lens_prev, lens_now, outs=None,
                        scale=1.0, one_call: bool = True):
        """One decode step where layer 0 (the anchor) selects for every layer.

        layers: dicts with Q, K, V (K/V already hold the appended token).
        outs: optional list of (O, lse) buffers per layer. one_call: the anchor
        layer's append, selection and attention through one
        sparse_attn_decode_step call (its block set is left in self.idx /
        self.cnt for the other layers), else three calls.
        """
        res = []
        for i, lay in enumerate(layers):
            O, lse = (outs[i] if outs is not None else (None, None))
            if O is None:
                O = torch.empty_like(self.O)
                lse = torch.empty_like(self.lse) if self.lse is not None else None
            if i == 0 and one_call:
                res.append(self.fused_step(lay["Q"], lay["Q"], lay["K"], lay["V"], Kc, lens_prev,
                                           lens_now, scale, O=O, lse=lse))
                continue
            if i == 0:
                self.append(lay["K"], Kc, lens_prev, lens_now)
                self.select(lay["Q"], Kc, lens_now)
            res.append(self.attend(lay["Q"], lay["K"], lay["V"], lens_now, O=O, lse=lse,
                                   scale=scale))
        return res


class LookaheadDecoder:
    """A decode step through several layers, each selecting its own blocks with
    its own Forecast (Eq. 4 with F_l, one vector per GQA group), where layer
    l+1's append and selection run on a second stream while layer l attends:
    the Forecast of the next layer is available before this layer's attention,
    so selection leaves the critical path (the lookahead the SparDA page
    describes between the Forecast and its use one layer later). Two sets of
    selection buffers alternate between layers; every dependency is an event
    (selection of layer l+1 waits for attention of layer l-1, which last read
    that buffer set; attention of layer l waits for its selection).
    """

    def __init__(self, B: int, Hq: int, Hkv: int, T_cap: int, top_k: int, n_init: int = 1,
                 n_local: int = 2, device="cuda", n_split: int = 0, out_dtype=torch.float32):
        self.dec = [SparseDecoder(B, Hq, Hkv, T_cap, top_k, n_init, n_local, "forecast", "raw_sum",
                                  device=device, n_split=n_split, out_dtype=out_dtype)
                    for _ in range(2)]
        self.device = torch.device(device)
        self.side = torch.cuda.Stream(device=self.device)   # default priority

    def new_kc(self, dtype) -> torch.Tensor:
        return self.dec[0].new_kc(dtype)

    def build(self, K, Kc, seq_lens):
        self.dec[0].build(K, Kc, seq_lens)

    def step(self, layers: Sequence[dict], lens_prev, lens_now, outs, scale=1.0,
             lookahead: bool = True):
        """layers: dicts with F (Forecast, [B, Hkv, d]), Q, K, V (K/V already hold
        the new token) and Kc (that layer's compressed keys); outs: list of
        (O, lse) per layer. With lookahead=False everything runs in order on the
        current stream (the same calls, for comparison)."""
        main = torch.cuda.current_stream(self.device)
        n = len(layers)
        if not lookahead:
            for l, lay in enumerate(layers):
                d = self.dec[l % 2]
                d.append(lay["K"], lay["Kc"], lens_prev, lens_now)
                d.select(lay["F"], lay["Kc"], lens_now)
                d.attend(lay["Q"], lay["K"], lay["V"], lens_now, O=outs[l][0], lse=outs[l][1],
                         scale=scale)
            return outs
        side = self.side
        side.wait_stream(main)                     # the step's inputs are in place

        def select_on_side(l):
            d, lay = self.dec[l % 2], layers[l]
            with torch.cuda.stream(side):
                d.append(lay["K"], lay["Kc"], lens_prev, lens_now)
                d.select(lay["F"], lay["Kc"], lens_now)
                ev = torch.cuda.Event()
                ev.record(side)
            return ev

        sel_done = select_on_side(0)
        att_done = [None] * n
        for l, lay in enumerate(layers):
            main.wait_event(sel_done)
            if l + 1 < n:
                if l >= 1:
                    side.wait_event(att_done[l - 1])   # buffers of layer l+1 = those of l-1
                next_done = select_on_side(l + 1)
            self.dec[l % 2].attend(lay["Q"], lay["K"], lay["V"], lens_now, O=outs[l][0],
                                   lse=outs[l][1], scale=scale)
            att_done[l] = torch.cuda.Event()
            att_done[l].record(main)
            if l + 1 < n:
                sel_done = next_done
        main.wait_stream(side)                     # join: the side stream is idle after the step
        return outs

    def step_one_call(self, layers: Sequence[dict], lens_prev, lens_now, outs, scale=1.0):
        """The same step in order on the current stream with one
        sparse_attn_decode_step call per layer (append, selection and attention
        of a layer in one call, so no selection is left to overlap)."""
        d = self.dec[0]
        for l, lay in enumerate(layers):
            d.fused_step(lay["Q"], lay["F"], lay["K"], lay["V"], lay["Kc"], lens_prev, lens_now,
                         scale, O=outs[l][0], lse=outs[l][1])
        return outs


class CobsDecoder(SparseDecoder):
    """A decode step whose selection uses per-block statistics (block mean and
    per-channel variance) instead of compressed keys: append writes the
    statistics of a block when the new token completes it, select scores the
    blocks by the first- or second-order block-mass estimate, attend is the
    block decode attention."""

    def __init__(self, *args, order: int = 2, **kw):
        super().__init__(*args, **kw)
        self.order = order
        p = make_params(self.top_k, self.n_init, self.n_local, self.score_mode)
        ws = cobs_select_workspace_size(self.B, self.Hkv, self.H_sel, self.T_cap, p)
        self.sel_ws = torch.empty(max(ws, 1), dtype=torch.uint8, device=self.device)
        self.nb_cap = n_blocks(self.T_cap)

    def new_stats(self, dtype) -> torch.Tensor:
        return torch.empty((self.B, self.Hkv, self.nb_cap, 2, 128), dtype=dtype, device=self.device)

    def build(self, K, stats, seq_lens):
        cobs_stats(K, stats, torch.zeros_like(seq_lens), seq_lens, max_new_blocks=self.nb_cap)

    def append(self, K, stats, lens_prev, lens_now, max_new_blocks: int = 1):
        cobs_stats(K, stats, lens_prev, lens_now, max_new_blocks=max_new_blocks)

    def select(self, sel, stats, seq_lens, block_scores=None, order=None):
        return cobs_select(sel, stats, seq_lens, self.T_cap, self.top_k, self.n_init, self.n_local,
                           self.score_mode, self.order if order is None else order, idx=self.idx,
                           cnt=self.cnt, block_scores=block_scores, workspace=self.sel_ws)

    def fused_step(self, Q, sel, K, V, stats, lens_prev, lens_now, scale=1.0, max_new_blocks=1,
                   O=None, lse=None):
        """The same step through sparse_attn_cobs_decode_step (one call)."""
        if getattr(self, "cobs_step_ws", None) is None:
            p = make_params(self.top_k, self.n_init, self.n_local, self.score_mode)
            need = cobs_decode_step_workspace_size(self.B, self.Hq, self.Hkv, self.H_sel,
                                                   self.T_cap, p, self.cap, self.n_split)
            self.cobs_step_ws = torch.empty(max(need, 1), dtype=torch.uint8, device=self.device)
        O, lse, _, _ = cobs_decode_step(Q, sel, K, V, stats, lens_prev, lens_now, self.top_k,
                                        self.n_init, self.n_local, self.score_mode, self.order,
                                        scale, max_new_blocks, idx=self.idx, cnt=self.cnt,
                                        O=self.O if O is None else O,
                                        lse=self.lse if lse is None else lse,
                                        want_lse=self.lse is not None or lse is not None,
                                        n_split=self.n_split, workspace=self.cobs_step_ws)
        return O, lse


class TokenIndexDecoder:
    """A decode step in which one token-level index, computed once from the
    anchor's index keys and selector, serves every layer (the CLSA routing
    index shared across layers): token_select once, then token_decode per
    layer over the same list. Buffers are allocated once."""

    def __init__(self, B: int, Hq: int, Hkv: int, T_cap: int, top_k: int, n_init: int = 64,
                 n_local: int = 128, device="cuda", n_split: int = 0, out_dtype=torch.float32):
        self.B, self.Hq, self.Hkv, self.T_cap = B, Hq, Hkv, T_cap
        self.top_k, self.n_init, self.n_local, self.n_split = top_k, n_init, n_local, n_split
        dev = torch.device(device)
        self.cap = top_k + n_init + n_local
        self.idx = torch.empty((B, Hkv, self.cap), dtype=torch.int32, device=dev)
        self.cnt = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
        self.sel_ws = torch.empty(max(token_select_workspace_size(B, Hkv, T_cap), 1),
                                  dtype=torch.uint8, device=dev)
        dws = token_decode_workspace_size(B, Hq, Hkv, self.cap, n_split)
        self.dec_ws = torch.empty(max(dws, 1), dtype=torch.uint8, device=dev)

    def select(self, sel, Ki, seq_lens):
        return token_select(sel, Ki, seq_lens, self.top_k, self.n_init, self.n_local,
                            idx=self.idx, cnt=self.cnt, workspace=self.sel_ws)

    def attend(self, Q, K, V, seq_lens, O, lse=None, scale=1.0):
        return token_decode(Q, K, V, seq_lens, self.idx, self.cnt, scale, O=O, lse=lse,
                            want_lse=lse is not None, n_split=self.n_split, workspace=self.dec_ws)

    def step(self, sel, Ki, layers: Sequence[dict], seq_lens, outs, scale=1.0):
        """layers: dicts with Q, K, V; outs: list of (O, lse) per layer."""
        self.select(sel, Ki, seq_lens)
        for lay, (O, lse) in zip(layers, outs):
            self.attend(lay["Q"], lay["K"], lay["V"], seq_lens, O, lse, scale)
        return outs


class SparsePrefill:
    """Buffers and call for chunked sparse prefill of one sequence."""

    def __init__(self, Hq: int, Hkv: int, q_start: int, Tq: int, top_k: int, n_init: int = 1,
                 n_local: int = 4, score_mode: str = "softmax_sum", device="cuda",
                 out_dtype=torch.float32):
        self.Hq, self.Hkv, self.q_start, self.Tq = Hq, Hkv, q_start, Tq
        self.top_k, self.n_init, self.n_local, self.score_mode = top_k, n_init, n_local, score_mode
        dev = torch.device(device)
        p = make_params(top_k, n_init, n_local, score_mode)
        self.cap = prefill_tile_cap(q_start, Tq, p)
        n_tiles = (Tq + 63) // 64
        self.tile_idx = torch.empty((n_tiles, Hkv, self.cap), dtype=torch.int32, device=dev)
        self.tile_cnt = torch.empty((n_tiles, Hkv), dtype=torch.int32, device=dev)
        ws = prefill_workspace_size(Hq, Hkv, q_start, Tq, p)
        self.ws = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
        self.O = torch.empty((Tq, Hq, 128), dtype=out_dtype, device=dev)
        self.lse = torch.empty((Tq, Hq), dtype=torch.float32, device=dev)

    def run(self, Q, K, V, Kc, scale=1.0):
        return prefill_chunk(Q, self.q_start, K, V, Kc, self.top_k, self.n_init, self.n_local,
                             self.score_mode, scale, O=self.O, lse=self.lse,
                             tile_idx=self.tile_idx, tile_cnt=self.tile_cnt, workspace=self.ws)

    def attend(self, Q, K, V, scale=1.0, O=None, lse=None):
        """Attention only, over the tile sets of the last run (reuse across layers)."""
        return prefill_attend(Q, self.q_start, K, V, self.tile_idx, self.tile_cnt, scale,
                              O=self.O if O is None else O, lse=self.lse if lse is None else lse)
