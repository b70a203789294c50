"""GPU parity of the lookahead decode step (layer l+1's Forecast selection on a
second stream while layer l attends): every layer's selection and output equal
the in-order step bit for bit (same kernels, only the order of independent work
changes), eagerly and replayed as a captured graph, and match the CPU oracle.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from block_sparse_attention_12_amd.pipeline import LookaheadDecoder
from oracle import SelectParams
from oracle.attention import block_tokens
from parity import selection_ok, gpu_rows, assert_close, to_np, assert_same_attention

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _setup(n_layers=3, T=8192, B=2):
    w = dataclasses.replace(synth.WORKLOADS["lookahead_forecast_bf16_128k"], name="t", B=B, Hq=8,
                            Hkv=2, T=T, top_k=16, planted=4, layers=n_layers)
    la = LookaheadDecoder(w.B, w.Hq, w.Hkv, w.T, w.top_k, w.n_init, w.n_local, device=DEV)
    layers, inps = [], []
    for l in range(n_layers):
        inp = synth.make_decode_inputs(w, device=DEV, layer=l)
        Kc = la.new_kc(inp["K"].dtype)
        la.build(inp["K"], Kc, inp["seq_lens"] - 1)
        layers.append(dict(Q=inp["Q"], F=inp["F"], K=inp["K"], V=inp["V"], Kc=Kc))
        inps.append(inp)
    lens = inps[0]["seq_lens"]
    return w, la, layers, inps, lens


def _outs(w, n):
    return [(torch.full((w.B, w.Hq, 128), float("nan"), device=DEV),
             torch.full((w.B, w.Hq), float("nan"), device=DEV)) for _ in range(n)]


def _snapshot(la, layers, lens, outs, lookahead):
    """Runs one step and returns per-layer (O, lse) copies."""
    la.step(layers, lens - 1, lens, outs, lookahead=lookahead)
    torch.cuda.synchronize()
    return [(o.clone(), s.clone()) for (o, s) in outs]


def test_lookahead_equals_in_order_eager_and_graph():
    w, la, layers, inps, lens = _setup()
    n = len(layers)
    kc0 = [lay["Kc"].clone() for lay in layers]

    def restore():
        for lay, kc in zip(layers, kc0):
            lay["Kc"].copy_(kc)

    ref_outs = _outs(w, n)
    ref = _snapshot(la, layers, lens, ref_outs, lookahead=False)
    # in-order step: each layer's selection is left in dec[l % 2]; keep the last two
    ref_idx = {n - 1: (la.dec[(n - 1) % 2].idx.clone(), la.dec[(n - 1) % 2].cnt.clone()),
               n - 2: (la.dec[(n - 2) % 2].idx.clone(), la.dec[(n - 2) % 2].cnt.clone())}
    kc_after = [lay["Kc"].clone() for lay in layers]
    for mode in ("eager", "graph"):
        restore()
        outs = _outs(w, n)
        if mode == "eager":
            got = _snapshot(la, layers, lens, outs, lookahead=True)
        else:
            g = la.dec[0].capture(lambda: la.step(layers, lens - 1, lens, outs, lookahead=True))
            for rep in range(3):                  # replays with eager work in between
                restore()
                for o, s in outs:
                    o.fill_(float("nan"))
                    s.fill_(float("nan"))
                torch.cuda.synchronize()
                g.replay()
                torch.cuda.synchronize()
                got = [(o.clone(), s.clone()) for (o, s) in outs]
                for l in range(n):
                    assert torch.equal(got[l][0], ref[l][0]), (mode, rep, l)
                    assert torch.equal(got[l][1], ref[l][1]), (mode, rep, l)
        for l in range(n):
            assert torch.equal(got[l][0], ref[l][0]), (mode, l)
            assert torch.equal(got[l][1], ref[l][1]), (mode, l)
            assert torch.equal(layers[l]["Kc"], kc_after[l]), (mode, l)
        for l, (idx, cnt) in ref_idx.items():
            d = la.dec[l % 2]
            assert torch.equal(d.idx, idx) and torch.equal(d.cnt, cnt), (mode, l)


def test_lookahead_layers_match_oracle():
    w, la, layers, inps, lens = _setup(n_layers=2)
    outs = _outs(w, 2)
    la.step(layers, lens - 1, lens, outs, lookahead=True)
    torch.cuda.synchronize()
    p = SelectParams(w.top_k, w.n_init, w.n_local, w.score_mode)
    for l in range(2):
        rows = gpu_rows(la.dec[l % 2].idx, la.dec[l % 2].cnt)
        inp = inps[l]
        F, Q = to_np(inp["F"]), to_np(inp["Q"])
        On, Ln = to_np(outs[l][0]), outs[l][1].cpu().numpy()
        for b in range(w.B):
            for h in range(w.Hkv):
                L = int(lens[b])
                K = inp["K"][b, h].float().cpu().numpy()
                V = inp["V"][b, h].float().cpu().numpy()
                Kc = oracle.compressed_keys(K, L, w.dtype)
                got_kc = layers[l]["Kc"][b, h, :Kc.shape[0]].float().cpu().numpy()
                assert np.array_equal(got_kc.view(np.uint32), Kc.view(np.uint32)), (l, b, h)
                ref, BS = oracle.select_blocks(F[b, h:h + 1], Kc, L, p, True)
                ok, why = selection_ok(rows[(b, h)], ref, BS, oracle.n_blocks(L), w.top_k,
                                       w.n_init, w.n_local)
                assert ok, (l, b, h, why)
                assert set(inp["planted"][b][h]) <= set(rows[(b, h)])
                o, lse = oracle.sparse_attention(Q[b, h * w.G:(h + 1) * w.G], K, V,
                                                 block_tokens(rows[(b, h)], L), 1.0)
                assert_close(On[b, h * w.G:(h + 1) * w.G], o, "bf16", f"O layer {l} {(b, h)}")
                assert_close(Ln[b, h * w.G:(h + 1) * w.G], lse, "bf16", f"LSE layer {l} {(b, h)}")


def test_one_call_schedule_equals_in_order():
    """One sparse_attn_decode_step call per layer gives every layer's
    compressed keys and block set bit for bit as the three-call in-order step
    and its outputs up to fp32 summation order; replays of the captured
    one-call step give the eager one-call step's bits."""
    w, la, layers, inps, lens = _setup()
    n = len(layers)
    kc0 = [lay["Kc"].clone() for lay in layers]
    ref = _snapshot(la, layers, lens, _outs(w, n), lookahead=False)
    last = (la.dec[(n - 1) % 2].idx.clone(), la.dec[(n - 1) % 2].cnt.clone())
    kc_after = [lay["Kc"].clone() for lay in layers]
    outs = _outs(w, n)
    g = la.dec[0].capture(lambda: la.step_one_call(layers, lens - 1, lens, outs))
    first = None
    for mode in ("eager", "graph", "graph"):
        for lay, kc in zip(layers, kc0):
            lay["Kc"].copy_(kc)
        for o, s in outs:
            o.fill_(float("nan"))
            s.fill_(float("nan"))
        torch.cuda.synchronize()
        if mode == "eager":
            la.step_one_call(layers, lens - 1, lens, outs)
        else:
            g.replay()
        torch.cuda.synchronize()
        if first is None:                  # the eager one-call step vs the in-order step
            for l in range(n):
                assert_same_attention(outs[l][0], ref[l][0], outs[l][1], ref[l][1], (mode, l))
            first = [(o.clone(), s.clone()) for o, s in outs]
        for l in range(n):                 # every replay: the eager one-call step's bits
            assert torch.equal(outs[l][0], first[l][0]), (mode, l)
            assert torch.equal(outs[l][1], first[l][1]), (mode, l)
            assert torch.equal(layers[l]["Kc"], kc_after[l]), (mode, l)
        assert torch.equal(la.dec[0].idx, last[0]) and torch.equal(la.dec[0].cnt, last[1]), mode
