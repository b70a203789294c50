"""End-to-end GPU parity at the workloads' full sizes, in the launch
configuration the benchmark times (library-chosen split counts, fp32 outputs).

Inputs come from the seeded generators (on the device for the large ones); the
oracle recomputes every step on the CPU, for all (sequence, KV head) units or a
fixed sample of them where a full pass would take too long.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from block_sparse_attention_12_amd.pipeline import SparseDecoder
from oracle import SelectParams
from oracle.attention import block_tokens
from parity import selection_ok, gpu_rows, assert_close, to_np, ulp_distance

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run_decode_workload(w, units=None, check_planted=True, fused=False):
    inp = synth.make_decode_inputs(w, device=DEV)
    lens = inp["seq_lens"]
    dec = SparseDecoder(w.B, w.Hq, w.Hkv, w.T, w.top_k, w.n_init, w.n_local, w.selector,
                        w.score_mode)
    Kc = dec.new_kc(inp["K"].dtype)
    sel = inp["F"] if w.selector == "forecast" else inp["Q"]
    if fused:   # the benchmark's step: entries up to L - 1 exist, one call appends, selects, attends
        dec.build(inp["K"], Kc, lens - 1)
        O, lse = dec.fused_step(inp["Q"], sel, inp["K"], inp["V"], Kc, lens - 1, lens)
    else:
        dec.build(inp["K"], Kc, lens)
        dec.select(sel, Kc, lens)
        O, lse = dec.attend(inp["Q"], inp["K"], inp["V"], lens)
    torch.cuda.synchronize()
    rows = gpu_rows(dec.idx, dec.cnt)
    On, Ln = to_np(O), lse.cpu().numpy()
    S, Q = to_np(sel), to_np(inp["Q"])
    Gs, G = S.shape[1] // w.Hkv, w.G
    p = SelectParams(w.top_k, w.n_init, w.n_local, w.score_mode)
    if units is None:
        units = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    kinds, errs = [], []
    for (b, h) in units:
        L = int(lens[b])
        Kbh = inp["K"][b, h].float().cpu().numpy()
        Vbh = inp["V"][b, h].float().cpu().numpy()
        Kc_ref = oracle.compressed_keys(Kbh, L, w.dtype)
        got_kc = Kc[b, h, :Kc_ref.shape[0]].float().cpu().numpy()
        assert np.array_equal(got_kc.view(np.uint32), Kc_ref.view(np.uint32)), (b, h)
        ref, BS = oracle.select_blocks(S[b, h * Gs:(h + 1) * Gs], Kc_ref, L, p, True)
        ok, why = selection_ok(rows[(b, h)], ref, BS, oracle.n_blocks(L), w.top_k, w.n_init,
                               w.n_local)
        assert ok, ((b, h), why)
        kinds.append(why)
        if check_planted:
            assert set(inp["planted"][b][h]) <= set(rows[(b, h)]), "planted block missed"
        o, l = oracle.sparse_attention(Q[b, h * G:(h + 1) * G], Kbh, Vbh,
                                       block_tokens(rows[(b, h)], L), 1.0)
        errs.append(assert_close(On[b, h * G:(h + 1) * G], o, w.dtype, f"O {(b, h)}"))
        assert_close(Ln[b, h * G:(h + 1) * G], l, w.dtype, f"LSE {(b, h)}")
    print(f"{w.name}: {len(units)} units, selections {dict((k, kinds.count(k)) for k in set(kinds))},"
          f" max |O err| {max(errs):.2e}", flush=True)


def test_decode_tiny_f32_8k_full():
    _run_decode_workload(synth.WORKLOADS["decode_tiny_f32_8k"])


def test_decode_gqa_bf16_32k_full():
    _run_decode_workload(synth.WORKLOADS["decode_gqa_bf16_32k"])


def test_decode_forecast_bf16_128k_full():
    _run_decode_workload(synth.WORKLOADS["decode_forecast_bf16_128k"])


def test_decode_forecast_bf16_128k_one_call_step_full():
    """The benchmark's launch configuration: sparse_attn_decode_step (append
    inside the scoring launch) on the full workload, every unit against the
    oracle, compressed keys after the step bit-exact."""
    _run_decode_workload(synth.WORKLOADS["decode_forecast_bf16_128k"], fused=True)


def test_decode_gqa_bf16_32k_one_call_step_full():
    _run_decode_workload(synth.WORKLOADS["decode_gqa_bf16_32k"], fused=True)


def _run_crosslayer(w, units=None, T_cap=None):
    steps = w.steps
    T_cap = w.T + steps if T_cap is None else T_cap
    layers = []
    for l in range(w.layers):
        inp = synth.make_decode_inputs(w, device=DEV, T_cap=T_cap, layer=l)
        qs = synth.make_decode_queries(w, steps, device=DEV, seed_offset=100 + l)
        layers.append(dict(K=inp["K"], V=inp["V"], qs=qs))
    lens0 = torch.full((w.B,), w.T, dtype=torch.int32, device=DEV)
    dec = SparseDecoder(w.B, w.Hq, w.Hkv, T_cap, w.top_k, w.n_init, w.n_local, "query",
                        w.score_mode)
    Kc = dec.new_kc(layers[0]["K"].dtype)
    dec.build(layers[0]["K"], Kc, lens0)
    if units is None:
        units = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    # oracle state for the checked units (the anchor layer's compressed keys)
    host = {}
    for (b, h) in units:
        host[(b, h)] = dict(K=[lay["K"][b, h].float().cpu().numpy() for lay in layers],
                            V=[lay["V"][b, h].float().cpu().numpy() for lay in layers])
        host[(b, h)]["Kc"] = oracle.compressed_keys(host[(b, h)]["K"][0], w.T, w.dtype)
    p = SelectParams(w.top_k, w.n_init, w.n_local, w.score_mode)
    lens = lens0
    G = w.G
    for s in range(steps):
        new = lens + 1
        for lay in layers:
            lay["Q"] = lay["qs"][s]
        outs = dec.crosslayer_step(layers, Kc, lens, new)
        torch.cuda.synchronize()
        rows = gpu_rows(dec.idx, dec.cnt)
        for (b, h) in units:
            L_old, L = int(lens[b]), int(new[b])
            hb = host[(b, h)]
            hb["Kc"] = oracle.append_compressed_keys(hb["K"][0], hb["Kc"], L_old, L, w.dtype)
            q0 = to_np(layers[0]["Q"][b, h * G:(h + 1) * G])
            ref, BS = oracle.select_blocks(q0, hb["Kc"], L, p, True)
            ok, why = selection_ok(rows[(b, h)], ref, BS, oracle.n_blocks(L), w.top_k, w.n_init,
                                   w.n_local)
            assert ok, (s, (b, h), why)
            for l, (O, lse) in enumerate(outs):
                q = to_np(layers[l]["Q"][b, h * G:(h + 1) * G])
                o, lv = oracle.sparse_attention(q, hb["K"][l], hb["V"][l],
                                                block_tokens(rows[(b, h)], L), 1.0)
                assert_close(to_np(O[b, h * G:(h + 1) * G]), o, w.dtype, f"step {s} layer {l}")
                assert_close(lse[b, h * G:(h + 1) * G].cpu().numpy(), lv, w.dtype, "lse")
        lens = new
    # compressed keys after all appends equal a bulk rebuild, for every unit
    ref_kc = torch.empty_like(Kc)
    dec.build(layers[0]["K"], ref_kc, lens)
    n = oracle.n_compressed(int(lens[0]))
    assert torch.equal(Kc[:, :, :n].view(torch.int16), ref_kc[:, :, :n].view(torch.int16))


def test_crosslayer_small_all_units():
    w = synth.scaled(synth.WORKLOADS["crosslayer_bf16_64k"], B=3, T=4090)
    _run_crosslayer(w)


def test_crosslayer_bf16_64k_full_sampled():
    """The cross-layer workload at full size (B = 32, 64K, 4 layers, 16 steps):
    32 of the 256 (sequence, KV head) units, two per even sequence on varying
    KV heads, checked at every step (selection, all 4 layers' outputs)."""
    w = synth.WORKLOADS["crosslayer_bf16_64k"]
    units = [(b, h) for b in range(0, w.B, 2) for h in sorted({b % w.Hkv, (3 * b + 5) % w.Hkv})]
    assert len(units) == 32                          # b % 8 and (3b + 5) % 8 differ for even b
    _run_crosslayer(w, units=units)


def test_tokenindex_forecast_bf16_128k_full():
    """The token-index workload at full size (B = 8, 128K tokens, 64-dim index,
    top 4096 + 64 + 128 tokens, 4 layers), in the benchmark's launch
    configuration; selection and every layer's output checked on every unit."""
    from block_sparse_attention_12_amd.pipeline import TokenIndexDecoder
    from parity import token_selection_ok

    w = synth.TOKEN_WORKLOADS["tokenindex_forecast_bf16_128k"]
    inp = synth.make_token_inputs(w, device=DEV)
    lens = inp["seq_lens"]
    dec = TokenIndexDecoder(w.B, w.Hq, w.Hkv, w.T, w.top_k, w.n_init, w.n_local)
    outs = [(torch.empty((w.B, w.Hq, w.d), device=DEV), torch.empty((w.B, w.Hq), device=DEV))
            for _ in range(w.layers)]
    dec.step(inp["Fi"], inp["Ki"], inp["layers"], lens, outs)
    torch.cuda.synchronize()
    rows = gpu_rows(dec.idx, dec.cnt)
    Fi = to_np(inp["Fi"])
    units = [(b, h) for b in range(w.B) for h in range(w.Hkv)]      # every unit
    for (b, h) in units:
        L = int(lens[b])
        Ki = inp["Ki"][b, h].float().cpu().numpy()
        ref, s = oracle.select_tokens(Fi[b, h:h + 1], Ki, L, w.top_k, w.n_init, w.n_local, True)
        bound = 2e-6 * (np.abs(Ki[:L].astype(np.float64)) @ np.abs(Fi[b, h].astype(np.float64)))
        ok, why = token_selection_ok(rows[(b, h)], ref, s, bound, w.top_k,
                                     oracle.token_candidates(L, w.n_init, w.n_local)[2])
        assert ok, ((b, h), why)
        assert len(rows[(b, h)]) == w.top_k + w.n_init + w.n_local
        for l, lay in enumerate(inp["layers"]):
            q = lay["Q"][b, h * w.G:(h + 1) * w.G].float().cpu().numpy()
            o, lse = oracle.token_decode_unit(q, lay["K"][b, h].float().cpu().numpy(),
                                              lay["V"][b, h].float().cpu().numpy(), rows[(b, h)], 1.0)
            assert_close(to_np(outs[l][0])[b, h * w.G:(h + 1) * w.G], o, w.dtype, f"O {l} {(b, h)}")
            assert_close(outs[l][1].cpu().numpy()[b, h * w.G:(h + 1) * w.G], lse, w.dtype,
                         f"LSE {l} {(b, h)}")


def test_decode_cobs_gqa_bf16_128k_full():
    """The block-statistic workload at full size (B = 8, 128K, G = 4, softmax
    form, second order), in the benchmark's launch configuration: statistics
    within one ulp, selection and attention checked on every unit."""
    from block_sparse_attention_12_amd.pipeline import CobsDecoder

    w = synth.WORKLOADS["decode_cobs_gqa_bf16_128k"]
    inp = synth.make_decode_inputs(w, device=DEV)
    lens = inp["seq_lens"]
    dec = CobsDecoder(w.B, w.Hq, w.Hkv, w.T, w.top_k, w.n_init, w.n_local, w.selector,
                      w.score_mode, order=2)
    S = dec.new_stats(inp["K"].dtype)
    dec.build(inp["K"], S, lens - 1)
    dec.append(inp["K"], S, lens - 1, lens)
    dec.select(inp["Q"], S, lens)
    O, lse = dec.attend(inp["Q"], inp["K"], inp["V"], lens)
    torch.cuda.synchronize()
    rows = gpu_rows(dec.idx, dec.cnt)
    Q = to_np(inp["Q"])
    p = SelectParams(w.top_k, w.n_init, w.n_local, w.score_mode)
    units = [(b, h) for b in range(w.B) for h in range(w.Hkv)]      # every unit
    for (b, h) in units:
        L = int(lens[b])
        Kbh = inp["K"][b, h].float().cpu().numpy()
        mu, var = oracle.block_stats(Kbh, L, w.dtype)
        got = S[b, h, :mu.shape[0]].float().cpu().numpy()
        assert ulp_distance(got[:, 0], mu, w.dtype).max() <= 1, (b, h)
        assert ulp_distance(got[:, 1], var, w.dtype).max() <= 1, (b, h)
        ref, BS = oracle.select_blocks_cobs(Q[b, h * w.G:(h + 1) * w.G], mu, var, L, p, 2, True)
        ok, why = selection_ok(rows[(b, h)], ref, BS, oracle.n_blocks(L), w.top_k, w.n_init,
                               w.n_local)
        assert ok, ((b, h), why)
        assert set(inp["spread"][b][h]) <= set(rows[(b, h)]), "spread block missed"
        o, l = oracle.sparse_attention(Q[b, h * w.G:(h + 1) * w.G], Kbh,
                                       inp["V"][b, h].float().cpu().numpy(),
                                       block_tokens(rows[(b, h)], L), 1.0)
        assert_close(to_np(O)[b, h * w.G:(h + 1) * w.G], o, w.dtype, f"O {(b, h)}")
        assert_close(lse.cpu().numpy()[b, h * w.G:(h + 1) * w.G], l, w.dtype, f"LSE {(b, h)}")
