"""The C-ABI library loads, exports every symbol its header declares, and its
host-side validation rejects bad arguments with the documented status before
any HIP call (so these run without a GPU; no call here reaches a kernel).
"""
import ctypes
import os
import re

import pytest
import torch

import block_sparse_attention_12_amd as sa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_attn.h")

FAKE = 0x1000          # never dereferenced: every call below fails validation first


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sparse_attn_\w+)\s*\(", src)))


def test_header_declarations_match_binding_list():
    assert declared_functions() == sorted(sa.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = sa.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value


def test_version_and_status_strings():
    assert sa.abi_version() == 1
    for code, text in ((0, "ok"), (-1, "invalid argument"), (-2, "unsupported configuration"),
                       (-3, "workspace missing or too small"), (-4, "output or cache capacity too small"),
                       (-5, "HIP launch error"), (7, "unknown status")):
        assert sa.status_string(code) == text


def _compress(**kw):
    a = dict(K=FAKE, Kc=FAKE, dtype=sa.SA_BF16, B=2, Hkv=2, d=128, T_cap=1000, nc_cap=61,
             lens_prev=FAKE, lens_now=FAKE, max_new=61, stream=None)
    a.update(kw)
    return sa.lib().sparse_attn_compress(a["K"], a["Kc"], a["dtype"], a["B"], a["Hkv"], a["d"],
                                         a["T_cap"], a["nc_cap"], a["lens_prev"], a["lens_now"],
                                         a["max_new"], a["stream"])


def test_compress_validation():
    assert _compress(K=None) == sa.SA_ERR_INVALID_ARG
    assert _compress(lens_now=None) == sa.SA_ERR_INVALID_ARG
    assert _compress(dtype=7) == sa.SA_ERR_INVALID_ARG
    assert _compress(B=0) == sa.SA_ERR_INVALID_ARG
    assert _compress(max_new=-1) == sa.SA_ERR_INVALID_ARG
    assert _compress(d=64) == sa.SA_ERR_UNSUPPORTED
    assert _compress(nc_cap=60) == sa.SA_ERR_CAPACITY           # n_c(1000) = 61
    assert _compress(max_new=0) == sa.SA_OK                     # nothing to do: no launch


def _select(**kw):
    p = kw.pop("params", sa.make_params(16, 1, 2, "softmax_sum"))
    a = dict(sel=FAKE, H_sel=8, Kc=FAKE, dtype=sa.SA_F32, B=1, Hkv=2, d=128, T_cap=8192,
             nc_cap=511, seq_lens=FAKE, idx=FAKE, idx_cap=19, cnt=FAKE, bs=None, ws=FAKE,
             ws_bytes=1 << 30, stream=None)
    a.update(kw)
    pp = None if p is None else ctypes.byref(p)
    return sa.lib().sparse_attn_select(a["sel"], a["H_sel"], a["Kc"], a["dtype"], a["B"], a["Hkv"],
                                       a["d"], a["T_cap"], a["nc_cap"], a["seq_lens"], pp, a["idx"],
                                       a["idx_cap"], a["cnt"], a["bs"], a["ws"], a["ws_bytes"],
                                       a["stream"])


def test_select_validation():
    assert _select(sel=None) == sa.SA_ERR_INVALID_ARG
    assert _select(params=None) == sa.SA_ERR_INVALID_ARG
    assert _select(H_sel=7) == sa.SA_ERR_INVALID_ARG            # not a multiple of Hkv
    assert _select(params=sa.make_params(-1)) == sa.SA_ERR_INVALID_ARG
    assert _select(params=sa.make_params(16, score_mode=5)) == sa.SA_ERR_INVALID_ARG
    assert _select(params=sa.make_params(16, block_size=128)) == sa.SA_ERR_UNSUPPORTED
    assert _select(params=sa.make_params(16, cmp_stride=8)) == sa.SA_ERR_UNSUPPORTED
    assert _select(H_sel=6) == sa.SA_ERR_UNSUPPORTED            # G = 3
    assert _select(d=96) == sa.SA_ERR_UNSUPPORTED
    assert _select(T_cap=64 * 32769) == sa.SA_ERR_UNSUPPORTED
    assert _select(nc_cap=510) == sa.SA_ERR_CAPACITY
    assert _select(idx_cap=18) == sa.SA_ERR_CAPACITY
    assert _select(ws=None) == sa.SA_ERR_WORKSPACE
    need = sa.select_workspace_size(1, 2, 8, 8192, sa.make_params(16))
    assert need > 0
    assert _select(ws_bytes=need - 1) == sa.SA_ERR_WORKSPACE


def test_select_workspace_sizes():
    soft = sa.select_workspace_size(8, 8, 32, 131072, sa.make_params(64, 1, 2, "softmax_sum"))
    raw = sa.select_workspace_size(8, 8, 8, 131072, sa.make_params(64, 1, 2, "raw_sum"))
    assert soft >= 64 * 4 * 8191 * 4                          # logits of every entry and head
    assert raw >= 64 * 2048 * 4                                # one score per block
    assert sa.select_workspace_size(8, 8, 7, 1000, sa.make_params(4)) == 0   # invalid -> 0


def _decode(**kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, dtype=sa.SA_BF16, B=2, Hq=8, Hkv=2, d=128, T_cap=4096,
             lens=FAKE, idx=FAKE, cnt=FAKE, idx_cap=19, scale=1.0, O=FAKE, out_dtype=sa.SA_F32,
             lse=None, n_split=4, ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return sa.lib().sparse_attn_decode(a["Q"], a["K"], a["V"], a["dtype"], a["B"], a["Hq"], a["Hkv"],
                                       a["d"], a["T_cap"], a["lens"], a["idx"], a["cnt"],
                                       a["idx_cap"], a["scale"], a["O"], a["out_dtype"], a["lse"],
                                       a["n_split"], a["ws"], a["ws_bytes"], a["stream"])


def test_decode_validation():
    assert _decode(O=None) == sa.SA_ERR_INVALID_ARG
    assert _decode(idx_cap=0) == sa.SA_ERR_INVALID_ARG
    assert _decode(Hq=7) == sa.SA_ERR_INVALID_ARG
    assert _decode(out_dtype=3) == sa.SA_ERR_INVALID_ARG
    assert _decode(scale=float("nan")) == sa.SA_ERR_INVALID_ARG
    assert _decode(Hq=6) == sa.SA_ERR_UNSUPPORTED               # G = 3
    assert _decode(Hq=32) == sa.SA_ERR_UNSUPPORTED              # G = 16
    assert _decode(n_split=65) == sa.SA_ERR_UNSUPPORTED
    assert _decode(idx_cap=4097) == sa.SA_ERR_UNSUPPORTED
    assert _decode(d=64) == sa.SA_ERR_UNSUPPORTED
    assert _decode(ws=None) == sa.SA_ERR_WORKSPACE
    assert _decode(ws_bytes=sa.decode_workspace_size(2, 8, 2, 19, 4) - 1) == sa.SA_ERR_WORKSPACE
    assert sa.decode_workspace_size(2, 8, 2, 19, 1) == 0        # one split writes O directly


def _prefill(**kw):
    p = kw.pop("params", sa.make_params(32, 1, 4))
    a = dict(Q=FAKE, q_start=1024, Tq=256, K=FAKE, V=FAKE, Kc=FAKE, dtype=sa.SA_BF16, Hq=32, Hkv=8,
             d=128, T_cap=1280, nc_cap=79, O=FAKE, out_dtype=sa.SA_F32, lse=None, tidx=FAKE,
             tcap=20, tcnt=FAKE, ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return sa.lib().sparse_attn_prefill_chunk(a["Q"], a["q_start"], a["Tq"], a["K"], a["V"], a["Kc"],
                                              a["dtype"], a["Hq"], a["Hkv"], a["d"], a["T_cap"],
                                              a["nc_cap"], ctypes.byref(p), 1.0, a["O"],
                                              a["out_dtype"], a["lse"], a["tidx"], a["tcap"],
                                              a["tcnt"], a["ws"], a["ws_bytes"], a["stream"])


def test_prefill_validation():
    assert sa.prefill_tile_cap(1024, 256, sa.make_params(32, 1, 4)) == 20       # nb(1280) = 20
    assert sa.prefill_tile_cap(129024, 2048, sa.make_params(32, 1, 4)) == 2048
    assert _prefill(q_start=1000) == sa.SA_ERR_INVALID_ARG                       # not block aligned
    assert _prefill(Tq=0) == sa.SA_ERR_INVALID_ARG
    assert _prefill(tidx=None) == sa.SA_ERR_INVALID_ARG
    assert _prefill(dtype=sa.SA_F32) == sa.SA_ERR_UNSUPPORTED
    assert _prefill(Hq=16) == sa.SA_ERR_UNSUPPORTED
    # a tile's block scores (64 queries x Hkv x blocks, fp32) must fit 31-bit offsets
    assert _prefill(Hq=2048, Hkv=512, q_start=64 * 32767, Tq=64, T_cap=64 * 32768,
                    nc_cap=4 * 32768) == sa.SA_ERR_UNSUPPORTED
    assert _prefill(T_cap=1279) == sa.SA_ERR_CAPACITY
    assert _prefill(nc_cap=78) == sa.SA_ERR_CAPACITY                             # n_c(1280) = 79
    assert _prefill(tcap=19) == sa.SA_ERR_CAPACITY


def test_binding_refuses_host_tensors():
    import torch
    K = torch.zeros(1, 1, 64, 128)
    with pytest.raises(ValueError):
        sa.compress(K, torch.zeros(1, 1, 3, 128), torch.zeros(1, dtype=torch.int32),
                    torch.zeros(1, dtype=torch.int32))


def test_prefill_attend_validation():
    L = sa.lib()

    def call(**kw):
        a = dict(Q=FAKE, q_start=1024, Tq=256, K=FAKE, V=FAKE, dtype=sa.SA_BF16, Hq=32, Hkv=8, d=128,
                 T_cap=1280, tidx=FAKE, tcap=20, tcnt=FAKE, O=FAKE, out=sa.SA_F32, lse=None)
        a.update(kw)
        return L.sparse_attn_prefill_attend(a["Q"], a["q_start"], a["Tq"], a["K"], a["V"], a["dtype"],
                                            a["Hq"], a["Hkv"], a["d"], a["T_cap"], a["tidx"], a["tcap"],
                                            a["tcnt"], 1.0, a["O"], a["out"], a["lse"], None)
    assert call(tidx=None) == sa.SA_ERR_INVALID_ARG
    assert call(q_start=65) == sa.SA_ERR_INVALID_ARG
    assert call(tcap=0) == sa.SA_ERR_INVALID_ARG
    assert call(Hq=8) == sa.SA_ERR_UNSUPPORTED
    assert call(dtype=sa.SA_F32) == sa.SA_ERR_UNSUPPORTED
    assert call(T_cap=1000) == sa.SA_ERR_CAPACITY


def test_stream_read_validation():
    L = sa.lib()
    assert L.sparse_attn_stream_read_blocks() > 0
    assert L.sparse_attn_stream_read(None, 1024, FAKE, None) == sa.SA_ERR_INVALID_ARG
    assert L.sparse_attn_stream_read(FAKE, 0, FAKE, None) == sa.SA_ERR_INVALID_ARG
    assert L.sparse_attn_stream_read(FAKE, 1000, FAKE, None) == sa.SA_ERR_INVALID_ARG   # not a multiple of 16
    assert L.sparse_attn_stream_read(FAKE + 8, 1024, FAKE, None) == sa.SA_ERR_INVALID_ARG  # misaligned
    assert L.sparse_attn_stream_read(FAKE, 1024, None, None) == sa.SA_ERR_INVALID_ARG


def test_block_mass_validation():
    L = sa.lib()

    def call(**kw):
        a = dict(Q=FAKE, K=FAKE, dtype=sa.SA_BF16, B=2, Hq=8, Hkv=2, d=128, T_cap=1000, lens=FAKE,
                 mass=FAKE, mass_cap=16, idx=None, cnt=None, idx_cap=0, recall=None, ws=FAKE,
                 ws_bytes=1 << 30)
        a.update(kw)
        return L.sparse_attn_block_mass(a["Q"], a["K"], a["dtype"], a["B"], a["Hq"], a["Hkv"], a["d"],
                                        a["T_cap"], a["lens"], 1.0, a["mass"], a["mass_cap"], a["idx"],
                                        a["cnt"], a["idx_cap"], a["recall"], a["ws"], a["ws_bytes"], None)
    assert call(Q=None) == sa.SA_ERR_INVALID_ARG
    assert call(mass=None) == sa.SA_ERR_INVALID_ARG
    assert call(dtype=9) == sa.SA_ERR_INVALID_ARG
    assert call(Hq=7) == sa.SA_ERR_INVALID_ARG
    assert call(idx=FAKE) == sa.SA_ERR_INVALID_ARG                   # set without cnt / recall
    assert call(Hq=16) == sa.SA_ERR_UNSUPPORTED                      # G = 8
    assert call(d=64) == sa.SA_ERR_UNSUPPORTED
    assert call(mass_cap=15) == sa.SA_ERR_CAPACITY                   # ceil(1000 / 64) = 16
    need = L.sparse_attn_block_mass_workspace_size(2, 8, 16)
    assert need == 2 * 2 * 8 * 16 * 4
    assert call(ws_bytes=need - 1) == sa.SA_ERR_WORKSPACE
    assert call(ws=None) == sa.SA_ERR_WORKSPACE


def test_token_select_validation():
    L = sa.lib()

    def call(**kw):
        a = dict(sel=FAKE, H_sel=2, Ki=FAKE, dtype=sa.SA_BF16, B=2, Hkv=2, d_i=64, T_cap=10000,
                 lens=FAKE, k=256, ni=64, nl=128, idx=FAKE, idx_cap=448, cnt=FAKE, scores=None,
                 ws=FAKE, ws_bytes=1 << 30)
        a.update(kw)
        return L.sparse_attn_token_select(a["sel"], a["H_sel"], a["Ki"], a["dtype"], a["B"], a["Hkv"],
                                          a["d_i"], a["T_cap"], a["lens"], a["k"], a["ni"], a["nl"],
                                          a["idx"], a["idx_cap"], a["cnt"], a["scores"], a["ws"],
                                          a["ws_bytes"], None)
    assert call(sel=None) == sa.SA_ERR_INVALID_ARG
    assert call(cnt=None) == sa.SA_ERR_INVALID_ARG
    assert call(dtype=5) == sa.SA_ERR_INVALID_ARG
    assert call(k=-1) == sa.SA_ERR_INVALID_ARG
    assert call(H_sel=3) == sa.SA_ERR_INVALID_ARG                     # not a multiple of Hkv
    assert call(d_i=96) == sa.SA_ERR_UNSUPPORTED
    assert call(H_sel=2 * 65) == sa.SA_ERR_UNSUPPORTED                # 65 selectors per group
    assert call(T_cap=1 << 24, d_i=128, dtype=sa.SA_F32) == sa.SA_ERR_UNSUPPORTED   # 8 GiB slice
    assert call(idx_cap=447) == sa.SA_ERR_CAPACITY
    need = L.sparse_attn_token_select_workspace_size(2, 2, 10000)
    chunks = 3                                                       # ceil(10000 / 4096)
    assert need >= 4 * chunks * 4096 * 4 + 4 * 4 * 256 * 4
    assert call(ws_bytes=need - 1) == sa.SA_ERR_WORKSPACE
    assert call(ws=None) == sa.SA_ERR_WORKSPACE
    assert L.sparse_attn_token_select_workspace_size(2, 2, 0) > 0      # one chunk even when empty


def test_token_decode_validation():
    L = sa.lib()

    def call(**kw):
        a = dict(Q=FAKE, K=FAKE, V=FAKE, dtype=sa.SA_BF16, B=2, Hq=8, Hkv=2, d=128, T_cap=10000,
                 lens=FAKE, idx=FAKE, cnt=FAKE, idx_cap=448, O=FAKE, out=sa.SA_F32, lse=None,
                 n_split=0, ws=FAKE, ws_bytes=1 << 30)
        a.update(kw)
        return L.sparse_attn_token_decode(a["Q"], a["K"], a["V"], a["dtype"], a["B"], a["Hq"],
                                          a["Hkv"], a["d"], a["T_cap"], a["lens"], a["idx"], a["cnt"],
                                          a["idx_cap"], 1.0, a["O"], a["out"], a["lse"], a["n_split"],
                                          a["ws"], a["ws_bytes"], None)
    assert call(Q=None) == sa.SA_ERR_INVALID_ARG
    assert call(idx_cap=0) == sa.SA_ERR_INVALID_ARG
    assert call(Hq=7) == sa.SA_ERR_INVALID_ARG
    assert call(d=64) == sa.SA_ERR_UNSUPPORTED
    assert call(Hq=6) == sa.SA_ERR_UNSUPPORTED                        # G = 3
    assert call(Hq=32) == sa.SA_ERR_UNSUPPORTED                       # G = 16
    assert call(n_split=65) == sa.SA_ERR_UNSUPPORTED
    assert call(idx_cap=64 * 64 * 64 + 1) == sa.SA_ERR_UNSUPPORTED    # more than 4096 tiles
    need = L.sparse_attn_token_decode_workspace_size(2, 8, 2, 448, 4)
    part = -(-(2 * 8 * 4 * 132 * 4) // 256) * 256                     # partials of 4 splits
    assert need == part + (2 + 2 * 2) * 8                             # + split-merge words
    assert call(n_split=4, ws_bytes=need - 1) == sa.SA_ERR_WORKSPACE


def test_cobs_validation():
    L = sa.lib()

    def stats_call(**kw):
        a = dict(K=FAKE, S=FAKE, dtype=sa.SA_BF16, B=2, Hkv=2, d=128, T_cap=1000, nb_cap=16,
                 lp=FAKE, ln=FAKE, mx=16)
        a.update(kw)
        return L.sparse_attn_cobs_stats(a["K"], a["S"], a["dtype"], a["B"], a["Hkv"], a["d"],
                                        a["T_cap"], a["nb_cap"], a["lp"], a["ln"], a["mx"], None)
    assert stats_call(K=None) == sa.SA_ERR_INVALID_ARG
    assert stats_call(mx=-1) == sa.SA_ERR_INVALID_ARG
    assert stats_call(d=64) == sa.SA_ERR_UNSUPPORTED
    assert stats_call(nb_cap=14) == sa.SA_ERR_CAPACITY                # 1000 // 64 = 15 complete
    assert stats_call(mx=0) == sa.SA_OK                               # nothing to do

    def sel_call(**kw):
        p = kw.pop("params", sa.make_params(8, 1, 2, "softmax_sum"))
        a = dict(sel=FAKE, H_sel=8, S=FAKE, dtype=sa.SA_BF16, B=2, Hkv=2, d=128, T_cap=1000,
                 nb_cap=16, lens=FAKE, order=2, idx=FAKE, idx_cap=11, cnt=FAKE, bs=None, ws=FAKE,
                 ws_bytes=1 << 30)
        a.update(kw)
        return L.sparse_attn_cobs_select(a["sel"], a["H_sel"], a["S"], a["dtype"], a["B"], a["Hkv"],
                                         a["d"], a["T_cap"], a["nb_cap"], a["lens"], ctypes.byref(p),
                                         a["order"], a["idx"], a["idx_cap"], a["cnt"], a["bs"],
                                         a["ws"], a["ws_bytes"], None)
    assert sel_call(sel=None) == sa.SA_ERR_INVALID_ARG
    assert sel_call(order=3) == sa.SA_ERR_INVALID_ARG
    assert sel_call(H_sel=7) == sa.SA_ERR_INVALID_ARG
    assert sel_call(H_sel=6) == sa.SA_ERR_UNSUPPORTED                 # G = 3
    assert sel_call(params=sa.make_params(8, block_size=32)) == sa.SA_ERR_UNSUPPORTED
    assert sel_call(nb_cap=15) == sa.SA_ERR_CAPACITY                  # ceil(1000 / 64) = 16
    assert sel_call(idx_cap=10) == sa.SA_ERR_CAPACITY
    need = L.sparse_attn_cobs_select_workspace_size(2, 2, 8, 1000, ctypes.byref(sa.make_params(8)))
    assert need >= 4 * 16 * 4 + 4 * 4 * 256 * 4                       # block scores + logits
    assert sel_call(ws_bytes=need - 1) == sa.SA_ERR_WORKSPACE


def test_cobs_decode_step_validation():
    L = sa.lib()
    p8 = sa.make_params(8, 1, 2, "softmax_sum")

    def step_call(**kw):
        p = kw.pop("params", p8)
        a = dict(Q=FAKE, sel=FAKE, H_sel=8, K=FAKE, V=FAKE, S=FAKE, dtype=sa.SA_BF16, B=2, Hq=8,
                 Hkv=2, d=128, T_cap=1000, nb_cap=16, lp=FAKE, ln=FAKE, mx=1, order=2, scale=1.0,
                 idx=FAKE, idx_cap=11, cnt=FAKE, O=FAKE, out_dtype=sa.SA_F32, lse=None, n_split=0,
                 ws=FAKE, ws_bytes=1 << 30)
        a.update(kw)
        return L.sparse_attn_cobs_decode_step(
            a["Q"], a["sel"], a["H_sel"], a["K"], a["V"], a["S"], a["dtype"], a["B"], a["Hq"],
            a["Hkv"], a["d"], a["T_cap"], a["nb_cap"], a["lp"], a["ln"], a["mx"], ctypes.byref(p),
            a["order"], a["scale"], a["idx"], a["idx_cap"], a["cnt"], a["O"], a["out_dtype"],
            a["lse"], a["n_split"], a["ws"], a["ws_bytes"], None)
    assert step_call(S=None) == sa.SA_ERR_INVALID_ARG
    assert step_call(mx=-1) == sa.SA_ERR_INVALID_ARG
    assert step_call(order=0) == sa.SA_ERR_INVALID_ARG
    assert step_call(scale=float("nan")) == sa.SA_ERR_INVALID_ARG
    assert step_call(H_sel=6) == sa.SA_ERR_UNSUPPORTED                # G = 3
    assert step_call(Hq=6) == sa.SA_ERR_UNSUPPORTED                   # 3 query heads per KV head
    assert step_call(n_split=65) == sa.SA_ERR_UNSUPPORTED
    assert step_call(nb_cap=15) == sa.SA_ERR_CAPACITY
    assert step_call(idx_cap=10) == sa.SA_ERR_CAPACITY
    need = L.sparse_attn_cobs_decode_step_workspace_size(2, 8, 2, 8, 1000, ctypes.byref(p8), 11, 0)
    assert need >= L.sparse_attn_cobs_select_workspace_size(2, 2, 8, 1000, ctypes.byref(p8))
    assert step_call(ws_bytes=need - 1) == sa.SA_ERR_WORKSPACE


def test_decode_step_noalloc_rejects_steps_beyond_its_scratch():
    """A step whose scratch exceeds the fixed per-GPU array is refused before
    any HIP call (softmax-sum logits of 512 units x 4 heads x 8192 entries)."""
    L = sa.lib()
    p = sa.make_params(64, 1, 2, "softmax_sum")
    need = L.sparse_attn_decode_step_workspace_size(64, 256, 8, 32, 131072, ctypes.byref(p), 67, 0)
    assert need > sa.NOALLOC_SCRATCH_BYTES
    st = L.sparse_attn_decode_step_noalloc(FAKE, FAKE, 32, FAKE, FAKE, FAKE, sa.SA_BF16, 64, 256, 8,
                                           128, 131072, 8191, FAKE, FAKE, 1, ctypes.byref(p), 1.0,
                                           FAKE, 67, FAKE, FAKE, sa.SA_F32, None, 0, None)
    assert st == sa.SA_ERR_WORKSPACE
    assert L.sparse_attn_decode_step_noalloc(FAKE, FAKE, 32, FAKE, FAKE, FAKE, sa.SA_BF16, 64, 256,
                                             8, 128, 131072, 8191, FAKE, FAKE, 1, None, 1.0, FAKE,
                                             67, FAKE, FAKE, sa.SA_F32, None, 0, None) \
        == sa.SA_ERR_INVALID_ARG


def test_decode_step_splits():
    """sparse_attn_decode_step_splits: the step's split count is the decode
    call's for the same arguments (so sparse_attn_decode with it reproduces
    the step's outputs up to fp32 order), an explicit count is kept (raised to
    the one that keeps every split within 64 list entries), and invalid
    arguments give 0."""
    L = sa.lib()
    raw = sa.make_params(64, 1, 2, "raw_sum")
    soft = sa.make_params(64, 1, 2, "softmax_sum")
    for p in (raw, soft):
        for dtype in (torch.bfloat16, torch.float32):
            for B, Hkv in ((8, 8), (16, 8), (1, 2), (32, 8)):
                s = sa.decode_step_splits(dtype, B, Hkv, 131072, p, 67)
                assert s >= 1
                ws = sa.decode_workspace_size(B, 4 * Hkv, Hkv, 67, s)
                assert ws == sa.decode_workspace_size(B, 4 * Hkv, Hkv, 67, 0)   # = automatic
                assert sa.decode_step_splits(dtype, B, Hkv, 131072, p, 67, 1, 3) == 3
    assert sa.decode_step_splits(torch.bfloat16, 1, 2, 131072, raw, 1000, 1, 3) == 16   # 1000 / 64
    bad = [(-1, 8, 8, 131072, 67, 1, 0), (1, 0, 8, 131072, 67, 1, 0), (1, 8, 0, 131072, 67, 1, 0),
           (1, 8, 8, -1, 67, 1, 0), (1, 8, 8, 131072, 0, 1, 0), (1, 8, 8, 131072, 67, -1, 0),
           (1, 8, 8, 131072, 67, 1, -1), (7, 8, 8, 131072, 67, 1, 0)]
    for dt, B, Hkv, T, cap, mx, ns in bad:
        assert L.sparse_attn_decode_step_splits(dt, B, Hkv, T, ctypes.byref(raw), cap, mx, ns) == 0
    assert L.sparse_attn_decode_step_splits(1, 8, 8, 131072, None, 67, 1, 0) == 0
