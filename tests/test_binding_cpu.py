"""The Python binding rejects mismatched tensors before any call into the
library (host only: CPU tensors stand in for device tensors, so a call whose
arguments all pass validation stops at the device-tensor check)."""
import pytest
import torch

import block_sparse_attention_12_amd as sa

bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
B, Hq, Hkv, T, d = 2, 8, 2, 256, 128


def good_decode_step():
    return dict(Q=torch.zeros(B, Hq, d, dtype=bf), sel=torch.zeros(B, Hkv, d, dtype=bf),
                K=torch.zeros(B, Hkv, T, d, dtype=bf), V=torch.zeros(B, Hkv, T, d, dtype=bf),
                Kc=torch.zeros(B, Hkv, 15, d, dtype=bf), lens_prev=torch.zeros(B, dtype=i32),
                lens_now=torch.zeros(B, dtype=i32), top_k=4)


def call_decode_step(a):
    return sa.decode_step(a["Q"], a["sel"], a["K"], a["V"], a["Kc"], a["lens_prev"], a["lens_now"],
                          a["top_k"], **a.get("kw", {}))


def expect_reject(fn, args, key, value, match):
    a = dict(args)
    if key.startswith("kw."):
        a["kw"] = {key[3:]: value}
    else:
        a[key] = value
    with pytest.raises(ValueError, match=match):
        fn(a)


def test_valid_arguments_reach_the_device_check():
    with pytest.raises(ValueError, match="device tensor"):
        call_decode_step(good_decode_step())


@pytest.mark.parametrize("key,value,match", [
    ("Q", torch.zeros(B, Hq, d, dtype=f32), "Q must have dtype"),
    ("sel", torch.zeros(B, Hkv, d, dtype=f32), "sel must have dtype"),
    ("V", torch.zeros(B, Hkv, T, d, dtype=f32), "V must have dtype"),
    ("Kc", torch.zeros(B, Hkv, 15, d, dtype=f32), "Kc must have dtype"),
    ("V", torch.zeros(B, Hkv, T - 1, d, dtype=bf), "V must have shape"),
    ("Kc", torch.zeros(B, Hkv + 1, 15, d, dtype=bf), "Kc must have shape"),
    ("Q", torch.zeros(B + 1, Hq, d, dtype=bf), "Q must have shape"),
    ("lens_prev", torch.zeros(B, dtype=torch.int64), "lens_prev must have dtype"),
    ("lens_now", torch.zeros(B + 1, dtype=i32), "lens_now must have shape"),
    ("kw.idx", torch.zeros(B, Hkv, 7, dtype=torch.int64), "idx must have dtype"),
    ("kw.cnt", torch.zeros(B, Hkv + 1, dtype=i32), "cnt must have shape"),
    ("kw.O", torch.zeros(B, Hq, d - 1, dtype=f32), "O must have shape"),
    ("kw.lse", torch.zeros(B, Hq, dtype=bf), "lse must have dtype"),
])
def test_decode_step_rejects(key, value, match):
    expect_reject(call_decode_step, good_decode_step(), key, value, match)


def good_decode():
    return dict(Q=torch.zeros(B, Hq, d, dtype=bf), K=torch.zeros(B, Hkv, T, d, dtype=bf),
                V=torch.zeros(B, Hkv, T, d, dtype=bf), seq_lens=torch.zeros(B, dtype=i32),
                idx=torch.zeros(B, Hkv, 7, dtype=i32), cnt=torch.zeros(B, Hkv, dtype=i32))


def call_decode(a):
    return sa.decode(a["Q"], a["K"], a["V"], a["seq_lens"], a["idx"], a["cnt"], **a.get("kw", {}))


def call_token_decode(a):
    return sa.token_decode(a["Q"], a["K"], a["V"], a["seq_lens"], a["idx"], a["cnt"],
                           **a.get("kw", {}))


@pytest.mark.parametrize("fn", [call_decode, call_token_decode])
@pytest.mark.parametrize("key,value,match", [
    ("Q", torch.zeros(B, Hq, d, dtype=f32), "Q must have dtype"),
    ("V", torch.zeros(B, Hkv, T, d, dtype=f32), "V must have dtype"),
    ("K", torch.zeros(B, Hkv, T, d, dtype=torch.float16), "K must have dtype"),
    ("seq_lens", torch.zeros(B, dtype=torch.int64), "seq_lens must have dtype"),
    ("idx", torch.zeros(B, Hkv + 1, 7, dtype=i32), "idx must have shape"),
    ("cnt", torch.zeros(B, Hkv, dtype=torch.int64), "cnt must have dtype"),
    ("kw.O", torch.zeros(B, Hq + 1, d, dtype=f32), "O must have shape"),
])
def test_decode_rejects(fn, key, value, match):
    with pytest.raises(ValueError, match="device tensor"):
        fn(good_decode())
    expect_reject(fn, good_decode(), key, value, match)


def test_select_rejects():
    Kc = torch.zeros(B, Hkv, 15, d, dtype=bf)
    lens = torch.zeros(B, dtype=i32)
    with pytest.raises(ValueError, match="device tensor"):
        sa.select(torch.zeros(B, Hq, d, dtype=bf), Kc, lens, T, 4)
    with pytest.raises(ValueError, match="sel must have dtype"):
        sa.select(torch.zeros(B, Hq, d, dtype=f32), Kc, lens, T, 4)
    with pytest.raises(ValueError, match="sel must have shape"):
        sa.select(torch.zeros(B, Hq, d // 2, dtype=bf), Kc, lens, T, 4)
    with pytest.raises(ValueError, match="seq_lens must have shape"):
        sa.select(torch.zeros(B, Hq, d, dtype=bf), Kc, torch.zeros(B + 1, dtype=i32), T, 4)
    with pytest.raises(ValueError, match="idx must have dtype"):
        sa.select(torch.zeros(B, Hq, d, dtype=bf), Kc, lens, T, 4,
                  idx=torch.zeros(B, Hkv, 7, dtype=torch.int64))


def test_cobs_and_prefill_reject():
    K = torch.zeros(B, Hkv, T, d, dtype=bf)
    S = torch.zeros(B, Hkv, 4, 2, d, dtype=bf)
    lens = torch.zeros(B, dtype=i32)
    Q = torch.zeros(B, Hq, d, dtype=bf)
    with pytest.raises(ValueError, match="device tensor"):
        sa.cobs_decode_step(Q, Q, K, K, S, lens, lens, 4)
    with pytest.raises(ValueError, match="stats must have dtype"):
        sa.cobs_decode_step(Q, Q, K, K, S.float(), lens, lens, 4)
    with pytest.raises(ValueError, match="stats must have shape"):
        sa.cobs_select(Q, torch.zeros(B, Hkv, 4, 3, d, dtype=bf), lens, T, 4)
    Kp = torch.zeros(Hkv, T, d, dtype=bf)
    Qp = torch.zeros(64, Hq, d, dtype=bf)
    Kc = torch.zeros(Hkv, 15, d, dtype=bf)
    with pytest.raises(ValueError, match="device tensor"):
        sa.prefill_chunk(Qp, 128, Kp, Kp, Kc, 4)
    with pytest.raises(ValueError, match="V must have dtype"):
        sa.prefill_chunk(Qp, 128, Kp, Kp.float(), Kc, 4)
    with pytest.raises(ValueError, match="Kc must have shape"):
        sa.prefill_chunk(Qp, 128, Kp, Kp, torch.zeros(Hkv + 1, 15, d, dtype=bf), 4)
    with pytest.raises(ValueError, match="tile_cnt must have shape"):
        sa.prefill_attend(Qp, 128, Kp, Kp, torch.zeros(1, Hkv, 9, dtype=i32),
                          torch.zeros(2, Hkv, dtype=i32))


def test_strided_tensors_are_refused_with_the_reason():
    a = good_decode()
    a["K"] = torch.zeros(B, Hkv, T, 2 * d, dtype=bf)[..., :d]          # right shape, not dense
    with pytest.raises(ValueError, match="K must be dense row-major"):
        call_decode(a)
