"""Python binding of libsparse_attn (MI355X / gfx950 block-sparse attention).

Argument marshalling only: every step of the method runs in the HIP kernels of
the shared library, reached through its C ABI (include/sparse_attn.h) with
ctypes. PyTorch supplies device memory and the current HIP stream. There is no
CPU or PyTorch fallback: if the library is not built, every call raises.

Entry points (same names as the C ABI):
    compress(K, Kc, lens_prev, lens_now)              compressed keys, Eq. 2
    select(sel, Kc, seq_lens, T_cap, top_k, ...)      scores + top-k + union, Eq. 1/4/6
    decode(Q, K, V, seq_lens, idx, cnt, ...)          sparse decode attention, Eq. 5
    prefill_chunk(Q, q_start, K, V, Kc, ...)          tile-shared sparse prefill
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libsparse_attn.so")

SA_OK = 0
SA_ERR_INVALID_ARG = -1
SA_ERR_UNSUPPORTED = -2
SA_ERR_WORKSPACE = -3
SA_ERR_CAPACITY = -4
SA_ERR_HIP = -5
SA_F32 = 0
SA_BF16 = 1
SA_SCORE_SOFTMAX_SUM = 0
SA_SCORE_RAW_SUM = 1

SCORE_MODES = {"softmax_sum": SA_SCORE_SOFTMAX_SUM, "raw_sum": SA_SCORE_RAW_SUM}

# exported symbols, as declared in include/sparse_attn.h
EXPORTS = [
    "sparse_attn_abi_version", "sparse_attn_status_string", "sparse_attn_compress",
    "sparse_attn_select_workspace_size", "sparse_attn_select",
    "sparse_attn_decode_workspace_size", "sparse_attn_decode",
    "sparse_attn_prefill_tile_cap", "sparse_attn_prefill_workspace_size",
    "sparse_attn_prefill_chunk", "sparse_attn_prefill_attend",
    "sparse_attn_block_mass_workspace_size", "sparse_attn_block_mass",
    "sparse_attn_stream_read_blocks", "sparse_attn_stream_read",
    "sparse_attn_token_select_workspace_size", "sparse_attn_token_select",
    "sparse_attn_token_decode_workspace_size", "sparse_attn_token_decode",
    "sparse_attn_cobs_stats", "sparse_attn_cobs_select_workspace_size", "sparse_attn_cobs_select",
    "sparse_attn_decode_step_workspace_size", "sparse_attn_decode_step_splits",
    "sparse_attn_decode_step",
    "sparse_attn_cobs_decode_step_workspace_size", "sparse_attn_cobs_decode_step",
    "sparse_attn_decode_step_noalloc",
]

# scratch bytes of sparse_attn_decode_step_noalloc's per-GPU array (SA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 32 << 20


class SelectParams(ctypes.Structure):
    _fields_ = [("block_size", ctypes.c_int32), ("cmp_kernel", ctypes.c_int32),
                ("cmp_stride", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("n_init", ctypes.c_int32), ("n_local", ctypes.c_int32),
                ("score_mode", ctypes.c_int32)]


def make_params(top_k: int, n_init: int = 1, n_local: int = 2, score_mode="softmax_sum",
                block_size: int = 64, cmp_kernel: int = 32, cmp_stride: int = 16) -> SelectParams:
    mode = SCORE_MODES[score_mode] if isinstance(score_mode, str) else int(score_mode)
    return SelectParams(block_size, cmp_kernel, cmp_stride, top_k, n_init, n_local, mode)


class SparseAttnError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: {text} (status {status})")
        self.status = status


_lib = None
_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_int = ctypes.c_int
_PP = ctypes.POINTER(SelectParams)


def lib() -> ctypes.CDLL:
    """Load libsparse_attn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libsparse_attn.so not built ({LIB_PATH}); run __graft_entry__.build() "
                           "or python block_sparse_attention_12_amd/_build.py")
    L = ctypes.CDLL(LIB_PATH)
    L.sparse_attn_abi_version.restype = _int
    L.sparse_attn_abi_version.argtypes = []
    L.sparse_attn_status_string.restype = ctypes.c_char_p
    L.sparse_attn_status_string.argtypes = [_int]
    L.sparse_attn_compress.restype = _int
    L.sparse_attn_compress.argtypes = [_vp, _vp, _int, _int, _int, _int, _i64, _i64, _vp, _vp, _i32, _vp]
    L.sparse_attn_select_workspace_size.restype = _sz
    L.sparse_attn_select_workspace_size.argtypes = [_int, _int, _int, _i64, _PP]
    L.sparse_attn_select.restype = _int
    L.sparse_attn_select.argtypes = [_vp, _int, _vp, _int, _int, _int, _int, _i64, _i64, _vp, _PP,
                                     _vp, _i32, _vp, _vp, _vp, _sz, _vp]
    L.sparse_attn_decode_workspace_size.restype = _sz
    L.sparse_attn_decode_workspace_size.argtypes = [_int, _int, _int, _i32, _i32]
    L.sparse_attn_decode.restype = _int
    L.sparse_attn_decode.argtypes = [_vp, _vp, _vp, _int, _int, _int, _int, _int, _i64, _vp, _vp, _vp,
                                     _i32, _f32, _vp, _int, _vp, _i32, _vp, _sz, _vp]
    L.sparse_attn_prefill_tile_cap.restype = _i32
    L.sparse_attn_prefill_tile_cap.argtypes = [_i64, _i64, _PP]
    L.sparse_attn_prefill_workspace_size.restype = _sz
    L.sparse_attn_prefill_workspace_size.argtypes = [_int, _int, _i64, _i64, _PP]
    L.sparse_attn_prefill_chunk.restype = _int
    L.sparse_attn_prefill_chunk.argtypes = [_vp, _i64, _i64, _vp, _vp, _vp, _int, _int, _int, _int,
                                            _i64, _i64, _PP, _f32, _vp, _int, _vp, _vp, _i32, _vp,
                                            _vp, _sz, _vp]
    L.sparse_attn_prefill_attend.restype = _int
    L.sparse_attn_prefill_attend.argtypes = [_vp, _i64, _i64, _vp, _vp, _int, _int, _int, _int, _i64,
                                             _vp, _i32, _vp, _f32, _vp, _int, _vp, _vp]
    L.sparse_attn_block_mass_workspace_size.restype = _sz
    L.sparse_attn_block_mass_workspace_size.argtypes = [_int, _int, _i64]
    L.sparse_attn_block_mass.restype = _int
    L.sparse_attn_block_mass.argtypes = [_vp, _vp, _int, _int, _int, _int, _int, _i64, _vp, _f32, _vp,
                                         _i64, _vp, _vp, _i32, _vp, _vp, _sz, _vp]
    L.sparse_attn_stream_read_blocks.restype = _int
    L.sparse_attn_stream_read_blocks.argtypes = []
    L.sparse_attn_stream_read.restype = _int
    L.sparse_attn_stream_read.argtypes = [_vp, _sz, _vp, _vp]
    L.sparse_attn_token_select_workspace_size.restype = _sz
    L.sparse_attn_token_select_workspace_size.argtypes = [_int, _int, _i64]
    L.sparse_attn_token_select.restype = _int
    L.sparse_attn_token_select.argtypes = [_vp, _int, _vp, _int, _int, _int, _int, _i64, _vp, _i32,
                                           _i32, _i32, _vp, _i32, _vp, _vp, _vp, _sz, _vp]
    L.sparse_attn_decode_step_workspace_size.restype = _sz
    L.sparse_attn_decode_step_workspace_size.argtypes = [_int, _int, _int, _int, _i64, _PP, _i32, _i32]
    L.sparse_attn_decode_step_splits.restype = _i32
    L.sparse_attn_decode_step_splits.argtypes = [_int, _int, _int, _i64, _PP, _i32, _i32, _i32]
    L.sparse_attn_decode_step.restype = _int
    L.sparse_attn_decode_step.argtypes = [_vp, _vp, _int, _vp, _vp, _vp, _int, _int, _int, _int, _int,
                                          _i64, _i64, _vp, _vp, _i32, _PP, _f32, _vp, _i32, _vp, _vp,
                                          _int, _vp, _i32, _vp, _sz, _vp]
    L.sparse_attn_decode_step_noalloc.restype = _int
    L.sparse_attn_decode_step_noalloc.argtypes = [_vp, _vp, _int, _vp, _vp, _vp, _int, _int, _int, _int,
                                                  _int, _i64, _i64, _vp, _vp, _i32, _PP, _f32, _vp,
                                                  _i32, _vp, _vp, _int, _vp, _i32, _vp]
    L.sparse_attn_cobs_stats.restype = _int
    L.sparse_attn_cobs_stats.argtypes = [_vp, _vp, _int, _int, _int, _int, _i64, _i64, _vp, _vp, _i32,
                                         _vp]
    L.sparse_attn_cobs_select_workspace_size.restype = _sz
    L.sparse_attn_cobs_select_workspace_size.argtypes = [_int, _int, _int, _i64, _PP]
    L.sparse_attn_cobs_select.restype = _int
    L.sparse_attn_cobs_select.argtypes = [_vp, _int, _vp, _int, _int, _int, _int, _i64, _i64, _vp,
                                          _PP, _i32, _vp, _i32, _vp, _vp, _vp, _sz, _vp]
    L.sparse_attn_cobs_decode_step_workspace_size.restype = _sz
    L.sparse_attn_cobs_decode_step_workspace_size.argtypes = [_int, _int, _int, _int, _i64, _PP, _i32,
                                                              _i32]
    L.sparse_attn_cobs_decode_step.restype = _int
    L.sparse_attn_cobs_decode_step.argtypes = [_vp, _vp, _int, _vp, _vp, _vp, _int, _int, _int, _int,
                                               _int, _i64, _i64, _vp, _vp, _i32, _PP, _i32, _f32,
                                               _vp, _i32, _vp, _vp, _int, _vp, _i32, _vp, _sz, _vp]
    L.sparse_attn_token_decode_workspace_size.restype = _sz
    L.sparse_attn_token_decode_workspace_size.argtypes = [_int, _int, _int, _i32, _i32]
    L.sparse_attn_token_decode.restype = _int
    L.sparse_attn_token_decode.argtypes = [_vp, _vp, _vp, _int, _int, _int, _int, _int, _i64, _vp,
                                           _vp, _vp, _i32, _f32, _vp, _int, _vp, _i32, _vp, _sz,
                                           _vp]
    _lib = L
    return L


def abi_version() -> int:
    return lib().sparse_attn_abi_version()


def status_string(status: int) -> str:
    return lib().sparse_attn_status_string(status).decode()


def _check(fn: str, status: int):
    if status != SA_OK:
        raise SparseAttnError(fn, status, status_string(status))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SA_F32
    if t.dtype == torch.bfloat16:
        return SA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t: torch.Tensor, name: str) -> int:
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be dense row-major (contiguous): the C ABI takes no strides")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return t.data_ptr()


def _expect(t, name: str, shape=None, dtype=None):
    """Raises ValueError unless t is a tensor of the given shape (None entries
    are free) and dtype (one dtype or a tuple of allowed ones)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be dense row-major (contiguous): the C ABI takes no strides")
    if shape is not None:
        if t.dim() != len(shape) or any(w is not None and int(g) != int(w)
                                        for g, w in zip(t.shape, shape)):
            want = "[" + ", ".join("*" if w is None else str(int(w)) for w in shape) + "]"
            raise ValueError(f"{name} must have shape {want}, got {list(t.shape)}")
    if dtype is not None:
        allowed = dtype if isinstance(dtype, tuple) else (dtype,)
        if t.dtype not in allowed:
            raise ValueError(f"{name} must have dtype {' or '.join(str(a) for a in allowed)}, "
                             f"got {t.dtype}")


_FLOAT = (torch.float32, torch.bfloat16)


def _check_kv(K, V, names=("K", "V")):
    """K, V [B, Hkv, T_cap, d] of one floating dtype; returns (B, Hkv, T_cap, d)."""
    _expect(K, names[0], (None, None, None, None), _FLOAT)
    if V is not None:
        _expect(V, names[1], tuple(K.shape), K.dtype)
    return tuple(int(x) for x in K.shape)


def _check_sets(idx, cnt, B, Hkv):
    if idx is not None:
        _expect(idx, "idx", (B, Hkv, None), torch.int32)
    if cnt is not None:
        _expect(cnt, "cnt", (B, Hkv), torch.int32)


def _check_out(O, lse, rows, Hq, d):
    if O is not None:
        _expect(O, "O", (rows, Hq, d), _FLOAT)
    if lse is not None:
        _expect(lse, "lse", (rows, Hq), torch.float32)


def _check_lens(B, **lens):
    for name, t in lens.items():
        _expect(t, name, (B,), torch.int32)


def _opt(t: Optional[torch.Tensor], name: str):
    return None if t is None else _dev(t, name)


def _stream(t: torch.Tensor, stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream(t.device)
    return s.cuda_stream


def n_compressed(L: int) -> int:
    return 0 if L < 32 else (L - 32) // 16 + 1


def n_blocks(L: int) -> int:
    return (L + 63) // 64


# ------------------------------------------------------------------ compress

def compress(K: torch.Tensor, Kc: torch.Tensor, lens_prev: torch.Tensor, lens_now: torch.Tensor,
             max_new_entries: Optional[int] = None, stream=None) -> torch.Tensor:
    """Write compressed-key entries [n_c(lens_prev), n_c(lens_now)) of Kc from K (in place)."""
    B, Hkv, T_cap, d = K.shape
    nc_cap = Kc.shape[2]
    if Kc.dtype != K.dtype or Kc.shape[:2] != K.shape[:2] or Kc.shape[3] != d:
        raise ValueError("Kc must be [B, Hkv, nc_cap, d] with K's dtype")
    _check_lens(B, lens_prev=lens_prev, lens_now=lens_now)
    if max_new_entries is None:
        max_new_entries = n_compressed(T_cap)
    st = lib().sparse_attn_compress(_dev(K, "K"), _dev(Kc, "Kc"), _dtype_code(K), B, Hkv, d, T_cap,
                                    nc_cap, _dev(lens_prev, "lens_prev"), _dev(lens_now, "lens_now"),
                                    int(max_new_entries), _stream(K, stream))
    _check("sparse_attn_compress", st)
    return Kc


# ------------------------------------------------------------------ select

def select_workspace_size(B, Hkv, H_sel, T_cap, params: SelectParams) -> int:
    return lib().sparse_attn_select_workspace_size(B, Hkv, H_sel, T_cap, ctypes.byref(params))


def select(sel: torch.Tensor, Kc: torch.Tensor, seq_lens: torch.Tensor, T_cap: int, top_k: int,
           n_init: int = 1, n_local: int = 2, score_mode="softmax_sum",
           idx: Optional[torch.Tensor] = None, cnt: Optional[torch.Tensor] = None,
           block_scores: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
           stream=None):
    """Block selection for every (sequence, KV head). Returns (idx, cnt, block_scores)."""
    _expect(Kc, "Kc", (None, None, None, None), _FLOAT)
    B, Hkv, nc_cap, d = Kc.shape
    _expect(sel, "sel", (B, None, d), Kc.dtype)
    H_sel = sel.shape[1]
    _check_lens(B, seq_lens=seq_lens)
    p = make_params(top_k, n_init, n_local, score_mode)
    cap = top_k + n_init + n_local
    dev = sel.device
    _check_sets(idx, cnt, B, Hkv)
    if isinstance(block_scores, torch.Tensor):
        _expect(block_scores, "block_scores", (B, Hkv, None), torch.float32)
    if idx is None:
        idx = torch.empty((B, Hkv, cap), dtype=torch.int32, device=dev)
    if cnt is None:
        cnt = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    if block_scores is True:
        block_scores = torch.empty((B, Hkv, n_blocks(T_cap)), dtype=torch.float32, device=dev)
    need = select_workspace_size(B, Hkv, H_sel, T_cap, p)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().sparse_attn_select(_dev(sel, "sel"), H_sel, _dev(Kc, "Kc"), _dtype_code(Kc), B, Hkv, d,
                                  T_cap, nc_cap, _dev(seq_lens, "seq_lens"), ctypes.byref(p),
                                  _dev(idx, "idx"), idx.shape[-1], _dev(cnt, "cnt"),
                                  _opt(block_scores if isinstance(block_scores, torch.Tensor) else None,
                                       "block_scores"),
                                  _opt(workspace, "workspace"), ws_bytes, _stream(sel, stream))
    _check("sparse_attn_select", st)
    return idx, cnt, (block_scores if isinstance(block_scores, torch.Tensor) else None)


# ------------------------------------------------------------------ decode

def decode_workspace_size(B, Hq, Hkv, idx_cap, n_split=0) -> int:
    return lib().sparse_attn_decode_workspace_size(B, Hq, Hkv, idx_cap, n_split)


def decode(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, seq_lens: torch.Tensor,
           idx: torch.Tensor, cnt: torch.Tensor, scale: float = 1.0,
           out_dtype=torch.float32, O: Optional[torch.Tensor] = None,
           lse: Optional[torch.Tensor] = None, want_lse: bool = True, n_split: int = 0,
           workspace: Optional[torch.Tensor] = None, stream=None):
    """Sparse decode attention over the selected blocks. Returns (O, lse)."""
    B, Hkv, T_cap, d = _check_kv(K, V)
    _expect(Q, "Q", (B, None, d), K.dtype)
    Hq = Q.shape[1]
    _check_lens(B, seq_lens=seq_lens)
    _expect(idx, "idx", (B, Hkv, None), torch.int32)
    _expect(cnt, "cnt", (B, Hkv), torch.int32)
    _check_out(O, lse, B, Hq, d)
    dev = Q.device
    if O is None:
        O = torch.empty((B, Hq, d), dtype=out_dtype, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    need = decode_workspace_size(B, Hq, Hkv, idx.shape[-1], n_split)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().sparse_attn_decode(_dev(Q, "Q"), _dev(K, "K"), _dev(V, "V"), _dtype_code(K), B, Hq, Hkv,
                                  d, T_cap, _dev(seq_lens, "seq_lens"), _dev(idx, "idx"),
                                  _dev(cnt, "cnt"), idx.shape[-1], float(scale), _dev(O, "O"),
                                  _dtype_code(O), _opt(lse, "lse"), int(n_split),
                                  _opt(workspace, "workspace"), ws_bytes, _stream(Q, stream))
    _check("sparse_attn_decode", st)
    return O, lse


# ------------------------------------------------------------------ prefill

def prefill_tile_cap(q_start: int, Tq: int, params: SelectParams) -> int:
    return lib().sparse_attn_prefill_tile_cap(q_start, Tq, ctypes.byref(params))


def prefill_workspace_size(Hq, Hkv, q_start, Tq, params: SelectParams) -> int:
    return lib().sparse_attn_prefill_workspace_size(Hq, Hkv, q_start, Tq, ctypes.byref(params))


def prefill_chunk(Q: torch.Tensor, q_start: int, K: torch.Tensor, V: torch.Tensor, Kc: torch.Tensor,
                  top_k: int, n_init: int = 1, n_local: int = 4, score_mode="softmax_sum",
                  scale: float = 1.0, out_dtype=torch.float32, O=None, lse=None, want_lse=True,
                  tile_idx=None, tile_cnt=None, workspace=None, stream=None):
    """Tile-shared sparse causal prefill of one chunk. Returns (O, lse, tile_idx, tile_cnt)."""
    K3 = K.reshape(K.shape[-3:]) if K.dim() == 4 and K.shape[0] == 1 else K
    _expect(K3, "K", (None, None, None), _FLOAT)
    Hkv, T_cap, d = K3.shape
    _expect(V, "V", tuple(K.shape), K.dtype)
    _expect(Q, "Q", (None, None, d), K.dtype)
    Tq, Hq = Q.shape[0], Q.shape[1]
    _expect(Kc, "Kc", tuple(K.shape[:-2]) + (None, d), K.dtype)
    nc_cap = Kc.shape[-2]
    _check_out(O, lse, Tq, Hq, d)
    p = make_params(top_k, n_init, n_local, score_mode)
    dev = Q.device
    n_tiles = (Tq + 63) // 64
    cap = prefill_tile_cap(q_start, Tq, p)
    if O is None:
        O = torch.empty((Tq, Hq, d), dtype=out_dtype, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((Tq, Hq), dtype=torch.float32, device=dev)
    if tile_idx is None:
        tile_idx = torch.empty((n_tiles, Hkv, cap), dtype=torch.int32, device=dev)
    if tile_cnt is None:
        tile_cnt = torch.empty((n_tiles, Hkv), dtype=torch.int32, device=dev)
    _expect(tile_idx, "tile_idx", (n_tiles, Hkv, None), torch.int32)
    _expect(tile_cnt, "tile_cnt", (n_tiles, Hkv), torch.int32)
    need = prefill_workspace_size(Hq, Hkv, q_start, Tq, p)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().sparse_attn_prefill_chunk(_dev(Q, "Q"), int(q_start), Tq, _dev(K, "K"), _dev(V, "V"),
                                         _dev(Kc, "Kc"), _dtype_code(K), Hq, Hkv, d, T_cap, nc_cap,
                                         ctypes.byref(p), float(scale), _dev(O, "O"), _dtype_code(O),
                                         _opt(lse, "lse"), _dev(tile_idx, "tile_idx"),
                                         tile_idx.shape[-1], _dev(tile_cnt, "tile_cnt"),
                                         _opt(workspace, "workspace"), ws_bytes, _stream(Q, stream))
    _check("sparse_attn_prefill_chunk", st)
    return O, lse, tile_idx, tile_cnt


def prefill_attend(Q: torch.Tensor, q_start: int, K: torch.Tensor, V: torch.Tensor,
                   tile_idx: torch.Tensor, tile_cnt: torch.Tensor, scale: float = 1.0,
                   out_dtype=torch.float32, O=None, lse=None, want_lse=True, stream=None):
    """Causal attention of a prefill chunk over given tile block sets. Returns (O, lse)."""
    K3 = K.reshape(K.shape[-3:]) if K.dim() == 4 and K.shape[0] == 1 else K
    _expect(K3, "K", (None, None, None), _FLOAT)
    Hkv, T_cap, d = K3.shape
    _expect(V, "V", tuple(K.shape), K.dtype)
    _expect(Q, "Q", (None, None, d), K.dtype)
    Tq, Hq = Q.shape[0], Q.shape[1]
    n_tiles = (Tq + 63) // 64
    _expect(tile_idx, "tile_idx", (n_tiles, Hkv, None), torch.int32)
    _expect(tile_cnt, "tile_cnt", (n_tiles, Hkv), torch.int32)
    _check_out(O, lse, Tq, Hq, d)
    dev = Q.device
    if O is None:
        O = torch.empty((Tq, Hq, d), dtype=out_dtype, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((Tq, Hq), dtype=torch.float32, device=dev)
    st = lib().sparse_attn_prefill_attend(_dev(Q, "Q"), int(q_start), Tq, _dev(K, "K"), _dev(V, "V"),
                                          _dtype_code(K), Hq, Hkv, d, T_cap,
                                          _dev(tile_idx, "tile_idx"), tile_idx.shape[-1],
                                          _dev(tile_cnt, "tile_cnt"), float(scale), _dev(O, "O"),
                                          _dtype_code(O), _opt(lse, "lse"), _stream(Q, stream))
    _check("sparse_attn_prefill_attend", st)
    return O, lse


def stream_read(buf: torch.Tensor, xor_out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Reads a contiguous device buffer once (HBM stream-read ceiling measurement).
    Returns the per-workgroup XOR words (int32 view of uint32)."""
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    nbytes = buf.numel() * buf.element_size()
    if xor_out is None:
        xor_out = torch.empty(lib().sparse_attn_stream_read_blocks(), dtype=torch.int32, device=buf.device)
    st = lib().sparse_attn_stream_read(_dev(buf, "buf"), nbytes, _dev(xor_out, "xor_out"), _stream(buf, stream))
    _check("sparse_attn_stream_read", st)
    return xor_out


def block_mass(Q: torch.Tensor, K: torch.Tensor, seq_lens: torch.Tensor, scale: float = 1.0,
               idx: Optional[torch.Tensor] = None, cnt: Optional[torch.Tensor] = None,
               mass: Optional[torch.Tensor] = None, recall: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None, stream=None):
    """Exact attention mass per 64-token block of each head's decode query, and
    the recall of (idx, cnt) if given. Returns (mass [B, Hq, nb], recall or None)."""
    B, Hkv, T_cap, d = _check_kv(K, None)
    _expect(Q, "Q", (B, None, d), K.dtype)
    Hq = Q.shape[1]
    _check_lens(B, seq_lens=seq_lens)
    if idx is not None or cnt is not None:
        _expect(idx, "idx", (B, Hkv, None), torch.int32)
        _expect(cnt, "cnt", (B, Hkv), torch.int32)
    if mass is not None:
        _expect(mass, "mass", (B, Hq, None), torch.float32)
    if recall is not None:
        _expect(recall, "recall", (B, Hq), torch.float32)
    nb = n_blocks(T_cap)
    if mass is None:
        mass = torch.empty((B, Hq, nb), dtype=torch.float32, device=Q.device)
    if idx is not None and recall is None:
        recall = torch.empty((B, Hq), dtype=torch.float32, device=Q.device)
    ws_need = lib().sparse_attn_block_mass_workspace_size(B, Hq, mass.shape[-1])
    if workspace is None:
        workspace = torch.empty(max(ws_need, 1), dtype=torch.uint8, device=Q.device)
    st = lib().sparse_attn_block_mass(_dev(Q, "Q"), _dev(K, "K"), _dtype_code(K), B, Hq, Hkv, d, T_cap,
                                      _dev(seq_lens, "seq_lens"), float(scale), _dev(mass, "mass"),
                                      mass.shape[-1], _opt(idx, "idx"), _opt(cnt, "cnt"),
                                      idx.shape[-1] if idx is not None else 0, _opt(recall, "recall"),
                                      _dev(workspace, "workspace"), workspace.numel(), _stream(Q, stream))
    _check("sparse_attn_block_mass", st)
    return mass, recall


# ------------------------------------------------------------------ token-level index

def token_select_workspace_size(B, Hkv, T_cap) -> int:
    return lib().sparse_attn_token_select_workspace_size(B, Hkv, T_cap)


def token_select(sel: torch.Tensor, Ki: torch.Tensor, seq_lens: torch.Tensor, top_k: int,
                 n_init: int = 64, n_local: int = 128, idx: Optional[torch.Tensor] = None,
                 cnt: Optional[torch.Tensor] = None, scores=None,
                 workspace: Optional[torch.Tensor] = None, stream=None):
    """Token-level index per (sequence, KV head): kept initial/local tokens and
    the top_k scored tokens, ascending. Returns (idx, cnt, scores or None)."""
    B, Hkv, T_cap, d_i = _check_kv(Ki, None, ("Ki", ""))
    _expect(sel, "sel", (B, None, d_i), Ki.dtype)
    H_sel = sel.shape[1]
    _check_lens(B, seq_lens=seq_lens)
    _check_sets(idx, cnt, B, Hkv)
    if isinstance(scores, torch.Tensor):
        _expect(scores, "scores", (B, Hkv, T_cap), torch.float32)
    dev = sel.device
    if idx is None:
        idx = torch.empty((B, Hkv, top_k + n_init + n_local), dtype=torch.int32, device=dev)
    if cnt is None:
        cnt = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    if scores is True:
        scores = torch.empty((B, Hkv, T_cap), dtype=torch.float32, device=dev)
    need = token_select_workspace_size(B, Hkv, T_cap)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    sc = scores if isinstance(scores, torch.Tensor) else None
    st = lib().sparse_attn_token_select(_dev(sel, "sel"), H_sel, _dev(Ki, "Ki"), _dtype_code(Ki), B,
                                        Hkv, d_i, T_cap, _dev(seq_lens, "seq_lens"), int(top_k),
                                        int(n_init), int(n_local), _dev(idx, "idx"), idx.shape[-1],
                                        _dev(cnt, "cnt"), _opt(sc, "scores"),
                                        _dev(workspace, "workspace"), ws_bytes, _stream(sel, stream))
    _check("sparse_attn_token_select", st)
    return idx, cnt, sc


def token_decode_workspace_size(B, Hq, Hkv, idx_cap, n_split=0) -> int:
    return lib().sparse_attn_token_decode_workspace_size(B, Hq, Hkv, idx_cap, n_split)


def token_decode(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, seq_lens: torch.Tensor,
                 idx: torch.Tensor, cnt: torch.Tensor, scale: float = 1.0,
                 out_dtype=torch.float32, O: Optional[torch.Tensor] = None,
                 lse: Optional[torch.Tensor] = None, want_lse: bool = True, n_split: int = 0,
                 workspace: Optional[torch.Tensor] = None, stream=None):
    """Sparse decode attention over token lists (gathered rows). Returns (O, lse)."""
    B, Hkv, T_cap, d = _check_kv(K, V)
    _expect(Q, "Q", (B, None, d), K.dtype)
    Hq = Q.shape[1]
    _check_lens(B, seq_lens=seq_lens)
    _expect(idx, "idx", (B, Hkv, None), torch.int32)
    _expect(cnt, "cnt", (B, Hkv), torch.int32)
    _check_out(O, lse, B, Hq, d)
    dev = Q.device
    if O is None:
        O = torch.empty((B, Hq, d), dtype=out_dtype, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    need = token_decode_workspace_size(B, Hq, Hkv, idx.shape[-1], n_split)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().sparse_attn_token_decode(_dev(Q, "Q"), _dev(K, "K"), _dev(V, "V"), _dtype_code(K), B,
                                        Hq, Hkv, d, T_cap, _dev(seq_lens, "seq_lens"),
                                        _dev(idx, "idx"), _dev(cnt, "cnt"), idx.shape[-1],
                                        float(scale), _dev(O, "O"), _dtype_code(O), _opt(lse, "lse"),
                                        int(n_split), _opt(workspace, "workspace"), ws_bytes,
                                        _stream(Q, stream))
    _check("sparse_attn_token_decode", st)
    return O, lse


# ------------------------------------------------------------------ second-order block statistic

def cobs_stats(K: torch.Tensor, stats: torch.Tensor, lens_prev: torch.Tensor, lens_now: torch.Tensor,
               max_new_blocks: Optional[int] = None, stream=None) -> torch.Tensor:
    """Write the mean and per-channel variance rows of the blocks completed
    between lens_prev and lens_now into stats [B, Hkv, nb_cap, 2, d] (in place)."""
    B, Hkv, T_cap, d = K.shape
    nb_cap = stats.shape[2]
    if stats.dtype != K.dtype or stats.shape[:2] != K.shape[:2] or stats.shape[3:] != (2, d):
        raise ValueError("stats must be [B, Hkv, nb_cap, 2, d] with K's dtype")
    _check_lens(B, lens_prev=lens_prev, lens_now=lens_now)
    if max_new_blocks is None:
        max_new_blocks = nb_cap
    st = lib().sparse_attn_cobs_stats(_dev(K, "K"), _dev(stats, "stats"), _dtype_code(K), B, Hkv, d,
                                      T_cap, nb_cap, _dev(lens_prev, "lens_prev"),
                                      _dev(lens_now, "lens_now"), int(max_new_blocks),
                                      _stream(K, stream))
    _check("sparse_attn_cobs_stats", st)
    return stats


def cobs_select_workspace_size(B, Hkv, H_sel, T_cap, params: SelectParams) -> int:
    return lib().sparse_attn_cobs_select_workspace_size(B, Hkv, H_sel, T_cap, ctypes.byref(params))


def cobs_select(sel: torch.Tensor, stats: torch.Tensor, seq_lens: torch.Tensor, T_cap: int, top_k: int,
                n_init: int = 1, n_local: int = 2, score_mode="softmax_sum", order: int = 2,
                idx: Optional[torch.Tensor] = None, cnt: Optional[torch.Tensor] = None,
                block_scores=None, workspace: Optional[torch.Tensor] = None, stream=None):
    """Block selection by the first- or second-order block-mass estimate.
    Returns (idx, cnt, block_scores or None)."""
    _expect(stats, "stats", (None, None, None, 2, None), _FLOAT)
    B, Hkv, nb_cap, _, d = stats.shape
    _expect(sel, "sel", (B, None, d), stats.dtype)
    H_sel = sel.shape[1]
    _check_lens(B, seq_lens=seq_lens)
    _check_sets(idx, cnt, B, Hkv)
    if isinstance(block_scores, torch.Tensor):
        _expect(block_scores, "block_scores", (B, Hkv, None), torch.float32)
    p = make_params(top_k, n_init, n_local, score_mode)
    dev = sel.device
    if idx is None:
        idx = torch.empty((B, Hkv, top_k + n_init + n_local), dtype=torch.int32, device=dev)
    if cnt is None:
        cnt = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    if block_scores is True:
        block_scores = torch.empty((B, Hkv, n_blocks(T_cap)), dtype=torch.float32, device=dev)
    bs = block_scores if isinstance(block_scores, torch.Tensor) else None
    need = cobs_select_workspace_size(B, Hkv, H_sel, T_cap, p)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().sparse_attn_cobs_select(_dev(sel, "sel"), H_sel, _dev(stats, "stats"),
                                       _dtype_code(stats), B, Hkv, d, T_cap, nb_cap,
                                       _dev(seq_lens, "seq_lens"), ctypes.byref(p), int(order),
                                       _dev(idx, "idx"), idx.shape[-1], _dev(cnt, "cnt"),
                                       _opt(bs, "block_scores"), _dev(workspace, "workspace"),
                                       ws_bytes, _stream(sel, stream))
    _check("sparse_attn_cobs_select", st)
    return idx, cnt, bs


def cobs_decode_step_workspace_size(B, Hq, Hkv, H_sel, T_cap, params: SelectParams, idx_cap,
                                    n_split=0) -> int:
    return lib().sparse_attn_cobs_decode_step_workspace_size(B, Hq, Hkv, H_sel, T_cap,
                                                             ctypes.byref(params), idx_cap, n_split)


def cobs_decode_step(Q: torch.Tensor, sel: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
                     stats: torch.Tensor, lens_prev: torch.Tensor, lens_now: torch.Tensor,
                     top_k: int, n_init: int = 1, n_local: int = 2, score_mode="softmax_sum",
                     order: int = 2, scale: float = 1.0, max_new_blocks: int = 1, idx=None,
                     cnt=None, O=None, lse=None, want_lse=True, out_dtype=torch.float32,
                     n_split: int = 0, workspace=None, stream=None):
    """Statistics append + selection by block statistics + decode attention in
    one call. Returns (O, lse, idx, cnt)."""
    B, Hkv, T_cap, d = _check_kv(K, V)
    _expect(Q, "Q", (B, None, d), K.dtype)
    _expect(sel, "sel", (B, None, d), K.dtype)
    _expect(stats, "stats", (B, Hkv, None, 2, d), K.dtype)
    Hq, H_sel = Q.shape[1], sel.shape[1]
    _check_lens(B, lens_prev=lens_prev, lens_now=lens_now)
    _check_sets(idx, cnt, B, Hkv)
    _check_out(O, lse, B, Hq, d)
    nb_cap = stats.shape[2]
    p = make_params(top_k, n_init, n_local, score_mode)
    dev = Q.device
    cap = top_k + n_init + n_local
    if idx is None:
        idx = torch.empty((B, Hkv, cap), dtype=torch.int32, device=dev)
    if cnt is None:
        cnt = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    if O is None:
        O = torch.empty((B, Hq, d), dtype=out_dtype, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    need = cobs_decode_step_workspace_size(B, Hq, Hkv, H_sel, T_cap, p, idx.shape[-1], n_split)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().sparse_attn_cobs_decode_step(_dev(Q, "Q"), _dev(sel, "sel"), H_sel, _dev(K, "K"),
                                            _dev(V, "V"), _dev(stats, "stats"), _dtype_code(K), B,
                                            Hq, Hkv, d, T_cap, nb_cap, _dev(lens_prev, "lens_prev"),
                                            _dev(lens_now, "lens_now"), int(max_new_blocks),
                                            ctypes.byref(p), int(order), float(scale),
                                            _dev(idx, "idx"), idx.shape[-1], _dev(cnt, "cnt"),
                                            _dev(O, "O"), _dtype_code(O), _opt(lse, "lse"),
                                            int(n_split), _dev(workspace, "workspace"), ws_bytes,
                                            _stream(Q, stream))
    _check("sparse_attn_cobs_decode_step", st)
    return O, lse, idx, cnt


# ------------------------------------------------------------------ whole decode step

def decode_step_workspace_size(B, Hq, Hkv, H_sel, T_cap, params: SelectParams, idx_cap,
                               n_split=0) -> int:
    return lib().sparse_attn_decode_step_workspace_size(B, Hq, Hkv, H_sel, T_cap, ctypes.byref(params),
                                                        idx_cap, n_split)


def decode_step_splits(dtype, B, Hkv, T_cap, params: SelectParams, idx_cap, max_new_tokens=1,
                       n_split=0) -> int:
    """Split-K workgroups per (b, kvh) of decode_step's attention with these
    arguments (dtype: the key dtype, torch.bfloat16 or torch.float32)."""
    code = {torch.bfloat16: 1, torch.float32: 0}[dtype]
    return lib().sparse_attn_decode_step_splits(code, B, Hkv, T_cap, ctypes.byref(params), idx_cap,
                                                int(max_new_tokens), int(n_split))


def decode_step(Q: torch.Tensor, sel: torch.Tensor, K: torch.Tensor, V: torch.Tensor, Kc: torch.Tensor,
                lens_prev: torch.Tensor, lens_now: torch.Tensor, top_k: int, n_init: int = 1,
                n_local: int = 2, score_mode="softmax_sum", scale: float = 1.0,
                max_new_tokens: int = 1, idx=None, cnt=None, O=None, lse=None, want_lse=True,
                out_dtype=torch.float32, n_split: int = 0, workspace=None, stream=None):
    """Append + select + decode attention in one call. Returns (O, lse, idx, cnt)."""
    B, Hkv, T_cap, d = _check_kv(K, V)
    _expect(Q, "Q", (B, None, d), K.dtype)
    _expect(sel, "sel", (B, None, d), K.dtype)
    _expect(Kc, "Kc", (B, Hkv, None, d), K.dtype)
    Hq, H_sel = Q.shape[1], sel.shape[1]
    _check_lens(B, lens_prev=lens_prev, lens_now=lens_now)
    _check_sets(idx, cnt, B, Hkv)
    _check_out(O, lse, B, Hq, d)
    nc_cap = Kc.shape[2]
    p = make_params(top_k, n_init, n_local, score_mode)
    dev = Q.device
    cap = top_k + n_init + n_local
    if idx is None:
        idx = torch.empty((B, Hkv, cap), dtype=torch.int32, device=dev)
    if cnt is None:
        cnt = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    if O is None:
        O = torch.empty((B, Hq, d), dtype=out_dtype, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    need = decode_step_workspace_size(B, Hq, Hkv, H_sel, T_cap, p, idx.shape[-1], n_split)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().sparse_attn_decode_step(_dev(Q, "Q"), _dev(sel, "sel"), H_sel, _dev(K, "K"), _dev(V, "V"),
                                       _dev(Kc, "Kc"), _dtype_code(K), B, Hq, Hkv, d, T_cap, nc_cap,
                                       _dev(lens_prev, "lens_prev"), _dev(lens_now, "lens_now"),
                                       int(max_new_tokens), ctypes.byref(p), float(scale),
                                       _dev(idx, "idx"), idx.shape[-1], _dev(cnt, "cnt"), _dev(O, "O"),
                                       _dtype_code(O), _opt(lse, "lse"), int(n_split),
                                       _dev(workspace, "workspace"), ws_bytes, _stream(Q, stream))
    _check("sparse_attn_decode_step", st)
    return O, lse, idx, cnt


def decode_step_noalloc(Q: torch.Tensor, sel: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
                        Kc: torch.Tensor, lens_prev: torch.Tensor, lens_now: torch.Tensor,
                        top_k: int, n_init: int = 1, n_local: int = 2, score_mode="softmax_sum",
                        scale: float = 1.0, max_new_tokens: int = 1, idx=None, cnt=None, O=None,
                        lse=None, want_lse=True, out_dtype=torch.float32, n_split: int = 0,
                        stream=None):
    """decode_step without a workspace: the library's fixed per-GPU scratch
    array serves as scratch (nothing is allocated for it). Calls that overlap
    on one GPU race on that array. Returns (O, lse, idx, cnt)."""
    B, Hkv, T_cap, d = _check_kv(K, V)
    _expect(Q, "Q", (B, None, d), K.dtype)
    _expect(sel, "sel", (B, None, d), K.dtype)
    _expect(Kc, "Kc", (B, Hkv, None, d), K.dtype)
    Hq, H_sel = Q.shape[1], sel.shape[1]
    _check_lens(B, lens_prev=lens_prev, lens_now=lens_now)
    _check_sets(idx, cnt, B, Hkv)
    _check_out(O, lse, B, Hq, d)
    nc_cap = Kc.shape[2]
    p = make_params(top_k, n_init, n_local, score_mode)
    dev = Q.device
    cap = top_k + n_init + n_local
    if idx is None:
        idx = torch.empty((B, Hkv, cap), dtype=torch.int32, device=dev)
    if cnt is None:
        cnt = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    if O is None:
        O = torch.empty((B, Hq, d), dtype=out_dtype, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    st = lib().sparse_attn_decode_step_noalloc(_dev(Q, "Q"), _dev(sel, "sel"), H_sel, _dev(K, "K"),
                                               _dev(V, "V"), _dev(Kc, "Kc"), _dtype_code(K), B, Hq,
                                               Hkv, d, T_cap, nc_cap, _dev(lens_prev, "lens_prev"),
                                               _dev(lens_now, "lens_now"), int(max_new_tokens),
                                               ctypes.byref(p), float(scale), _dev(idx, "idx"),
                                               idx.shape[-1], _dev(cnt, "cnt"), _dev(O, "O"),
                                               _dtype_code(O), _opt(lse, "lse"), int(n_split),
                                               _stream(Q, stream))
    _check("sparse_attn_decode_step_noalloc", st)
    return O, lse, idx, cnt
