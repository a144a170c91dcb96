"""Python binding of libqsa.so, the MI355X (gfx950) QSA micro-block sparse
attention hot path.

Argument marshalling only: torch tensors become device pointers and the
current HIP stream; every step runs in the library's HIP kernels.  The C
declarations, with the meaning, layout and error behaviour of every argument,
are in ``include/qsa.h``.  The functions keep the C names:

    qsa_compress_keys, qsa_block_scores, qsa_decode_scores_refresh, qsa_topk_blocks, qsa_topk_blocks_ws,
    qsa_sparse_attn_decode, qsa_sparse_attn_extend, qsa_merge_lse,
    qsa_decode_fused (scores + top-k + attention + merge in one launch),
    qsa_sparse_attn_decode_noalloc (decode attention with no workspace: static device scratch)

Importing this module does not need a GPU; calling a function that launches
work does.  If ``libqsa.so`` has not been built, loading fails with an error:
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libqsa.so")

QSA_OK = 0
QSA_ERR_INVALID_ARG = -1
QSA_ERR_UNSUPPORTED = -2
QSA_ERR_HIP = -3
HEAD_DIM = 256
MICROBLOCK = 4
DEFAULT_TOPK = 512
MAX_TOPK = 2048
MAX_SPLITS = 64
CKEY_FP32 = 0
CKEY_BF16 = 1
CKEY_FP8 = 2
KV_BF16 = 0
KV_FP8 = 1

EXPORTS = ("qsa_version", "qsa_last_error", "qsa_compress_keys", "qsa_block_scores", "qsa_topk_blocks",
           "qsa_sparse_attn_decode", "qsa_decode_workspace_bytes", "qsa_sparse_attn_extend", "qsa_merge_lse",
           "qsa_decode_fused", "qsa_decode_fused_workspace_bytes", "qsa_topk_blocks_ws",
           "qsa_topk_workspace_bytes", "qsa_decode_scores_refresh", "qsa_sparse_attn_decode_noalloc",
           "qsa_sparse_attn_extend_union", "qsa_sparse_attn_extend_split", "qsa_extend_workspace_bytes")


class QsaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{msg} (status {code})")
        self.code = code


class qsa_kv_t(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("ckey", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("batch", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
        ("ckey_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libqsa.so (raises if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        kvp = ctypes.POINTER(qsa_kv_t)
        L.qsa_version.argtypes, L.qsa_version.restype = [], ctypes.c_int
        L.qsa_last_error.argtypes, L.qsa_last_error.restype = [], ctypes.c_char_p
        L.qsa_compress_keys.argtypes = [kvp, vp, i32, vp]
        L.qsa_block_scores.argtypes = [kvp, vp, i64, vp, vp, i32, i32, vp, i32, vp]
        L.qsa_decode_scores_refresh.argtypes = [kvp, vp, i64, i32, vp, i32, vp]
        L.qsa_topk_blocks.argtypes = [vp, i32, vp, i32, i32, i32, vp, vp, vp]
        L.qsa_topk_blocks_ws.argtypes = [vp, i32, vp, i32, i32, i32, vp, vp, vp, sz, vp]
        L.qsa_topk_workspace_bytes.argtypes, L.qsa_topk_workspace_bytes.restype = [i32, i32, i32, i32], sz
        L.qsa_sparse_attn_decode.argtypes = [kvp, vp, i64, i32, vp, vp, i32, f32, i32, vp, i64, vp, vp, vp, vp, sz, vp]
        L.qsa_decode_workspace_bytes.argtypes, L.qsa_decode_workspace_bytes.restype = [i32, i32, i32], sz
        L.qsa_sparse_attn_decode_noalloc.argtypes = [kvp, vp, i64, i32, vp, vp, i32, f32, i32, vp, i64, vp, vp]
        L.qsa_sparse_attn_extend.argtypes = [kvp, vp, i64, vp, vp, i32, i32, vp, vp, i32, f32, vp, i64, vp, vp]
        L.qsa_sparse_attn_extend_union.argtypes = [kvp, vp, i64, vp, vp, i32, i32, vp, vp, i32, f32, vp, i64, vp, vp]
        L.qsa_sparse_attn_extend_split.argtypes = [kvp, vp, i64, vp, vp, i32, i32, vp, vp, i32, f32, i32, vp, i64, vp,
                                                   vp, sz, vp]
        L.qsa_extend_workspace_bytes.argtypes, L.qsa_extend_workspace_bytes.restype = [i32, i32, i32], sz
        L.qsa_merge_lse.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp]
        L.qsa_decode_fused.argtypes = [kvp, vp, i64, i32, i32, f32, i32, vp, vp, vp, i64, vp, vp, sz, vp]
        L.qsa_decode_fused_workspace_bytes.argtypes = [kvp, i32, i32, i32]
        L.qsa_decode_fused_workspace_bytes.restype = sz
        for f in ("qsa_compress_keys", "qsa_block_scores", "qsa_decode_scores_refresh", "qsa_topk_blocks",
                  "qsa_topk_blocks_ws", "qsa_sparse_attn_decode", "qsa_sparse_attn_extend", "qsa_merge_lse",
                  "qsa_decode_fused", "qsa_sparse_attn_decode_noalloc", "qsa_sparse_attn_extend_union",
                  "qsa_sparse_attn_extend_split"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int):
    if rc != QSA_OK:
        raise QsaError(rc, lib().qsa_last_error().decode())


def _ptr(t) -> Optional[int]:
    """Device address of a tensor (None -> NULL); ints pass through (raw pointers)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch

    return torch.cuda.current_stream().cuda_stream


@dataclass
class KVCache:
    """A paged cache as torch tensors (device memory owned by the caller).

    k, v: bf16 [num_pages][Hkv][page_size][256]; ckey: fp32 or bf16 [num_pages][Hkv][page_size/4][256]
    (its dtype selects the block-key format);
    block_table: int32 [batch][max_pages]; seq_lens: int32 [batch]; max_seq_len: host bound."""

    k: object
    v: object
    ckey: object
    block_table: object
    seq_lens: object
    max_seq_len: int

    def descriptor(self) -> qsa_kv_t:
        num_pages, hkv, page_size, d = self.k.shape
        dt = str(getattr(self.ckey, "dtype", "")) if self.ckey is not None else ""
        ckey_dtype = {"torch.bfloat16": CKEY_BF16, "torch.float8_e4m3fn": CKEY_FP8}.get(dt, CKEY_FP32)
        kv_dtype = KV_FP8 if str(getattr(self.k, "dtype", "")) == "torch.float8_e4m3fn" else KV_BF16
        return qsa_kv_t(_ptr(self.k), _ptr(self.v), _ptr(self.ckey), _ptr(self.block_table), _ptr(self.seq_lens),
                        int(self.block_table.shape[0]), int(hkv), int(d), int(page_size), int(num_pages),
                        int(self.block_table.shape[1]), int(self.max_seq_len), ckey_dtype, kv_dtype)


def _kv(kv) -> qsa_kv_t:
    return kv.descriptor() if isinstance(kv, KVCache) else kv


def qsa_version() -> int:
    return int(lib().qsa_version())


def qsa_last_error() -> str:
    return lib().qsa_last_error().decode()


def qsa_compress_keys(kv, first_token=None, max_new_tokens: int = 0, stream=None) -> None:
    d = _kv(kv)
    _check(lib().qsa_compress_keys(ctypes.byref(d), _ptr(first_token), max_new_tokens, _stream(stream)))


def qsa_block_scores(kv, q, q_row_stride: int, q_seq, q_pos, R: int, Hq: int, scores, score_stride: int,
                     stream=None) -> None:
    d = _kv(kv)
    _check(lib().qsa_block_scores(ctypes.byref(d), _ptr(q), q_row_stride, _ptr(q_seq), _ptr(q_pos), R, Hq,
                                  _ptr(scores), score_stride, _stream(stream)))


def qsa_decode_scores_refresh(kv, q, q_row_stride: int, Hq: int, scores, score_stride: int, stream=None) -> None:
    d = _kv(kv)
    _check(lib().qsa_decode_scores_refresh(ctypes.byref(d), _ptr(q), q_row_stride, Hq, _ptr(scores), score_stride,
                                           _stream(stream)))


def qsa_topk_blocks(scores, score_stride: int, q_pos, R: int, Hkv: int, k: int, sel_idx, sel_cnt,
                    stream=None) -> None:
    _check(lib().qsa_topk_blocks(_ptr(scores), score_stride, _ptr(q_pos), R, Hkv, k, _ptr(sel_idx), _ptr(sel_cnt),
                                 _stream(stream)))


def qsa_topk_workspace_bytes(R: int, Hkv: int, k: int, score_stride: int) -> int:
    return int(lib().qsa_topk_workspace_bytes(R, Hkv, k, score_stride))


def qsa_topk_blocks_ws(scores, score_stride: int, q_pos, R: int, Hkv: int, k: int, sel_idx, sel_cnt,
                       workspace=None, workspace_bytes: int = 0, stream=None) -> None:
    _check(lib().qsa_topk_blocks_ws(_ptr(scores), score_stride, _ptr(q_pos), R, Hkv, k, _ptr(sel_idx),
                                    _ptr(sel_cnt), _ptr(workspace), workspace_bytes, _stream(stream)))


def qsa_decode_workspace_bytes(batch: int, Hq: int, num_splits: int) -> int:
    return int(lib().qsa_decode_workspace_bytes(batch, Hq, num_splits))


def qsa_sparse_attn_decode(kv, q, q_row_stride: int, Hq: int, sel_idx, sel_cnt, k: int, scale: float,
                           num_splits: int, out, out_row_stride: int, lse=None, part_out=None, part_lse=None,
                           workspace=None, workspace_bytes: int = 0, stream=None) -> None:
    d = _kv(kv)
    _check(lib().qsa_sparse_attn_decode(ctypes.byref(d), _ptr(q), q_row_stride, Hq, _ptr(sel_idx), _ptr(sel_cnt), k,
                                        scale, num_splits, _ptr(out), out_row_stride, _ptr(lse), _ptr(part_out),
                                        _ptr(part_lse), _ptr(workspace), workspace_bytes, _stream(stream)))


def qsa_sparse_attn_decode_noalloc(kv, q, q_row_stride: int, Hq: int, sel_idx, sel_cnt, k: int, scale: float,
                                   num_splits: int, out, out_row_stride: int, lse=None, stream=None) -> None:
    d = _kv(kv)
    _check(lib().qsa_sparse_attn_decode_noalloc(ctypes.byref(d), _ptr(q), q_row_stride, Hq, _ptr(sel_idx),
                                                _ptr(sel_cnt), k, scale, num_splits, _ptr(out), out_row_stride,
                                                _ptr(lse), _stream(stream)))


def qsa_sparse_attn_extend(kv, q, q_row_stride: int, q_seq, q_pos, R: int, Hq: int, sel_idx, sel_cnt, k: int,
                           scale: float, out, out_row_stride: int, lse=None, stream=None) -> None:
    d = _kv(kv)
    _check(lib().qsa_sparse_attn_extend(ctypes.byref(d), _ptr(q), q_row_stride, _ptr(q_seq), _ptr(q_pos), R, Hq,
                                        _ptr(sel_idx), _ptr(sel_cnt), k, scale, _ptr(out), out_row_stride,
                                        _ptr(lse), _stream(stream)))


def qsa_extend_workspace_bytes(R: int, Hq: int, num_splits: int) -> int:
    return int(lib().qsa_extend_workspace_bytes(R, Hq, num_splits))


def qsa_sparse_attn_extend_split(kv, q, q_row_stride: int, q_seq, q_pos, R: int, Hq: int, sel_idx, sel_cnt, k: int,
                                 scale: float, num_splits: int, out, out_row_stride: int, lse=None, workspace=None,
                                 workspace_bytes: int = 0, stream=None) -> None:
    d = _kv(kv)
    _check(lib().qsa_sparse_attn_extend_split(ctypes.byref(d), _ptr(q), q_row_stride, _ptr(q_seq), _ptr(q_pos), R, Hq,
                                              _ptr(sel_idx), _ptr(sel_cnt), k, scale, num_splits, _ptr(out),
                                              out_row_stride, _ptr(lse), _ptr(workspace), workspace_bytes,
                                              _stream(stream)))


def qsa_sparse_attn_extend_union(kv, q, q_row_stride: int, q_seq, q_pos, R: int, Hq: int, sel_idx, sel_cnt, k: int,
                                 scale: float, out, out_row_stride: int, lse=None, stream=None) -> None:
    d = _kv(kv)
    _check(lib().qsa_sparse_attn_extend_union(ctypes.byref(d), _ptr(q), q_row_stride, _ptr(q_seq), _ptr(q_pos), R, Hq,
                                              _ptr(sel_idx), _ptr(sel_cnt), k, scale, _ptr(out), out_row_stride,
                                              _ptr(lse), _stream(stream)))


def qsa_merge_lse(part_out, part_lse, S: int, N: int, D: int, out, out_lse=None, stream=None) -> None:
    _check(lib().qsa_merge_lse(_ptr(part_out), _ptr(part_lse), S, N, D, _ptr(out), _ptr(out_lse), _stream(stream)))


def qsa_decode_fused_workspace_bytes(kv, Hq: int, k: int, num_splits: int = 0) -> int:
    d = _kv(kv)
    return int(lib().qsa_decode_fused_workspace_bytes(ctypes.byref(d), Hq, k, num_splits))


def qsa_decode_fused(kv, q, q_row_stride: int, Hq: int, k: int, scale: float, num_splits: int, sel_idx, sel_cnt,
                     out, out_row_stride: int, lse=None, workspace=None, workspace_bytes: int = 0,
                     stream=None) -> None:
    d = _kv(kv)
    _check(lib().qsa_decode_fused(ctypes.byref(d), _ptr(q), q_row_stride, Hq, k, scale, num_splits, _ptr(sel_idx),
                                  _ptr(sel_cnt), _ptr(out), out_row_stride, _ptr(lse), _ptr(workspace),
                                  workspace_bytes, _stream(stream)))
