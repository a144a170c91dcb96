"""Step drivers: the QSA decode and extend passes as sequences of libqsa calls.

Buffers are torch tensors on the current device (plumbing); every step runs in
the library's HIP kernels, in the order of the method -- block keys, block
scores, top-k selection, sparse attention, log-sum-exp merge.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import (HEAD_DIM, KVCache, qsa_block_scores, qsa_compress_keys, qsa_decode_fused, qsa_decode_scores_refresh,
               qsa_decode_fused_workspace_bytes, qsa_decode_workspace_bytes, qsa_sparse_attn_decode,
               qsa_extend_workspace_bytes, qsa_sparse_attn_extend, qsa_sparse_attn_extend_split,
               qsa_sparse_attn_extend_union, qsa_topk_blocks, qsa_topk_blocks_ws, qsa_topk_workspace_bytes)


@dataclass
class DecodeBuffers:
    """Intermediate and output buffers of one decode step."""

    scores: torch.Tensor      # fp32 [B][Hkv][score_stride]
    sel_idx: torch.Tensor     # int32 [B][Hkv][k]
    sel_cnt: torch.Tensor     # int32 [B][Hkv]
    out: torch.Tensor         # bf16 [B][Hq][256]
    lse: torch.Tensor         # fp32 [B][Hq]
    workspace: Optional[torch.Tensor]
    topk_workspace: Optional[torch.Tensor]  # candidates of the two-stage select (long rows)
    score_stride: int
    k: int

    @staticmethod
    def allocate(B: int, Hq: int, Hkv: int, score_stride: int, k: int, num_splits: int = 0,
                 device="cuda") -> "DecodeBuffers":
        ws_bytes = qsa_decode_workspace_bytes(B, Hq, num_splits)
        tk_bytes = qsa_topk_workspace_bytes(B, Hkv, k, score_stride)
        return DecodeBuffers(
            scores=torch.empty((B, Hkv, score_stride), dtype=torch.float32, device=device),
            sel_idx=torch.empty((B, Hkv, max(k, 1)), dtype=torch.int32, device=device),
            sel_cnt=torch.empty((B, Hkv), dtype=torch.int32, device=device),
            out=torch.empty((B, Hq, HEAD_DIM), dtype=torch.bfloat16, device=device),
            lse=torch.empty((B, Hq), dtype=torch.float32, device=device),
            workspace=torch.empty(ws_bytes, dtype=torch.uint8, device=device) if ws_bytes else None,
            topk_workspace=torch.empty(tk_bytes, dtype=torch.uint8, device=device) if tk_bytes else None,
            score_stride=score_stride, k=k)


def decode_step(kv: KVCache, q: torch.Tensor, q_pos: torch.Tensor, buf: DecodeBuffers, scale: float = 0.0,
                num_splits: int = 0, refresh_keys: bool = True, stream=None) -> None:
    """One decode step for every sequence of `kv`: refresh the block key holding the
    newest token and score (one launch), select, attend (and merge the splits).
    q: bf16 [B][Hq][256] (rows may be strided); q_pos = L - 1 per sequence."""
    B, Hq = q.shape[0], q.shape[1]
    Hkv = kv.k.shape[1]
    if refresh_keys:
        qsa_decode_scores_refresh(kv, q, q.stride(0), Hq, buf.scores, buf.score_stride, stream=stream)
    else:
        qsa_block_scores(kv, q, q.stride(0), None, None, B, Hq, buf.scores, buf.score_stride, stream=stream)
    tw = buf.topk_workspace
    qsa_topk_blocks_ws(buf.scores, buf.score_stride, q_pos, B, Hkv, buf.k, buf.sel_idx, buf.sel_cnt, workspace=tw,
                       workspace_bytes=0 if tw is None else tw.numel(), stream=stream)
    ws = buf.workspace
    qsa_sparse_attn_decode(kv, q, q.stride(0), Hq, buf.sel_idx, buf.sel_cnt, buf.k, scale, num_splits, buf.out,
                           buf.out.stride(0), buf.lse, workspace=ws, workspace_bytes=0 if ws is None else ws.numel(),
                           stream=stream)


@dataclass
class FusedDecodeBuffers:
    """Outputs and workspace of the fused decode step.  The workspace is zeroed
    once here; the library keeps its control area consistent from then on."""

    sel_idx: torch.Tensor     # int32 [B][Hkv][k]
    sel_cnt: torch.Tensor     # int32 [B][Hkv]
    out: torch.Tensor         # bf16 [B][Hq][256]
    lse: torch.Tensor         # fp32 [B][Hq]
    workspace: torch.Tensor   # uint8, zero-filled at allocation
    k: int
    num_splits: int

    @staticmethod
    def allocate(kv: KVCache, Hq: int, k: int, num_splits: int = 0, device="cuda") -> "FusedDecodeBuffers":
        B, Hkv = kv.block_table.shape[0], kv.k.shape[1]
        ws = qsa_decode_fused_workspace_bytes(kv, Hq, k, num_splits)
        if ws == 0:
            raise ValueError("invalid fused decode shape")
        return FusedDecodeBuffers(
            sel_idx=torch.empty((B, Hkv, max(k, 1)), dtype=torch.int32, device=device),
            sel_cnt=torch.empty((B, Hkv), dtype=torch.int32, device=device),
            out=torch.empty((B, Hq, HEAD_DIM), dtype=torch.bfloat16, device=device),
            lse=torch.empty((B, Hq), dtype=torch.float32, device=device),
            workspace=torch.zeros(ws, dtype=torch.uint8, device=device), k=k, num_splits=num_splits)


def decode_step_fused(kv: KVCache, q: torch.Tensor, q_pos: torch.Tensor, buf: FusedDecodeBuffers, scale: float = 0.0,
                      stream=None) -> None:
    """The decode step in one launch: the newest token's block key rebuilt, then
    scores, selection, attention and merge (q_pos is implied: L - 1)."""
    Hq = q.shape[1]
    qsa_decode_fused(kv, q, q.stride(0), Hq, buf.k, scale, buf.num_splits, buf.sel_idx, buf.sel_cnt, buf.out,
                     buf.out.stride(0), buf.lse, workspace=buf.workspace, workspace_bytes=buf.workspace.numel(),
                     stream=stream)


@dataclass
class ExtendBuffers:
    scores: torch.Tensor      # fp32 [R][Hkv][score_stride]
    sel_idx: torch.Tensor     # int32 [R][Hkv][k]
    sel_cnt: torch.Tensor     # int32 [R][Hkv]
    out: torch.Tensor         # bf16 [R][Hq][256]
    lse: torch.Tensor         # fp32 [R][Hq]
    score_stride: int
    k: int
    workspace: Optional[torch.Tensor] = None  # split partials of qsa_sparse_attn_extend_split

    @staticmethod
    def allocate(R: int, Hq: int, Hkv: int, score_stride: int, k: int, device="cuda",
                 max_splits: int = 1) -> "ExtendBuffers":
        """max_splits: the largest split count the chunk's attention may use (0: any the library chooses)."""
        ws = qsa_extend_workspace_bytes(R, Hq, max_splits)
        return ExtendBuffers(
            scores=torch.empty((R, Hkv, score_stride), dtype=torch.float32, device=device),
            sel_idx=torch.empty((R, Hkv, max(k, 1)), dtype=torch.int32, device=device),
            sel_cnt=torch.empty((R, Hkv), dtype=torch.int32, device=device),
            out=torch.empty((R, Hq, HEAD_DIM), dtype=torch.bfloat16, device=device),
            lse=torch.empty((R, Hq), dtype=torch.float32, device=device),
            score_stride=score_stride, k=k,
            workspace=torch.empty(ws, dtype=torch.uint8, device=device) if ws else None)


def extend_step(kv: KVCache, q: torch.Tensor, q_seq: torch.Tensor, q_pos: torch.Tensor, buf: ExtendBuffers,
                first_new: Optional[torch.Tensor] = None, max_new_tokens: int = 0, scale: float = 0.0,
                stream=None, union_tiles: bool = False, num_splits: int = 1) -> None:
    """One extend chunk: block keys of the new tokens (first_new [B] = first new
    position per sequence), then per-row scores, selection and attention (with
    union_tiles, the query-tile union kernel: the same result sets, usually slower;
    with num_splits != 1, the split read merged by log-sum-exp, for chunks of few
    rows; 0 lets the library choose the split count)."""
    R, Hq = q.shape[0], q.shape[1]
    Hkv = kv.k.shape[1]
    if first_new is not None:
        qsa_compress_keys(kv, first_new, max_new_tokens, stream=stream)
    qsa_block_scores(kv, q, q.stride(0), q_seq, q_pos, R, Hq, buf.scores, buf.score_stride, stream=stream)
    qsa_topk_blocks(buf.scores, buf.score_stride, q_pos, R, Hkv, buf.k, buf.sel_idx, buf.sel_cnt, stream=stream)
    if num_splits != 1:
        if union_tiles:
            raise ValueError("the query-tile union kernel has no split read")
        ws = buf.workspace
        qsa_sparse_attn_extend_split(kv, q, q.stride(0), q_seq, q_pos, R, Hq, buf.sel_idx, buf.sel_cnt, buf.k, scale,
                                     num_splits, buf.out, buf.out.stride(0), buf.lse, workspace=ws,
                                     workspace_bytes=ws.numel() if ws is not None else 0, stream=stream)
        return
    attend = qsa_sparse_attn_extend_union if union_tiles else qsa_sparse_attn_extend
    attend(kv, q, q.stride(0), q_seq, q_pos, R, Hq, buf.sel_idx, buf.sel_cnt, buf.k, scale, buf.out, buf.out.stride(0),
           buf.lse, stream=stream)


class DecodeGraph:
    """A decode step captured once in a HIP graph and replayed.

    The library never allocates, synchronises or memsets, so the launches of a
    step record as plain kernel nodes.  Inputs are read from the buffers given at
    capture time: update them in place (q, q_pos, the cache) between replays."""

    def __init__(self, kv: KVCache, q: torch.Tensor, q_pos: torch.Tensor, buf: DecodeBuffers, scale: float = 0.0,
                 num_splits: int = 0, warmup: int = 2):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(warmup):
                decode_step(kv, q, q_pos, buf, scale=scale, num_splits=num_splits)
        torch.cuda.current_stream().wait_stream(side)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            decode_step(kv, q, q_pos, buf, scale=scale, num_splits=num_splits)
        self._keep = (kv, q, q_pos, buf)

    def replay(self) -> None:
        self.graph.replay()
