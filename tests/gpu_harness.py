"""Device-side harness for the GPU tests: uploads a synth.Case and runs the libqsa
entry points on it through the Python binding (which calls the C ABI)."""
from __future__ import annotations

import numpy as np
import torch

import block_sparse_attention_compress_amd as qsa
import synth


def log(msg: str):
    print(f"[gpu] {msg}", flush=True)


class Dev:
    def __init__(self, case: synth.Case, device: str = "cuda"):
        self.case = case
        self.device = device
        self.t = synth.to_device(case, device)
        self.kv = qsa.KVCache(self.t["k"], self.t["v"], self.t["ckey"], self.t["block_table"], self.t["seq_lens"],
                              max(case.max_len, 1))
        self.stride = max([1] + [case.nb(i) for i in range(case.B)])

    # ------------------------------------------------------------ steps
    def compress(self, first=None, max_new: int = 0):
        qsa.qsa_compress_keys(self.kv, first, max_new)

    def scores(self, extend: bool = False, q=None) -> torch.Tensor:
        c = self.case
        q = self.t["q"] if q is None else q
        s = torch.full((c.R, c.Hkv, self.stride), float("nan"), dtype=torch.float32, device=self.device)
        if extend:
            qsa.qsa_block_scores(self.kv, q, q.stride(0), self.t["q_seq"], self.t["q_pos"], c.R, c.Hq, s, self.stride)
        else:
            qsa.qsa_block_scores(self.kv, q, q.stride(0), None, None, c.R, c.Hq, s, self.stride)
        return s

    def topk(self, scores: torch.Tensor, k: int, q_pos=None):
        c = self.case
        R, Hkv, stride = scores.shape
        sel = torch.full((R, Hkv, max(k, 1)), -7, dtype=torch.int32, device=self.device)
        cnt = torch.full((R, Hkv), -7, dtype=torch.int32, device=self.device)
        qsa.qsa_topk_blocks(scores, stride, self.t["q_pos"] if q_pos is None else q_pos, R, Hkv, k, sel, cnt)
        return sel, cnt

    def decode_attn(self, sel, cnt, k: int, num_splits: int = 0, scale: float = 0.0, q=None, out=None):
        c = self.case
        q = self.t["q"] if q is None else q
        out = torch.full((c.B, c.Hq, 256), float("nan"), dtype=torch.bfloat16, device=self.device) if out is None \
            else out
        lse = torch.full((c.B, c.Hq), float("nan"), dtype=torch.float32, device=self.device)
        wsb = qsa.qsa_decode_workspace_bytes(c.B, c.Hq, num_splits)
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=self.device)
        qsa.qsa_sparse_attn_decode(self.kv, q, q.stride(0), c.Hq, sel, cnt, k, scale, num_splits, out, out.stride(0),
                                   lse, workspace=ws, workspace_bytes=wsb)
        return out, lse

    def decode_partials(self, sel, cnt, k: int, S: int, scale: float = 0.0):
        c = self.case
        po = torch.full((S, c.B, c.Hq, 256), float("nan"), dtype=torch.float32, device=self.device)
        pl = torch.full((S, c.B, c.Hq), float("nan"), dtype=torch.float32, device=self.device)
        q = self.t["q"]
        qsa.qsa_sparse_attn_decode(self.kv, q, q.stride(0), c.Hq, sel, cnt, k, scale, S, None, 0, None, po, pl)
        return po, pl

    def extend_attn(self, sel, cnt, k: int, scale: float = 0.0):
        c = self.case
        q = self.t["q"]
        out = torch.full((c.R, c.Hq, 256), float("nan"), dtype=torch.bfloat16, device=self.device)
        lse = torch.full((c.R, c.Hq), float("nan"), dtype=torch.float32, device=self.device)
        qsa.qsa_sparse_attn_extend(self.kv, q, q.stride(0), self.t["q_seq"], self.t["q_pos"], c.R, c.Hq, sel, cnt, k,
                                   scale, out, out.stride(0), lse)
        return out, lse

    # ------------------------------------------------------------ views
    def ckey_logical(self, i: int) -> np.ndarray:
        """Block keys of sequence i as [Hkv][nb][256] float32 (bf16 keys widened), gathered
        from the pool."""
        c = self.case
        nb = c.nb(i)
        t = self.t["ckey"]
        if t.dtype == torch.float8_e4m3fn:  # decoded to float32 (exact)
            pool = t.cpu().to(torch.float32).numpy()
        elif t.dtype == torch.bfloat16:  # widened to float32 (exact)
            pool = synth.bf16_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16))
        else:
            pool = t.cpu().numpy()
        b = np.arange(nb)
        pages = c.block_table[i][(4 * b) // c.page_size]
        slots = ((4 * b) % c.page_size) // 4
        return np.ascontiguousarray(pool[pages, :, slots, :].transpose(1, 0, 2))

    def ckey_codes(self, i: int) -> np.ndarray:
        """fp8 block-key codes of sequence i as uint8 [Hkv][nb][256]."""
        c = self.case
        b = np.arange(c.nb(i))
        pool = self.t["ckey"].view(torch.uint8).cpu().numpy()
        pages = c.block_table[i][(4 * b) // c.page_size]
        slots = ((4 * b) % c.page_size) // 4
        return np.ascontiguousarray(pool[pages, :, slots, :].transpose(1, 0, 2))


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()
