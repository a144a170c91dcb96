"""Seeded synthetic inputs for the QSA decode and extend workloads.

Holds no attention arithmetic: it draws numbers (``synth.c`` defines the
counter-based generator) and lays them out, in the logical per-sequence layout
the CPU oracle reads and in the paged layout the HIP library reads.  The same
case object feeds both sides.

Workload recipes (each has its own seed; every tensor has its own stream):

* ``C1``  1 sequence x 8192 tokens, (16, 2) heads, N(0,1) q/K/V, one
  contiguous page (page_size 8192), top-512.
* ``C2``  32 sequences, lengths uniform on [32768, 65536], (16, 2) heads,
  K and V multiplied by an independent U(0.5, 2) factor per
  (sequence, token, KV head) before bf16 rounding, 64-token pages under a
  seeded permutation of the pool.
* ``C3``  8 sequences x 262144 tokens, (24, 2) heads, 1 % of the
  microblocks of every (sequence, KV head) (655 of 65536, drawn without
  replacement) get every key shifted by 3 times the unit vector of the
  group-summed decode query; 64-token pages, shuffled.
* ``C4``  extend: 1 sequence of 32768 tokens whose last 4096 are new query
  rows at positions 28672..32767, (12, 1) heads, one contiguous page.
* ``C5``  64 sequences, lengths uniform on [65536, 131072], (6, 1) heads,
  64-token pages, shuffled; decoded with 4 interleaved KV splits.

The microblock size (4), the top-512 budget, head_dim 256 and the head pairs
follow the QSA description on "Qwen 4 QSA krijgt decode-contextparallellisme"
(section "Wat de pull request daadwerkelijk verandert") and the head shapes on
"Qwen4-Exp QSA komt naar Huawei's Ascend" (section "Wat de pull request
daadwerkelijk toevoegt").
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")

# stream ids (upper 32 bits of the stream number; the lower 32 bits hold the sequence)
S_K, S_V, S_Q, S_LEN, S_PERM, S_KJIT, S_VJIT, S_BIAS, S_QBASE = 1, 2, 3, 4, 5, 6, 7, 8, 9


def build(verbose: bool = False) -> str:
    """Compile libsynth.so with gcc (no GPU code)."""
    import subprocess

    cmd = ["gcc", "-O2", "-Wall", "-shared", "-fPIC", "-pthread", "-ffp-contract=off",
           os.path.join(_HERE, "synth.c"), "-o", _LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(_LIB_PATH)
        u64, i64, i32, dbl = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
        vp = ctypes.c_void_p
        L.synth_key.argtypes, L.synth_key.restype = [u64, u64], u64
        L.synth_u64.argtypes, L.synth_u64.restype = [u64, u64], u64
        L.synth_uniform.argtypes, L.synth_uniform.restype = [u64, u64], dbl
        L.synth_normal.argtypes, L.synth_normal.restype = [u64, u64], dbl
        L.synth_normal_bf16.argtypes, L.synth_normal_bf16.restype = [u64, u64, i64, dbl, vp, ctypes.c_int], None
        L.synth_normal_f32.argtypes, L.synth_normal_f32.restype = [u64, u64, i64, dbl, vp, ctypes.c_int], None
        L.synth_kv.argtypes = [u64, u64, vp, vp, dbl, i32, i64, i32, i32, vp, vp, vp, ctypes.c_int]
        L.synth_kv.restype = ctypes.c_int
        L.synth_permutation.argtypes, L.synth_permutation.restype = [u64, i64, vp], None
        L.synth_choose.argtypes, L.synth_choose.restype = [u64, i64, i64, vp, vp], None
        L.synth_uniform_int.argtypes, L.synth_uniform_int.restype = [u64, u64, i64, i64], i64
        L.synth_bf16_from_float.argtypes, L.synth_bf16_from_float.restype = [ctypes.c_float], ctypes.c_uint16
        _lib = L
    return _lib


def threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def key(seed: int, tensor: int, seq: int = 0) -> int:
    return int(lib().synth_key(seed, (tensor << 32) | seq))


def normal_bf16(seed: int, tensor: int, seq: int, shape, scale: float = 1.0) -> np.ndarray:
    out = np.empty(shape, dtype=np.uint16)
    lib().synth_normal_bf16(key(seed, tensor, seq), 0, out.size, scale, _ptr(out), threads())
    return out


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 values (exact)."""
    return (a.astype(np.uint32) << 16).view(np.float32)


def bf16_to_e4m3(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp8 E4M3 codes (uint8): round to nearest even, values
    held within +-448.  How an fp8 cache is filled from bf16 keys and values."""
    import torch

    flat = np.ascontiguousarray(bits, dtype=np.uint16).reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    step = 1 << 26
    for a in range(0, flat.size, step):
        t = torch.from_numpy(flat[a:a + step].view(np.int16)).view(torch.bfloat16).float().clamp_(-448.0, 448.0)
        out[a:a + step] = t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return out.reshape(bits.shape)


def e4m3_to_bf16(codes: np.ndarray) -> np.ndarray:
    """fp8 E4M3 codes -> bf16 bit patterns of the same values (exact)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 bit patterns, nearest-even (inputs finite)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


@dataclass
class Case:
    """One synthetic workload: a paged KV cache plus query rows.

    Rows are decode rows (one per sequence, at position L-1) unless
    ``q_seq``/``q_pos`` say otherwise (extend).
    """

    name: str
    seed: int
    Hq: int
    Hkv: int
    lens: np.ndarray                 # int32 [B]
    page_size: int
    q_seq: np.ndarray                # int32 [R]
    q_pos: np.ndarray                # int32 [R]
    topk: int = 512
    scale: float = 1.0 / 16.0
    splits: int = 1
    D: int = 256
    jitter: bool = False
    bias_frac: float = 0.0
    bias_mag: float = 3.0
    shuffle: bool = True
    shared_prefix_pages: int = 0     # sequence i>0 reuses the first pages of sequence 0
    ckey_dtype: str = "fp32"         # storage of the block keys: "fp32", "bf16" or "fp8"
    kv_dtype: str = "bf16"           # storage of K and V: "bf16", or "fp8" (E4M3 codes of the bf16 draws)
    q_share: float = 0.0             # > 0: each query row is sqrt(q_share) parts a vector its sequence's rows share
    block_table: np.ndarray = field(default=None, repr=False)   # int32 [B][max_pages]
    num_pages: int = 0
    _q: Optional[np.ndarray] = field(default=None, repr=False)
    _bias: dict = field(default_factory=dict, repr=False)

    @property
    def B(self) -> int:
        return int(self.lens.shape[0])

    @property
    def R(self) -> int:
        return int(self.q_seq.shape[0])

    @property
    def g(self) -> int:
        return self.Hq // self.Hkv

    @property
    def max_len(self) -> int:
        return int(self.lens.max()) if self.B else 0

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])

    def nb(self, i: int) -> int:
        return (int(self.lens[i]) + 3) // 4

    # -------------------------------------------------------------- queries
    @property
    def q(self) -> np.ndarray:
        """bf16 bit patterns [R][Hq][D].  N(0,1) per element; with q_share = s > 0 each
        row is sqrt(s) * (its sequence's shared N(0,1) vector) + sqrt(1 - s) * (its own
        N(0,1) draw), rounded to bf16, so that the rows of a sequence select overlapping
        blocks."""
        if self._q is None:
            q = normal_bf16(self.seed, S_Q, 0, (self.R, self.Hq, self.D))
            if self.q_share > 0.0:
                base = bf16_to_f32(normal_bf16(self.seed, S_QBASE, 0, (self.B, self.Hq, self.D))).astype(np.float64)
                own = bf16_to_f32(q).astype(np.float64)
                mix = np.sqrt(self.q_share) * base[self.q_seq] + np.sqrt(1.0 - self.q_share) * own
                q = f32_to_bf16(mix.astype(np.float32))
            self._q = q
        return self._q

    # ----------------------------------------------------------------- bias
    def bias(self, i: int):
        """(direction [Hkv][D] float32, mask [Hkv][nb] uint8) for sequence i, or (None, None)."""
        if self.bias_frac <= 0.0:
            return None, None
        if i not in self._bias:
            nb = self.nb(i)
            n_b = int(round(self.bias_frac * nb))
            rows = np.nonzero(self.q_seq == i)[0]
            r = rows[np.argmax(self.q_pos[rows])]  # the sequence's last query row
            qd = bf16_to_f32(self.q[r]).astype(np.float64).reshape(self.Hkv, self.g, self.D)
            qsum = qd.sum(axis=1)
            direction = (qsum / np.linalg.norm(qsum, axis=1, keepdims=True)).astype(np.float32)
            mask = np.zeros((self.Hkv, nb), dtype=np.uint8)
            scratch = np.empty(nb, dtype=np.int32)
            chosen = np.empty(n_b, dtype=np.int32)
            for h in range(self.Hkv):
                lib().synth_choose(key(self.seed, S_BIAS, (i << 8) | h), nb, n_b, _ptr(scratch), _ptr(chosen))
                mask[h, chosen] = 1
            self._bias[i] = (np.ascontiguousarray(direction), mask)
        return self._bias[i]

    # ------------------------------------------------------------ K / V
    def _gen(self, tensor: str, i: int, logical, paged):
        tid, jid = (S_K, S_KJIT) if tensor == "k" else (S_V, S_VJIT)
        kj = key(self.seed, jid, i) if self.jitter else 0
        bdir, bmask = self.bias(i) if tensor == "k" else (None, None)
        rc = lib().synth_kv(key(self.seed, tid, i), kj, _ptr(bdir), _ptr(bmask), self.bias_mag, self.Hkv,
                            int(self.lens[i]), self.D, self.page_size,
                            _ptr(self.block_table[i]) if paged is not None else None,
                            _ptr(logical), _ptr(paged), threads())
        if rc != 0:
            raise RuntimeError("synth_kv failed")

    def logical(self, tensor: str, i: int) -> np.ndarray:
        """bf16 bit patterns [Hkv][L_i][D] of sequence i (tensor 'k' or 'v'): the
        values the cache holds (with an fp8 cache, the decoded fp8 values)."""
        L = int(self.lens[i])
        if self.shared_prefix_pages and i > 0:
            # content of aliased pages comes from the paged pool: gather it
            out = self.gather_logical(self.paged(tensor), i)
        else:
            out = np.empty((self.Hkv, L, self.D), dtype=np.uint16)
            self._gen(tensor, i, out, None)
        if self.kv_dtype == "fp8":
            out = e4m3_to_bf16(bf16_to_e4m3(out))
        return out

    def paged(self, tensor: str) -> np.ndarray:
        """bf16 bit patterns [num_pages][Hkv][page_size][D] of the whole pool."""
        cache = getattr(self, "_paged_" + tensor, None)
        if cache is not None:
            return cache
        out = np.zeros((self.num_pages, self.Hkv, self.page_size, self.D), dtype=np.uint16)
        for i in range(self.B):
            self._gen(tensor, i, None, out)
        if self.shared_prefix_pages:
            # sequences > 0 wrote their own values into the pages they share with
            # sequence 0; writing sequence 0 again gives those pages its content
            self._gen(tensor, 0, None, out)
        setattr(self, "_paged_" + tensor, out)
        return out

    def paged_device(self, tensor: str) -> np.ndarray:
        """The pool as the cache stores it: bf16 bit patterns (uint16), or fp8 E4M3
        codes (uint8) with kv_dtype "fp8"."""
        pool = self.paged(tensor)
        return bf16_to_e4m3(pool) if self.kv_dtype == "fp8" else pool

    def drop_paged(self):
        for t in ("k", "v"):
            if hasattr(self, "_paged_" + t):
                delattr(self, "_paged_" + t)

    def gather_logical(self, pool: np.ndarray, i: int) -> np.ndarray:
        L = int(self.lens[i])
        pos = np.arange(L)
        pages = self.block_table[i][pos // self.page_size]
        slots = pos % self.page_size
        return np.ascontiguousarray(pool[pages, :, slots, :].transpose(1, 0, 2))


def to_device(case: Case, device="cuda", ckey: bool = True):
    """Upload a case's paged pool, tables and queries as torch tensors (layout only).

    Returns a dict: k, v (bf16, or fp8 E4M3 with kv_dtype "fp8", [num_pages][Hkv][page_size][D]), ckey (fp32, bf16 or fp8
    E4M3 as the case stores block keys, zeroed),
    block_table, seq_lens, q_seq, q_pos (int32), q (bf16 [R][Hq][D])."""
    import torch

    def bf16(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)

    def kv(tensor):
        a = case.paged_device(tensor)
        if case.kv_dtype == "fp8":
            return torch.from_numpy(a).view(torch.float8_e4m3fn).to(device)
        return bf16(a)

    out = {
        "k": kv("k"),
        "v": kv("v"),
        "block_table": torch.from_numpy(case.block_table).to(device),
        "seq_lens": torch.from_numpy(case.lens).to(device),
        "q_seq": torch.from_numpy(case.q_seq).to(device),
        "q_pos": torch.from_numpy(case.q_pos).to(device),
        "q": bf16(case.q),
    }
    if ckey:
        dt = {"bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}.get(case.ckey_dtype, torch.float32)
        out["ckey"] = torch.zeros((case.num_pages, case.Hkv, case.page_size // 4, case.D), dtype=dt, device=device)
    return out


def _block_table(seed: int, lens: np.ndarray, page_size: int, shuffle: bool, shared_prefix_pages: int):
    npg = [(int(L) + page_size - 1) // page_size for L in lens]
    max_pages = max(max(npg) if npg else 1, 1)
    total = sum(npg)
    if shared_prefix_pages:
        total -= shared_prefix_pages * (len(lens) - 1)
    perm = np.arange(total, dtype=np.int32)
    if shuffle and total > 1:
        lib().synth_permutation(key(seed, S_PERM, 0), total, _ptr(perm))
    bt = np.zeros((len(lens), max_pages), dtype=np.int32)
    off = 0
    for i, n in enumerate(npg):
        if shared_prefix_pages and i > 0:
            s = min(shared_prefix_pages, n)
            bt[i, :s] = bt[0, :s]
            bt[i, s:n] = perm[off:off + n - s]
            off += n - s
        else:
            bt[i, :n] = perm[off:off + n]
            off += n
    return bt, max(total, 1)


def make_case(name: str, seed: int, Hq: int, Hkv: int, lens, page_size: int, *, q_seq=None, q_pos=None,
              topk: int = 512, scale: float = 1.0 / 16.0, splits: int = 1, jitter: bool = False,
              bias_frac: float = 0.0, shuffle: bool = True, shared_prefix_pages: int = 0, D: int = 256,
              ckey_dtype: str = "fp32", kv_dtype: str = "bf16", q_share: float = 0.0) -> Case:
    lens = np.asarray(lens, dtype=np.int32)
    if q_seq is None:  # decode: one row per sequence at its last position
        q_seq = np.arange(lens.shape[0], dtype=np.int32)
        q_pos = (lens - 1).astype(np.int32)
    bt, num_pages = _block_table(seed, lens, page_size, shuffle, shared_prefix_pages)
    return Case(name=name, seed=seed, Hq=Hq, Hkv=Hkv, lens=lens, page_size=page_size,
                q_seq=np.asarray(q_seq, dtype=np.int32), q_pos=np.asarray(q_pos, dtype=np.int32), topk=topk,
                scale=scale, splits=splits, D=D, jitter=jitter, bias_frac=bias_frac, shuffle=shuffle,
                shared_prefix_pages=shared_prefix_pages, block_table=bt, num_pages=num_pages, ckey_dtype=ckey_dtype,
                kv_dtype=kv_dtype, q_share=q_share)


def uniform_lengths(seed: int, B: int, lo: int, hi: int) -> np.ndarray:
    k = key(seed, S_LEN, 0)
    return np.array([lib().synth_uniform_int(k, i, lo, hi) for i in range(B)], dtype=np.int32)


def extend_rows(total: int, new: int, seq: int = 0):
    q_pos = np.arange(total - new, total, dtype=np.int32)
    return np.full(new, seq, dtype=np.int32), q_pos


# ------------------------------------------------------------------ the five workloads

def config(name: str, *, B: Optional[int] = None, L: Optional[int] = None, L_range=None,
           new: Optional[int] = None, q_share: float = 0.0) -> Case:
    """The named workload, optionally shrunk (fewer sequences / shorter contexts) with
    the same recipe otherwise.  q_share (extend only) mixes a per-sequence shared
    component into the queries (Case.q)."""
    if name == "C1":
        L1 = L or 8192
        return make_case("C1", 1, 16, 2, [L1] * (B or 1), page_size=L1, shuffle=False)
    if name == "C2":
        lo, hi = L_range or (32768, 65536)
        return make_case("C2", 2, 16, 2, uniform_lengths(2, B or 32, lo, hi), page_size=64, jitter=True)
    if name == "C3":
        L3 = L or 262144
        return make_case("C3", 3, 24, 2, [L3] * (B or 8), page_size=64, bias_frac=0.01)
    if name == "C4":
        total = L or 32768
        n_new = new or 4096
        q_seq, q_pos = extend_rows(total, n_new)
        return make_case("C4", 4, 12, 1, [total], page_size=total, q_seq=q_seq, q_pos=q_pos, shuffle=False,
                         q_share=q_share)
    if name == "C5":
        lo, hi = L_range or (65536, 131072)
        return make_case("C5", 5, 6, 1, uniform_lengths(5, B or 64, lo, hi), page_size=64, splits=4)
    raise KeyError(name)


CONFIGS = ("C1", "C2", "C3", "C4", "C5")
