"""CPU oracle for the QSA hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never calls it and
shares no code with it; both are fed the same seeded inputs from ``synth``.

``oracle.c`` holds the arithmetic (fp64 except the block-key mean, whose fp32
definition is pinned); this module only marshals numpy arrays and runs
independent (row, KV head) units on a thread pool (ctypes releases the GIL
during each call).

Steps, in the order of the QSA description on "Qwen 4 QSA krijgt
decode-contextparallellisme" (section "Wat de pull request daadwerkelijk
verandert"): ``compress`` (keys -> 4-token block keys), ``scores`` (block keys
against the group-summed query), ``topk`` (the best k blocks), ``attend``
(exact softmax attention over the selected blocks' uncompressed tokens) and
``merge`` (log-sum-exp combination of partial results, the combine step of
decode context parallelism described on the same page).

Parity unpinned: agreement with the real model's learned indexer -- the pages
print no worked example and no weights exist here.  Every function below is
pinned against closed forms, brute force and invariants in
``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    """Compile liboracle.so with gcc: -O2, no fast-math, no FMA contraction."""
    import subprocess

    cmd = ["gcc", "-O2", "-Wall", "-shared", "-fPIC", "-ffp-contract=off", "-fno-fast-math",
           os.path.join(_HERE, "oracle.c"), "-o", _LIB_PATH + ".tmp", "-lm"]
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
        vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.oracle_compress.argtypes = [vp, i64, i32, vp]
        L.oracle_compress_bf16.argtypes = [vp, i64, i32, vp]
        L.oracle_compress_fp8.argtypes = [vp, i64, i32, vp, vp]
        L.oracle_scores.argtypes = [vp, i32, i32, vp, i64, vp]
        L.oracle_topk.argtypes = [vp, i64, i32, vp, vp]
        L.oracle_attend.argtypes = [vp, i32, i32, vp, vp, i64, i64, vp, i32, dbl, i32, i32, vp, vp]
        L.oracle_merge.argtypes = [vp, vp, i32, i64, i32, vp, vp]
        for f in ("oracle_compress", "oracle_scores", "oracle_topk", "oracle_attend", "oracle_merge"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what} failed ({rc})")


# ----------------------------------------------------------------------- steps

def compress(keys: np.ndarray, ckey_dtype: str = "fp32") -> np.ndarray:
    """keys bf16 bits [L][D] -> block keys float32 [ceil(L/4)][D]; with
    ckey_dtype "bf16" / "fp8", the fp32 means rounded to bf16 / fp8 E4M3
    (returned decoded to float32)."""
    keys = np.ascontiguousarray(keys, dtype=np.uint16)
    L, D = keys.shape
    out = np.empty(((L + 3) // 4, D), dtype=np.float32)
    if ckey_dtype == "bf16":
        _check(lib().oracle_compress_bf16(_p(keys), L, D, _p(out)), "oracle_compress_bf16")
    elif ckey_dtype == "fp8":
        _check(lib().oracle_compress_fp8(_p(keys), L, D, _p(out), None), "oracle_compress_fp8")
    else:
        assert ckey_dtype == "fp32", ckey_dtype
        _check(lib().oracle_compress(_p(keys), L, D, _p(out)), "oracle_compress")
    return out


def compress_fp8_codes(keys: np.ndarray) -> np.ndarray:
    """keys bf16 bits [L][D] -> fp8 E4M3 block-key codes uint8 [ceil(L/4)][D]."""
    keys = np.ascontiguousarray(keys, dtype=np.uint16)
    L, D = keys.shape
    out = np.empty(((L + 3) // 4, D), dtype=np.float32)
    codes = np.empty(((L + 3) // 4, D), dtype=np.uint8)
    _check(lib().oracle_compress_fp8(_p(keys), L, D, _p(out), _p(codes)), "oracle_compress_fp8")
    return codes


def scores(q_group: np.ndarray, ckey: np.ndarray, n_elig: int) -> np.ndarray:
    """q_group bf16 bits [g][D], ckey float32 [>=n_elig][D] -> float64 [n_elig]."""
    q_group = np.ascontiguousarray(q_group, dtype=np.uint16)
    ckey = np.ascontiguousarray(ckey, dtype=np.float32)
    g, D = q_group.shape
    assert ckey.shape[1] == D and ckey.shape[0] >= n_elig
    out = np.empty(max(n_elig, 1), dtype=np.float64)
    _check(lib().oracle_scores(_p(q_group), g, D, _p(ckey), n_elig, _p(out)), "oracle_scores")
    return out[:n_elig]


def topk(s: np.ndarray, k: int) -> Tuple[np.ndarray, int]:
    """float64 scores [n] -> (ascending indices, -1 padded, int32 [k]; count)."""
    s = np.ascontiguousarray(s, dtype=np.float64)
    sel = np.empty(max(k, 1), dtype=np.int32)
    cnt = np.zeros(1, dtype=np.int32)
    _check(lib().oracle_topk(_p(s), s.shape[0], k, _p(sel), _p(cnt)), "oracle_topk")
    return sel[:k], int(cnt[0])


def attend(q_group: np.ndarray, K: np.ndarray, V: np.ndarray, t: int, sel: np.ndarray, cnt: int, scale: float,
           S: int = 1, s: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of g heads over the selected blocks' tokens (split s of S).

    q_group bf16 bits [g][D]; K, V bf16 bits [L][D] -> (out float64 [g][D], lse float64 [g])."""
    q_group = np.ascontiguousarray(q_group, dtype=np.uint16)
    K = np.ascontiguousarray(K, dtype=np.uint16)
    V = np.ascontiguousarray(V, dtype=np.uint16)
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    g, D = q_group.shape
    L = K.shape[0]
    assert K.shape == (L, D) and V.shape == (L, D)
    out = np.empty((g, D), dtype=np.float64)
    lse = np.empty(g, dtype=np.float64)
    sel_buf = sel if sel.size else np.zeros(1, dtype=np.int32)
    _check(lib().oracle_attend(_p(q_group), g, D, _p(K), _p(V), L, t, _p(sel_buf), cnt, scale, S, s, _p(out),
                               _p(lse)), "oracle_attend")
    return out, lse


def merge(part_out: np.ndarray, part_lse: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """part_out [S][N][D], part_lse [S][N] (float64) -> (out [N][D], lse [N])."""
    part_out = np.ascontiguousarray(part_out, dtype=np.float64)
    part_lse = np.ascontiguousarray(part_lse, dtype=np.float64)
    S, N, D = part_out.shape
    out = np.empty((N, D), dtype=np.float64)
    lse = np.empty(N, dtype=np.float64)
    _check(lib().oracle_merge(_p(part_out), _p(part_lse), S, N, D, _p(out), _p(lse)), "oracle_merge")
    return out, lse


# ------------------------------------------------------------- whole-step driver

def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:
        return os.cpu_count() or 1


@dataclass
class StepResult:
    """Oracle results for a set of (row, KV head) units of one case."""

    rows: np.ndarray                                   # the row indices computed
    scores: Dict[Tuple[int, int], np.ndarray] = field(default_factory=dict)   # (r, h) -> float64 [n_elig]
    sel: Dict[Tuple[int, int], np.ndarray] = field(default_factory=dict)      # (r, h) -> int32 [k]
    cnt: Dict[Tuple[int, int], int] = field(default_factory=dict)
    out: Dict[int, np.ndarray] = field(default_factory=dict)                  # r -> float64 [Hq][D]
    lse: Dict[int, np.ndarray] = field(default_factory=dict)                  # r -> float64 [Hq]
    part_out: Dict[int, np.ndarray] = field(default_factory=dict)             # r -> float64 [S][Hq][D]
    part_lse: Dict[int, np.ndarray] = field(default_factory=dict)             # r -> float64 [S][Hq]


class CaseData:
    """Logical K/V and block keys of a synth.Case, generated per sequence on demand."""

    def __init__(self, case):
        self.case = case
        self._k: Dict[int, np.ndarray] = {}
        self._v: Dict[int, np.ndarray] = {}
        self._ckey: Dict[Tuple[int, int], np.ndarray] = {}

    def K(self, i: int) -> np.ndarray:
        if i not in self._k:
            self._k[i] = self.case.logical("k", i)
        return self._k[i]

    def V(self, i: int) -> np.ndarray:
        if i not in self._v:
            self._v[i] = self.case.logical("v", i)
        return self._v[i]

    def ckey(self, i: int, h: int) -> np.ndarray:
        if (i, h) not in self._ckey:
            self._ckey[(i, h)] = compress(self.K(i)[h], self.case.ckey_dtype)
        return self._ckey[(i, h)]

    def prefetch(self, seqs, threads: int):
        """Build the block keys of the given sequences (all heads) in parallel."""
        seqs = sorted(set(int(i) for i in seqs))
        for i in seqs:
            self.K(i)
        units = [(i, h) for i in seqs for h in range(self.case.Hkv) if (i, h) not in self._ckey]
        with ThreadPoolExecutor(max_workers=threads) as ex:
            for (i, h), ck in zip(units, ex.map(lambda u: compress(self.K(u[0])[u[1]], self.case.ckey_dtype),
                                                units)):
                self._ckey[(i, h)] = ck

    def release(self, i: int):
        self._k.pop(i, None)
        self._v.pop(i, None)
        for h in range(self.case.Hkv):
            self._ckey.pop((i, h), None)


def run_unit(data: CaseData, r: int, h: int, k: int, S: int, sel_override: Optional[np.ndarray] = None,
             cnt_override: Optional[int] = None, keep_scores: bool = True):
    """Scores, selection and attention of one (row, KV head) unit."""
    case = data.case
    g, D = case.g, case.D
    i, t = int(case.q_seq[r]), int(case.q_pos[r])
    qg = case.q[r, h * g:(h + 1) * g]
    s = None
    if sel_override is None:
        n_elig = min(t // 4 + 1, case.nb(i))
        s = scores(qg, data.ckey(i, h), n_elig)
        sel, cnt = topk(s, k)
    else:
        sel, cnt = sel_override, int(cnt_override)
    K, V, L = data.K(i)[h], data.V(i)[h], int(case.lens[i])
    if S == 1:
        out, lse = attend(qg, K, V, t, sel, cnt, case.scale)
        parts = None
    else:
        po = np.empty((S, g, D))
        pl = np.empty((S, g))
        for sp in range(S):
            po[sp], pl[sp] = attend(qg, K, V, t, sel, cnt, case.scale, S, sp)
        out, lse = merge(po, pl)
        parts = (po, pl)
    return (s if keep_scores else None), sel, cnt, out, lse, parts


def run_case(case, rows=None, *, splits: Optional[int] = None, threads: Optional[int] = None,
             sel_override: Optional[Dict[Tuple[int, int], Tuple[np.ndarray, int]]] = None,
             keep_scores: bool = True, data: Optional[CaseData] = None) -> StepResult:
    """Run the whole oracle step on the given rows (default: all rows)."""
    threads = threads or default_threads()
    S = case.splits if splits is None else splits
    rows = np.arange(case.R) if rows is None else np.asarray(rows)
    data = data or CaseData(case)
    data.prefetch(case.q_seq[rows], threads)
    for i in set(int(x) for x in case.q_seq[rows]):
        data.V(i)
    res = StepResult(rows=rows)
    units = [(int(r), h) for r in rows for h in range(case.Hkv)]

    def work(u):
        r, h = u
        so = sel_override.get(u) if sel_override else None
        if so is None:
            return run_unit(data, r, h, case.topk, S, keep_scores=keep_scores)
        return run_unit(data, r, h, case.topk, S, so[0], so[1], keep_scores=keep_scores)

    g, D = case.g, case.D
    with ThreadPoolExecutor(max_workers=threads) as ex:
        results = list(ex.map(work, units))
    for (r, h), (s, sel, cnt, out, lse, parts) in zip(units, results):
        if s is not None:
            res.scores[(r, h)] = s
        res.sel[(r, h)] = sel
        res.cnt[(r, h)] = cnt
        if r not in res.out:
            res.out[r] = np.zeros((case.Hq, D))
            res.lse[r] = np.zeros(case.Hq)
            if S > 1:
                res.part_out[r] = np.zeros((S, case.Hq, D))
                res.part_lse[r] = np.zeros((S, case.Hq))
        res.out[r][h * g:(h + 1) * g] = out
        res.lse[r][h * g:(h + 1) * g] = lse
        if parts is not None:
            res.part_out[r][:, h * g:(h + 1) * g] = parts[0]
            res.part_lse[r][:, h * g:(h + 1) * g] = parts[1]
    return res
