#!/usr/bin/env python3
"""QSA decode benchmark on one MI355X.

A step is one pass of the whole decode hot path for every sequence of the batch:
refresh the block key holding the newest token, score every eligible block
against the group-summed query, keep the top-512 blocks, run the sparse attention
over their uncompressed K/V (split-KV partials merged by log-sum-exp).  Inputs are
seeded synthetic tensors (``synth``) already resident in HBM when timing starts.

Headline workload (``value``): 32 sequences with lengths uniform on
[32768, 65536], 16 query / 2 KV heads, head_dim 256, bf16 K/V with a U(0.5, 2)
norm jitter per token, 64-token pages under a shuffled block table, top-512
blocks.  The default run also measures the other decode workloads, each with its
own roofline and CPU oracle baseline, under ``configs``:

* C1  1 sequence of 8192 tokens, (16,2) heads, one contiguous page;
* C3  8 sequences of 262144 tokens, (24,2) heads, 1 % of the microblocks biased
      toward the query, 64-token shuffled pages;
* C5  64 sequences of 65536..131072 tokens, (6,1) heads, 64-token shuffled
      pages, timed as configured -- 4 token-interleaved split partials merged by
      ``qsa_merge_lse`` -- and beside it with the library's internal split;

and the extend chunk (4096 new tokens on 28672 cached, (12,1) heads) under
``extend``.

Prints one JSON line.  Per workload: queries/s, ms per step, per-kernel HIP-event
times, the roofline of the dominant kernel (the block-score scan, HBM-bound: the
algorithmic bytes of that launch over its event time) with the step's
own fraction beside it, and the CPU oracle timed on a bounded sample of the same
workload on the host cores.  Algorithmic bytes are what the method must move:
the block-key scan, the selected tokens' K and V, q, out, lse, the block table
and the lengths; scores, the rebuilt newest block key and split partials are the
implementation's overhead and are reported apart.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--config C2|C1|C3|C5|all]
    python bench.py --copy-calibration      # plain copy kernel for counter scaling
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "QSA decode queries/s and achieved HBM GB/s (% of MI355X peak) at 64K ctx"
HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
SCORES_SRC = [os.path.join(ROOT, "block_sparse_attention_compress_amd", "csrc", f)
              for f in ("scores.hip", "scan_body.h", "qsa_device.h")]
DTYPE = "fp32 block-key scores; bf16 K/V on bf16 MFMA with fp32 accumulate (P rounded to bf16)"
DECODE_CONFIGS = ("C2", "C1", "C3", "C5")


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", default="all", choices=["all", "C1", "C2", "C3", "C5"],
                   help="decode workload(s): all = C2 (headline) then C1, C3, C5")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extend", action="store_true", help="skip the extend (prefill chunk) figures")
    p.add_argument("--extend-only", action="store_true",
                   help="print only the extend chunk's figures (one JSON object; for profiling the chunk alone)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="oracle timing span for the headline workload (seconds of wall time; the other "
                        "workloads take 40 %% of it)")
    p.add_argument("--copy-calibration", action="store_true")
    p.add_argument("--graph", action="store_true", help="time a replayed HIP graph of the step instead of eager launches")
    p.add_argument("--splits", type=int, default=None, help="decode split count (default: the library's choice)")
    p.add_argument("--no-fused", action="store_true", help="do not time the fused step (the default)")
    p.add_argument("--fused", action="store_true",
                   help="also time the single-launch fused step (qsa_decode_fused); slower than the separate calls "
                        "on every workload measured, so not part of the default run")
    p.add_argument("--flush", action="store_true",
                   help="also time single steps after a 1 GiB read that evicts the caches (MALL included)")
    p.add_argument("--kv", choices=["bf16", "fp8"], default="bf16",
                   help="main cache storage (bf16; fp8: E4M3 codes of the same draws)")
    p.add_argument("--q-share", type=float, default=0.0,
                   help="extend only: queries share a per-sequence component with this weight (0.9: 8 adjacent rows "
                        "select a quarter as many distinct blocks as 8 x 512), for the query-tile union kernel")
    p.add_argument("--ckey", choices=["fp32", "bf16", "fp8"], default="fp32",
                   help="block-key storage (fp32: the method's definition; bf16 / fp8: the rounded-mean variants)")
    return p.parse_args()


LENGTH_RANGE = {"C2": "drawn uniformly from [32768, 65536]", "C5": "drawn uniformly from [65536, 131072]"}


def describe(case) -> str:
    """One line naming the decode workload by its shape."""
    lo, hi = int(case.lens.min()), int(case.lens.max())
    lens = f"length {lo}" if lo == hi else f"lengths {lo}..{hi} {LENGTH_RANGE.get(case.name, '')}".rstrip()
    if case.block_table.shape[1] == 1:
        cache = f"contiguous {case.kv_dtype} KV"
    else:
        cache = f"{case.kv_dtype} paged KV ({case.page_size}-token pages{', shuffled' if case.shuffle else ''})"
    extra = []
    if case.jitter:
        extra.append("per-token key/value norm jitter x U(0.5, 2)")
    if case.bias_frac:
        extra.append(f"{case.bias_frac:.0%} of microblocks biased +{case.bias_mag:g} sigma toward the query")
    if case.splits > 1:
        extra.append(f"{case.splits} token-interleaved split-KV partials merged by log-sum-exp")
    if case.ckey_dtype == "bf16":
        extra.append("bf16 block keys (fp32 means rounded to nearest even)")
    if case.ckey_dtype == "fp8":
        extra.append("fp8 E4M3 block keys (fp32 means rounded to nearest even, held at +-448)")
    if case.kv_dtype == "fp8":
        extra.append("fp8 E4M3 main K/V cache (codes of the bf16 draws, unit scale)")
    return (f"{case.name}: decode, {case.B} sequence{'s' if case.B > 1 else ''}, {lens}, ({case.Hq},{case.Hkv}) heads, "
            f"head_dim 256, {cache}, top-{case.topk} microblocks of 4" + "".join("; " + e for e in extra))


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def copy_calibration():
    """A plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}))


def decode_bytes(case, sel, cnt, page_size, splits):
    """Algorithmic HBM bytes of one decode step and the implementation's
    overhead bytes, for the step and for the block-score launch.

    Algorithmic, per (sequence, KV head): the block-key scan (nb * 1 KiB for fp32
    keys, 512 B bf16, 256 B fp8) and the K and V rows of the selected tokens
    (512 B each, 256 B for an fp8 cache); per row: q and out (bf16) and lse
    (fp32); the block-table entries and the lengths.  The block-score launch's
    share is the scan, q, the table and the lengths.
    Overhead: the scores written by the scan and read back by the top-k (4 B per
    block each way), the newest block key rebuilt in the scan (1..4 K rows read,
    one key written) and the split partials (fp32 out + lse, written and read)."""
    import numpy as np

    B, Hkv, Hq = case.B, case.Hkv, case.Hq
    nb = np.array([case.nb(i) for i in range(B)], dtype=np.int64)
    key_bytes = 256 * {"bf16": 2, "fp8": 1}.get(case.ckey_dtype, 4)
    ckey = int(nb.sum()) * Hkv * key_bytes
    row_bytes = 256 if case.kv_dtype == "fp8" else 512  # one K or V row
    tokens = 0
    for i in range(B):
        L = int(case.lens[i])
        for h in range(Hkv):
            c = int(cnt[i, h])
            blocks = sel[i, h, :c].astype(np.int64)
            tokens += int(np.minimum(L - 4 * blocks, 4).sum())
    kv_bytes = tokens * row_bytes * 2
    q_bytes = B * Hq * 256 * 2
    qo = q_bytes * 2 + B * Hq * 4
    table = int(sum((int(L) + page_size - 1) // page_size for L in case.lens)) * 4 + B * 4
    step = ckey + kv_bytes + qo + table
    scan = ckey + q_bytes + table
    refresh = sum((int(L) - 4 * ((int(L) - 1) // 4)) * row_bytes + key_bytes for L in case.lens if L > 0) * Hkv
    score_rw = int(nb.sum()) * Hkv * 4
    partials = (splits * B * Hq * (256 + 1) * 4 * 2) if splits > 1 else 0
    return {"step": step, "scan": scan, "tokens": tokens,
            "scan_overhead": score_rw + refresh, "step_overhead": 2 * score_rw + refresh + partials}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(case, target_s: float, max_rows: int):
    """The CPU oracle as it stands, timed on a sample of the same workload: on
    every host thread it may use (one (row, KV head) unit per thread), and on one
    thread (a shorter sample)."""
    import oracle

    threads = oracle.default_threads()
    rows = list(range(min(case.B, max_rows)))
    data = oracle.CaseData(case)
    data.prefetch([case.q_seq[r] for r in rows], threads)      # logical K and block keys: not timed
    for r in rows:
        data.V(int(case.q_seq[r]))

    def timed(rows_, nthreads, span):
        reps = 0
        t0 = time.perf_counter()
        while True:
            oracle.run_case(case, rows=rows_, threads=nthreads, data=data, keep_scores=False)
            reps += 1
            if time.perf_counter() - t0 >= span:
                break
        return reps, time.perf_counter() - t0

    reps, dt = timed(rows, threads, target_s)
    reps1, dt1 = timed(rows[:1], 1, max(1.0, target_s / 4))
    used = min(threads, len(rows) * case.Hkv)
    return {"value": round(reps * len(rows) / dt, 3), "unit": "queries/s", "cores": used, "kind": "oracle",
            "sample": f"fp64 oracle decode step (scores, top-{case.topk}, attention"
                      f"{', 4 interleaved splits merged' if case.splits > 1 else ''}) on sequences "
                      f"0..{len(rows) - 1} of the {case.B}-sequence workload ({len(rows) * case.Hkv} (sequence, "
                      f"KV head) units on {used} threads), {reps} repetitions in {dt:.2f} s, block keys precomputed",
            "single_thread_value": round(reps1 / dt1, 3),
            "single_thread_sample": f"sequence 0 on 1 thread, {reps1} repetitions in {dt1:.2f} s",
            "host_threads": threads, "cpu_model": cpu_model()}


def extend_cpu_baseline(case, target_s: float, nrows: int = 128):
    """The CPU oracle on a sample of the extend chunk's rows (rows spread evenly over
    the chunk), all host threads; and a short single-thread sample."""
    import numpy as np

    import oracle

    threads = oracle.default_threads()
    rows = [int(r) for r in np.linspace(0, case.R - 1, nrows).round()]
    data = oracle.CaseData(case)
    data.prefetch([0], threads)  # logical K and block keys: not timed
    data.V(0)

    def timed(rows_, nthreads, span):
        reps = 0
        t0 = time.perf_counter()
        while True:
            oracle.run_case(case, rows=rows_, threads=nthreads, data=data, keep_scores=False)
            reps += 1
            if time.perf_counter() - t0 >= span:
                break
        return reps, time.perf_counter() - t0

    reps, dt = timed(rows, threads, target_s)
    reps1, dt1 = timed(rows[:8], 1, max(1.0, target_s / 4))
    return {"value": round(reps * len(rows) / dt, 3), "unit": "new tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 oracle extend rows (scores, top-{case.topk}, causal attention) for {len(rows)} of the "
                      f"chunk's {case.R} new tokens, spread evenly over it, on {threads} threads, {reps} repetitions "
                      f"in {dt:.2f} s, block keys precomputed",
            "single_thread_value": round(reps1 * 8 / dt1, 3),
            "single_thread_sample": f"8 of those rows on 1 thread, {reps1} repetitions in {dt1:.2f} s",
            "host_threads": threads, "cpu_model": cpu_model()}


def traffic_record(case):
    """HBM bytes per launch of the scan from the committed PMC summary of this
    workload, or None when the scan's sources changed since it was taken."""
    path = os.path.join(PROFILES, f"scores_stream_kernel_{case.name}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if (rec.get("source_sha256_16") == source_hash(SCORES_SRC) and rec.get("workload") == case.name
            and rec.get("ckey_dtype", "fp32") == case.ckey_dtype and rec.get("kv_dtype", "bf16") == case.kv_dtype):
        return rec.get("hbm_bytes_per_launch")
    return None


class Timer:
    """HIP events on the current stream (the one the library launches on)."""

    def __init__(self, steps: int, marks: int):
        import torch

        self.ev = [[torch.cuda.Event(enable_timing=True) for _ in range(marks)] for _ in range(steps)]

    def ms(self):
        import numpy as np

        return np.array([[ev[j].elapsed_time(ev[j + 1]) for j in range(len(ev) - 1)] for ev in self.ev])


def decode_record(name: str, args, headline: bool) -> dict:
    """Measure one decode workload: the step, its kernels, its roofline and (unless
    disabled) its CPU oracle baseline."""
    import numpy as np
    import torch

    import block_sparse_attention_compress_amd as qsa
    import synth
    from block_sparse_attention_compress_amd.pipeline import (DecodeBuffers, DecodeGraph, FusedDecodeBuffers,
                                                             decode_step, decode_step_fused)

    case = synth.config(name)
    case.ckey_dtype = args.ckey
    case.kv_dtype = args.kv
    log(f"workload {case.name}: B={case.B} lens {int(case.lens.min())}..{int(case.lens.max())} "
        f"heads ({case.Hq},{case.Hkv}) page {case.page_size}")
    t0 = time.perf_counter()
    dev = synth.to_device(case, "cuda")
    case.drop_paged()
    log(f"{name}: inputs generated and uploaded in {time.perf_counter() - t0:.1f} s")
    kv = qsa.KVCache(dev["k"], dev["v"], dev["ckey"], dev["block_table"], dev["seq_lens"], case.max_len)
    q, q_pos = dev["q"], dev["q_pos"]
    stride = (max(case.nb(i) for i in range(case.B)) + 63) // 64 * 64  # 16-byte rows for the selection's loads
    buf = DecodeBuffers.allocate(case.B, case.Hq, case.Hkv, stride, case.topk, 0, "cuda")
    steps, warmup = args.steps, args.warmup

    # full block-key build (prefill-time work, timed on its own)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    qsa.qsa_compress_keys(kv)
    e0.record()
    qsa.qsa_compress_keys(kv)
    e1.record()
    torch.cuda.synchronize()
    compress_full_ms = e0.elapsed_time(e1)

    internal = 0 if args.splits is None else args.splits
    ws, tw = buf.workspace, buf.topk_workspace
    S = case.splits                                            # > 1: the workload names interleaved partials
    part_out = part_lse = None
    if S > 1:
        part_out = torch.empty((S, case.B, case.Hq, 256), dtype=torch.float32, device="cuda")
        part_lse = torch.empty((S, case.B, case.Hq), dtype=torch.float32, device="cuda")
    N = case.B * case.Hq

    def scan():
        qsa.qsa_decode_scores_refresh(kv, q, q.stride(0), case.Hq, buf.scores, stride)

    def topk():
        qsa.qsa_topk_blocks_ws(buf.scores, stride, q_pos, case.B, case.Hkv, case.topk, buf.sel_idx, buf.sel_cnt,
                               workspace=tw, workspace_bytes=0 if tw is None else tw.numel())

    def attn_internal():
        qsa.qsa_sparse_attn_decode(kv, q, q.stride(0), case.Hq, buf.sel_idx, buf.sel_cnt, case.topk, case.scale,
                                   internal, buf.out, buf.out.stride(0), buf.lse, workspace=ws,
                                   workspace_bytes=0 if ws is None else ws.numel())

    def attn_partials():
        qsa.qsa_sparse_attn_decode(kv, q, q.stride(0), case.Hq, buf.sel_idx, buf.sel_cnt, case.topk, case.scale,
                                   S, None, 0, None, part_out, part_lse)

    def merge():
        qsa.qsa_merge_lse(part_out, part_lse, S, N, 256, buf.out, buf.lse)

    # the step as the workload names it: for C5 the interleaved partials and the merge
    launches = [scan, topk] + ([attn_partials, merge] if S > 1 else [attn_internal])
    names = ["refresh_and_scores", "topk"] + (["attention_partials", "merge_lse"] if S > 1 else
                                              ["attention_and_merge"])

    def step(ev=None):
        for j, f in enumerate(launches):
            if ev is not None:
                ev[j].record()
            f()
        if ev is not None:
            ev[len(launches)].record()

    def wall(fn, n):
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t) / n * 1e3

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # (1) eager steps with HIP events between the launches: per-kernel times
    tm = Timer(steps, len(launches) + 1)
    for i in range(steps):
        step(tm.ev[i])
    torch.cuda.synchronize()
    part_ms = tm.ms().mean(axis=0)
    # (2) eager steps, nothing between the launches
    eager_ms = wall(step, steps)
    ms_per_step, mode = eager_ms, "eager"
    # (3) optionally, the step captured once in a HIP graph and replayed
    if args.graph and S == 1:
        graph = DecodeGraph(kv, q, q_pos, buf, scale=case.scale, num_splits=internal)
        for _ in range(warmup):
            graph.replay()
        ms_per_step, mode = wall(graph.replay, steps), "hip-graph replay"

    # the internal split beside the named interleaved path (C5)
    internal_rec = None
    if S > 1:
        for _ in range(warmup):
            decode_step(kv, q, q_pos, buf, scale=case.scale, num_splits=internal)
        ims = wall(lambda: decode_step(kv, q, q_pos, buf, scale=case.scale, num_splits=internal), steps)
        internal_rec = {"ms_per_step": round(ims, 4), "queries_per_s": round(case.B / (ims / 1e3), 1),
                        "path": "qsa_decode_scores_refresh, qsa_topk_blocks_ws, qsa_sparse_attn_decode with the "
                                "library's split count (contiguous block ranges, merged inside the call)"}

    # (4) optionally, cold-cache steps: a 1 GiB read before each one evicts L2 and the MALL
    cold = None
    if args.flush:
        junk = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        cold_ms = []
        for i in range(steps):
            junk.sum()
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record()
            step()
            c1.record()
            torch.cuda.synchronize()
            cold_ms.append(c0.elapsed_time(c1))
        del junk
        cm = float(np.median(cold_ms))
        cold = {"ms_per_step_median": round(cm, 4), "queries_per_s": round(case.B / (cm / 1e3), 1),
                "flush_bytes_read": 1 << 30}

    # (5) optionally, the fused single-launch step (qsa_decode_fused), beside the step
    fused = None
    if args.fused:
        fb = FusedDecodeBuffers.allocate(kv, case.Hq, case.topk, internal)
        for _ in range(warmup):
            decode_step_fused(kv, q, q_pos, fb, scale=case.scale)
        fms = wall(lambda: decode_step_fused(kv, q, q_pos, fb, scale=case.scale), steps)
        fused = {"ms_per_step": round(fms, 4), "queries_per_s": round(case.B / (fms / 1e3), 1),
                 "vs_step": round(ms_per_step / fms, 3),
                 "selection_equal": bool(torch.equal(fb.sel_idx, buf.sel_idx)),
                 "abandoned_waits": int(fb.workspace[8:12].view(torch.int32).item())}
        del fb

    # the selection of the timed path (identical for every path: same scores, same select)
    step()
    torch.cuda.synchronize()
    sel = buf.sel_idx.cpu().numpy()
    cnt = buf.sel_cnt.cpu().numpy()
    by = decode_bytes(case, sel, cnt, case.page_size, S)
    scan_ms = float(part_ms[0])
    achieved = by["scan"] / (scan_ms / 1e3) / 1e9
    step_gbs = by["step"] / (ms_per_step / 1e3) / 1e9

    rec = {
        "workload": describe(case),
        "batch": case.B, "mean_context": float(case.lens.mean()), "topk_blocks": case.topk,
        "queries_per_s": round(case.B / (ms_per_step / 1e3), 1),
        "ms_per_step": round(ms_per_step, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_record(case),
                     "kernel": "scores_stream_kernel (newest block key rebuilt + block-score scan)",
                     "algorithmic_bytes_per_launch": by["scan"],
                     "overhead_bytes_per_launch": by["scan_overhead"],
                     "avg_launch_ms": round(scan_ms, 5),
                     "step_algorithmic_bytes": by["step"],
                     "step_achieved": round(step_gbs, 1),
                     "step_frac": round(step_gbs / HBM_PEAK_GBS, 4)},
        "step": {"path": " -> ".join(names), "selected_tokens": by["tokens"],
                 "overhead_bytes": by["step_overhead"],
                 "event_ms": {n: round(float(m), 5) for n, m in zip(names, part_ms)},
                 "execution": mode, "eager_ms_per_step": round(eager_ms, 4),
                 "internal_split": internal_rec, "fused_single_launch": fused, "cold_cache": cold,
                 "full_block_key_build_ms": round(compress_full_ms, 4)},
    }
    del dev, kv, q, q_pos, buf, part_out, part_lse
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        secs = args.cpu_seconds if headline else 0.4 * args.cpu_seconds
        rows = {"C1": 1, "C2": 8, "C3": 4, "C5": 16}[name]
        t0 = time.perf_counter()
        rec["cpu_baseline"] = cpu_baseline(case, secs, rows)
        log(f"{name}: cpu baseline in {time.perf_counter() - t0:.1f} s")
    return rec


def extend_figures(steps: int, flush: bool = False, ckey_dtype: str = "fp32", kv_dtype: str = "bf16",
                   q_share: float = 0.0, cpu_seconds: float = 0.0):
    """Extend chunk: 4096 new query tokens on 28672 cached (32768 total), (12, 1) heads."""
    import numpy as np
    import torch

    import block_sparse_attention_compress_amd as qsa
    import synth
    from block_sparse_attention_compress_amd.pipeline import ExtendBuffers, extend_step

    case = synth.config("C4", q_share=q_share)
    case.ckey_dtype, case.kv_dtype = ckey_dtype, kv_dtype
    dev = synth.to_device(case, "cuda")
    kv = qsa.KVCache(dev["k"], dev["v"], dev["ckey"], dev["block_table"], dev["seq_lens"], case.max_len)
    first = torch.tensor([int(case.q_pos[0])], dtype=torch.int32, device="cuda")
    qsa.qsa_compress_keys(kv)                                  # cached blocks
    stride = case.nb(0)
    buf = ExtendBuffers.allocate(case.R, case.Hq, case.Hkv, stride, 512, "cuda")
    q, q_seq, q_pos = dev["q"], dev["q_seq"], dev["q_pos"]
    R, Hq, Hkv = case.R, case.Hq, case.Hkv
    launches = [
        lambda: qsa.qsa_compress_keys(kv, first, 0),
        lambda: qsa.qsa_block_scores(kv, q, q.stride(0), q_seq, q_pos, R, Hq, buf.scores, stride),
        lambda: qsa.qsa_topk_blocks(buf.scores, stride, q_pos, R, Hkv, 512, buf.sel_idx, buf.sel_cnt),
        lambda: qsa.qsa_sparse_attn_extend(kv, q, q.stride(0), q_seq, q_pos, R, Hq, buf.sel_idx, buf.sel_cnt, 512,
                                           case.scale, buf.out, buf.out.stride(0), buf.lse),
    ]
    names = ["block_keys", "scores", "topk", "attention"]
    for _ in range(2):
        extend_step(kv, q, q_seq, q_pos, buf, first, scale=case.scale)
    torch.cuda.synchronize()
    tm = Timer(steps, len(launches) + 1)
    for i in range(steps):
        for j, f in enumerate(launches):
            tm.ev[i][j].record()
            f()
        tm.ev[i][len(launches)].record()
    torch.cuda.synchronize()
    part_ms = tm.ms().mean(axis=0)
    t0 = time.perf_counter()
    for _ in range(steps):
        extend_step(kv, q, q_seq, q_pos, buf, first, scale=case.scale)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    cold = None
    if flush:  # a 1 GiB read before each chunk evicts L2 and the MALL
        junk = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        ms = []
        for i in range(steps):
            junk.sum()
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record()
            extend_step(kv, q, q_seq, q_pos, buf, first, scale=case.scale)
            c1.record()
            torch.cuda.synchronize()
            ms.append(c0.elapsed_time(c1))
        del junk
        cold = round(float(np.median(ms)), 4)
    # matrix-core work: scores 2*256 per eligible block per row; attention 2 * 2 * 256
    # per (selected token, real head)
    elig = sum(min(int(t) // 4 + 1, stride) for t in case.q_pos)
    # the query-tile union kernel on the same selection (an alternative entry point, timed beside)
    uo = torch.empty_like(buf.out)
    ul = torch.empty_like(buf.lse)
    union = lambda: qsa.qsa_sparse_attn_extend_union(kv, q, q.stride(0), q_seq, q_pos, R, Hq, buf.sel_idx,
                                                     buf.sel_cnt, 512, case.scale, uo, uo.stride(0), ul)
    union()
    torch.cuda.synchronize()
    ut = Timer(steps, 2)
    for i in range(steps):
        ut.ev[i][0].record()
        union()
        ut.ev[i][1].record()
    torch.cuda.synchronize()
    union_ms = float(ut.ms().mean(axis=0)[0])
    cnt = buf.sel_cnt.cpu().numpy()
    score_flops = 2 * 256 * elig
    attn_flops = 4 * 256 * case.Hq * int(cnt.sum()) * 4
    return {"workload": f"extend: 4096 new tokens on 28672 cached, (12,1) heads, top-512 per query, "
                        f"{kv_dtype} K/V, {ckey_dtype} block keys"
                        + (f", queries with a shared per-sequence component (weight {q_share})" if q_share else ""),
            "new_tokens_per_s": round(case.R / dt, 1), "ms_per_chunk": round(dt * 1e3, 4),
            "tflops": round((score_flops + attn_flops) / dt / 1e12, 2),
            "event_ms": {n: round(float(m), 5) for n, m in zip(names, part_ms)},
            # the scores run on bf16 matrix cores with each fp32 operand split into three
            # bf16 pieces: 6 bf16 products per fp32 product (3 with bf16 or fp8 block keys)
            "scores_tflops": round(score_flops / (part_ms[1] / 1e3) / 1e12, 2),
            "scores_frac_of_fp32_matrix_peak": round(score_flops / (part_ms[1] / 1e3) / 157.3e12, 4),
            "scores_bf16_mfma_frac": round((6 if ckey_dtype == "fp32" else 3) * score_flops / (part_ms[1] / 1e3)
                                           / 2.5e15, 4),
            "attention_tflops": round(attn_flops / (part_ms[3] / 1e3) / 1e12, 2),
            "union_attention_event_ms": round(union_ms, 5),
            "cold_cache_ms_per_chunk_median": cold,
            "cpu_baseline": extend_cpu_baseline(case, cpu_seconds) if cpu_seconds > 0 else None}


def small_chunk_figures(steps: int, kv_dtype: str = "bf16", ckey_dtype: str = "fp32", rows=(32, 64, 128)):
    """Extend chunks of few rows: the newest R tokens of one 32,768-token sequence, (12,1)
    heads, top-512.  The chunk's attention with one workgroup per (row, KV head) against
    the split read merged by log-sum-exp (qsa_sparse_attn_extend_split, the library's split
    count), and the whole chunk (block keys of the new tokens, scores, top-k, attention)
    both ways."""
    import torch

    import block_sparse_attention_compress_amd as qsa
    import synth
    from block_sparse_attention_compress_amd.pipeline import ExtendBuffers, extend_step

    def wall(fn, n):
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t) / n * 1e3

    total = 32768
    out = []
    for R in rows:
        q_pos = list(range(total - R, total))
        case = synth.make_case(f"small{R}", 700 + R, 12, 1, [total], page_size=total, q_seq=[0] * R, q_pos=q_pos,
                               shuffle=False, ckey_dtype=ckey_dtype, kv_dtype=kv_dtype)
        dev = synth.to_device(case, "cuda")
        kv = qsa.KVCache(dev["k"], dev["v"], dev["ckey"], dev["block_table"], dev["seq_lens"], case.max_len)
        qsa.qsa_compress_keys(kv)
        first = torch.tensor([total - R], dtype=torch.int32, device="cuda")
        stride = case.nb(0)
        buf = ExtendBuffers.allocate(R, case.Hq, case.Hkv, stride, 512, "cuda", max_splits=0)
        q, q_seq, qp = dev["q"], dev["q_seq"], dev["q_pos"]
        ws = buf.workspace
        wsb = ws.numel() if ws is not None else 0
        attn = {
            "unsplit": lambda: qsa.qsa_sparse_attn_extend(kv, q, q.stride(0), q_seq, qp, R, case.Hq, buf.sel_idx,
                                                          buf.sel_cnt, 512, case.scale, buf.out, buf.out.stride(0),
                                                          buf.lse),
            "split": lambda: qsa.qsa_sparse_attn_extend_split(kv, q, q.stride(0), q_seq, qp, R, case.Hq, buf.sel_idx,
                                                              buf.sel_cnt, 512, case.scale, 0, buf.out,
                                                              buf.out.stride(0), buf.lse, workspace=ws,
                                                              workspace_bytes=wsb),
        }
        extend_step(kv, q, q_seq, qp, buf, first, scale=case.scale)
        torch.cuda.synchronize()
        rec = {"new_tokens": R, "context": total}
        for name, f in attn.items():
            f()
            rec[f"attention_ms_{name}"] = round(wall(f, steps), 5)
        for name, S in (("unsplit", 1), ("split", 0)):
            step = lambda: extend_step(kv, q, q_seq, qp, buf, first, scale=case.scale, num_splits=S)
            step()
            rec[f"chunk_ms_{name}"] = round(wall(step, steps), 5)
        log(f"small extend chunk {R} rows: attention {rec['attention_ms_unsplit']} -> {rec['attention_ms_split']} ms, "
            f"chunk {rec['chunk_ms_unsplit']} -> {rec['chunk_ms_split']} ms")
        out.append(rec)
        del dev, kv, buf
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the library has no multi-GPU path; "
              f"run it with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.copy_calibration:
        copy_calibration()
        return
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.extend_only:
        print(json.dumps(extend_figures(args.steps, args.flush, args.ckey, args.kv, args.q_share)), flush=True)
        return
    import block_sparse_attention_compress_amd as qsa

    qsa.lib()
    names = DECODE_CONFIGS if args.config == "all" else (args.config,)
    records = {}
    for i, name in enumerate(names):
        records[name] = decode_record(name, args, headline=(i == 0))
    head_name = names[0]
    head = records[head_name]
    result = {
        "metric": METRIC,
        "value": head["queries_per_s"],
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE if (args.ckey, args.kv) == ("fp32", "bf16") else f"{args.ckey} block keys, {args.kv} K/V",
        "data": "synthetic (seeded SplitMix64/Box-Muller bf16 K/V and queries)",
        "config": {"workload": head["workload"], "batch": head["batch"], "mean_context": head["mean_context"],
                   "topk_blocks": head["topk_blocks"], "parallelism": "1 GPU"},
        "roofline": head["roofline"],
        "step": head["step"],
    }
    if "cpu_baseline" in head:
        result["cpu_baseline"] = head["cpu_baseline"]
    if len(names) > 1:
        result["configs"] = {n: records[n] for n in names[1:]}
    if not args.no_extend:
        result["extend"] = extend_figures(max(20, args.steps // 2), args.flush, args.ckey, args.kv,
                                          cpu_seconds=0.0 if args.no_cpu_baseline else 0.4 * args.cpu_seconds)
        result["extend"]["small_chunks"] = small_chunk_figures(max(20, args.steps // 2), args.kv, args.ckey)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
