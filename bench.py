#!/usr/bin/env python3
"""QSA decode benchmark on one MI355X.

A step is one pass of the whole decode hot path for every sequence of the batch:
refresh the block key holding the newest token, score every eligible block
against the group-summed query, keep the top-512 blocks, run the sparse attention
over their uncompressed K/V (split-KV partials merged by log-sum-exp).  Inputs are
seeded synthetic tensors (``synth``) already resident in HBM when timing starts.

Default workload: 32 sequences with lengths uniform on [32768, 65536], 16 query /
2 KV heads, head_dim 256, bf16 K/V with a U(0.5, 2) norm jitter per token,
64-token pages under a shuffled block table, top-512 blocks.

Prints one JSON line: queries/s for the step, the roofline of the dominant kernel
(the block-score scan over fp32 block keys, HBM-bound), and the CPU oracle timed
on a bounded sample of the same workload on the host cores.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--config C2]
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scores_stream_kernel_C2_traffic.json")
SCORES_SRC = [os.path.join(ROOT, "block_sparse_attention_compress_amd", "csrc", f)
              for f in ("scores.hip", "scan_body.h", "qsa_device.h")]


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", default="C2", choices=["C1", "C2", "C3", "C5"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extend", action="store_true", help="skip the extend (prefill chunk) figures")
    p.add_argument("--extend-only", action="store_true",
                   help="print only the extend chunk's figures (one JSON object; for profiling the chunk alone)")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="target oracle timing span (seconds of wall time)")
    p.add_argument("--copy-calibration", action="store_true")
    p.add_argument("--graph", action="store_true", help="time a replayed HIP graph of the step instead of eager launches")
    p.add_argument("--splits", type=int, default=None, help="decode split count (default: the library's choice)")
    p.add_argument("--no-fused", action="store_true", help="skip the single-launch fused step figures")
    p.add_argument("--flush", action="store_true",
                   help="also time single steps after a 1 GiB read that evicts the caches (MALL included)")
    p.add_argument("--kv", choices=["bf16", "fp8"], default="bf16",
                   help="main cache storage (bf16; fp8: E4M3 codes of the same draws)")
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
        extra.append(f"{case.splits} split-KV partitions merged by log-sum-exp")
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


def decode_bytes(case, sel, cnt, page_size):
    """Algorithmic HBM bytes of one decode step, and of its refresh-and-score launch.

    step: per (sequence, KV head) the block-key scan (nb * 1 KiB for fp32 keys,
    nb * 512 B for bf16 keys, nb * 256 B for fp8 keys), the rebuilt newest block key (its 1..4 bf16 K rows
    read, one block key written) and the bf16 K and V rows of the selected tokens
    (512 B each), plus q and out rows (bf16), lse (fp32), the block table and the
    lengths.
    refresh-and-score launch: the block-key scan, the rebuilt key, the q rows,
    the score writes (4 B per block) and the block table."""
    import numpy as np

    B, Hkv, Hq = case.B, case.Hkv, case.Hq
    nb = np.array([case.nb(i) for i in range(B)], dtype=np.int64)
    key_bytes = 256 * {"bf16": 2, "fp8": 1}.get(case.ckey_dtype, 4)
    ckey = int(nb.sum()) * Hkv * key_bytes
    row_bytes = 256 if case.kv_dtype == "fp8" else 512  # one K or V row
    refresh = sum((int(L) - 4 * ((int(L) - 1) // 4)) * row_bytes + key_bytes for L in case.lens if L > 0) * Hkv
    tokens = 0
    for i in range(B):
        L = int(case.lens[i])
        for h in range(Hkv):
            c = int(cnt[i, h])
            blocks = sel[i, h, :c].astype(np.int64)
            tokens += int(np.minimum(L - 4 * blocks, 4).sum())
    kv_bytes = tokens * row_bytes * 2
    qo = B * Hq * 256 * 2 * 2 + B * Hq * 4
    table = int(sum((int(L) + page_size - 1) // page_size for L in case.lens)) * 4 + B * 4
    step = ckey + refresh + kv_bytes + qo + table
    scores = ckey + refresh + B * Hq * 256 * 2 + int(nb.sum()) * Hkv * 4 + table
    return step, scores, tokens


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(case, target_s: float):
    """The CPU oracle as it stands, timed on a sample of the same workload: on
    every host thread it may use, and on one thread (a shorter sample)."""
    import oracle

    threads = oracle.default_threads()
    rows = list(range(min(case.B, 8)))
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
    return {"value": round(reps * len(rows) / dt, 3), "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 oracle decode step (scores, top-512, attention) on sequences 0..{len(rows) - 1} of "
                      f"the {case.B}-sequence workload, {reps} repetitions in {dt:.2f} s, block keys precomputed",
            "single_thread_value": round(reps1 / dt1, 3),
            "single_thread_sample": f"sequence 0 on 1 thread, {reps1} repetitions in {dt1:.2f} s",
            "cpu_model": cpu_model()}


def extend_figures(steps: int, flush: bool = False, ckey_dtype: str = "fp32", kv_dtype: str = "bf16"):
    """Extend chunk: 4096 new query tokens on 28672 cached (32768 total), (12, 1) heads."""
    import torch

    import block_sparse_attention_compress_amd as qsa
    import synth
    from block_sparse_attention_compress_amd.pipeline import ExtendBuffers, extend_step

    case = synth.config("C4")
    case.ckey_dtype, case.kv_dtype = ckey_dtype, kv_dtype
    dev = synth.to_device(case, "cuda")
    kv = qsa.KVCache(dev["k"], dev["v"], dev["ckey"], dev["block_table"], dev["seq_lens"], case.max_len)
    first = torch.tensor([int(case.q_pos[0])], dtype=torch.int32, device="cuda")
    qsa.qsa_compress_keys(kv)                                  # cached blocks
    stride = case.nb(0)
    buf = ExtendBuffers.allocate(case.R, case.Hq, case.Hkv, stride, 512, "cuda")
    for _ in range(2):
        extend_step(kv, dev["q"], dev["q_seq"], dev["q_pos"], buf, first, case.R, scale=case.scale)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        extend_step(kv, dev["q"], dev["q_seq"], dev["q_pos"], buf, first, case.R, scale=case.scale)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    cold = None
    if flush:  # a 1 GiB read before each chunk evicts L2 and the MALL
        import numpy as np
        junk = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        ms = []
        for i in range(steps):
            junk.sum()
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record()
            extend_step(kv, dev["q"], dev["q_seq"], dev["q_pos"], buf, first, case.R, scale=case.scale)
            c1.record()
            torch.cuda.synchronize()
            ms.append(c0.elapsed_time(c1))
        del junk
        cold = round(float(np.median(ms)), 4)
    # MFMA work: scores 2*256 per eligible block per row; attention 2 * 2 * 256 per
    # (selected token, real head)
    elig = sum(min(int(t) // 4 + 1, stride) for t in case.q_pos)
    cnt = buf.sel_cnt.cpu().numpy()
    flops = 2 * 256 * elig + 4 * 256 * case.Hq * int(cnt.sum()) * 4
    return {"workload": f"extend: 4096 new tokens on 28672 cached, (12,1) heads, top-512 per query, "
                        f"{kv_dtype} K/V, {ckey_dtype} block keys",
            "new_tokens_per_s": round(case.R / dt, 1), "ms_per_chunk": round(dt * 1e3, 4),
            "tflops": round(flops / dt / 1e12, 2), "cold_cache_ms_per_chunk_median": cold}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the library has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.copy_calibration:
        copy_calibration()
        return
    if args.extend_only:
        assert torch.cuda.is_available(), "bench.py needs a GPU"
        print(json.dumps(extend_figures(args.steps, args.flush, args.ckey, args.kv)), flush=True)
        return
    import block_sparse_attention_compress_amd as qsa
    import synth
    from block_sparse_attention_compress_amd.pipeline import (DecodeBuffers, DecodeGraph, FusedDecodeBuffers,
                                                             decode_step, decode_step_fused)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    qsa.lib()
    case = synth.config(args.config)
    case.ckey_dtype = args.ckey
    case.kv_dtype = args.kv
    log(f"workload {case.name}: B={case.B} lens {int(case.lens.min())}..{int(case.lens.max())} "
        f"heads ({case.Hq},{case.Hkv}) page {case.page_size}")
    t0 = time.perf_counter()
    dev = synth.to_device(case, "cuda")
    case.drop_paged()
    log(f"inputs generated and uploaded in {time.perf_counter() - t0:.1f} s")
    kv = qsa.KVCache(dev["k"], dev["v"], dev["ckey"], dev["block_table"], dev["seq_lens"], case.max_len)
    q, q_pos = dev["q"], dev["q_pos"]
    stride = (max(case.nb(i) for i in range(case.B)) + 63) // 64 * 64  # 16-byte rows for the selection's loads
    buf = DecodeBuffers.allocate(case.B, case.Hq, case.Hkv, stride, case.topk, 0, "cuda")

    # full block-key build (prefill-time work, timed on its own)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    qsa.qsa_compress_keys(kv)
    e0.record()
    qsa.qsa_compress_keys(kv)
    e1.record()
    torch.cuda.synchronize()
    compress_full_ms = e0.elapsed_time(e1)

    splits = (0 if case.splits == 1 else case.splits) if args.splits is None else args.splits
    ws, tw = buf.workspace, buf.topk_workspace

    def step(ev=None):
        # the same calls as pipeline.decode_step, with events between the launches
        if ev is not None:
            ev[0].record()
        qsa.qsa_decode_scores_refresh(kv, q, q.stride(0), case.Hq, buf.scores, stride)
        if ev is not None:
            ev[1].record()
        qsa.qsa_topk_blocks_ws(buf.scores, stride, q_pos, case.B, case.Hkv, case.topk, buf.sel_idx, buf.sel_cnt,
                               workspace=tw, workspace_bytes=0 if tw is None else tw.numel())
        if ev is not None:
            ev[2].record()
        qsa.qsa_sparse_attn_decode(kv, q, q.stride(0), case.Hq, buf.sel_idx, buf.sel_cnt, case.topk, case.scale,
                                   splits, buf.out, buf.out.stride(0), buf.lse, workspace=ws,
                                   workspace_bytes=0 if ws is None else ws.numel())
        if ev is not None:
            ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # (1) eager steps with HIP events between the launches: per-kernel times
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    parts = np.array([[ev[j].elapsed_time(ev[j + 1]) for j in range(3)] for ev in events])  # ms
    part_ms = parts.mean(axis=0)
    # (2) eager steps, nothing between the launches
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        decode_step(kv, q, q_pos, buf, scale=case.scale, num_splits=splits)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t1) / args.steps * 1e3
    # (3) optionally, the same step captured once in a HIP graph and replayed (on
    # this stack the eager launches already run back to back, so eager is faster)
    ms_per_step = eager_ms
    mode = "eager"
    if args.graph:
        graph = DecodeGraph(kv, q, q_pos, buf, scale=case.scale, num_splits=splits)
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        ms_per_step = (time.perf_counter() - t0) / args.steps * 1e3
        mode = "hip-graph replay"

    # (3b) optionally, cold-cache steps: a 1 GiB read before each one evicts L2 and
    # the 256 MB MALL (a read, so no dirty lines are left to write back during the
    # step); HIP events bracket the step alone (median reported)
    cold = None
    if args.flush:
        junk = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        cold_ms = []
        for i in range(args.steps):
            junk.sum()
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record()
            decode_step(kv, q, q_pos, buf, scale=case.scale, num_splits=splits)
            c1.record()
            torch.cuda.synchronize()
            cold_ms.append(c0.elapsed_time(c1))
        del junk
        cm = float(np.median(cold_ms))
        cold = {"ms_per_step_median": round(cm, 4), "queries_per_s": round(case.B / (cm / 1e3), 1),
                "flush_bytes_read": 1 << 30}

    # (4) the fused single-launch step (qsa_decode_fused), reported beside the
    # headline; its selection must equal the separate calls'
    fused = None
    if not args.no_fused:
        fb = FusedDecodeBuffers.allocate(kv, case.Hq, case.topk, splits)
        for _ in range(args.warmup):
            decode_step_fused(kv, q, q_pos, fb, scale=case.scale)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        for _ in range(args.steps):
            decode_step_fused(kv, q, q_pos, fb, scale=case.scale)
        torch.cuda.synchronize()
        fused_ms = (time.perf_counter() - t2) / args.steps * 1e3
        fused = {"ms_per_step": round(fused_ms, 4), "queries_per_s": round(case.B / (fused_ms / 1e3), 1),
                 "selection_equal": bool(torch.equal(fb.sel_idx, buf.sel_idx)),
                 "abandoned_waits": int(fb.workspace[8:12].view(torch.int32).item())}
        del fb

    sel = buf.sel_idx.cpu().numpy()
    cnt = buf.sel_cnt.cpu().numpy()
    step_bytes, scores_bytes, tokens = decode_bytes(case, sel, cnt, case.page_size)
    scores_s = part_ms[0] / 1e3
    achieved = scores_bytes / scores_s / 1e9

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        rec = json.load(open(TRAFFIC_FILE))
        if (rec.get("source_sha256_16") == source_hash(SCORES_SRC) and rec.get("workload") == case.name
                and rec.get("ckey_dtype", "fp32") == case.ckey_dtype and rec.get("kv_dtype", "bf16") == case.kv_dtype):
            traffic = rec.get("hbm_bytes_per_launch")

    result = {
        "metric": METRIC,
        "value": round(case.B / (ms_per_step / 1e3), 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic (seeded SplitMix64/Box-Muller bf16 K/V and queries)",
        "config": {"workload": describe(case),
                   "batch": case.B, "mean_context": float(case.lens.mean()), "topk_blocks": case.topk,
                   "parallelism": "1 GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "scores_stream_kernel (newest block key rebuilt + block-score scan)",
                     "algorithmic_bytes_per_launch": scores_bytes, "avg_launch_ms": round(part_ms[0], 5)},
        "step": {"algorithmic_bytes": step_bytes, "algorithmic_GBps": round(step_bytes / (ms_per_step / 1e3) / 1e9, 1),
                 "selected_tokens": tokens,
                 "event_ms": {"refresh_and_scores": round(part_ms[0], 5), "topk": round(part_ms[1], 5),
                              "attention_and_merge": round(part_ms[2], 5)},
                 "execution": mode, "eager_ms_per_step": round(eager_ms, 4), "fused_single_launch": fused,
                 "cold_cache": cold,
                 "full_block_key_build_ms": round(compress_full_ms, 4)},
    }
    if not args.no_extend:
        result["extend"] = extend_figures(max(3, args.steps // 4), args.flush, args.ckey, args.kv)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
