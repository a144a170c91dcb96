"""The benchmark's host-side contract, checked without a GPU: it refuses more than
one GPU with a message and exit status 2, and its byte model counts what the
roofline object states (block keys at their storage width, q rows, table and
lengths as algorithmic bytes; score writes and the refreshed key as overhead)."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_scan_bytes_follow_the_key_storage_width():
    case = synth.config("C2", B=3, L_range=(4096, 8192))
    B, Hkv = case.B, case.Hkv
    nb = np.array([case.nb(i) for i in range(B)])
    sel = np.zeros((B, Hkv, case.topk), dtype=np.int32)
    cnt = np.zeros((B, Hkv), dtype=np.int32)
    per_key = {}
    for ck in ("fp32", "bf16", "fp8"):
        case.ckey_dtype = ck
        by = bench.decode_bytes(case, sel, cnt, case.page_size, 1)
        per_key[ck] = by["scan"]
    keys = int(nb.sum()) * Hkv * 256
    # the scan's algorithmic bytes differ only in the block keys: 4, 2 and 1 bytes per element
    assert per_key["fp32"] - per_key["bf16"] == keys * 2
    assert per_key["bf16"] - per_key["fp8"] == keys


def test_scan_overhead_is_reported_apart_from_algorithmic_bytes():
    case = synth.config("C2", B=2, L_range=(3000, 5000))
    sel = np.zeros((case.B, case.Hkv, case.topk), dtype=np.int32)
    cnt = np.zeros((case.B, case.Hkv), dtype=np.int32)
    by = bench.decode_bytes(case, sel, cnt, case.page_size, 1)
    nb_total = sum(case.nb(i) for i in range(case.B))
    # algorithmic: keys (1 KiB each for fp32), the bf16 query rows, table entries and lengths
    pages = sum((int(L) + case.page_size - 1) // case.page_size for L in case.lens)
    assert by["scan"] == nb_total * case.Hkv * 1024 + case.B * case.Hq * 512 + pages * 4 + case.B * 4
    # overhead: 4 B of score per block and KV head, plus the refreshed newest key (its K rows and the key)
    refresh = sum((int(L) - 4 * ((int(L) - 1) // 4)) * 512 + 1024 for L in case.lens) * case.Hkv
    assert by["scan_overhead"] == nb_total * case.Hkv * 4 + refresh
