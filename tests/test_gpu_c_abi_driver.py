"""A decode step and an extend chunk driven from C++ through include/qsa.h alone
(tests/c_abi_driver.cpp: no Python and no torch in that process; it allocates its
own device memory and stream).  Its results are held to the bars of the
Python-driven parity tests: block keys bit-exact against the oracle, the selection
bit-exact on the driver's own fp32 scores and within the swap window against the
oracle, outputs and lse within |gpu - oracle| <= 1e-2 + 1e-2 |oracle|.  The driver
also checks that an out-of-range argument is rejected with a message."""
import os
import subprocess
from types import SimpleNamespace

import numpy as np
import pytest

import oracle
import synth
from test_gpu_parity import check_decode_against_oracle

pytestmark = pytest.mark.gpu

DRIVER = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_driver")
KV_CODE = {"bf16": 0, "fp8": 1}
CKEY_CODE = {"fp32": 0, "bf16": 1, "fp8": 2}


def ckey_logical(case, pool: np.ndarray, i: int) -> np.ndarray:
    """Block keys of sequence i, [Hkv][nb][256], gathered from the driver's pool."""
    nb = case.nb(i)
    b = np.arange(nb)
    pages = case.block_table[i][(4 * b) // case.page_size]
    slots = ((4 * b) % case.page_size) // 4
    return np.ascontiguousarray(pool[pages, :, slots, :].transpose(1, 0, 2))


def run_driver(tmp_path, case, mode):
    assert os.path.exists(DRIVER), "tests/c_abi_driver is not built: run __graft_entry__.build()"
    stride = (max(case.nb(i) for i in range(case.B)) + 63) // 64 * 64 if mode == "decode" else case.nb(0)
    k = case.topk
    d = tmp_path
    (d / "meta.txt").write_text(f"{case.B} {case.Hq} {case.Hkv} {case.page_size} {case.num_pages} {case.max_pages} "
                                f"{case.max_len} {k} {stride} {KV_CODE[case.kv_dtype]} {CKEY_CODE[case.ckey_dtype]} "
                                f"{case.R}\n")
    case.paged_device("k").tofile(d / "k.bin")
    case.paged_device("v").tofile(d / "v.bin")
    np.ascontiguousarray(case.block_table, dtype=np.int32).tofile(d / "table.bin")
    np.ascontiguousarray(case.lens, dtype=np.int32).tofile(d / "lens.bin")
    np.ascontiguousarray(case.q).tofile(d / "q.bin")
    if mode == "extend":
        np.ascontiguousarray(case.q_seq, dtype=np.int32).tofile(d / "q_seq.bin")
        np.ascontiguousarray(case.q_pos, dtype=np.int32).tofile(d / "q_pos.bin")
    print(f"[c_abi_driver] {mode}, {case.kv_dtype} cache, {case.ckey_dtype} block keys, lens={case.lens.tolist()}, "
          f"rows={case.R}", flush=True)
    r = subprocess.run([DRIVER, str(d), mode], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "rejected as expected" in r.stdout, r.stdout

    R, Hq, Hkv = case.R, case.Hq, case.Hkv
    ckey_dt = {"fp32": np.float32, "bf16": np.uint16}[case.ckey_dtype]
    pool = np.fromfile(d / "ckey.bin", ckey_dt).reshape(case.num_pages, Hkv, case.page_size // 4, 256)
    if case.ckey_dtype == "bf16":
        pool = (pool.astype(np.uint32) << 16).view(np.float32)
    for i in range(case.B):
        got = ckey_logical(case, pool, i)
        K = case.logical("k", i)
        for h in range(Hkv):
            want = oracle.compress(K[h], case.ckey_dtype)
            assert np.array_equal(got[h].view(np.uint32), want.view(np.uint32)), (i, h)

    scores = np.fromfile(d / "scores.bin", np.float32).reshape(R, Hkv, stride)
    sel = np.fromfile(d / "sel.bin", np.int32).reshape(R, Hkv, k)
    cnt = np.fromfile(d / "cnt.bin", np.int32).reshape(R, Hkv)
    out = synth.bf16_to_f32(np.fromfile(d / "out.bin", np.uint16).reshape(R, Hq, 256))
    lse = np.fromfile(d / "lse.bin", np.float32).reshape(R, Hq)
    check_decode_against_oracle(case, SimpleNamespace(stride=stride), scores, sel, cnt, out, lse, k)


@pytest.mark.parametrize("kv_dtype,ckey_dtype", [("bf16", "fp32"), ("fp8", "bf16")])
def test_decode_step_through_the_c_abi_alone(tmp_path, kv_dtype, ckey_dtype):
    case = synth.make_case(f"cabi{kv_dtype}", 93, 16, 2, [3000, 4097, 130, 20000], page_size=64, jitter=True,
                           kv_dtype=kv_dtype, ckey_dtype=ckey_dtype)
    run_driver(tmp_path, case, "decode")


def test_extend_chunk_through_the_c_abi_alone(tmp_path):
    total, new = 5000, 300
    q_seq, q_pos = synth.extend_rows(total, new)
    case = synth.make_case("cabix", 94, 12, 1, [total], page_size=64, q_seq=q_seq, q_pos=q_pos, jitter=True)
    run_driver(tmp_path, case, "extend")
