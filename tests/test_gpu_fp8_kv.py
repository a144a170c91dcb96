"""An fp8 main cache (QSA_KV_FP8: K and V rows stored as OCP E4M3 codes) through the
C ABI.  Every kernel must behave as on a bf16 cache holding the decoded values: the
block keys bit-exact against the oracle's means of the decoded keys, the refresh
launch equal to the separate calls, selections exact up to swaps within 1e-4 of
the k-th score, outputs within |gpu - oracle| <= 1e-2 + 1e-2 |oracle| -- for
decode (page sizes, head pairs, splits), extend, the fused launch and the
full-size decode workload."""
import numpy as np
import pytest
import torch

import block_sparse_attention_compress_amd as qsa
import oracle
import synth
from gpu_harness import Dev, log, to_np
from parity import check_close, check_lse
from test_gpu_parity import check_decode_against_oracle, run_decode, run_extend

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def kv8_case(name, seed, Hq, Hkv, lens, page_size=64, **kw):
    return synth.make_case(name, seed, Hq, Hkv, lens, page_size=page_size, kv_dtype="fp8", **kw)


@pytest.mark.parametrize("ckey_dtype", ["fp32", "bf16", "fp8"])
@pytest.mark.parametrize("page_size,lens", [(64, [4096, 4097, 4098, 4099]), (4, [37, 64, 1]), (8192, [8192])])
def test_block_keys_from_fp8_keys(ckey_dtype, page_size, lens):
    case = kv8_case(f"k8c{page_size}", 160 + page_size, 8, 2, lens, page_size, jitter=True, ckey_dtype=ckey_dtype)
    log(f"fp8 cache compress page_size={page_size} lens={lens} ckey={ckey_dtype}")
    d = Dev(case)
    assert d.t["k"].dtype == torch.float8_e4m3fn and d.kv.descriptor().kv_dtype == qsa.KV_FP8
    d.compress()
    torch.cuda.synchronize()
    for i in range(case.B):
        K = case.logical("k", i)
        if ckey_dtype == "fp8":
            got = d.ckey_codes(i)
            for h in range(case.Hkv):
                assert np.array_equal(got[h], oracle.compress_fp8_codes(K[h])), (i, h)
        else:
            got = d.ckey_logical(i)
            for h in range(case.Hkv):
                want = oracle.compress(K[h], ckey_dtype)
                assert np.array_equal(got[h].view(np.uint32), want.view(np.uint32)), (i, h)


@pytest.mark.parametrize("page_size", [4, 16, 64, 8192])
def test_decode_step_page_sizes(page_size):
    lens = [8192, 5000, 777] if page_size == 8192 else [7000, 5000, 777]
    case = kv8_case(f"k8p{page_size}", 520 + page_size, 16, 2, lens, page_size, jitter=True,
                    shuffle=page_size < 8192)
    log(f"fp8 cache decode page_size={page_size}")
    res = run_decode(case)
    check_decode_against_oracle(case, *res, case.topk)


@pytest.mark.parametrize("Hq,Hkv", [(24, 2), (12, 1), (6, 1), (3, 1)])
def test_decode_step_head_pairs(Hq, Hkv):
    case = kv8_case(f"k8h{Hq}", 620 + Hq, Hq, Hkv, [2051, 4097, 9000, 130], jitter=True)
    res = run_decode(case)
    check_decode_against_oracle(case, *res, case.topk)


@pytest.mark.parametrize("S", [3, 4])
def test_split_partials(S):
    case = kv8_case(f"k8s{S}", 700 + S, 6, 1, [5001, 7000, 2222, 12000])
    d = Dev(case)
    d.compress()
    sc = d.scores()
    sel, cnt = d.topk(sc, 512)
    po, pl = d.decode_partials(sel, cnt, 512, S)
    internal, ilse = d.decode_attn(sel, cnt, 512, num_splits=S)
    torch.cuda.synchronize()
    sel_np, cnt_np = to_np(sel), to_np(cnt)
    override = {(r, 0): (sel_np[r, 0], int(cnt_np[r, 0])) for r in range(case.R)}
    ref = oracle.run_case(case, splits=S, sel_override=override)
    po, pl = to_np(po), to_np(pl)
    for r in range(case.R):
        check_close(po[:, r], ref.part_out[r], f"partials row {r}")
        check_lse(pl[:, r], ref.part_lse[r], f"partial lse row {r}")
        check_close(to_np(internal)[r], ref.out[r], f"internal row {r}")
        check_lse(to_np(ilse)[r], ref.lse[r], f"internal lse row {r}")


def test_extend_step():
    total, nq = 3000, 257
    q_seq, q_pos = synth.extend_rows(total, nq)
    case = synth.make_case("k8ext", 514, 12, 1, [total], page_size=64, q_seq=q_seq, q_pos=q_pos, kv_dtype="fp8")
    res = run_extend(case)
    check_decode_against_oracle(case, *res, case.topk)


def test_fused_decode():
    from test_gpu_fused import check_fused
    case = kv8_case("k8fused", 16, 16, 2, [9000, 4097, 6000, 20000])
    check_fused(case)


def test_refresh_scores_equal_separate_calls():
    from test_gpu_refresh import both_paths
    for ck in ("fp32", "fp8"):
        case = kv8_case(f"k8rf{ck}", 730, 16, 2, [4096, 4097, 4098, 4099, 1, 5], jitter=True, ckey_dtype=ck)
        both_paths(case)


def test_full_size_decode_all_rows():
    """32 sequences of 32K-64K tokens on an fp8 cache, in the benchmark's launch
    configuration, against the oracle on every row."""
    from test_gpu_configs import all_row_properties, compare_rows, upload
    from block_sparse_attention_compress_amd.pipeline import DecodeBuffers, decode_step
    case = synth.config("C2")
    case.kv_dtype = "fp8"
    dev, kv = upload(case)
    assert dev["k"].dtype == torch.float8_e4m3fn
    qsa.qsa_compress_keys(kv)
    stride = (max(case.nb(i) for i in range(case.B)) + 63) // 64 * 64
    buf = DecodeBuffers.allocate(case.B, case.Hq, case.Hkv, stride, case.topk, 0, "cuda")
    decode_step(kv, dev["q"], dev["q_pos"], buf, scale=case.scale)
    torch.cuda.synchronize()
    sel, cnt, out, lse = to_np(buf.sel_idx), to_np(buf.sel_cnt), to_np(buf.out), to_np(buf.lse)
    all_row_properties(case, sel, cnt, out, lse)
    compare_rows(case, list(range(case.B)), sel, cnt, out, lse, stride)
