"""bf16 block keys (QSA_CKEY_BF16) through the C ABI: the stored keys must equal the
oracle's rounded means bit for bit; scores, selections and outputs must meet the
same bars as with fp32 block keys, against the oracle run on the same bf16 keys
(selection exact up to swaps within 1e-4 of the k-th score, outputs within
|gpu - oracle| <= 1e-2 + 1e-2 |oracle|)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_harness import Dev, log, to_np
from parity import check_close, check_lse, score_bound
from test_gpu_parity import check_decode_against_oracle, run_decode, run_extend

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def bf16_case(name, seed, Hq, Hkv, lens, page_size=64, **kw):
    return synth.make_case(name, seed, Hq, Hkv, lens, page_size=page_size, ckey_dtype="bf16", **kw)


@pytest.mark.parametrize("page_size,lens", [
    (64, [4096, 4097, 4098, 4099]),
    (4, [37, 64, 1]),
    (16, [500, 3]),
    (8192, [8192]),
])
def test_bf16_compress_bitwise(page_size, lens):
    case = bf16_case(f"bcmp{page_size}", 100 + page_size, 8, 2, lens, page_size, jitter=True)
    log(f"bf16 compress page_size={page_size} lens={lens}")
    d = Dev(case)
    assert d.t["ckey"].dtype == torch.bfloat16
    d.compress()
    torch.cuda.synchronize()
    for i in range(case.B):
        got = d.ckey_logical(i)
        K = case.logical("k", i)
        for h in range(case.Hkv):
            want = oracle.compress(K[h], "bf16")
            assert np.array_equal(got[h].view(np.uint32), want.view(np.uint32)), (i, h)


@pytest.mark.parametrize("Hq,Hkv", [(16, 2), (6, 1)])
def test_bf16_decode_scores_within_fp32_bound(Hq, Hkv):
    case = bf16_case(f"bsc{Hq}", 200 + Hq, Hq, Hkv, [2051, 700, 4096])
    d = Dev(case)
    d.compress()
    sc = to_np(d.scores())
    for r in range(case.R):
        i = int(case.q_seq[r])
        ck = d.ckey_logical(i)
        for h in range(case.Hkv):
            n = case.nb(i)
            qg = case.q[r, h * case.g:(h + 1) * case.g]
            want = oracle.scores(qg, ck[h], n)
            bound = score_bound(synth.bf16_to_f32(qg).astype(np.float64), ck[h][:n])
            assert np.all(np.abs(sc[r, h, :n] - want) <= bound + 1e-30), (r, h)


@pytest.mark.parametrize("Hq,Hkv", [(16, 2), (24, 2), (12, 1)])
def test_bf16_decode_step(Hq, Hkv):
    case = bf16_case(f"bdec{Hq}", 300 + Hq, Hq, Hkv, [2051, 4097, 9000, 130], jitter=True)
    log(f"bf16 decode heads=({Hq},{Hkv})")
    res = run_decode(case)
    check_decode_against_oracle(case, *res, case.topk)


def test_bf16_extend_step():
    total, nq = 3000, 257
    q_seq, q_pos = synth.extend_rows(total, nq)
    case = synth.make_case("bext", 512, 12, 1, [total], page_size=64, q_seq=q_seq, q_pos=q_pos, ckey_dtype="bf16")
    res = run_extend(case)
    check_decode_against_oracle(case, *res, case.topk)


def test_bf16_fused_decode():
    from test_gpu_fused import check_fused
    case = bf16_case("bfused", 14, 16, 2, [9000, 4097, 6000, 20000])
    check_fused(case)


def test_bf16_full_size_decode_all_rows():
    """32 sequences of 32K-64K tokens with bf16 block keys, in the benchmark's
    launch configuration, against the oracle on every row."""
    from test_gpu_configs import all_row_properties, compare_rows, upload
    import block_sparse_attention_compress_amd as qsa
    from block_sparse_attention_compress_amd.pipeline import DecodeBuffers, decode_step
    case = synth.config("C2")
    case.ckey_dtype = "bf16"
    dev, kv = upload(case)
    assert dev["ckey"].dtype == torch.bfloat16
    qsa.qsa_compress_keys(kv)
    stride = (max(case.nb(i) for i in range(case.B)) + 63) // 64 * 64
    buf = DecodeBuffers.allocate(case.B, case.Hq, case.Hkv, stride, case.topk, 0, "cuda")
    decode_step(kv, dev["q"], dev["q_pos"], buf, scale=case.scale)
    torch.cuda.synchronize()
    sel, cnt, out, lse = to_np(buf.sel_idx), to_np(buf.sel_cnt), to_np(buf.out), to_np(buf.lse)
    all_row_properties(case, sel, cnt, out, lse)
    compare_rows(case, list(range(case.B)), sel, cnt, out, lse, stride)
