"""fp8 block keys (QSA_CKEY_FP8, OCP E4M3) through the C ABI: the stored codes must
equal the oracle's (the fp32 mean rounded to nearest even, held at +-448) byte for
byte, including saturated and subnormal keys; scores, selections and outputs must
meet the same bars as with fp32 block keys, against the oracle run on the same
fp8 keys (selection exact up to swaps within 1e-4 of the k-th score, outputs
within |gpu - oracle| <= 1e-2 + 1e-2 |oracle|)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_harness import Dev, log, to_np
from parity import score_bound
from test_gpu_parity import check_decode_against_oracle, run_decode, run_extend

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def fp8_case(name, seed, Hq, Hkv, lens, page_size=64, **kw):
    return synth.make_case(name, seed, Hq, Hkv, lens, page_size=page_size, ckey_dtype="fp8", **kw)


def scaled_bf16(bits: np.ndarray, factor: float) -> np.ndarray:
    """bf16 bit patterns times a power of two (exact while in range)."""
    return synth.f32_to_bf16(synth.bf16_to_f32(bits) * np.float32(factor))


@pytest.mark.parametrize("page_size,lens,factor", [
    (64, [4096, 4097, 4098, 4099], 1.0),
    (4, [37, 64, 1], 1.0),
    (16, [500, 3], 512.0),        # means past 448: saturated codes
    (64, [700, 1302], 2.0 ** -8),  # means below 2^-6: subnormal codes
    (8192, [8192], 1.0),
])
def test_fp8_compress_bytewise(page_size, lens, factor):
    case = fp8_case(f"fcmp{page_size}", 150 + page_size, 8, 2, lens, page_size, jitter=True)
    log(f"fp8 compress page_size={page_size} lens={lens} key factor {factor}")
    d = Dev(case)
    assert d.t["ckey"].dtype == torch.float8_e4m3fn
    if factor != 1.0:
        d.t["k"].mul_(factor)
    d.compress()
    torch.cuda.synchronize()
    saturated = subnormal = 0
    for i in range(case.B):
        got = d.ckey_codes(i)
        K = case.logical("k", i)
        for h in range(case.Hkv):
            want = oracle.compress_fp8_codes(scaled_bf16(K[h], factor) if factor != 1.0 else K[h])
            assert np.array_equal(got[h], want), (i, h, int(np.sum(got[h] != want)))
            saturated += int(np.sum((want & 0x7F) == 0x7E))
            subnormal += int(np.sum(((want & 0x78) == 0) & ((want & 0x7) != 0)))
    if factor > 1:
        assert saturated > 0
    if factor < 1:
        assert subnormal > 0


@pytest.mark.parametrize("Hq,Hkv", [(16, 2), (6, 1)])
def test_fp8_decode_scores_within_fp32_bound(Hq, Hkv):
    case = fp8_case(f"fsc{Hq}", 250 + Hq, Hq, Hkv, [2051, 700, 4096])
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


@pytest.mark.parametrize("Hq,Hkv", [(16, 2), (24, 2), (12, 1), (3, 1)])
def test_fp8_decode_step(Hq, Hkv):
    case = fp8_case(f"fdec{Hq}", 350 + Hq, Hq, Hkv, [2051, 4097, 9000, 130], jitter=True)
    log(f"fp8 decode heads=({Hq},{Hkv})")
    res = run_decode(case)
    check_decode_against_oracle(case, *res, case.topk)


def test_fp8_extend_step():
    total, nq = 3000, 257
    q_seq, q_pos = synth.extend_rows(total, nq)
    case = synth.make_case("fext", 513, 12, 1, [total], page_size=64, q_seq=q_seq, q_pos=q_pos, ckey_dtype="fp8")
    res = run_extend(case)
    check_decode_against_oracle(case, *res, case.topk)


def test_fp8_fused_decode():
    from test_gpu_fused import check_fused
    case = fp8_case("ffused", 15, 16, 2, [9000, 4097, 6000, 20000])
    check_fused(case)


def test_fp8_full_size_decode_all_rows():
    """32 sequences of 32K-64K tokens with fp8 block keys, in the benchmark's
    launch configuration, against the oracle on every row."""
    from test_gpu_configs import all_row_properties, compare_rows, upload
    import block_sparse_attention_compress_amd as qsa
    from block_sparse_attention_compress_amd.pipeline import DecodeBuffers, decode_step
    case = synth.config("C2")
    case.ckey_dtype = "fp8"
    dev, kv = upload(case)
    assert dev["ckey"].dtype == torch.float8_e4m3fn
    qsa.qsa_compress_keys(kv)
    stride = (max(case.nb(i) for i in range(case.B)) + 63) // 64 * 64
    buf = DecodeBuffers.allocate(case.B, case.Hq, case.Hkv, stride, case.topk, 0, "cuda")
    decode_step(kv, dev["q"], dev["q_pos"], buf, scale=case.scale)
    torch.cuda.synchronize()
    sel, cnt, out, lse = to_np(buf.sel_idx), to_np(buf.sel_cnt), to_np(buf.out), to_np(buf.lse)
    all_row_properties(case, sel, cnt, out, lse)
    compare_rows(case, list(range(case.B)), sel, cnt, out, lse, stride)
