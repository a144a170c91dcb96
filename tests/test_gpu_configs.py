"""The five workloads at full size, in the launch configuration the benchmark times,
against the CPU oracle on every row (selections by the swap rule, outputs within
the tolerance), plus properties checked on every row.  The Ascend page's
long-prefill shape (7,810 queries on a 65,536-token cache, (24,2) heads) is an
extra extend case, checked on every row as well.  Tests at still larger shapes
(the longest sequence, a batch of 1,024) compare sampled rows."""
import numpy as np
import pytest
import torch

import block_sparse_attention_compress_amd as qsa
import oracle
import synth
from block_sparse_attention_compress_amd.pipeline import DecodeBuffers, ExtendBuffers, decode_step, extend_step
from gpu_harness import log, to_np
from parity import check_close, check_lse, check_selection, tol_ratio

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def upload(case):
    dev = synth.to_device(case, "cuda")
    case.drop_paged()
    kv = qsa.KVCache(dev["k"], dev["v"], dev["ckey"], dev["block_table"], dev["seq_lens"], case.max_len)
    return dev, kv


def compare_rows(case, rows, sel, cnt, out, lse, stride, splits=1):
    """Oracle on the given rows; selections by the swap rule, outputs on the GPU's selection."""
    ref = oracle.run_case(case, rows=rows, splits=1)
    override = {}
    for r in rows:
        for h in range(case.Hkv):
            same = check_selection(sel[r, h], int(cnt[r, h]), ref.sel[(r, h)], ref.cnt[(r, h)], ref.scores[(r, h)],
                                   case.topk, f"{case.name} row {r} head {h}")
            if not same:
                override[(r, h)] = (sel[r, h, :case.topk].copy(), int(cnt[r, h]))
    if override:
        log(f"{case.name}: {len(override)} (row, head) selections differ within the swap window")
        ref = oracle.run_case(case, rows=rows, sel_override=override, splits=splits)
    elif splits > 1:
        ref = oracle.run_case(case, rows=rows, splits=splits)
    worst_o = worst_l = 0.0
    for r in rows:
        check_close(out[r], ref.out[r], f"{case.name} out row {r}")
        check_lse(lse[r], ref.lse[r], f"{case.name} lse row {r}")
        worst_o = max(worst_o, tol_ratio(out[r], ref.out[r]))
        worst_l = max(worst_l, tol_ratio(lse[r], ref.lse[r]))
    # the share of the |gpu - oracle| <= 1e-2 + 1e-2 |oracle| budget used (1 = at the bound)
    log(f"{case.name}: tolerance used on {len(rows)} rows: out {worst_o:.4f}, lse {worst_l:.4f}")
    return ref


def all_row_properties(case, sel, cnt, out, lse):
    for r in range(case.R):
        n_elig = int(case.q_pos[r]) // 4 + 1
        for h in range(case.Hkv):
            c = int(cnt[r, h])
            assert c == min(case.topk, n_elig)
            s = sel[r, h, :c]
            assert np.all(np.diff(s) > 0) and s[0] >= 0 and s[-1] < n_elig
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))


def decode_full(name, sample, num_splits=0):
    case = synth.config(name)
    log(f"{name}: B={case.B} lens {int(case.lens.min())}..{int(case.lens.max())} heads ({case.Hq},{case.Hkv})")
    dev, kv = upload(case)
    qsa.qsa_compress_keys(kv)
    stride = (max(case.nb(i) for i in range(case.B)) + 63) // 64 * 64  # as the benchmark
    buf = DecodeBuffers.allocate(case.B, case.Hq, case.Hkv, stride, case.topk, num_splits, "cuda")
    decode_step(kv, dev["q"], dev["q_pos"], buf, scale=case.scale, num_splits=num_splits)
    torch.cuda.synchronize()
    sel, cnt, out, lse = to_np(buf.sel_idx), to_np(buf.sel_cnt), to_np(buf.out), to_np(buf.lse)
    all_row_properties(case, sel, cnt, out, lse)
    log(f"{name}: oracle on rows {sample}")
    compare_rows(case, sample, sel, cnt, out, lse, stride)
    return case, dev, kv, buf


def test_c1_full():
    decode_full("C1", [0])


def test_c2_all_rows():
    decode_full("C2", list(range(32)))


def test_c3_all_rows():
    case, dev, kv, buf = decode_full("C3", list(range(8)))
    # the 1 % biased blocks dominate the selection: most selected blocks are biased ones
    sel, cnt = to_np(buf.sel_idx), to_np(buf.sel_cnt)
    for r in (0, 7):
        _, mask = case.bias(r)
        for h in range(case.Hkv):
            frac = mask[h][sel[r, h, :cnt[r, h]]].mean()
            assert frac > 0.9, frac


def test_c5_split4_merge_equals_unsplit():
    case = synth.config("C5")
    log(f"C5: B={case.B} lens {int(case.lens.min())}..{int(case.lens.max())}")
    dev, kv = upload(case)
    qsa.qsa_compress_keys(kv)
    stride = (max(case.nb(i) for i in range(case.B)) + 63) // 64 * 64  # as the benchmark
    buf = DecodeBuffers.allocate(case.B, case.Hq, case.Hkv, stride, case.topk, 4, "cuda")
    decode_step(kv, dev["q"], dev["q_pos"], buf, scale=case.scale, num_splits=4)
    # the same selection: explicit partials + merge, and unsplit
    S = 4
    q = dev["q"]
    po = torch.empty((S, case.B, case.Hq, 256), dtype=torch.float32, device="cuda")
    pl = torch.empty((S, case.B, case.Hq), dtype=torch.float32, device="cuda")
    qsa.qsa_sparse_attn_decode(kv, q, q.stride(0), case.Hq, buf.sel_idx, buf.sel_cnt, case.topk, case.scale, S,
                               None, 0, None, po, pl)
    merged = torch.empty((case.B, case.Hq, 256), dtype=torch.bfloat16, device="cuda")
    mlse = torch.empty((case.B, case.Hq), dtype=torch.float32, device="cuda")
    qsa.qsa_merge_lse(po, pl, S, case.B * case.Hq, 256, merged, mlse)
    unsplit = torch.empty_like(merged)
    ulse = torch.empty_like(mlse)
    qsa.qsa_sparse_attn_decode(kv, q, q.stride(0), case.Hq, buf.sel_idx, buf.sel_cnt, case.topk, case.scale, 1,
                               unsplit, unsplit.stride(0), ulse)
    torch.cuda.synchronize()
    sel, cnt = to_np(buf.sel_idx), to_np(buf.sel_cnt)
    all_row_properties(case, sel, cnt, to_np(merged), to_np(mlse))
    for r in range(case.B):
        check_close(to_np(merged)[r], to_np(unsplit)[r], f"C5 merged vs unsplit row {r}")
        check_close(to_np(buf.out)[r], to_np(unsplit)[r], f"C5 internal split vs unsplit row {r}")
        check_lse(to_np(mlse)[r], to_np(ulse)[r], f"C5 lse row {r}")
    rows = list(range(case.B))
    ref = compare_rows(case, rows, sel, cnt, to_np(merged), to_np(mlse), stride, splits=S)
    po, pl = to_np(po), to_np(pl)
    for r in rows:
        check_close(po[:, r], ref.part_out[r], f"C5 partials row {r}")
        check_lse(pl[:, r], ref.part_lse[r], f"C5 partial lse row {r}")


def extend_full(case, sample):
    dev, kv = upload(case)
    first = torch.tensor([int(case.q_pos.min())], dtype=torch.int32, device="cuda")
    # cached blocks first, then the chunk refreshes the blocks of the new tokens
    qsa.qsa_compress_keys(kv)
    stride = case.nb(0)
    buf = ExtendBuffers.allocate(case.R, case.Hq, case.Hkv, stride, case.topk, "cuda")
    extend_step(kv, dev["q"], dev["q_seq"], dev["q_pos"], buf, first, case.R, scale=case.scale)
    torch.cuda.synchronize()
    sel, cnt, out, lse = to_np(buf.sel_idx), to_np(buf.sel_cnt), to_np(buf.out), to_np(buf.lse)
    all_row_properties(case, sel, cnt, out, lse)
    log(f"{case.name}: oracle on {len(sample)} of {case.R} rows")
    compare_rows(case, sample, sel, cnt, out, lse, stride)


def test_c4_extend_all_rows():
    """All 4,096 rows of the extend chunk against the oracle."""
    case = synth.config("C4")
    extend_full(case, list(range(case.R)))


def test_c4_extend_shuffled_pages_sampled():
    total, new = 32768, 4096
    q_seq, q_pos = synth.extend_rows(total, new)
    case = synth.make_case("C4-paged", 44, 12, 1, [total], page_size=64, q_seq=q_seq, q_pos=q_pos)
    extend_full(case, [0, 777, 2048, 4095])


def test_long_prefill_shape_of_the_ascend_tests():
    """7,810 query rows appended to a cache totalling 65,536 tokens, (24,2) heads; every
    row against the oracle, as the Ascend page's own test did on sampled rows."""
    total, new = 65536, 7810
    q_seq, q_pos = synth.extend_rows(total, new)
    case = synth.make_case("prefill7810", 7810, 24, 2, [total], page_size=64, q_seq=q_seq, q_pos=q_pos)
    extend_full(case, list(range(case.R)))


def test_longest_sequence_decode():
    """One sequence at the library's length limit (2^20 tokens, 262,144 blocks per
    row: two-stage top-k over 32 slices) next to a short one, decode step against
    the oracle on both rows."""
    case = synth.make_case("maxlen", 41, 16, 2, [1 << 20, 3001], page_size=64, jitter=True)
    log(f"max length decode: lens {case.lens.tolist()}")
    dev, kv = upload(case)
    qsa.qsa_compress_keys(kv)
    stride = (max(case.nb(i) for i in range(case.B)) + 63) // 64 * 64
    buf = DecodeBuffers.allocate(case.B, case.Hq, case.Hkv, stride, case.topk, 0, "cuda")
    assert buf.topk_workspace is not None
    decode_step(kv, dev["q"], dev["q_pos"], buf, scale=case.scale)
    torch.cuda.synchronize()
    sel, cnt, out, lse = to_np(buf.sel_idx), to_np(buf.sel_cnt), to_np(buf.out), to_np(buf.lse)
    all_row_properties(case, sel, cnt, out, lse)
    compare_rows(case, [0, 1], sel, cnt, out, lse, stride)


def test_large_batch_decode():
    """1,024 sequences of 1K-5K tokens, (16,2) heads: 2,048 (row, KV head) units,
    so the selection takes its many-row form (512 threads per row) and attention
    one split per unit; against the oracle on sampled rows."""
    case = synth.make_case("bigbatch", 43, 16, 2, synth.uniform_lengths(43, 1024, 1000, 5000), page_size=64,
                           jitter=True)
    log(f"large batch decode: B={case.B}")
    dev, kv = upload(case)
    qsa.qsa_compress_keys(kv)
    stride = (max(case.nb(i) for i in range(case.B)) + 63) // 64 * 64
    buf = DecodeBuffers.allocate(case.B, case.Hq, case.Hkv, stride, case.topk, 0, "cuda")
    decode_step(kv, dev["q"], dev["q_pos"], buf, scale=case.scale)
    torch.cuda.synchronize()
    sel, cnt, out, lse = to_np(buf.sel_idx), to_np(buf.sel_cnt), to_np(buf.out), to_np(buf.lse)
    all_row_properties(case, sel, cnt, out, lse)
    compare_rows(case, [0, 1, 511, 777, 1023], sel, cnt, out, lse, stride)


def test_most_rows_per_call():
    """65,535 query rows, the most one call takes, on one 4,096-token sequence at
    random positions, (12,1) heads: block scores, selection and attention, with
    properties on every row and the oracle on sampled rows."""
    rng = np.random.default_rng(65535)
    R, L = 65535, 4096
    q_seq = np.zeros(R, dtype=np.int32)
    q_pos = rng.integers(0, L, size=R).astype(np.int32)
    case = synth.make_case("rows65535", 65535, 12, 1, [L], page_size=64, q_seq=q_seq, q_pos=q_pos)
    log(f"{case.name}: {R} rows on one {L}-token sequence")
    dev, kv = upload(case)
    qsa.qsa_compress_keys(kv)
    stride = case.nb(0)
    buf = ExtendBuffers.allocate(R, case.Hq, case.Hkv, stride, case.topk, "cuda")
    extend_step(kv, dev["q"], dev["q_seq"], dev["q_pos"], buf, None, 0, scale=case.scale)
    torch.cuda.synchronize()
    sel, cnt, out, lse = to_np(buf.sel_idx), to_np(buf.sel_cnt), to_np(buf.out), to_np(buf.lse)
    all_row_properties(case, sel, cnt, out, lse)
    sample = sorted(set([0, 1, R - 2, R - 1] + rng.choice(R, 60, replace=False).tolist()))
    compare_rows(case, sample, sel, cnt, out, lse, stride)
