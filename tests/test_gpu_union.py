"""The query-tile union kernel (qsa_sparse_attn_extend_union) against the oracle.

It computes the same per-row sets as qsa_sparse_attn_extend, so every case here
runs the extend path up to the selection, gives that selection to the union
kernel, and holds its outputs to the oracle's bars on that selection: outputs and
lse within |gpu - oracle| <= 1e-2 + 1e-2 |oracle|, selections by the swap rule.
Cases: the C4 chunk on every row, with independent and with shared-component
queries; ragged tiles and tiles spanning sequences (random shapes, both cache
types); two union windows (rows over 8,192 blocks) at k = 2,048; rows that see
nothing (k = 0, empty selections, an empty sequence); strided q and out rows."""
import numpy as np
import pytest
import torch

import block_sparse_attention_compress_amd as qsa
import oracle
import synth
from gpu_harness import Dev, log, to_np
from parity import check_close, check_lse, tol_ratio
from test_gpu_configs import all_row_properties, compare_rows, upload
from test_gpu_parity import check_decode_against_oracle
from test_gpu_random_shapes import random_extend

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def union_attn(kv, q, q_seq, q_pos, R, Hq, sel, cnt, k, scale=0.0):
    out = torch.full((R, Hq, 256), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((R, Hq), float("nan"), dtype=torch.float32, device="cuda")
    qsa.qsa_sparse_attn_extend_union(kv, q, q.stride(0), q_seq, q_pos, R, Hq, sel, cnt, k, scale, out, out.stride(0),
                                     lse)
    return out, lse


def extend_select(case, k):
    """Block keys, extend scores and top-k on the GPU: (Dev, scores as numpy, sel, cnt)."""
    d = Dev(case)
    d.compress()
    sc = d.scores(extend=True)
    sel, cnt = d.topk(sc, k)
    return d, to_np(sc), sel, cnt


def union_full(case):
    """Extend chunk through the per-row path, then the union kernel on the same
    selection: every row against the oracle, and against the per-row kernel."""
    from block_sparse_attention_compress_amd.pipeline import ExtendBuffers, extend_step
    dev, kv = upload(case)
    first = torch.tensor([int(case.q_pos.min())], dtype=torch.int32, device="cuda")
    qsa.qsa_compress_keys(kv)
    stride = case.nb(0)
    buf = ExtendBuffers.allocate(case.R, case.Hq, case.Hkv, stride, case.topk, "cuda")
    extend_step(kv, dev["q"], dev["q_seq"], dev["q_pos"], buf, first, case.R, scale=case.scale)
    uo, ul = union_attn(kv, dev["q"], dev["q_seq"], dev["q_pos"], case.R, case.Hq, buf.sel_idx, buf.sel_cnt,
                        case.topk, case.scale)
    torch.cuda.synchronize()
    sel, cnt = to_np(buf.sel_idx), to_np(buf.sel_cnt)
    uo, ul, po, pl = to_np(uo), to_np(ul), to_np(buf.out), to_np(buf.lse)
    all_row_properties(case, sel, cnt, uo, ul)
    worst = 0.0
    for r in range(case.R):  # the two kernels sum the same tokens in different orders
        check_close(uo[r], po[r], f"{case.name} union vs per-row out row {r}")
        check_lse(ul[r], pl[r], f"{case.name} union vs per-row lse row {r}")
        worst = max(worst, tol_ratio(uo[r], po[r]))
    log(f"{case.name}: union vs per-row kernel, tolerance used: {worst:.4f}")
    compare_rows(case, list(range(case.R)), sel, cnt, uo, ul, stride)


def test_union_c4_all_rows():
    """The C4 chunk (4,096 rows of one 32,768-token sequence, (12,1) heads): every row."""
    union_full(synth.config("C4"))


def test_union_c4_shared_queries_all_rows():
    """C4 with queries sharing a per-sequence component (q_share 0.9: 8 adjacent rows
    select about a quarter as many distinct blocks as 8 x 512): every row."""
    case = synth.config("C4", q_share=0.9)
    case.name = "C4-shared"
    union_full(case)


@pytest.mark.parametrize("i", range(12))
def test_union_random_shapes(i):
    """The random extend shapes: several sequences' rows per launch (tiles spanning
    sequences), ragged last tiles, head pairs down to (3,1), page sizes 4-256, k 1-512,
    bf16 and fp8 caches."""
    case, k = random_extend(i)
    log(f"union random {i}: heads=({case.Hq},{case.Hkv}) page={case.page_size} lens={case.lens.tolist()} "
        f"rows={case.R} k={k} cache={case.kv_dtype}")
    d, sc, sel, cnt = extend_select(case, k)
    out, lse = union_attn(d.kv, d.t["q"], d.t["q_seq"], d.t["q_pos"], case.R, case.Hq, sel, cnt, k)
    torch.cuda.synchronize()
    check_decode_against_oracle(case, d, sc, to_np(sel), to_np(cnt), to_np(out), to_np(lse), k)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_union_two_windows_largest_k(kv_dtype):
    """Rows of a 40,000-token sequence (10,000 blocks: two union windows of 8,192)
    at k = 2,048, 21 rows (a ragged last tile), shuffled 64-token pages."""
    total, nq = 40000, 21
    q_seq, q_pos = synth.extend_rows(total, nq)
    case = synth.make_case("union2w", 611, 16, 2, [total], page_size=64, q_seq=q_seq, q_pos=q_pos, topk=2048,
                           kv_dtype=kv_dtype, q_share=0.5)
    d, sc, sel, cnt = extend_select(case, 2048)
    out, lse = union_attn(d.kv, d.t["q"], d.t["q_seq"], d.t["q_pos"], case.R, case.Hq, sel, cnt, 2048)
    torch.cuda.synchronize()
    sel_np, cnt_np = to_np(sel), to_np(cnt)
    assert sel_np.max() >= 8192 and (sel_np[sel_np >= 0] < 8192).any()  # both windows are used
    check_decode_against_oracle(case, d, sc, sel_np, cnt_np, to_np(out), to_np(lse), 2048)


def test_union_rows_that_see_nothing():
    """k = 0, a row whose selection count is 0, and rows of an empty sequence next to
    ordinary rows in one tile: zero output and -inf lse for the empty rows, the
    per-row kernel's results (within rounding) for the others."""
    lens = [3000, 0, 2000]
    q_seq = [0, 0, 0, 1, 1, 2, 2, 2, 2, 0, 2]
    q_pos = [2999, 10, 1500, -1, -1, 1999, 3, 1000, 0, 2998, 1999]  # t < 0: the empty sequence's rows see nothing
    case = synth.make_case("union-empty", 612, 12, 1, lens, page_size=16, q_seq=q_seq, q_pos=q_pos, topk=64)
    d, _, sel, cnt = extend_select(case, 64)
    cnt[0, 0] = 0  # row 0 selects nothing
    for k in (64, 0):
        ref_o, ref_l = d.extend_attn(sel, cnt, k)
        out, lse = union_attn(d.kv, d.t["q"], d.t["q_seq"], d.t["q_pos"], case.R, case.Hq, sel, cnt, k)
        torch.cuda.synchronize()
        out, lse, ref_o, ref_l = to_np(out), to_np(lse), to_np(ref_o), to_np(ref_l)
        empty = [r for r in range(case.R) if k == 0 or r == 0 or q_seq[r] == 1]
        for r in range(case.R):
            if r in empty:
                assert np.all(out[r] == 0) and np.all(np.isneginf(lse[r])), r
            else:
                check_close(out[r], ref_o[r], f"k={k} row {r}")
                check_lse(lse[r], ref_l[r], f"k={k} lse row {r}")
    # the non-empty rows against the oracle on the GPU's selection
    rows = [r for r in range(case.R) if r != 0 and q_seq[r] != 1]
    override = {(r, 0): (to_np(sel)[r, 0, :64].copy(), int(to_np(cnt)[r, 0])) for r in rows}
    ref = oracle.run_case(case, rows=rows, sel_override=override)
    out, lse = union_attn(d.kv, d.t["q"], d.t["q_seq"], d.t["q_pos"], case.R, case.Hq, sel, cnt, 64)
    torch.cuda.synchronize()
    out, lse = to_np(out), to_np(lse)
    for r in rows:
        check_close(out[r], ref.out[r], f"oracle row {r}")
        check_lse(lse[r], ref.lse[r], f"oracle lse row {r}")


def test_union_strided_query_and_output_rows():
    """q rows and out rows that are views into wider tensors: results equal the
    contiguous call's bit for bit, and the columns past each row are not written."""
    total, nq = 3000, 37
    q_seq, q_pos = synth.extend_rows(total, nq)
    case = synth.make_case("union-stride", 613, 12, 1, [total], page_size=64, q_seq=q_seq, q_pos=q_pos)
    d, _, sel, cnt = extend_select(case, case.topk)
    o1, l1 = union_attn(d.kv, d.t["q"], d.t["q_seq"], d.t["q_pos"], case.R, case.Hq, sel, cnt, case.topk)
    qbig = torch.zeros((case.R, case.Hq + 4, 256), dtype=torch.bfloat16, device="cuda")
    qbig[:, :case.Hq] = d.t["q"]
    qv = qbig[:, :case.Hq]
    obig = torch.full((case.R, case.Hq + 3, 256), 7.0, dtype=torch.bfloat16, device="cuda")
    ov = obig[:, :case.Hq]
    l2 = torch.full((case.R, case.Hq), float("nan"), dtype=torch.float32, device="cuda")
    qsa.qsa_sparse_attn_extend_union(d.kv, qv, qv.stride(0), d.t["q_seq"], d.t["q_pos"], case.R, case.Hq, sel, cnt,
                                     case.topk, 0.0, ov, ov.stride(0), l2)
    torch.cuda.synchronize()
    assert torch.all(obig[:, case.Hq:] == 7.0)
    assert torch.equal(ov.contiguous().view(torch.int16), o1.view(torch.int16))
    assert torch.equal(l2.view(torch.int32), l1.view(torch.int32))


def test_union_through_the_extend_step():
    """extend_step(..., union_tiles=True) gives the direct union call's outputs bit for bit."""
    from block_sparse_attention_compress_amd.pipeline import ExtendBuffers, extend_step
    total, nq = 5000, 61
    q_seq, q_pos = synth.extend_rows(total, nq)
    case = synth.make_case("union-step", 614, 24, 2, [total], page_size=64, q_seq=q_seq, q_pos=q_pos, q_share=0.5)
    dev, kv = upload(case)
    qsa.qsa_compress_keys(kv)
    buf = ExtendBuffers.allocate(case.R, case.Hq, case.Hkv, case.nb(0), case.topk, "cuda")
    extend_step(kv, dev["q"], dev["q_seq"], dev["q_pos"], buf, scale=case.scale, union_tiles=True)
    out, lse = union_attn(kv, dev["q"], dev["q_seq"], dev["q_pos"], case.R, case.Hq, buf.sel_idx, buf.sel_cnt,
                          case.topk, case.scale)
    torch.cuda.synchronize()
    assert torch.equal(buf.out.view(torch.int16), out.view(torch.int16))
    assert torch.equal(buf.lse.view(torch.int32), lse.view(torch.int32))
