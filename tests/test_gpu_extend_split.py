"""Extend attention with a split read (qsa_sparse_attn_extend_split) against the oracle.

Each case runs the extend path up to the selection on the GPU, gives that selection
to the split entry point, and holds its outputs to the oracle's bars on that
selection: outputs and lse within |gpu - oracle| <= 1e-2 + 1e-2 |oracle|,
selections by the swap rule.  The merged result must also agree with the unsplit
extend call within the same tolerance (only the order of the sums differs).
Cases: the random extend shapes (several sequences per launch, head pairs down to
(3,1), page sizes 4-256, k 1-512, bf16 and fp8 caches) at split counts 0 (the
library's choice), 2, 3, 5, 16 and 64; a small chunk on a long context (the shape
the split read is for); the largest k (2,048) at 16 and 64 splits; rows that see
nothing; strided query rows; the pipeline's extend step."""
import numpy as np
import pytest
import torch

import block_sparse_attention_compress_amd as qsa
import oracle
import synth
from gpu_harness import Dev, log, to_np
from parity import check_close, check_lse, tol_ratio
from test_gpu_parity import check_decode_against_oracle
from test_gpu_random_shapes import random_extend

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def split_attn(d: Dev, sel, cnt, k: int, S: int, scale: float = 0.0, q=None):
    c = d.case
    q = d.t["q"] if q is None else q
    out = torch.full((c.R, c.Hq, 256), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((c.R, c.Hq), float("nan"), dtype=torch.float32, device="cuda")
    wsb = qsa.qsa_extend_workspace_bytes(c.R, c.Hq, S)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    qsa.qsa_sparse_attn_extend_split(d.kv, q, q.stride(0), d.t["q_seq"], d.t["q_pos"], c.R, c.Hq, sel, cnt, k, scale,
                                     S, out, out.stride(0), lse, workspace=ws, workspace_bytes=wsb)
    return out, lse


def select(case, k):
    d = Dev(case)
    d.compress()
    sc = d.scores(extend=True)
    sel, cnt = d.topk(sc, k)
    return d, to_np(sc), sel, cnt


def agree_with_unsplit(d, sel, cnt, k, out, lse, what):
    ro, rl = d.extend_attn(sel, cnt, k)
    torch.cuda.synchronize()
    ro, rl = to_np(ro), to_np(rl)
    worst = 0.0
    for r in range(d.case.R):
        check_close(out[r], ro[r], f"{what} split vs unsplit out row {r}")
        check_lse(lse[r], rl[r], f"{what} split vs unsplit lse row {r}")
        worst = max(worst, tol_ratio(out[r], ro[r]))
    log(f"{what}: split vs unsplit, tolerance used: {worst:.4f}")


SPLITS = [0, 2, 3, 5, 16, 64]


@pytest.mark.parametrize("i", range(12))
def test_extend_split_random_shapes(i):
    case, k = random_extend(i)
    S = SPLITS[i % len(SPLITS)]
    log(f"extend split random {i}: heads=({case.Hq},{case.Hkv}) page={case.page_size} lens={case.lens.tolist()} "
        f"rows={case.R} k={k} S={S} cache={case.kv_dtype}")
    d, sc, sel, cnt = select(case, k)
    out, lse = split_attn(d, sel, cnt, k, S)
    torch.cuda.synchronize()
    out, lse = to_np(out), to_np(lse)
    check_decode_against_oracle(case, d, sc, to_np(sel), to_np(cnt), out, lse, k)
    agree_with_unsplit(d, sel, cnt, k, out, lse, f"random {i}")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_extend_split_small_chunk_on_long_context(kv_dtype):
    """48 new tokens at the end of a 20,000-token sequence, (12,1) heads, shuffled
    64-token pages: 48 (row, KV head) units, so the library splits each row's 512
    blocks over 6 workgroups.  Every row against the oracle and the unsplit call."""
    total, nq = 20000, 48
    q_pos = list(range(total - nq, total))
    case = synth.make_case(f"xsplit-{kv_dtype}", 621, 12, 1, [total], page_size=64, q_seq=[0] * nq, q_pos=q_pos,
                           jitter=True, kv_dtype=kv_dtype)
    log(f"extend split small chunk: rows={nq} len={total} cache={kv_dtype}")
    d, sc, sel, cnt = select(case, case.topk)
    out, lse = split_attn(d, sel, cnt, case.topk, 0)
    torch.cuda.synchronize()
    out, lse = to_np(out), to_np(lse)
    check_decode_against_oracle(case, d, sc, to_np(sel), to_np(cnt), out, lse, case.topk)
    agree_with_unsplit(d, sel, cnt, case.topk, out, lse, f"small chunk {kv_dtype}")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("S", [0, 64])
def test_extend_split_largest_k(S, kv_dtype):
    """k = 2,048 (8,192 selected tokens per row) on rows of a 40,000-token sequence and
    of a short one in one launch, shuffled 64-token pages, (16,2) heads: the library's
    split count (16) and 64 splits of 32 blocks."""
    lens = [40000, 700]
    q_seq = [0] * 9 + [1] * 4
    q_pos = [39999, 39998, 39000, 30001, 20000, 12345, 8191, 8192, 100] + [699, 698, 300, 3]
    case = synth.make_case(f"xsplit-k2048-{S}-{kv_dtype}", 625 + S, 16, 2, lens, page_size=64, q_seq=q_seq,
                           q_pos=q_pos, topk=2048, kv_dtype=kv_dtype)
    log(f"extend split k=2048 S={S} cache={kv_dtype}")
    d, sc, sel, cnt = select(case, 2048)
    out, lse = split_attn(d, sel, cnt, 2048, S)
    torch.cuda.synchronize()
    out, lse = to_np(out), to_np(lse)
    check_decode_against_oracle(case, d, sc, to_np(sel), to_np(cnt), out, lse, 2048)
    agree_with_unsplit(d, sel, cnt, 2048, out, lse, f"k=2048 S={S} {kv_dtype}")


def test_extend_split_rows_that_see_nothing():
    """k = 0, a row whose selection count is 0, and rows of an empty sequence next to
    ordinary rows: zero output and -inf lse for the empty rows; the others against the
    oracle on the GPU's selection.  S = 8 leaves most splits of the short rows empty."""
    lens = [3000, 0, 2000]
    q_seq = [0, 0, 0, 1, 1, 2, 2, 2, 2, 0, 2]
    q_pos = [2999, 10, 1500, -1, -1, 1999, 3, 1000, 0, 2998, 1999]
    case = synth.make_case("xsplit-empty", 622, 12, 1, lens, page_size=16, q_seq=q_seq, q_pos=q_pos, topk=64)
    d, _, sel, cnt = select(case, 64)
    cnt[0, 0] = 0
    for k in (64, 0):
        out, lse = split_attn(d, sel, cnt, k, 8)
        torch.cuda.synchronize()
        out, lse = to_np(out), to_np(lse)
        empty = [r for r in range(case.R) if k == 0 or r == 0 or q_seq[r] == 1]
        for r in empty:
            assert np.all(out[r] == 0) and np.all(np.isneginf(lse[r])), r
    rows = [r for r in range(case.R) if r != 0 and q_seq[r] != 1]
    override = {(r, 0): (to_np(sel)[r, 0, :64].copy(), int(to_np(cnt)[r, 0])) for r in rows}
    ref = oracle.run_case(case, rows=rows, sel_override=override)
    out, lse = split_attn(d, sel, cnt, 64, 8)
    torch.cuda.synchronize()
    out, lse = to_np(out), to_np(lse)
    for r in rows:
        check_close(out[r], ref.out[r], f"oracle row {r}")
        check_lse(lse[r], ref.lse[r], f"oracle lse row {r}")


def test_extend_split_one_split_is_the_unsplit_call():
    """S = 1 gives qsa_sparse_attn_extend's outputs bit for bit; strided query rows
    give the contiguous call's outputs bit for bit."""
    total, nq = 3000, 37
    q_seq, q_pos = synth.extend_rows(total, nq)
    case = synth.make_case("xsplit-one", 623, 24, 2, [total], page_size=64, q_seq=q_seq, q_pos=q_pos)
    d, _, sel, cnt = select(case, case.topk)
    o1, l1 = split_attn(d, sel, cnt, case.topk, 1)
    o0, l0 = d.extend_attn(sel, cnt, case.topk)
    assert torch.equal(o1.view(torch.int16), o0.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l0.view(torch.int32))
    o4, l4 = split_attn(d, sel, cnt, case.topk, 4)
    qbig = torch.zeros((case.R, case.Hq + 4, 256), dtype=torch.bfloat16, device="cuda")
    qbig[:, :case.Hq] = d.t["q"]
    o4s, l4s = split_attn(d, sel, cnt, case.topk, 4, q=qbig[:, :case.Hq])
    torch.cuda.synchronize()
    assert torch.equal(o4s.view(torch.int16), o4.view(torch.int16))
    assert torch.equal(l4s.view(torch.int32), l4.view(torch.int32))


def test_extend_split_through_the_extend_step():
    """extend_step(..., num_splits=0) gives the direct split call's outputs bit for bit,
    and both agree with the oracle."""
    from block_sparse_attention_compress_amd.pipeline import ExtendBuffers, extend_step
    total, nq = 6000, 24
    q_pos = list(range(total - nq, total))
    case = synth.make_case("xsplit-step", 624, 16, 2, [total], page_size=64, q_seq=[0] * nq, q_pos=q_pos)
    d = Dev(case)
    d.compress()
    buf = ExtendBuffers.allocate(case.R, case.Hq, case.Hkv, d.stride, case.topk, "cuda", max_splits=0)
    extend_step(d.kv, d.t["q"], d.t["q_seq"], d.t["q_pos"], buf, scale=case.scale, num_splits=0)
    out, lse = split_attn(d, buf.sel_idx, buf.sel_cnt, case.topk, 0, case.scale)
    torch.cuda.synchronize()
    assert torch.equal(buf.out.view(torch.int16), out.view(torch.int16))
    assert torch.equal(buf.lse.view(torch.int32), lse.view(torch.int32))
    check_decode_against_oracle(case, d, to_np(buf.scores), to_np(buf.sel_idx), to_np(buf.sel_cnt), to_np(buf.out),
                                to_np(buf.lse), case.topk)
