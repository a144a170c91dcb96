"""The fused decode entry point (block scores, top-k, attention and merge in one
launch) through the C ABI: its selection must equal the separate calls' bit for
bit (the same fp32 scores decide it), and its output must meet the oracle bar
|gpu - oracle| <= 1e-2 + 1e-2 |oracle| like the separate path.  The workspace's
control area must be zero again after every call, with no abandoned waits."""
import numpy as np
import pytest
import torch

import block_sparse_attention_compress_amd as qsa
import synth
from block_sparse_attention_compress_amd.pipeline import FusedDecodeBuffers, decode_step_fused
from gpu_harness import Dev, log, to_np
from parity import check_close, check_lse
from test_gpu_parity import check_decode_against_oracle, small_decode

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def check_control(ws: torch.Tensor, units: int, calls_before: int):
    """The control area after a call: ticket, finished and abandoned-wait counters
    zero, the call counter advanced by one, every unit's arrival counters zero and
    its ready word holding the number of this call."""
    ctl = ws[:256].view(torch.int32).cpu().numpy()
    assert ctl[0] == 0 and ctl[1] == 0, f"ticket counters not returned to zero: {ctl[:4]}"
    assert ctl[2] == 0, "a wait was abandoned"
    assert ctl[3] == calls_before + 1, f"call counter {ctl[3]}, expected {calls_before + 1}"
    unit = ws[256:256 + 16 * units].view(torch.int32).cpu().numpy().reshape(units, 4)
    assert np.all(unit[:, 0] == 0) and np.all(unit[:, 2] == 0), "arrival counters not returned to zero"
    assert np.all(unit[:, 1] == ctl[3]), "a unit's ready word was not raised by this call"


def fused(d: Dev, k=None, num_splits=0, scale=0.0, ws=None):
    c = d.case
    k = c.topk if k is None else k
    q = d.t["q"]
    sel = torch.full((c.B, c.Hkv, max(k, 1)), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((c.B, c.Hkv), -7, dtype=torch.int32, device="cuda")
    out = torch.full((c.B, c.Hq, 256), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((c.B, c.Hq), float("nan"), dtype=torch.float32, device="cuda")
    wsb = qsa.qsa_decode_fused_workspace_bytes(d.kv, c.Hq, k, num_splits)
    assert wsb > 0
    if ws is None:
        ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    assert ws.numel() >= wsb
    calls_before = int(ws[12:16].view(torch.int32).item())
    qsa.qsa_decode_fused(d.kv, q, q.stride(0), c.Hq, k, scale, num_splits, sel, cnt, out, out.stride(0), lse,
                         workspace=ws, workspace_bytes=ws.numel())
    torch.cuda.synchronize()
    check_control(ws, c.B * c.Hkv, calls_before)
    return to_np(sel), to_np(cnt), to_np(out), to_np(lse)


def check_fused(case, k=None, num_splits=0, scale=0.0):
    """Fused vs the separate calls (selection bit-exact) and vs the oracle."""
    k = case.topk if k is None else k
    d = Dev(case)
    d.compress()
    sc = d.scores()
    sel_ref, cnt_ref = d.topk(sc, k)
    fsel, fcnt, fout, flse = fused(d, k=k, num_splits=num_splits, scale=scale)
    sel_ref, cnt_ref = to_np(sel_ref), to_np(cnt_ref)
    assert np.array_equal(fcnt, cnt_ref)
    assert np.array_equal(fsel[:, :, :k], sel_ref[:, :, :k])
    check_decode_against_oracle(case, d, to_np(sc), fsel, fcnt, fout, flse, k)
    return d, fsel, fcnt, fout, flse


@pytest.mark.parametrize("Hq,Hkv", [(16, 2), (24, 2), (12, 1), (6, 1), (3, 1)])
def test_fused_head_pairs(Hq, Hkv):
    lens = [2051, 4097, 9000, 130]
    case = small_decode(f"fdec{Hq}", 300 + Hq, Hq, Hkv, lens, 64, jitter=True)
    log(f"fused heads=({Hq},{Hkv}) lens={lens}")
    check_fused(case)


@pytest.mark.parametrize("L,k", [(1, 1), (63, 16), (64, 16), (65, 17), (2051, 513)])
def test_fused_selection_widths(L, k):
    case = small_decode(f"fw{L}", 400 + L, 16, 2, [L, L], 64, topk=k)
    log(f"fused width L={L} k={k}")
    check_fused(case, k=k)


def test_fused_largest_k():
    """k = 2048, the most allowed: the fused selection's lists and the attention's
    8,192-token loop at their largest."""
    case = small_decode("fk2048", 90, 16, 2, [10000, 9001, 300], 64, topk=2048, jitter=True)
    log("fused k=2048")
    check_fused(case, k=2048)


@pytest.mark.parametrize("page_size", [4, 16, 256, 16384])
def test_fused_page_sizes(page_size):
    lens = [16384, 5000, 777] if page_size == 16384 else [7000, 5000, 777]
    case = small_decode(f"fps{page_size}", 500 + page_size, 16, 2, lens, page_size, shuffle=page_size < 16384)
    log(f"fused page_size={page_size} lens={lens}")
    check_fused(case)


@pytest.mark.parametrize("S", [1, 3, 16])
def test_fused_explicit_splits(S):
    case = small_decode(f"fs{S}", 600 + S, 12, 1, [9000, 3001, 4096], 64)
    log(f"fused splits={S}")
    check_fused(case, num_splits=S)


@pytest.mark.parametrize("scale", [0.03125, 0.2])
def test_fused_explicit_scale(scale):
    case = small_decode("fscale", 9, 16, 2, [3000, 2500], 64)
    case.scale = scale
    check_fused(case, scale=scale)


def test_fused_zero_k():
    case = small_decode("fk0", 5, 16, 2, [1000, 77], 64, topk=0)
    d = Dev(case)
    d.compress()
    sel, cnt, out, lse = fused(d, k=0)
    assert np.all(cnt == 0) and np.all(out == 0) and np.all(np.isneginf(lse))


def test_fused_empty_and_tiny_sequences():
    case = small_decode("fL0", 6, 8, 2, [0, 300, 1, 3], 64)
    d, sel, cnt, out, lse = check_fused(case)
    assert np.all(cnt[0] == 0) and np.all(sel[0] == -1)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))


def test_fused_ties_resolved_in_lds_and_in_memory():
    """A zero query makes every score 0: one histogram bin holds every block.  With
    1,500 blocks the bin is resolved from LDS, with 5,000 from memory; both must give
    blocks 0..511 (the lower index wins)."""
    case = small_decode("fq0", 8, 16, 2, [6000, 20000], 64)
    case._q = np.zeros_like(case.q)
    d, sel, cnt, out, lse = check_fused(case)
    for r in range(case.R):
        for h in range(case.Hkv):
            assert np.array_equal(sel[r, h], np.arange(512))


def test_fused_workspace_reused_by_a_smaller_call():
    """Three calls on one workspace, the second with fewer sequences: all correct, and
    the control area consistent after each (checked inside fused()): the smaller
    call leaves the larger call's later units untouched, and the third call's waits
    are not satisfied by ready words of the earlier calls."""
    big = small_decode("fbig", 12, 16, 2, [9000, 7000, 5000, 3000], 64)
    small = small_decode("fsmall", 13, 16, 2, [4000, 2500], 64)
    dbig, dsmall = Dev(big), Dev(small)
    dbig.compress()
    dsmall.compress()
    ws = torch.zeros(qsa.qsa_decode_fused_workspace_bytes(dbig.kv, big.Hq, big.topk, 0), dtype=torch.uint8,
                     device="cuda")
    for d in (dbig, dsmall, dbig):
        sc = d.scores()
        sel_ref, cnt_ref = d.topk(sc, d.case.topk)
        fsel, fcnt, fout, flse = fused(d, ws=ws)
        assert np.array_equal(fsel, to_np(sel_ref)) and np.array_equal(fcnt, to_np(cnt_ref))
        check_decode_against_oracle(d.case, d, to_np(sc), fsel, fcnt, fout, flse, d.case.topk)


def test_fused_matches_separate_path_at_full_size():
    """32 sequences of 32K-64K tokens, (16,2) heads, shuffled 64-token pages: the
    benchmark's decode workload.  Selections equal the separate calls'; outputs
    agree with theirs and with the oracle on every row."""
    case = synth.config("C2")
    log(f"C2 fused: B={case.B} lens {int(case.lens.min())}..{int(case.lens.max())}")
    d = Dev(case)
    case.drop_paged()
    d.compress()
    sc = d.scores()
    sel_ref, cnt_ref = d.topk(sc, case.topk)
    out_ref, lse_ref = d.decode_attn(sel_ref, cnt_ref, case.topk)
    fsel, fcnt, fout, flse = fused(d)
    assert np.array_equal(fsel, to_np(sel_ref)) and np.array_equal(fcnt, to_np(cnt_ref))
    out_ref, lse_ref = to_np(out_ref), to_np(lse_ref)
    for r in range(case.B):
        check_close(fout[r], out_ref[r], f"C2 fused vs separate out row {r}")
        check_lse(flse[r], lse_ref[r], f"C2 fused vs separate lse row {r}")
    from test_gpu_configs import compare_rows
    compare_rows(case, list(range(case.B)), fsel, fcnt, fout, flse, d.stride)


def test_fused_pipeline_step_and_graph_replay():
    """decode_step_fused captured in a HIP graph: every replay equals the eager step."""
    case = small_decode("fgraph", 14, 16, 2, [9000, 4097, 6000], 64)
    d = Dev(case)
    d.compress()
    q, q_pos = d.t["q"], d.t["q_pos"]
    buf = FusedDecodeBuffers.allocate(d.kv, case.Hq, case.topk)
    decode_step_fused(d.kv, q, q_pos, buf, scale=case.scale)
    torch.cuda.synchronize()
    eager = buf.out.clone(), buf.lse.clone(), buf.sel_idx.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        decode_step_fused(d.kv, q, q_pos, buf, scale=case.scale)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        decode_step_fused(d.kv, q, q_pos, buf, scale=case.scale)
    for i in range(3):
        buf.out.fill_(0)
        buf.lse.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(buf.sel_idx, eager[2]), i
        assert torch.equal(buf.out, eager[0]), i
        assert torch.equal(buf.lse, eager[1]), i
    # two eager calls and three replays on the workspace
    check_control(buf.workspace, case.B * case.Hkv, 4)


def test_fused_abandoned_wait_gives_nan_and_leaves_no_stale_flag(monkeypatch):
    """The bounded wait's time-out, forced from the host with a one-poll limit: a
    unit whose selection was not ready when its attention item polled reports NaN
    out and lse (never a result from a stale selection), the abandoned waits are
    counted, and a later call on the same workspace with the normal limit is exact
    again -- ready words raised late by the short-limit call do not satisfy it."""
    case = small_decode("ftimeout", 15, 16, 2, [9000, 4097, 6000, 12000, 3000, 7000], 64)
    d = Dev(case)
    d.compress()
    U = case.B * case.Hkv
    ws = torch.zeros(qsa.qsa_decode_fused_workspace_bytes(d.kv, case.Hq, case.topk, 0), dtype=torch.uint8,
                     device="cuda")
    ref_sel, ref_cnt, ref_out, ref_lse = fused(d, ws=ws)            # normal limit: exact, checked in fused()
    monkeypatch.setenv("QSA_FUSED_SPIN_LIMIT", "1")
    q = d.t["q"]
    nan_units = 0
    for rep in range(3):
        sel = torch.full((case.B, case.Hkv, case.topk), -7, dtype=torch.int32, device="cuda")
        cnt = torch.full((case.B, case.Hkv), -7, dtype=torch.int32, device="cuda")
        out = torch.zeros((case.B, case.Hq, 256), dtype=torch.bfloat16, device="cuda")
        lse = torch.zeros((case.B, case.Hq), dtype=torch.float32, device="cuda")
        before = int(ws[8:12].view(torch.int32).item())
        qsa.qsa_decode_fused(d.kv, q, q.stride(0), case.Hq, case.topk, 0.0, 0, sel, cnt, out, out.stride(0), lse,
                             workspace=ws, workspace_bytes=ws.numel())
        torch.cuda.synchronize()
        abandoned = int(ws[8:12].view(torch.int32).item()) - before
        o, l = to_np(out), to_np(lse)
        nan_here = 0
        for r in range(case.B):
            for h in range(case.Hkv):
                heads = slice(h * case.g, (h + 1) * case.g)
                if np.isnan(l[r, heads]).any() or np.isnan(o[r, heads]).any():
                    assert np.isnan(l[r, heads]).all() and np.isnan(o[r, heads]).all(), (rep, r, h)
                    nan_here += 1
                else:
                    assert np.array_equal(o[r, heads], ref_out[r, heads]), (rep, r, h)
                    assert np.array_equal(l[r, heads], ref_lse[r, heads]), (rep, r, h)
        assert (abandoned > 0) == (nan_here > 0) and nan_here <= abandoned, (rep, abandoned, nan_here)
        assert np.array_equal(to_np(sel), ref_sel) and np.array_equal(to_np(cnt), ref_cnt), rep
        nan_units += nan_here
    log(f"fused one-poll limit: {nan_units} of {3 * U} units reported NaN")
    monkeypatch.delenv("QSA_FUSED_SPIN_LIMIT")
    abandoned_total = int(ws[8:12].view(torch.int32).item())
    sel, cnt, out, lse = fused_counted(d, ws)
    assert int(ws[8:12].view(torch.int32).item()) == abandoned_total
    assert np.array_equal(sel, ref_sel) and np.array_equal(cnt, ref_cnt)
    assert np.array_equal(out, ref_out) and np.array_equal(lse, ref_lse)


def fused_counted(d: Dev, ws: torch.Tensor):
    """One fused call on a workspace that may carry abandoned waits from earlier calls
    (the abandoned-wait word is not reset): outputs and the rest of the control area."""
    c = d.case
    q = d.t["q"]
    sel = torch.full((c.B, c.Hkv, c.topk), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((c.B, c.Hkv), -7, dtype=torch.int32, device="cuda")
    out = torch.full((c.B, c.Hq, 256), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((c.B, c.Hq), float("nan"), dtype=torch.float32, device="cuda")
    calls_before = int(ws[12:16].view(torch.int32).item())
    qsa.qsa_decode_fused(d.kv, q, q.stride(0), c.Hq, c.topk, 0.0, 0, sel, cnt, out, out.stride(0), lse,
                         workspace=ws, workspace_bytes=ws.numel())
    torch.cuda.synchronize()
    ctl = ws[:16].view(torch.int32).cpu().numpy()
    assert ctl[0] == 0 and ctl[1] == 0 and ctl[3] == calls_before + 1
    unit = ws[256:256 + 16 * c.B * c.Hkv].view(torch.int32).cpu().numpy().reshape(-1, 4)
    assert np.all(unit[:, 0] == 0) and np.all(unit[:, 2] == 0) and np.all(unit[:, 1] == ctl[3])
    return to_np(sel), to_np(cnt), to_np(out), to_np(lse)


@pytest.mark.parametrize("ckey_dtype,kv_dtype", [("fp32", "bf16"), ("bf16", "bf16"), ("fp8", "fp8")])
def test_fused_rebuilds_the_newest_block_key(ckey_dtype, kv_dtype):
    """The fused launch rebuilds the block key holding each sequence's newest token,
    as qsa_decode_scores_refresh does: with those keys spoilt beforehand, its block-key
    pool, selection and output equal the separate path's (refresh-and-score launch,
    top-k, attention) bit for bit."""
    from test_gpu_refresh import spoil_newest
    case = small_decode("frefresh", 16, 16, 2, [4096, 4097, 4098, 4099, 1, 5, 9000], 64, jitter=True,
                        ckey_dtype=ckey_dtype, kv_dtype=kv_dtype)
    d = Dev(case)
    d.compress()
    spoil_newest(d)
    spoiled = d.t["ckey"].clone()
    q = d.t["q"]
    stride = d.stride
    s = torch.empty((case.B, case.Hkv, stride), dtype=torch.float32, device="cuda")
    qsa.qsa_decode_scores_refresh(d.kv, q, q.stride(0), case.Hq, s, stride)
    sel_ref, cnt_ref = d.topk(s, case.topk)
    out_ref, lse_ref = d.decode_attn(sel_ref, cnt_ref, case.topk)
    torch.cuda.synchronize()
    pool_ref = d.t["ckey"].clone()
    d.t["ckey"].copy_(spoiled)
    fsel, fcnt, fout, flse = fused(d)
    assert torch.equal(d.t["ckey"].view(torch.uint8), pool_ref.view(torch.uint8)), "block-key pool differs"
    assert np.array_equal(fsel, to_np(sel_ref)) and np.array_equal(fcnt, to_np(cnt_ref))
    check_decode_against_oracle(case, d, to_np(s), fsel, fcnt, fout, flse, case.topk)
    ro, rl = to_np(out_ref), to_np(lse_ref)
    for r in range(case.B):
        check_close(fout[r], ro[r], f"fused vs separate out row {r}")
        check_lse(flse[r], rl[r], f"fused vs separate lse row {r}")
