"""A decode step, an extend chunk (also one with the split read), and the query-tile union attention, captured in a
HIP graph replay to the same bits as the eager calls, on several replays with eager
work and synchronisations in between."""
import numpy as np
import pytest
import torch

import block_sparse_attention_compress_amd as qsa
import synth
from block_sparse_attention_compress_amd.pipeline import (DecodeBuffers, DecodeGraph, ExtendBuffers, decode_step,
                                                         extend_step)
from gpu_harness import log

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("num_splits,L_range", [(0, (9000, 17000)), (1, (9000, 17000)), (4, (9000, 17000)),
                                                (0, (70000, 90000))])  # rows over 16,384 blocks: two-stage top-k
def test_graph_replays_match_eager(num_splits, L_range):
    case = synth.config("C2", B=6, L_range=L_range)
    log(f"graph replay, num_splits={num_splits}, lengths {L_range}")
    dev = synth.to_device(case, "cuda")
    kv = qsa.KVCache(dev["k"], dev["v"], dev["ckey"], dev["block_table"], dev["seq_lens"], case.max_len)
    qsa.qsa_compress_keys(kv)
    stride = max(case.nb(i) for i in range(case.B))
    buf = DecodeBuffers.allocate(case.B, case.Hq, case.Hkv, stride, case.topk, num_splits, "cuda")
    assert (buf.topk_workspace is not None) == (stride > 16384)
    decode_step(kv, dev["q"], dev["q_pos"], buf, scale=case.scale, num_splits=num_splits)
    torch.cuda.synchronize()
    want = (buf.sel_idx.clone(), buf.sel_cnt.clone(), buf.out.clone(), buf.lse.clone())

    g = DecodeGraph(kv, dev["q"], dev["q_pos"], buf, scale=case.scale, num_splits=num_splits)
    for rep in range(4):
        buf.out.fill_(float("nan"))
        buf.lse.fill_(float("nan"))
        buf.sel_idx.fill_(-9)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (buf.sel_idx, buf.sel_cnt, buf.out, buf.lse)
        for a, b in zip(got, want):
            assert torch.equal(a, b), f"replay {rep} differs"
        # eager work between replays
        decode_step(kv, dev["q"], dev["q_pos"], buf, scale=case.scale, num_splits=num_splits)
        torch.cuda.synchronize()
    # a replay after changing the query in place follows the new query
    dev["q"].mul_(-1)
    g.replay()
    torch.cuda.synchronize()
    got = buf.out.clone()
    decode_step(kv, dev["q"], dev["q_pos"], buf, scale=case.scale, num_splits=num_splits)
    torch.cuda.synchronize()
    assert torch.equal(got, buf.out)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_extend_chunk_graph_replays_match_eager(kv_dtype):
    """The extend chunk's four calls (block keys of the new tokens, tiled block
    scores, many-row top-k, extend attention) in one captured graph."""
    total, new = 6000, 1100   # 1,100 rows: the many-row top-k
    q_seq, q_pos = synth.extend_rows(total, new)
    case = synth.make_case(f"xgraph{kv_dtype}", 61, 12, 1, [total], page_size=64, q_seq=q_seq, q_pos=q_pos,
                           jitter=True, kv_dtype=kv_dtype)
    log(f"extend graph replay, {kv_dtype} cache")
    dev = synth.to_device(case, "cuda")
    kv = qsa.KVCache(dev["k"], dev["v"], dev["ckey"], dev["block_table"], dev["seq_lens"], case.max_len)
    qsa.qsa_compress_keys(kv)
    first = torch.tensor([total - new], dtype=torch.int32, device="cuda")
    stride = case.nb(0)
    buf = ExtendBuffers.allocate(case.R, case.Hq, case.Hkv, stride, case.topk, "cuda")

    def chunk():
        extend_step(kv, dev["q"], dev["q_seq"], dev["q_pos"], buf, first, new, scale=case.scale)

    chunk()
    torch.cuda.synchronize()
    want = (buf.sel_idx.clone(), buf.sel_cnt.clone(), buf.out.clone(), buf.lse.clone(), dev["ckey"].clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        chunk()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        chunk()
    for rep in range(4):
        buf.out.fill_(float("nan"))
        buf.lse.fill_(float("nan"))
        buf.sel_idx.fill_(-9)
        buf.scores.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (buf.sel_idx, buf.sel_cnt, buf.out, buf.lse, dev["ckey"])
        for a, b in zip(got, want):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep} differs"
        chunk()  # eager work between replays
        torch.cuda.synchronize()


def test_split_extend_chunk_graph_replays_match_eager():
    """A chunk of few rows with the split read (extend_step(num_splits=0): block keys,
    tiled scores, top-k, split attention, merge) in one captured graph: every replay
    bit-equal to the eager chunk, with the workspace poisoned between replays."""
    total, new = 9000, 40   # 40 (row, KV head) units: the library splits each row 7 ways
    q_pos = list(range(total - new, total))
    case = synth.make_case("xsplitgraph", 62, 12, 1, [total], page_size=64, q_seq=[0] * new, q_pos=q_pos,
                           jitter=True)
    log("split extend graph replay")
    dev = synth.to_device(case, "cuda")
    kv = qsa.KVCache(dev["k"], dev["v"], dev["ckey"], dev["block_table"], dev["seq_lens"], case.max_len)
    qsa.qsa_compress_keys(kv)
    first = torch.tensor([total - new], dtype=torch.int32, device="cuda")
    buf = ExtendBuffers.allocate(case.R, case.Hq, case.Hkv, case.nb(0), case.topk, "cuda", max_splits=0)

    def chunk():
        extend_step(kv, dev["q"], dev["q_seq"], dev["q_pos"], buf, first, new, scale=case.scale, num_splits=0)

    chunk()
    torch.cuda.synchronize()
    want = (buf.sel_idx.clone(), buf.sel_cnt.clone(), buf.out.clone(), buf.lse.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        chunk()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        chunk()
    for rep in range(4):
        buf.out.fill_(float("nan"))
        buf.lse.fill_(float("nan"))
        buf.workspace.fill_(0xFF)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (buf.sel_idx, buf.sel_cnt, buf.out, buf.lse)
        for a, b in zip(got, want):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep} differs"
        chunk()  # eager work between replays
        torch.cuda.synchronize()


def test_union_extend_attention_graph_replays_match_eager():
    """The query-tile union kernel captured after the extend chunk's selection: each
    replay's outputs equal the eager call's bit for bit, with eager work between."""
    total, new = 6000, 300
    q_seq, q_pos = synth.extend_rows(total, new)
    case = synth.make_case("ugraph", 62, 16, 2, [total], page_size=64, q_seq=q_seq, q_pos=q_pos, q_share=0.5)
    log("union extend attention graph replay")
    dev = synth.to_device(case, "cuda")
    kv = qsa.KVCache(dev["k"], dev["v"], dev["ckey"], dev["block_table"], dev["seq_lens"], case.max_len)
    qsa.qsa_compress_keys(kv)
    stride = case.nb(0)
    buf = ExtendBuffers.allocate(case.R, case.Hq, case.Hkv, stride, case.topk, "cuda")
    extend_step(kv, dev["q"], dev["q_seq"], dev["q_pos"], buf, scale=case.scale)
    q = dev["q"]

    def union():
        qsa.qsa_sparse_attn_extend_union(kv, q, q.stride(0), dev["q_seq"], dev["q_pos"], case.R, case.Hq, buf.sel_idx,
                                         buf.sel_cnt, case.topk, case.scale, buf.out, buf.out.stride(0), buf.lse)

    union()
    torch.cuda.synchronize()
    want = (buf.out.clone(), buf.lse.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        union()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        union()
    for rep in range(4):
        buf.out.fill_(float("nan"))
        buf.lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip((buf.out, buf.lse), want):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep} differs"
        union()  # eager work between replays
        torch.cuda.synchronize()
