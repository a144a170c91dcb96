"""A decode step captured in a HIP graph replays to the same bits as the eager step,
on several replays with eager work and synchronisations in between."""
import numpy as np
import pytest
import torch

import block_sparse_attention_compress_amd as qsa
import synth
from block_sparse_attention_compress_amd.pipeline import DecodeBuffers, DecodeGraph, decode_step
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
