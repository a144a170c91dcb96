"""qsa_sparse_attn_decode_noalloc -- decode attention whose split partials live in
the library's static device scratch -- against qsa_sparse_attn_decode with a
caller workspace, through the C ABI: bit for bit on the same selection, on two
calls in a row (the second with a smaller input, so it runs on what the first
left in the scratch), and against the oracle; and the size limit."""
import numpy as np
import pytest
import torch

import block_sparse_attention_compress_amd as qsa
from gpu_harness import Dev, log, to_np
from test_gpu_parity import check_decode_against_oracle, small_decode

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def both_paths(case, num_splits):
    d = Dev(case)
    d.compress()
    sc = d.scores()
    sel, cnt = d.topk(sc, case.topk)
    ref_out, ref_lse = d.decode_attn(sel, cnt, case.topk, num_splits=num_splits)
    out = torch.full_like(ref_out, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    q = d.t["q"]
    qsa.qsa_sparse_attn_decode_noalloc(d.kv, q, q.stride(0), case.Hq, sel, cnt, case.topk, 0.0, num_splits, out,
                                       out.stride(0), lse)
    torch.cuda.synchronize()
    return d, to_np(sc), to_np(sel), to_np(cnt), ref_out, ref_lse, out, lse


@pytest.mark.parametrize("num_splits", [0, 4, 64])
def test_noalloc_equals_workspace_entry_point_on_two_calls(num_splits):
    big = small_decode("noalloc-big", 71, 16, 2, [9000, 4097, 6000, 12000, 3001, 7000], 64, jitter=True)
    small = small_decode("noalloc-small", 72, 6, 1, [5000, 2051], 64)
    for case in (big, small):
        log(f"noalloc {case.name} splits={num_splits} heads=({case.Hq},{case.Hkv}) lens={case.lens.tolist()}")
        d, sc, sel, cnt, ro, rl, o, l = both_paths(case, num_splits)
        assert torch.equal(o, ro), f"{case.name}: out differs from qsa_sparse_attn_decode"
        assert torch.equal(l, rl), f"{case.name}: lse differs from qsa_sparse_attn_decode"
        check_decode_against_oracle(case, d, sc, sel, cnt, to_np(o), to_np(l), case.topk)


def test_noalloc_rejects_partials_beyond_the_scratch():
    """64 splits of 600 rows x 16 heads need about 630 MB of partials: rejected with a
    message before anything is launched; one split needs no scratch and runs."""
    case = small_decode("noalloc-limit", 73, 16, 2, [64] * 600, 64)
    d = Dev(case)
    d.compress()
    sel, cnt = d.topk(d.scores(), case.topk)
    q = d.t["q"]
    out = torch.zeros((case.B, case.Hq, 256), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((case.B, case.Hq), dtype=torch.float32, device="cuda")
    with pytest.raises(qsa.QsaError) as e:
        qsa.qsa_sparse_attn_decode_noalloc(d.kv, q, q.stride(0), case.Hq, sel, cnt, case.topk, 0.0, 64, out,
                                           out.stride(0), lse)
    assert e.value.code == qsa.QSA_ERR_UNSUPPORTED and "scratch" in str(e.value)
    ref_out, ref_lse = d.decode_attn(sel, cnt, case.topk, num_splits=1)
    qsa.qsa_sparse_attn_decode_noalloc(d.kv, q, q.stride(0), case.Hq, sel, cnt, case.topk, 0.0, 1, out,
                                       out.stride(0), lse)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
