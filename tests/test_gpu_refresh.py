"""qsa_decode_scores_refresh through the C ABI: one launch that rebuilds the block
key holding each sequence's newest token and scores every block must give, bit
for bit, the scores and the block-key pool of the two separate calls
(qsa_compress_keys from L - 1, then qsa_block_scores).  The newest blocks' stored
keys are overwritten with a wrong value first, so a score taken from the stale
key, or a key left unwritten, shows."""
import numpy as np
import pytest
import torch

import block_sparse_attention_compress_amd as qsa
from gpu_harness import Dev, log
from test_gpu_parity import small_decode

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def spoil_newest(d: Dev):
    c = d.case
    ck = d.t["ckey"]
    for i in range(c.B):
        L = int(c.lens[i])
        if L == 0:
            continue
        b = (L - 1) // 4
        page = int(c.block_table[i][(4 * b) // c.page_size])
        ck[page, :, ((4 * b) % c.page_size) // 4, :] = 5.0


def both_paths(case, stride=None, drop_host=False):
    d = Dev(case)
    if drop_host:
        case.drop_paged()
    d.compress()
    spoil_newest(d)
    spoiled = d.t["ckey"].clone()
    stride = d.stride if stride is None else stride
    c = case
    q = d.t["q"]
    first = torch.from_numpy(np.maximum(c.lens - 1, 0).astype(np.int32)).cuda()
    out = []
    for fused in (False, True):
        d.t["ckey"].copy_(spoiled)
        s = torch.full((c.B, c.Hkv, stride), float("nan"), dtype=torch.float32, device="cuda")
        if fused:
            qsa.qsa_decode_scores_refresh(d.kv, q, q.stride(0), c.Hq, s, stride)
        else:
            qsa.qsa_compress_keys(d.kv, first, 1)
            qsa.qsa_block_scores(d.kv, q, q.stride(0), None, None, c.B, c.Hq, s, stride)
        torch.cuda.synchronize()
        out.append((s.view(torch.int32).clone(), d.t["ckey"].clone()))
    (s0, k0), (s1, k1) = out
    assert torch.equal(s0, s1), "scores differ from the separate calls"
    assert torch.equal(k0.view(torch.uint8), k1.view(torch.uint8)), "block-key pool differs from the separate calls"
    assert not torch.equal(k1.view(torch.uint8), spoiled.view(torch.uint8)) or int(c.lens.max()) == 0
    return d, s1


@pytest.mark.parametrize("ckey_dtype", ["fp32", "bf16", "fp8"])
@pytest.mark.parametrize("page_size,lens", [
    (64, [4096, 4097, 4098, 4099, 1, 5]),   # L mod 4 = 0..3; one- and two-block rows
    (4, [37, 64, 1, 2]),
    (16, [500, 3, 0]),                      # an empty sequence is skipped
    (256, [1000, 2051]),
    (8192, [8192, 8191]),                   # contiguous pages
])
def test_refresh_scores_equal_separate_calls(ckey_dtype, page_size, lens):
    case = small_decode(f"rf{page_size}", 700 + page_size, 16, 2, lens, page_size, jitter=True,
                        ckey_dtype=ckey_dtype)
    log(f"refresh+scores page_size={page_size} lens={lens} ckey={ckey_dtype}")
    both_paths(case)


@pytest.mark.parametrize("Hq,Hkv", [(24, 2), (6, 1), (3, 1)])
def test_refresh_head_ratios(Hq, Hkv):
    case = small_decode(f"rfh{Hq}", 800 + Hq, Hq, Hkv, [9001, 130, 2050], 64)
    both_paths(case)


def test_refresh_rows_cut_short_by_the_stride():
    """score_stride below a row's block count: the first score_stride blocks are
    scored, and the newest block's key is still rebuilt."""
    case = small_decode("rfcut", 900, 16, 2, [4003, 90, 2000], 64)
    both_paths(case, stride=100)


def test_refresh_full_size_decode_workload():
    import synth
    case = synth.config("C2")
    log(f"C2 refresh: B={case.B}")
    both_paths(case, stride=(max(case.nb(i) for i in range(case.B)) + 63) // 64 * 64, drop_host=True)


def test_refresh_with_shared_prefix_pages():
    """Sequences sharing their first 20 pages (a common prefix): the newest blocks
    lie in each sequence's own pages, as the refresh launch requires."""
    case = small_decode("rfpre", 950, 16, 2, [4096, 5000, 4500], 64, shared_prefix_pages=20)
    both_paths(case)
