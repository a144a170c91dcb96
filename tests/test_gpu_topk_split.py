"""The two-stage top-k for long rows (qsa_topk_blocks_ws) through the C ABI.

Its selection must equal, bit for bit, both the oracle's (score descending, lower
block index first) and the one-stage qsa_topk_blocks on the same fp32 scores:
long rows, a short last slice, rows that fit one slice, heavy ties across
slices, signed zeros, eligibility from q_pos, strides and k that rule out
16-byte loads, and one workspace reused by a smaller call."""
import numpy as np
import pytest
import torch

import block_sparse_attention_compress_amd as qsa
import oracle
from gpu_harness import log, to_np

pytestmark = pytest.mark.gpu

SLICE = 8192


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def select(scores_np, q_pos_np, k, ws=None):
    R, Hkv, stride = scores_np.shape
    s = torch.from_numpy(np.ascontiguousarray(scores_np, dtype=np.float32)).cuda()
    qp = None if q_pos_np is None else torch.from_numpy(np.asarray(q_pos_np, dtype=np.int32)).cuda()
    out = []
    for two_stage in (True, False):
        sel = torch.full((R, Hkv, max(k, 1)), -7, dtype=torch.int32, device="cuda")
        cnt = torch.full((R, Hkv), -7, dtype=torch.int32, device="cuda")
        if two_stage:
            need = qsa.qsa_topk_workspace_bytes(R, Hkv, k, stride)
            w = ws if ws is not None else (torch.empty(need, dtype=torch.uint8, device="cuda") if need else None)
            if w is not None:
                w.fill_(0xFF)  # contents on entry must not matter
            qsa.qsa_topk_blocks_ws(s, stride, qp, R, Hkv, k, sel, cnt, workspace=w,
                                   workspace_bytes=0 if w is None else w.numel())
        else:
            qsa.qsa_topk_blocks(s, stride, qp, R, Hkv, k, sel, cnt)
        torch.cuda.synchronize()
        out.append((to_np(sel), to_np(cnt)))
    return out


def check(scores_np, q_pos_np, k, ws=None):
    (sel, cnt), (sel1, cnt1) = select(scores_np, q_pos_np, k, ws)
    assert np.array_equal(cnt, cnt1) and np.array_equal(sel[..., :k], sel1[..., :k]), "two-stage != one-stage"
    R, Hkv, stride = scores_np.shape
    for r in range(R):
        n = stride if q_pos_np is None else max(0, min(int(q_pos_np[r]) // 4 + 1, stride))
        if q_pos_np is not None and int(q_pos_np[r]) < 0:
            n = 0
        for h in range(Hkv):
            want, wc = oracle.topk(scores_np[r, h, :n].astype(np.float64), k)
            assert cnt[r, h] == wc, (r, h, cnt[r, h], wc)
            assert np.array_equal(sel[r, h, :k], want), (r, h)


@pytest.mark.parametrize("n,k", [(16385, 512), (16384 + 513, 512), (24577, 2048), (20000, 17), (65536, 512),
                                 (65536, 1), (65536, 2048), (100003, 512), (262144, 512)])
def test_long_rows_equal_oracle_and_one_stage(n, k):
    rng = np.random.default_rng(n + 3 * k)
    s = (rng.standard_normal((2, 2, n)) * 30).astype(np.float32)
    log(f"topk two-stage n={n} k={k}")
    check(s, None, k)


def test_long_rows_biased_blocks():
    """1 % of the blocks lifted by +3 sigma, as in the long-context decode
    workload: the top k crowd into few slices."""
    rng = np.random.default_rng(77)
    s = rng.standard_normal((3, 2, 65536)).astype(np.float32)
    hot = rng.random((3, 2, 65536)) < 0.01
    s[hot] += 3.0
    s[2, :, 40000:41000] += 10.0  # one slice holds all 512
    check(s, None, 512)


def test_ties_across_slices_and_signed_zero():
    rng = np.random.default_rng(5)
    s = rng.integers(-3, 4, size=(4, 1, 40000)).astype(np.float32)  # every slice full of ties at the k-th value
    s[1] = 0.0                                                       # all equal: blocks 0..k-1
    s[2, 0, ::2] = -0.0
    s[2, 0, 1::2] = 0.0
    s[3, 0, :] = -1.0
    s[3, 0, 30000:] = 2.0                                            # the top k lie in the last slices
    check(s, None, 512)
    (sel, _), _ = select(np.zeros((1, 2, 30000), np.float32), None, 512)
    assert np.array_equal(sel[0, 0], np.arange(512)) and np.array_equal(sel[0, 1], np.arange(512))


def test_eligibility_from_q_pos():
    """n_elig = 0, 1, 512, 513, one slice, one slice + 1, two slices, a short
    last slice, the whole row."""
    rng = np.random.default_rng(9)
    stride = 40000
    s = rng.standard_normal((11, 2, stride)).astype(np.float32)
    n_elig = [0, 1, 512, 513, SLICE, SLICE + 1, 2 * SLICE, 2 * SLICE + 300, 4 * SLICE + 1, stride, 33333]
    q_pos = np.array([-1 if n == 0 else 4 * n - 1 for n in n_elig], dtype=np.int32)
    check(s, q_pos, 512)


def test_strides_and_k_without_16_byte_loads():
    rng = np.random.default_rng(11)
    check(rng.standard_normal((2, 1, 20001)).astype(np.float32), None, 512)  # stride % 4 != 0
    check(rng.standard_normal((2, 1, 33000)).astype(np.float32), None, 19)   # candidate rows of 5 x 19


def test_k_zero_and_short_rows_need_no_workspace():
    assert qsa.qsa_topk_workspace_bytes(2, 2, 0, 65536) == 0
    assert qsa.qsa_topk_workspace_bytes(2, 2, 512, 16384) == 0
    rng = np.random.default_rng(13)
    check(rng.standard_normal((2, 2, 65536)).astype(np.float32), None, 0)
    check(rng.standard_normal((2, 2, 16384)).astype(np.float32), None, 512)


def test_workspace_reused_by_a_smaller_call():
    rng = np.random.default_rng(17)
    big = rng.standard_normal((4, 2, 70000)).astype(np.float32)
    small = rng.standard_normal((2, 1, 20000)).astype(np.float32)
    ws = torch.empty(qsa.qsa_topk_workspace_bytes(4, 2, 512, 70000), dtype=torch.uint8, device="cuda")
    for sc in (big, small, big):
        check(sc, None, 512, ws=ws)


def test_many_rows_use_the_many_row_kernel_bit_exact():
    """1,100 rows of one KV head: the launch takes 512 threads per row.  Random,
    heavily tied (bins crowded past 512 candidates: the radix passes), all-equal
    and short rows, with eligibility from q_pos, against the oracle."""
    rng = np.random.default_rng(23)
    R, stride = 1100, 5000
    s = (rng.standard_normal((R, 1, stride)) * 20).astype(np.float32)
    s[100:200] = rng.integers(-3, 4, size=(100, 1, stride)).astype(np.float32)
    s[200:210] = 1.5
    s[210:220, 0, ::2] = -0.0
    s[210:220, 0, 1::2] = 0.0
    q_pos = np.full(R, 4 * stride - 1, dtype=np.int32)
    q_pos[300:400] = rng.integers(-1, 4 * stride, size=100)
    q_pos[400:410] = [0, 3, 4, 2043, 2047, 2048, 2051, 7, 11, 15]
    for k in (512, 37):
        log(f"topk many rows k={k}")
        check(s, q_pos, k)
