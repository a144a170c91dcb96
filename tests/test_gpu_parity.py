"""HIP path versus the CPU oracle on seeded inputs, through the C ABI.

Sizes span several tiles (64-token pages, 32-token attention tiles, 256-block score
chunks) and ragged tails (L mod 4 = 0..3, partial pages).  Bars: block keys and
selections on identical scores bit-exact; selections from the full path exact up
to swaps within 1e-4 relative of the k-th score; outputs and lse within
|gpu - oracle| <= 1e-2 + 1e-2 |oracle|.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import check_close, check_lse, check_selection, score_bound
from gpu_harness import Dev, log, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def small_decode(name, seed, Hq, Hkv, lens, page_size=64, **kw):
    return synth.make_case(name, seed, Hq, Hkv, lens, page_size=page_size, **kw)


# ------------------------------------------------------------------------- a1

@pytest.mark.parametrize("page_size,lens", [
    (64, [4096, 4097, 4098, 4099]),      # L mod 4 = 0..3, partial last page
    (4, [37, 64, 1]),
    (16, [500, 3]),
    (256, [1000, 2051]),
    (8192, [8192]),                       # one contiguous page
])
def test_compress_bitwise(page_size, lens):
    case = small_decode(f"cmp{page_size}", 100 + page_size, 8, 2, lens, page_size, jitter=True)
    log(f"compress page_size={page_size} lens={lens}")
    d = Dev(case)
    d.compress()
    torch.cuda.synchronize()
    for i in range(case.B):
        got = d.ckey_logical(i)
        K = case.logical("k", i)
        for h in range(case.Hkv):
            want = oracle.compress(K[h])
            assert np.array_equal(got[h].view(np.uint32), want.view(np.uint32)), (i, h)


def test_compress_refresh_from_first_token():
    case = small_decode("cmpfirst", 7, 4, 2, [300, 517], 64)
    d = Dev(case)
    d.t["ckey"].fill_(float("nan"))
    first = torch.tensor([201, 517 - 1], dtype=torch.int32, device="cuda")
    d.compress(first, max_new=100)
    torch.cuda.synchronize()
    for i, f in enumerate([201, 516]):
        got = d.ckey_logical(i)
        K = case.logical("k", i)
        for h in range(case.Hkv):
            want = oracle.compress(K[h])
            b0 = f // 4      # blocks with 4b + 3 >= first
            assert np.all(np.isnan(got[h, :b0]))
            assert np.array_equal(got[h, b0:].view(np.uint32), want[b0:].view(np.uint32))


# ------------------------------------------------------------------------- a2

@pytest.mark.parametrize("Hq,Hkv", [(16, 2), (24, 2), (12, 1), (6, 1), (3, 1)])
def test_decode_scores_within_fp32_bound(Hq, Hkv):
    case = small_decode(f"sc{Hq}", 200 + Hq, Hq, Hkv, [2051, 700, 4096], 64)
    log(f"decode scores heads=({Hq},{Hkv})")
    d = Dev(case)
    d.compress()
    s = to_np(d.scores())
    g = case.g
    for r in range(case.R):
        i = r
        ck = d.ckey_logical(i)
        for h in range(Hkv):
            qg = case.q[r, h * g:(h + 1) * g]
            ne = case.nb(i)
            ref = oracle.scores(qg, ck[h], ne)
            bound = score_bound(synth.bf16_to_f32(qg).astype(np.float64), ck[h][:ne])
            assert np.all(np.abs(s[r, h, :ne] - ref) <= bound), (r, h)
            assert np.all(np.isnan(s[r, h, ne:]))        # not written past n_elig


def test_extend_scores_within_fp32_bound_mixed_sequences():
    # rows of two sequences interleaved inside one 16-row tile, and a causal mask
    lens = [600, 900]
    q_seq = np.array([0, 1] * 20 + [1] * 9, dtype=np.int32)
    q_pos = np.array([min(lens[s] - 1, 17 * j + 3) for j, s in enumerate(q_seq)], dtype=np.int32)
    case = synth.make_case("scx", 31, 12, 1, lens, page_size=64, q_seq=q_seq, q_pos=q_pos)
    log("extend scores mixed sequences")
    d = Dev(case)
    d.compress()
    s = to_np(d.scores(extend=True))
    cks = [d.ckey_logical(i) for i in range(case.B)]
    for r in range(case.R):
        i, t = int(q_seq[r]), int(q_pos[r])
        ne = min(t // 4 + 1, d.stride)
        qg = case.q[r]
        ref = oracle.scores(qg, cks[i][0], ne)
        bound = score_bound(synth.bf16_to_f32(qg).astype(np.float64), cks[i][0][:ne])
        assert np.all(np.abs(s[r, 0, :ne] - ref) <= 2 * bound), r
        assert np.all(np.isnan(s[r, 0, ne:]))


def extend_scores_bound_check(case, d, s, rows=None):
    """Every written score of the given rows within the fp32 Higham bound of the
    fp64 oracle score; nothing written past the row's eligible blocks."""
    cks = [d.ckey_logical(i) for i in range(case.B)]
    rows = range(case.R) if rows is None else rows
    worst = 0.0
    for i in range(case.B):
        rr = [r for r in rows if int(case.q_seq[r]) == i]
        if not rr:
            continue
        ck = cks[i][0].astype(np.float64)                       # [nb][256], one KV head
        qg = synth.bf16_to_f32(case.q[rr]).astype(np.float64)   # [n][g][256]
        qsum = qg.sum(axis=1)
        ref = qsum @ ck.T                                       # fp64 scores, [n][nb]
        bound = score_bound_rows(qg, ck)
        for j, r in enumerate(rr):
            ne = min(int(case.q_pos[r]) // 4 + 1, d.stride)
            err = np.abs(s[r, 0, :ne] - ref[j, :ne])
            assert np.all(err <= bound[j, :ne]), (r, float((err - bound[j, :ne]).max()))
            worst = max(worst, float((err / np.maximum(bound[j, :ne], 1e-300)).max()))
            assert np.all(np.isnan(s[r, 0, ne:]))
    return worst


def score_bound_rows(qg, ck):
    """score_bound for many rows: gamma_n sum_d sum_j |q_jd| |ckey_d|, n = g + 256 + 2."""
    g = qg.shape[1]
    n = g + ck.shape[1] + 2
    u = 2.0 ** -24
    gamma = n * u / (1 - n * u)
    return gamma * (np.abs(qg).sum(axis=1) @ np.abs(ck).T)


@pytest.mark.parametrize("ckey_dtype", ["fp32", "bf16", "fp8"])
def test_extend_scores_within_fp32_bound_one_sequence(ckey_dtype):
    """Rows of one sequence (the shared-tile path on bf16 matrix cores with split
    operands): every score within the fp32 bound, partial chunks and page tables of
    4-token pages included."""
    for page_size, L, n in ((64, 9000, 300), (4, 2100, 130)):
        q_seq, q_pos = synth.extend_rows(L, n)
        case = synth.make_case(f"sc1{page_size}", 41 + page_size, 12, 1, [L], page_size=page_size, q_seq=q_seq,
                               q_pos=q_pos, ckey_dtype=ckey_dtype)
        log(f"extend scores one sequence page_size={page_size} L={L} rows={n} ckey={ckey_dtype}")
        d = Dev(case)
        d.compress()
        s = to_np(d.scores(extend=True))
        worst = extend_scores_bound_check(case, d, s)
        log(f"  worst |gpu - fp64| / bound = {worst:.4f}")


def test_extend_scores_within_fp32_bound_full_chunk():
    """All 4,096 rows x up to 8,192 blocks of the extend chunk (28,672 cached + 4,096
    new tokens, (12,1) heads): every score within the fp32 bound of the fp64 score."""
    case = synth.config("C4")
    log("extend scores C4, all rows")
    d = Dev(case)
    case.drop_paged()
    d.compress()
    s = to_np(d.scores(extend=True))
    worst = extend_scores_bound_check(case, d, s)
    log(f"C4 scores: worst |gpu - fp64| / fp32 bound = {worst:.4f}")


# ------------------------------------------------------------------------- a3

def gpu_topk_exact(scores_np: np.ndarray, q_pos_np, k: int):
    R, Hkv, stride = scores_np.shape
    s = torch.from_numpy(np.ascontiguousarray(scores_np, dtype=np.float32)).cuda()
    qp = None if q_pos_np is None else torch.from_numpy(np.asarray(q_pos_np, dtype=np.int32)).cuda()
    sel = torch.full((R, Hkv, max(k, 1)), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((R, Hkv), -7, dtype=torch.int32, device="cuda")
    import block_sparse_attention_compress_amd as qsa
    qsa.qsa_topk_blocks(s, stride, qp, R, Hkv, k, sel, cnt)
    sel, cnt = to_np(sel), to_np(cnt)
    for r in range(R):
        n = stride if q_pos_np is None else min(int(q_pos_np[r]) // 4 + 1, stride)
        for h in range(Hkv):
            want, wc = oracle.topk(scores_np[r, h, :n].astype(np.float64), k)
            assert cnt[r, h] == wc, (r, h, cnt[r, h], wc)
            assert np.array_equal(sel[r, h, :k], want), (r, h)


@pytest.mark.parametrize("n,k", [(1, 512), (511, 512), (512, 512), (513, 512), (2048, 512), (12289, 512),
                                 (65536, 512), (8192, 1), (8192, 2048), (3000, 0), (700, 17)])
def test_topk_bit_exact_on_identical_scores(n, k):
    rng = np.random.default_rng(n * 7 + k)
    s = rng.standard_normal((2, 2, n)).astype(np.float32) * 30
    log(f"topk n={n} k={k}")
    gpu_topk_exact(s, None, k)


def test_topk_ties_and_signed_zero():
    rng = np.random.default_rng(5)
    s = rng.integers(-3, 4, size=(3, 1, 5000)).astype(np.float32)     # heavy ties
    s[1] = 0.0
    s[2, 0, ::2] = -0.0                                                # -0 equals +0
    s[2, 0, 1::2] = 0.0
    gpu_topk_exact(s, None, 512)
    # the tie-break keeps blocks 0..511 when every score is 0
    gpu_topk_exact(np.zeros((1, 2, 4000), np.float32), None, 512)


def test_topk_eligibility_from_q_pos():
    rng = np.random.default_rng(9)
    s = rng.standard_normal((5, 2, 3000)).astype(np.float32)
    q_pos = np.array([0, 3, 4, 2047, 11999], dtype=np.int32)           # n_elig = 1, 1, 2, 512, 3000
    gpu_topk_exact(s, q_pos, 512)


# ---------------------------------------------------------------- a4 / full step

def run_decode(case, k=None, num_splits=0, scale=0.0):
    d = Dev(case)
    d.compress()
    k = case.topk if k is None else k
    sc = d.scores()
    sel, cnt = d.topk(sc, k)
    out, lse = d.decode_attn(sel, cnt, k, num_splits=num_splits, scale=scale)
    torch.cuda.synchronize()
    return d, to_np(sc), to_np(sel), to_np(cnt), to_np(out), to_np(lse)


def check_decode_against_oracle(case, d, scores, sel, cnt, out, lse, k):
    ref = oracle.run_case(case)
    g = case.g
    override = {}
    for r in range(case.R):
        for h in range(case.Hkv):
            # the decision from identical fp32 scores is bit-exact ...
            n = min(int(case.q_pos[r]) // 4 + 1, d.stride)
            w, wc = oracle.topk(scores[r, h, :n].astype(np.float64), k)
            assert np.array_equal(sel[r, h, :k], w), (r, h)
            # ... and against the fp64 oracle only swaps inside the window are allowed
            same = check_selection(sel[r, h], int(cnt[r, h]), ref.sel[(r, h)], ref.cnt[(r, h)],
                                   ref.scores[(r, h)], k, f"row {r} head {h}")
            if not same:
                override[(r, h)] = (sel[r, h, :k].copy(), int(cnt[r, h]))
    if override:
        ref = oracle.run_case(case, sel_override=override)
    for r in range(case.R):
        check_close(out[r], ref.out[r], f"out row {r}")
        check_lse(lse[r], ref.lse[r], f"lse row {r}")
    return ref


@pytest.mark.parametrize("Hq,Hkv", [(16, 2), (24, 2), (12, 1), (6, 1), (3, 1)])
def test_decode_step_head_pairs(Hq, Hkv):
    lens = [2051, 4097, 9000, 130]
    case = small_decode(f"dec{Hq}", 300 + Hq, Hq, Hkv, lens, 64, jitter=True)
    log(f"decode step heads=({Hq},{Hkv}) lens={lens}")
    res = run_decode(case)
    check_decode_against_oracle(case, *res, case.topk)


@pytest.mark.parametrize("L,k", [(1, 1), (63, 16), (64, 16), (65, 17), (2051, 513)])
def test_selection_widths(L, k):
    """Selected widths of 1, 63, 64, 65 and 2051 tokens (the last: 512 full blocks and a
    3-token tail), as in the Ascend page's operator tests."""
    case = small_decode(f"w{L}", 400 + L, 16, 2, [L, L], 64, topk=k)
    log(f"width L={L} k={k}")
    res = run_decode(case, k=k)
    check_decode_against_oracle(case, *res, k)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("num_splits", [0, 1, 5])
def test_largest_k(num_splits, kv_dtype):
    """k = 2048, the most allowed: 8,192 selected tokens per (row, KV head), the
    largest slot table and token loop, with the library's splits, one split and 5,
    for both cache types; a 300-token row selects all of its 75 blocks."""
    case = small_decode(f"k2048s{num_splits}{kv_dtype}", 88 + num_splits, 16, 2, [10000, 9001, 300], 64, topk=2048,
                        jitter=True, kv_dtype=kv_dtype)
    log(f"k=2048 splits={num_splits} cache={kv_dtype}")
    res = run_decode(case, k=2048, num_splits=num_splits)
    check_decode_against_oracle(case, *res, 2048)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_largest_k_extend(kv_dtype):
    total, nq = 12000, 65
    q_seq, q_pos = synth.extend_rows(total, nq)
    case = synth.make_case(f"k2048ext{kv_dtype}", 89, 12, 1, [total], page_size=64, q_seq=q_seq, q_pos=q_pos,
                           topk=2048, kv_dtype=kv_dtype)
    log(f"extend k=2048 cache={kv_dtype}")
    res = run_extend(case, k=2048)
    check_decode_against_oracle(case, *res, 2048)


def test_zero_k_gives_zero_output_and_neg_inf_lse():
    case = small_decode("k0", 5, 16, 2, [1000, 77], 64, topk=0)
    d, sc, sel, cnt, out, lse = run_decode(case, k=0)
    assert np.all(cnt == 0)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_empty_sequence():
    case = small_decode("L0", 6, 8, 2, [0, 300], 64)
    d, sc, sel, cnt, out, lse = run_decode(case)
    assert np.all(cnt[0] == 0) and np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    check_decode_against_oracle(case, d, sc, sel, cnt, out, lse, case.topk)


def test_zero_query_selects_first_blocks():
    case = small_decode("q0", 8, 16, 2, [6000, 3001], 64)
    case._q = np.zeros_like(case.q)
    d, sc, sel, cnt, out, lse = run_decode(case)
    for r in range(case.R):
        for h in range(case.Hkv):
            assert np.array_equal(sel[r, h], np.arange(512))
    check_decode_against_oracle(case, d, sc, sel, cnt, out, lse, case.topk)


@pytest.mark.parametrize("scale", [0.0, 0.03125, 0.2])
def test_default_and_explicit_scale(scale):
    case = small_decode("scale", 9, 16, 2, [3000, 2500], 64)
    case.scale = scale if scale > 0 else 1 / 16
    res = run_decode(case, scale=scale)
    check_decode_against_oracle(case, *res, case.topk)


def test_strided_query_and_output_rows():
    case = small_decode("stride", 10, 12, 1, [3000, 4000, 1234], 64)
    d = Dev(case)
    d.compress()
    qbig = torch.zeros((case.B, case.Hq + 4, 256), dtype=torch.bfloat16, device="cuda")
    qbig[:, :case.Hq] = d.t["q"]
    qv = qbig[:, :case.Hq]
    sc = d.scores(q=qv)
    sel, cnt = d.topk(sc, case.topk)
    obig = torch.full((case.B, case.Hq + 3, 256), 7.0, dtype=torch.bfloat16, device="cuda")
    ov = obig[:, :case.Hq]
    out, lse = d.decode_attn(sel, cnt, case.topk, num_splits=1, q=qv, out=ov)
    torch.cuda.synchronize()
    assert torch.all(obig[:, case.Hq:] == 7.0)
    check_decode_against_oracle(case, d, to_np(sc), to_np(sel), to_np(cnt), to_np(ov), to_np(lse), case.topk)


def test_shared_prefix_and_cache_reuse():
    case = small_decode("prefix", 11, 16, 2, [4096, 5000, 4500], 64, shared_prefix_pages=20)
    d, sc, sel, cnt, out, lse = run_decode(case)
    check_decode_against_oracle(case, d, sc, sel, cnt, out, lse, case.topk)
    # a second pass over the same cache, without recompressing, is bit-identical
    sc2 = d.scores()
    sel2, cnt2 = d.topk(sc2, case.topk)
    out2, lse2 = d.decode_attn(sel2, cnt2, case.topk)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(sel2), sel) and np.array_equal(to_np(out2), out)
    assert np.array_equal(to_np(lse2), lse, equal_nan=True)


# -------------------------------------------------------------- split-KV / a5

@pytest.mark.parametrize("S", [2, 3, 4, 7])
def test_split_partials_merge_and_unsplit(S):
    case = small_decode(f"split{S}", 12 + S, 6, 1, [5001, 7000, 2222, 12000], 64)
    log(f"split S={S}")
    d = Dev(case)
    d.compress()
    sc = d.scores()
    sel, cnt = d.topk(sc, 512)
    po, pl = d.decode_partials(sel, cnt, 512, S)
    import block_sparse_attention_compress_amd as qsa
    N = case.B * case.Hq
    merged = torch.empty((case.B, case.Hq, 256), dtype=torch.bfloat16, device="cuda")
    mlse = torch.empty((case.B, case.Hq), dtype=torch.float32, device="cuda")
    qsa.qsa_merge_lse(po, pl, S, N, 256, merged, mlse)
    unsplit, ulse = d.decode_attn(sel, cnt, 512, num_splits=1)
    auto, alse = d.decode_attn(sel, cnt, 512, num_splits=0)
    internal, ilse = d.decode_attn(sel, cnt, 512, num_splits=S)
    torch.cuda.synchronize()
    sel_np, cnt_np = to_np(sel), to_np(cnt)
    override = {(r, 0): (sel_np[r, 0], int(cnt_np[r, 0])) for r in range(case.R)}
    ref = oracle.run_case(case, splits=S, sel_override=override)
    po, pl = to_np(po), to_np(pl)
    for r in range(case.R):
        check_close(po[:, r], ref.part_out[r], f"partials row {r}")
        check_lse(pl[:, r], ref.part_lse[r], f"partial lse row {r}")
        for name, o, l in (("merged", merged, mlse), ("unsplit", unsplit, ulse), ("auto", auto, alse),
                           ("internal", internal, ilse)):
            check_close(to_np(o)[r], ref.out[r], f"{name} row {r}")
            check_lse(to_np(l)[r], ref.lse[r], f"{name} lse row {r}")
        check_close(to_np(merged)[r], to_np(unsplit)[r], f"merged vs unsplit row {r}")
    # the oracle's merged partials equal its unsplit attention (exact algebra)
    ref1 = oracle.run_case(case, splits=1, sel_override=override)
    for r in range(case.R):
        np.testing.assert_allclose(ref.out[r], ref1.out[r], atol=1e-12)


@pytest.mark.parametrize("kv_dtype,S", [("bf16", 16), ("fp8", 16), ("bf16", 64)])
def test_splits_without_tokens(kv_dtype, S):
    """16 or 64 (the most allowed) splits over sequences of 1 to 33 tokens (1 to 9
    blocks selected): most splits hold no token, and their partials must be 0 with
    lse -inf, as the oracle gives.  The merged partials and the library's internal
    S-way split must still equal the oracle."""
    import block_sparse_attention_compress_amd as qsa
    case = small_decode(f"s{S}{kv_dtype}", 77, 16, 2, [1, 5, 9, 33], 64, jitter=True, kv_dtype=kv_dtype)
    log(f"{S} splits, few tokens, {kv_dtype} cache")
    d = Dev(case)
    d.compress()
    sc = d.scores()
    sel, cnt = d.topk(sc, 512)
    po, pl = d.decode_partials(sel, cnt, 512, S)
    N = case.B * case.Hq
    merged = torch.empty((case.B, case.Hq, 256), dtype=torch.bfloat16, device="cuda")
    mlse = torch.empty((case.B, case.Hq), dtype=torch.float32, device="cuda")
    qsa.qsa_merge_lse(po, pl, S, N, 256, merged, mlse)
    internal, ilse = d.decode_attn(sel, cnt, 512, num_splits=S)
    torch.cuda.synchronize()
    sel_np, cnt_np = to_np(sel), to_np(cnt)
    assert np.array_equal(cnt_np[:, 0], [1, 2, 3, 9]) and np.array_equal(cnt_np[:, 1], [1, 2, 3, 9])
    override = {(r, h): (sel_np[r, h], int(cnt_np[r, h])) for r in range(case.R) for h in range(case.Hkv)}
    ref = oracle.run_case(case, splits=S, sel_override=override)
    po, pl = to_np(po), to_np(pl)
    for r in range(case.R):
        n_tok = int(case.lens[r])
        for s_ in range(n_tok, S):  # token p goes to split p mod S: these splits are empty
            assert np.all(po[s_, r] == 0) and np.all(np.isneginf(pl[s_, r])), (r, s_)
        check_close(po[:, r], ref.part_out[r], f"partials row {r}")
        check_lse(pl[:, r], ref.part_lse[r], f"partial lse row {r}")
        for name, o, l in (("merged", merged, mlse), ("internal", internal, ilse)):
            check_close(to_np(o)[r], ref.out[r], f"{name} row {r}")
            check_lse(to_np(l)[r], ref.lse[r], f"{name} lse row {r}")


def test_merge_kernel_against_oracle_with_empty_partials():
    import block_sparse_attention_compress_amd as qsa
    rng = np.random.default_rng(3)
    S, N, D = 5, 37, 512
    po = rng.standard_normal((S, N, D)).astype(np.float32)
    pl = (rng.standard_normal((S, N)) * 3).astype(np.float32)
    pl[1, :10] = -np.inf
    pl[:, 20] = -np.inf                 # a row with no tokens at all
    po[:, 20] = 0
    out = torch.empty((N, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(N, dtype=torch.float32, device="cuda")
    qsa.qsa_merge_lse(torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda(), S, N, D, out, lse)
    ro, rl = oracle.merge(po.astype(np.float64), pl.astype(np.float64))
    check_close(to_np(out), ro, "merge out")
    check_lse(to_np(lse), rl, "merge lse")
    assert np.all(to_np(out)[20] == 0)


@pytest.mark.parametrize("D", [4, 64, 260, 1000])
@pytest.mark.parametrize("S", [2, 17, 64])
def test_merge_kernel_any_width_and_split_count(S, D):
    """Widths that are not a multiple of 256 leave some lanes without dims on the
    last pass; split counts above 16 take several load batches.  Every output must
    still be the oracle's merge."""
    import block_sparse_attention_compress_amd as qsa
    rng = np.random.default_rng(1000 * S + D)
    N = 9
    po = rng.standard_normal((S, N, D)).astype(np.float32)
    pl = (rng.standard_normal((S, N)) * 3).astype(np.float32)
    pl[S - 1, 2] = -np.inf              # an empty last split
    pl[:, 5] = -np.inf                  # a row with no tokens at all
    po[:, 5] = 0
    out = torch.full((N, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
    qsa.qsa_merge_lse(torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda(), S, N, D, out, lse)
    ro, rl = oracle.merge(po.astype(np.float64), pl.astype(np.float64))
    check_close(to_np(out), ro, f"merge out S={S} D={D}")
    check_lse(to_np(lse), rl, f"merge lse S={S} D={D}")
    assert np.all(to_np(out)[5] == 0)


# ------------------------------------------------------------------- extend

def run_extend(case, k=None):
    d = Dev(case)
    d.compress()
    k = case.topk if k is None else k
    sc = d.scores(extend=True)
    sel, cnt = d.topk(sc, k)
    out, lse = d.extend_attn(sel, cnt, k)
    torch.cuda.synchronize()
    return d, to_np(sc), to_np(sel), to_np(cnt), to_np(out), to_np(lse)


def test_extend_strided_query_and_output_rows():
    """Extend with q rows and out rows that are views into wider tensors (row
    strides above Hq * 256): the scores, the selection and the outputs equal the
    oracle's, and the columns past each row are not written."""
    import block_sparse_attention_compress_amd as qsa
    total, nq = 3000, 200
    q_seq, q_pos = synth.extend_rows(total, nq)
    case = synth.make_case("xstride", 515, 12, 1, [total], page_size=64, q_seq=q_seq, q_pos=q_pos)
    d = Dev(case)
    d.compress()
    qbig = torch.zeros((case.R, case.Hq + 4, 256), dtype=torch.bfloat16, device="cuda")
    qbig[:, :case.Hq] = d.t["q"]
    qv = qbig[:, :case.Hq]
    sc = d.scores(extend=True, q=qv)
    sel, cnt = d.topk(sc, case.topk)
    obig = torch.full((case.R, case.Hq + 3, 256), 7.0, dtype=torch.bfloat16, device="cuda")
    ov = obig[:, :case.Hq]
    lse = torch.full((case.R, case.Hq), float("nan"), dtype=torch.float32, device="cuda")
    qsa.qsa_sparse_attn_extend(d.kv, qv, qv.stride(0), d.t["q_seq"], d.t["q_pos"], case.R, case.Hq, sel, cnt,
                               case.topk, 0.0, ov, ov.stride(0), lse)
    torch.cuda.synchronize()
    assert torch.all(obig[:, case.Hq:] == 7.0)
    check_decode_against_oracle(case, d, to_np(sc), to_np(sel), to_np(cnt), to_np(ov), to_np(lse), case.topk)


@pytest.mark.parametrize("Hq,Hkv", [(16, 2), (24, 2), (12, 1), (6, 1), (3, 1)])
@pytest.mark.parametrize("nq", [1, 257])
def test_extend_head_pairs(Hq, Hkv, nq):
    total = 3000
    q_seq, q_pos = synth.extend_rows(total, nq)
    case = synth.make_case(f"ext{Hq}", 500 + Hq + nq, Hq, Hkv, [total], page_size=64, q_seq=q_seq, q_pos=q_pos)
    log(f"extend heads=({Hq},{Hkv}) nq={nq}")
    res = run_extend(case)
    check_decode_against_oracle(case, *res, case.topk)


def test_extend_last_row_equals_decode():
    total, nq = 4099, 64
    q_seq, q_pos = synth.extend_rows(total, nq)
    ext = synth.make_case("extdec", 77, 12, 1, [total], page_size=64, q_seq=q_seq, q_pos=q_pos)
    d, sc, sel, cnt, out, lse = run_extend(ext)
    dec = synth.make_case("extdec", 77, 12, 1, [total], page_size=64)
    dec._q = ext.q[-1:].copy()
    res = run_decode(dec, num_splits=1)
    assert np.array_equal(res[2][0], sel[-1])
    check_close(out[-1], res[4][0], "extend last row vs decode")
