"""Pins of the CPU oracle against closed forms, brute force, library routines and
invariants -- never against a retyped copy of its own formulas.

Each test names the oracle step it pins (O1 compress, O2 scores, O3 select,
O4 attend, O5 merge, extend) and the plausible mistake it would catch.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import bf16_to_f32, f32_to_bf16

RNG = np.random.default_rng(1234)


def rand_bf16(shape, scale=1.0, rng=RNG):
    return f32_to_bf16((rng.standard_normal(shape) * scale).astype(np.float32))


def frac_to_f32(x: Fraction) -> np.float32:
    """Round an exact rational to the nearest float32 (ties to even), exactly."""
    if x == 0:
        return np.float32(0.0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    # fix e so that 2^e <= a < 2^(e+1)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - 23)
    q, r = divmod(a, ulp)
    q = int(q)
    if r * 2 > ulp or (r * 2 == ulp and q % 2 == 1):
        q += 1
    return np.float32(sign * float(q * ulp))


# --------------------------------------------------------------------------- O1

def test_o1_mean_is_exact_when_sums_are_exact():
    """For keys with a narrow exponent range the fp32 adds are exact, so the block key
    must equal the exactly rounded mean.  Catches a wrong divisor, a dropped key or a
    wrong block-to-token mapping."""
    L, D = 4 * 37 + 3, 16
    mag = RNG.uniform(0.25, 4.0, size=(L, D)) * RNG.choice([-1.0, 1.0], size=(L, D))
    keys = f32_to_bf16(mag.astype(np.float32))
    kv = bf16_to_f32(keys)
    ck = oracle.compress(keys)
    assert ck.shape == ((L + 3) // 4, D)
    for b in range(ck.shape[0]):
        n = min(4, L - 4 * b)
        for d in range(D):
            exact = sum(Fraction(float(kv[4 * b + u, d])) for u in range(n)) / n
            assert ck[b, d] == frac_to_f32(exact), (b, d, n)


def test_o1_pinned_add_order():
    """Hand-worked cases in which fp32 rounding depends on the add order.
    (a) k = (2^24, 1, 1, 0): the pinned ((k0+k1)+(k2+k3)) rounds 2^24+1 to 2^24 (ties to
        even) twice and gives 2^22, while the exact mean is 2^22 + 0.5.
    (b) k = (1, 1, 2^24, 0): (1+1) + (2^24+0) = 2^24 + 2 is exact, giving 2^22 + 0.5;
        a sum that starts with k2 + k1 would round to 2^24 first.
    (c) k = (2^24, 1, 0, 1): pinned (2^24 + 1 -> 2^24) + (0 + 1) -> 2^24 -> 2^22, while
        pairing k1 with k3 first would give 2^24 + 2 -> 2^22 + 0.5."""
    def ck(vals):
        keys = f32_to_bf16(np.array(vals, dtype=np.float32)[:, None])
        return oracle.compress(keys)[0, 0]

    assert ck([2.0 ** 24, 1.0, 1.0, 0.0]) == np.float32(2.0 ** 22)
    assert ck([1.0, 1.0, 2.0 ** 24, 0.0]) == np.float32(2.0 ** 22 + 0.5)
    assert ck([2.0 ** 24, 1.0, 0.0, 1.0]) == np.float32(2.0 ** 22)
    # a plain fp64 mean would give 2^22 + 0.5 for all three: the pinned order matters
    assert frac_to_f32(Fraction(2 ** 24 + 2, 4)) == np.float32(2.0 ** 22 + 0.5)


def test_o1_special_cases():
    """Four equal keys give that key; zero keys give 0; a 1-key tail is the key itself;
    L = 0 gives no block."""
    D = 8
    k = rand_bf16((1, D))
    keys = np.repeat(k, 4, axis=0)
    assert np.array_equal(oracle.compress(keys)[0], bf16_to_f32(k[0]))
    assert np.all(oracle.compress(np.zeros((8, D), np.uint16)) == 0)
    keys = rand_bf16((5, D))
    assert np.array_equal(oracle.compress(keys)[1], bf16_to_f32(keys[4]))
    assert oracle.compress(np.zeros((0, D), np.uint16)).shape == (0, D)


def test_o1_tail_divisor_three():
    """Tail of 3 keys (1, 1, 1) / 3 must be the float nearest to 1 (not 4/3 from a divisor
    of 4 with the wrong count, not 0.75 from always dividing by 4)."""
    keys = f32_to_bf16(np.array([[5.0], [5.0], [5.0], [5.0], [1.0], [1.0], [1.0]], np.float32))
    ck = oracle.compress(keys)
    assert ck[0, 0] == 5.0 and ck[1, 0] == 1.0
    keys = f32_to_bf16(np.array([[1.0], [2.0], [2.0]], np.float32))
    assert oracle.compress(keys)[0, 0] == frac_to_f32(Fraction(5, 3))


def test_o1c_fp8_block_keys_match_torch_e4m3fn():
    """O1c: within range, the fp8 block key is torch's float32 -> float8_e4m3fn
    conversion (round to nearest, ties to even) of the O1 mean: codes and decoded
    values, signed zeros and subnormal steps included (catches the bias-8 variant,
    truncation, or rounding the keys before the mean)."""
    for L, scale in ((64, 3.0), (61, 0.02), (7, 1.0), (1, 0.004), (4099, 2.0)):
        keys = rand_bf16((L, 256), scale=scale)
        mean = oracle.compress(keys)
        t = torch.from_numpy(mean).to(torch.float8_e4m3fn)
        codes = oracle.compress_fp8_codes(keys)
        assert codes.dtype == np.uint8 and codes.shape == mean.shape
        assert np.array_equal(codes, t.view(torch.uint8).numpy()), (L, scale)
        got = oracle.compress(keys, "fp8")
        assert np.array_equal(got.view(np.uint32), t.to(torch.float32).numpy().view(np.uint32)), (L, scale)


def test_o1c_saturation_ties_and_signed_zero():
    """O1c closed forms: means at or past 448 are held at +-448 (code 0x7E / 0xFE;
    torch would give NaN there); halfway means go to the even code in the normal
    and the subnormal range; the smallest normal 2^-6 is reached by rounding up; an
    all -0 block stays -0 (code 0x80)."""
    def block(vals):
        keys = np.zeros((4, 256), dtype=np.float32)
        keys[:, 0] = vals
        k = f32_to_bf16(keys)
        return oracle.compress_fp8_codes(k)[0, 0], oracle.compress(k, "fp8")[0, 0]

    assert block([1000.0] * 4) == (0x7E, np.float32(448.0))
    assert block([-1.0e4] * 4) == (0xFE, np.float32(-448.0))
    assert block([464.0] * 4) == (0x7E, np.float32(448.0))      # tie between 448 and 480: even code
    assert block([460.0] * 4) == (0x7E, np.float32(448.0))
    assert block([1.0625] * 4) == (0x38, np.float32(1.0))       # tie between 1 and 1.125 -> 1
    assert block([1.1875] * 4) == (0x3A, np.float32(1.25))      # tie between 1.125 and 1.25 -> 1.25
    assert block([1.5 * 2.0 ** -9] * 4) == (0x02, np.float32(2.0 ** -8))   # subnormal tie -> even
    assert block([2.0 ** -10] * 4) == (0x00, np.float32(0.0))              # half the smallest step -> 0
    assert block([0.75 * 2.0 ** -9] * 4) == (0x01, np.float32(2.0 ** -9))
    assert block([2.0 ** -7 * 1.9921875] * 4) == (0x08, np.float32(2.0 ** -6))
    c, v = block([-0.0] * 4)
    assert c == 0x80 and v == 0.0 and np.signbit(v)


# --------------------------------------------------------------------------- O2

def test_o1b_bf16_block_keys_match_torch_rounding():
    """O1b: the bf16 block key is the O1 mean rounded to nearest bf16, ties to even.
    Pinned against torch's own float32 -> bfloat16 conversion (catches truncation
    instead of rounding, or rounding the keys before the mean)."""
    for L in (64, 61, 7, 1):
        keys = rand_bf16((L, 256), scale=3.0)
        mean = oracle.compress(keys)
        want = torch.from_numpy(mean).to(torch.bfloat16).to(torch.float32).numpy()
        got = oracle.compress(keys, "bf16")
        assert got.dtype == np.float32 and got.shape == mean.shape
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), L


def test_o1b_ties_go_to_even_and_exact_means_stay():
    """O1b closed forms: a mean already in bf16 is kept; a mean exactly halfway
    between two bf16 values goes to the one with the even last bit (catches
    round-half-up)."""
    u = 2.0 ** -7  # bf16 spacing on [1, 2)

    def block(vals):
        keys = np.zeros((4, 256), dtype=np.float32)
        keys[:, 0] = vals
        keys[:, 1] = [3.0, 3.0, 3.0, 3.0]
        return oracle.compress(f32_to_bf16(keys), "bf16")[0]

    ck = block([1.0, 1.0, 1.0 + u, 1.0 + u])            # mean 1 + u/2: tie -> 1 (even)
    assert ck[0] == np.float32(1.0) and ck[1] == np.float32(3.0)
    ck = block([1.0 + u, 1.0 + u, 1.0 + 2 * u, 1.0 + 2 * u])  # mean 1 + 3u/2: tie -> 1 + 2u (even)
    assert ck[0] == np.float32(1.0 + 2 * u)
    ck = block([1.0, 1.0, 1.0, 1.0 + u])                 # mean 1 + u/4: below the tie -> 1
    assert ck[0] == np.float32(1.0)
    ck = block([1.0, 1.0 + u, 1.0 + u, 1.0 + u])         # mean 1 + 3u/4: above the tie -> 1 + u
    assert ck[0] == np.float32(1.0 + u)


def test_o2_zero_query_and_unit_query():
    """Zero q gives all-zero scores; q = e_d in one head of the group gives the d-th
    component of each block key.  Catches a transposed operand or a scale applied."""
    g, D, nb = 3, 16, 11
    ck = bf16_to_f32(rand_bf16((nb, D))).astype(np.float32)
    assert np.all(oracle.scores(np.zeros((g, D), np.uint16), ck, nb) == 0)
    for d in (0, 7, 15):
        q = np.zeros((g, D), np.float32)
        q[1, d] = 1.0
        s = oracle.scores(f32_to_bf16(q), ck, nb)
        assert np.array_equal(s, ck[:, d].astype(np.float64))


def test_o2_brute_force_exact_with_error_bound():
    """Exact rational score (sum over heads, then dot product) versus the fp64 oracle,
    within the Higham bound gamma_n * sum |qsum_d ckey_d| with u = 2^-53."""
    g, D, nb = 4, 32, 9
    q = rand_bf16((g, D))
    ck = (RNG.standard_normal((nb, D)) * 0.5).astype(np.float32)
    s = oracle.scores(q, ck, nb)
    qv = bf16_to_f32(q)
    u = 2.0 ** -53
    n = D + g
    gamma = n * u / (1 - n * u)
    for b in range(nb):
        qs = [sum(Fraction(float(qv[j, d])) for j in range(g)) for d in range(D)]
        exact = sum(qs[d] * Fraction(float(ck[b, d])) for d in range(D))
        bound = gamma * float(sum(abs(qs[d] * Fraction(float(ck[b, d]))) for d in range(D)))
        assert abs(s[b] - float(exact)) <= bound + 1e-300


def test_o2_group_mapping_is_contiguous():
    """Query head j scores KV head j // g: with only head 3 nonzero (g = 4), KV head 0 sees
    it and KV head 1 sees zeros.  Catches j % Hkv grouping."""
    case = synth.make_case("grp", 11, 8, 2, [64], page_size=64, topk=4)
    q = np.zeros((1, 8, 256), np.uint16)
    q[0, 3] = rand_bf16((256,))
    case._q = q
    res = oracle.run_case(case)
    assert np.any(res.scores[(0, 0)] != 0)
    assert np.all(res.scores[(0, 1)] == 0)


# --------------------------------------------------------------------------- O3

def brute_topk(s, k):
    n = len(s)
    sel = []
    for b in range(n):
        ahead = sum(1 for c in range(n) if s[c] > s[b] or (s[c] == s[b] and c < b))
        if ahead < k:
            sel.append(b)
    return sel


@pytest.mark.parametrize("n,k", [(0, 3), (1, 1), (5, 9), (40, 7), (64, 64), (97, 16), (200, 512)])
def test_o3_matches_rank_count_definition(n, k):
    """Selection equals the rank-count definition (b kept iff fewer than k blocks come
    before it in (score desc, index asc)); heavy ties from a small integer range."""
    s = RNG.integers(-3, 4, size=n).astype(np.float64)
    sel, cnt = oracle.topk(s, k)
    want = brute_topk(list(s), k)
    assert cnt == len(want) == min(n, k)
    assert list(sel[:cnt]) == want
    assert np.all(sel[cnt:] == -1)


def test_o3_invariants_and_special_cases():
    s = RNG.standard_normal(1000)
    sel, cnt = oracle.topk(s, 512)
    chosen = sel[:cnt]
    assert cnt == 512 and np.all(np.diff(chosen) > 0)
    rest = np.setdiff1d(np.arange(1000), chosen)
    assert s[chosen].min() >= s[rest].max()
    # zero scores: the tie-break keeps blocks 0..k-1
    sel, cnt = oracle.topk(np.zeros(3000), 512)
    assert np.array_equal(sel, np.arange(512))
    # -0 and +0 tie: the lower index wins
    sel, cnt = oracle.topk(np.array([-0.0, 0.0]), 1)
    assert sel[0] == 0
    sel, cnt = oracle.topk(np.array([0.0, -0.0, 1e-300]), 2)
    assert list(sel) == [0, 2]
    sel, cnt = oracle.topk(np.arange(10.0), 0)
    assert cnt == 0 and sel.shape == (0,)


# --------------------------------------------------------------------------- O4

def sdpa_f64(q, K, V, scale):
    """torch's textbook attention in float64 on the CPU: q [g][D], K/V [T][D]."""
    qt = torch.from_numpy(q)[None, :, None, :]          # [1, g, 1, D]
    kt = torch.from_numpy(K)[None, None].expand(1, q.shape[0], -1, -1)
    vt = torch.from_numpy(V)[None, None].expand(1, q.shape[0], -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    return o[0, :, 0, :].numpy()


@pytest.mark.parametrize("L", [1, 2, 3, 4, 61, 62, 63, 64, 65, 257])
def test_o4_dense_special_case_matches_sdpa(L):
    """With k >= number of blocks the method is plain softmax attention over all L tokens."""
    g, D = 3, 256
    q = rand_bf16((g, D))
    K = rand_bf16((L, D))
    V = rand_bf16((L, D))
    nb = (L + 3) // 4
    sel = np.arange(nb, dtype=np.int32)
    out, lse = oracle.attend(q, K, V, L - 1, sel, nb, 1 / 16)
    want = sdpa_f64(bf16_to_f32(q).astype(np.float64), bf16_to_f32(K).astype(np.float64),
                    bf16_to_f32(V).astype(np.float64), 1 / 16)
    np.testing.assert_allclose(out, want, rtol=1e-10, atol=1e-12)
    x = (bf16_to_f32(q).astype(np.float64) @ bf16_to_f32(K).astype(np.float64).T) / 16
    np.testing.assert_allclose(lse, np.log(np.exp(x).sum(axis=1)), rtol=1e-12)


def test_o4_causal_row_matches_sdpa_prefix():
    """An extend row at position t attends exactly to tokens 0..t of its blocks."""
    g, D, L = 2, 256, 50
    q = rand_bf16((g, D))
    K, V = rand_bf16((L, D)), rand_bf16((L, D))
    for t in (0, 1, 2, 3, 4, 21, 48, 49):
        nb = t // 4 + 1
        out, _ = oracle.attend(q, K, V, t, np.arange(nb, dtype=np.int32), nb, 0.07)
        f = lambda a: bf16_to_f32(a).astype(np.float64)
        want = sdpa_f64(f(q), f(K[:t + 1]), f(V[:t + 1]), 0.07)
        np.testing.assert_allclose(out, want, rtol=1e-10, atol=1e-12)


def test_o4_layout_identity_of_the_ascend_adapter():
    """With C = [K, V] (head dim 512) used as keys and values and Q' = [Q, 0], the scale
    kept at 1/16, softmax(scale Q' C^T) C stacks P K and P V ("Qwen4-Exp QSA komt naar
    Huawei's Ascend", section "Wat de pull request daadwerkelijk toevoegt")."""
    g, D, L = 4, 256, 203
    q, K, V = rand_bf16((g, D)), rand_bf16((L, D)), rand_bf16((L, D))
    C = np.concatenate([K, V], axis=1)
    qp = np.concatenate([q, np.zeros_like(q)], axis=1)
    sel = np.array([0, 3, 7, 20, 33, 50], dtype=np.int32)
    big, lse_big = oracle.attend(qp, C, C, L - 1, sel, len(sel), 1 / 16)
    pk, lse_k = oracle.attend(q, K, K, L - 1, sel, len(sel), 1 / 16)
    pv, lse_v = oracle.attend(q, K, V, L - 1, sel, len(sel), 1 / 16)
    np.testing.assert_allclose(big[:, :D], pk, atol=1e-12, rtol=0)
    np.testing.assert_allclose(big[:, D:], pv, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse_big, lse_v, atol=1e-12, rtol=0)


def test_o4_tiny_brute_force():
    """Tiny inputs, every k: direct exp-sum formula (no max shift) over the selected tokens."""
    rng = np.random.default_rng(7)
    for trial in range(40):
        L = int(rng.integers(1, 17))
        D = int(rng.integers(1, 9))
        g = int(rng.integers(1, 4))
        q, K, V = rand_bf16((g, D), rng=rng), rand_bf16((L, D), rng=rng), rand_bf16((L, D), rng=rng)
        nb = (L + 3) // 4
        t = int(rng.integers(0, L))
        elig = t // 4 + 1
        for k in range(0, nb + 1):
            sel = np.sort(rng.choice(elig, size=min(k, elig), replace=False)).astype(np.int32)
            out, lse = oracle.attend(q, K, V, t, sel, len(sel), 0.3)
            toks = [4 * b + u for b in sel for u in range(4) if 4 * b + u < L and 4 * b + u <= t]
            qf, kf, vf = (bf16_to_f32(a).astype(float) for a in (q, K, V))
            for h in range(g):
                if not toks:
                    assert np.all(out[h] == 0) and lse[h] == -np.inf
                    continue
                w = [math.exp(0.3 * sum(qf[h, d] * kf[p, d] for d in range(D))) for p in toks]
                z = sum(w)
                for d in range(D):
                    ref = sum(wi * vf[p, d] for wi, p in zip(w, toks)) / z
                    assert abs(out[h, d] - ref) <= 1e-12 * (1 + abs(ref))
                assert abs(lse[h] - math.log(z)) <= 1e-12 * (1 + abs(math.log(z)))


def test_o4_metamorphic():
    """K + w leaves the output unchanged; V + w shifts it by w; one token gives its v;
    identical keys give the mean of V over the selected tokens.  Values on a 1/8 grid
    keep K + w and V + w exact in bf16."""
    g, D, L = 2, 64, 40
    rng = np.random.default_rng(3)
    grid = lambda shape: f32_to_bf16(np.clip(np.round(rng.standard_normal(shape) * 8) / 8, -4, 4).astype(np.float32))
    q, K, V = grid((g, D)), grid((L, D)), grid((L, D))
    w = np.clip(np.round(rng.standard_normal(D) * 8) / 8, -2, 2).astype(np.float32)
    Kw = f32_to_bf16(bf16_to_f32(K) + w)
    Vw = f32_to_bf16(bf16_to_f32(V) + w)
    assert np.array_equal(bf16_to_f32(Kw) - bf16_to_f32(K), np.broadcast_to(w, K.shape))
    assert np.array_equal(bf16_to_f32(Vw) - bf16_to_f32(V), np.broadcast_to(w, V.shape))
    sel = np.array([1, 4, 9], dtype=np.int32)
    base, lse0 = oracle.attend(q, K, V, L - 1, sel, 3, 1 / 16)
    o_k, _ = oracle.attend(q, Kw, V, L - 1, sel, 3, 1 / 16)
    np.testing.assert_allclose(o_k, base, atol=1e-12)
    o_v, lse_v = oracle.attend(q, K, Vw, L - 1, sel, 3, 1 / 16)
    np.testing.assert_allclose(o_v, base + w, atol=1e-12)
    np.testing.assert_array_equal(lse_v, lse0)
    # one token: L = 1
    o1, _ = oracle.attend(q, K[:1], V[:1], 0, np.array([0], np.int32), 1, 1 / 16)
    np.testing.assert_array_equal(o1, np.broadcast_to(bf16_to_f32(V[0]).astype(float), (g, D)))
    # identical keys: uniform weights -> mean of V over the tokens
    Ksame = np.repeat(K[:1], L, axis=0)
    o_s, _ = oracle.attend(q, Ksame, V, L - 1, sel, 3, 1 / 16)
    toks = [4 * b + u for b in sel for u in range(4)]
    np.testing.assert_allclose(o_s, np.broadcast_to(bf16_to_f32(V[toks]).astype(float).mean(0), (g, D)),
                               atol=1e-13)


def test_o4_empty_selection():
    g, D, L = 3, 256, 10
    q, K, V = rand_bf16((g, D)), rand_bf16((L, D)), rand_bf16((L, D))
    out, lse = oracle.attend(q, K, V, L - 1, np.zeros(0, np.int32), 0, 1 / 16)
    assert np.all(out == 0) and np.all(lse == -np.inf)
    # a selected block that starts after t contributes nothing
    out, lse = oracle.attend(q, K, V, 3, np.array([1], np.int32), 1, 1 / 16)
    assert np.all(out == 0) and np.all(lse == -np.inf)


# --------------------------------------------------------------------------- O5

@pytest.mark.parametrize("S", [1, 2, 3, 4, 7])
def test_o5_any_partition_merges_to_unsplit(S):
    g, D, L = 4, 256, 183
    q, K, V = rand_bf16((g, D)), rand_bf16((L, D)), rand_bf16((L, D))
    sel = np.sort(RNG.choice(46, size=20, replace=False)).astype(np.int32)
    full, lse_full = oracle.attend(q, K, V, L - 1, sel, 20, 1 / 16)
    po = np.empty((S, g, D))
    pl = np.empty((S, g))
    for s in range(S):
        po[s], pl[s] = oracle.attend(q, K, V, L - 1, sel, 20, 1 / 16, S, s)
    out, lse = oracle.merge(po, pl)
    np.testing.assert_allclose(out, full, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, lse_full, atol=1e-12, rtol=0)
    if S == 1:
        np.testing.assert_array_equal(po[0], full)


def test_o5_empty_partials():
    N, D = 3, 8
    o = RNG.standard_normal((1, N, D))
    l = RNG.standard_normal((1, N))
    po = np.concatenate([o, np.zeros((2, N, D))])
    pl = np.concatenate([l, np.full((2, N), -np.inf)])
    out, lse = oracle.merge(po, pl)
    np.testing.assert_allclose(out, o[0], atol=1e-15)
    np.testing.assert_allclose(lse, l[0], atol=1e-15)
    out, lse = oracle.merge(np.zeros((4, N, D)), np.full((4, N), -np.inf))
    assert np.all(out == 0) and np.all(lse == -np.inf)
    # two equal partials with equal lse: average, lse + ln 2
    out, lse = oracle.merge(np.stack([o[0], 3 * o[0]]), np.stack([l[0], l[0]]))
    np.testing.assert_allclose(out, 2 * o[0], atol=1e-14)
    np.testing.assert_allclose(lse, l[0] + math.log(2), atol=1e-14)


def test_o5_interleaved_split_of_full_blocks_takes_one_token_per_block():
    """With S = 4 and full blocks, split s holds exactly token 4b + s of every block."""
    g, D, L = 1, 8, 64
    q = np.zeros((g, D), np.uint16)          # uniform weights: output = mean of the split's V
    K = rand_bf16((L, D))
    V = f32_to_bf16(np.arange(L, dtype=np.float32)[:, None].repeat(D, 1))
    sel = np.array([2, 5, 11], np.int32)
    for s in range(4):
        out, _ = oracle.attend(q, K, V, L - 1, sel, 3, 1.0, 4, s)
        np.testing.assert_allclose(out[0], np.mean([4 * b + s for b in sel]), atol=1e-12)


# ---------------------------------------------------------------------- extend

def test_extend_last_row_equals_decode_and_future_is_masked():
    total, new = 300, 40
    ext = synth.make_case("ext", 21, 6, 2, [total], page_size=32, q_seq=np.zeros(new, np.int32),
                          q_pos=np.arange(total - new, total, dtype=np.int32), topk=16)
    dec = synth.make_case("ext", 21, 6, 2, [total], page_size=32, topk=16)
    dec._q = ext.q[-1:].copy()
    r_ext = oracle.run_case(ext)
    r_dec = oracle.run_case(dec)
    np.testing.assert_array_equal(r_ext.out[new - 1], r_dec.out[0])
    for h in range(2):
        assert np.array_equal(r_ext.sel[(new - 1, h)], r_dec.sel[(0, h)])
    # changing K and V after a row's position leaves the row unchanged (selection uses
    # block keys built from the cache as it is, so only V after t is changed here; the
    # block holding t keeps its keys)
    data = oracle.CaseData(ext)
    r = 5
    t = int(ext.q_pos[r])
    Vmod = data.V(0).copy()
    Vmod[:, t + 1:] = rand_bf16(Vmod[:, t + 1:].shape)
    data._v[0] = Vmod
    r_mod = oracle.run_case(ext, rows=[r], data=data)
    np.testing.assert_array_equal(r_mod.out[r], r_ext.out[r])


def test_step_selection_invariant_under_key_shift():
    """Adding the same vector to every key shifts every block score by the same amount,
    so the selection is unchanged (scores compared in exact arithmetic)."""
    g, D, L = 2, 16, 64
    q = rand_bf16((g, D))
    K = f32_to_bf16((np.round(RNG.standard_normal((L, D)) * 8) / 8).astype(np.float32))
    Kw = f32_to_bf16(bf16_to_f32(K) + np.float32(0.125))
    s0 = oracle.scores(q, oracle.compress(K), 16)
    s1 = oracle.scores(q, oracle.compress(Kw), 16)
    shift = s1 - s0
    np.testing.assert_allclose(shift, shift[0], atol=1e-12)
    assert np.array_equal(oracle.topk(s0, 5)[0], oracle.topk(s1, 5)[0])
