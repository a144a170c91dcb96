"""The seeded generator (published SplitMix64 outputs, distribution, layouts) and the
constants the pages state (closed-form checks of their arithmetic)."""
import os

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "qsa_page_constants.txt")


def page_constants():
    out = {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, rest = line.split("=", 1)
        out[name.strip()] = rest.split("|")[0].strip()
    return out


def test_splitmix64_published_outputs():
    """SplitMix64 started from state 0 yields 0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4,
    0x06C45D188009454F (the published reference sequence)."""
    L = synth.lib()
    assert L.synth_u64(0, 0) == 0xE220A8397B1DCDAF
    assert L.synth_u64(0, 1) == 0x6E789E6AA1B965F4
    assert L.synth_u64(0, 2) == 0x06C45D188009454F


def test_normals_have_unit_moments():
    x = synth.bf16_to_f32(synth.normal_bf16(9, 1, 0, (1 << 18,))).astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    assert abs(np.mean(np.abs(x) > 3) - 0.0027) < 0.001


def test_bf16_rounding_is_nearest_even():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5], np.float32)
    assert list(synth.bf16_to_f32(synth.f32_to_bf16(f))) == [1.0, 1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -2.5]
    for v in f:
        assert synth.lib().synth_bf16_from_float(float(v)) == synth.f32_to_bf16(np.array([v]))[0]


def test_fp8_cache_recipe():
    """An fp8 cache holds the E4M3 codes of the bf16 draws (nearest even, within
    +-448); the logical view the oracle reads is the decoded values, and decoding
    is exact.  Codes checked against the format's closed forms."""
    vals = np.array([1.0, 1.0625, 1.1875, 448.0, 500.0, -1000.0, 2.0 ** -9, 1.5 * 2.0 ** -9, -0.0, 0.0], np.float32)
    codes = synth.bf16_to_e4m3(synth.f32_to_bf16(vals))
    assert list(codes) == [0x38, 0x38, 0x3A, 0x7E, 0x7E, 0xFE, 0x01, 0x02, 0x80, 0x00]
    back = synth.bf16_to_f32(synth.e4m3_to_bf16(codes))
    assert list(back[:8]) == [1.0, 1.0, 1.25, 448.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -8]
    allc = np.arange(256, dtype=np.uint8)
    finite = allc[(allc & 0x7F) != 0x7F]
    assert np.array_equal(synth.bf16_to_e4m3(synth.e4m3_to_bf16(finite)), finite)  # every code round-trips
    c = synth.make_case("f8", 3, 16, 2, [100, 37], page_size=16, kv_dtype="fp8", jitter=True)
    for t in ("k", "v"):
        pool = c.paged_device(t)
        assert pool.dtype == np.uint8
        for i in range(c.B):
            assert np.array_equal(c.gather_logical(synth.e4m3_to_bf16(pool), i), c.logical(t, i))


def test_paged_and_logical_layouts_agree():
    c = synth.config("C2", B=3, L_range=(100, 300))
    pk, pv = c.paged("k"), c.paged("v")
    for i in range(c.B):
        assert np.array_equal(c.gather_logical(pk, i), c.logical("k", i))
        assert np.array_equal(c.gather_logical(pv, i), c.logical("v", i))
    # the shuffled table is a permutation of the pool
    used = np.concatenate([c.block_table[i, :(int(c.lens[i]) + 63) // 64] for i in range(c.B)])
    assert np.array_equal(np.sort(used), np.arange(c.num_pages))


def test_shared_prefix_pages_alias_content():
    c = synth.make_case("sp", 31, 4, 2, [256, 300], page_size=64, shared_prefix_pages=2)
    assert np.array_equal(c.block_table[0, :2], c.block_table[1, :2])
    k0, k1 = c.logical("k", 0), c.logical("k", 1)
    assert np.array_equal(k0[:, :128], k1[:, :128])
    assert not np.array_equal(k0[:, 128:256], k1[:, 128:256])


def test_c3_bias_recipe():
    c = synth.config("C3", B=1, L=4096)
    d, m = c.bias(0)
    assert m.shape == (2, 1024) and int(m[0].sum()) == round(0.01 * 1024)
    np.testing.assert_allclose(np.linalg.norm(d, axis=1), 1, rtol=1e-6)
    k = synth.bf16_to_f32(c.logical("k", 0)).astype(np.float64)
    blocks = k.reshape(2, 1024, 4, 256)
    proj = np.einsum("hbd,hd->hb", blocks.mean(2), d.astype(np.float64))
    assert proj[0][m[0] == 1].mean() > 2.5 and abs(proj[0][m[0] == 0].mean()) < 0.2


def test_page_constants_closed_forms():
    c = page_constants()
    assert int(c["microblock_tokens"]) * int(c["topk_blocks"]) == int(c["approx_positions"])
    # 262144 tokens x 2 KV heads x 256 dims x 2 bytes x (K, V) = 512 MiB
    assert int(c["packed_cap_tokens"]) * 2 * int(c["head_dim"]) * 2 * 2 == int(c["packed_cap_mib"]) << 20
    pairs = [tuple(map(int, p.split(":"))) for p in c["local_head_pairs"].split(",")]
    assert all(hq % hkv == 0 and hq // hkv <= 16 for hq, hkv in pairs)
    hq, hkv = map(int, c["model_heads"].split(":"))
    # four of the local pairs are the model's 24:2 split over 1, 2, 4 or 8 ranks of heads
    assert {(hq // r, max(hkv // r, 1)) for r in (1, 2, 4, 8)} <= set(pairs)
    q, cache, slots = map(int, c["long_prefill"].split(","))
    # 2051 selected slots = 512 full blocks + a 3-token causal tail
    assert slots == int(c["topk_blocks"]) * int(c["microblock_tokens"]) + 3
