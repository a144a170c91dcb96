"""The C ABI without a GPU: the library loads, exports every declared entry point,
and rejects bad arguments on the host before launching anything."""
import ctypes
import os
import re

import pytest

import block_sparse_attention_compress_amd as qsa

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "qsa.h")

# fake but well-aligned device addresses: validation never dereferences them and a
# rejected call launches nothing
P = 0x10000


def declared():
    text = open(HEADER).read()
    return re.findall(r"QSA_API\s+[\w\s\*]+?\b(qsa_\w+)\s*\(", text)


def kv(**over):
    f = dict(k=P, v=P, ckey=P, block_table=P, seq_lens=P, batch=2, num_kv_heads=2, head_dim=256, page_size=64,
             num_pages=100, max_pages_per_seq=50, max_seq_len=3200)
    f.update(over)
    return qsa.qsa_kv_t(**f)


def status(fn, *args):
    return getattr(qsa.lib(), fn)(*args)


def test_every_declared_symbol_is_exported():
    names = declared()
    assert set(names) == set(qsa.EXPORTS)
    lib = ctypes.CDLL(qsa.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert qsa.qsa_version() >= 100


def test_header_constants_match_binding():
    text = open(HEADER).read()
    consts = dict(re.findall(r"#define (QSA_\w+) \(?(-?\d+)", text))
    assert int(consts["QSA_HEAD_DIM"]) == qsa.HEAD_DIM == 256
    assert int(consts["QSA_MICROBLOCK"]) == qsa.MICROBLOCK == 4
    assert int(consts["QSA_DEFAULT_TOPK"]) == qsa.DEFAULT_TOPK == 512
    assert int(consts["QSA_MAX_TOPK"]) == qsa.MAX_TOPK
    assert int(consts["QSA_ERR_INVALID_ARG"]) == qsa.QSA_ERR_INVALID_ARG
    assert int(consts["QSA_CKEY_FP32"]) == qsa.CKEY_FP32 == 0
    assert int(consts["QSA_CKEY_BF16"]) == qsa.CKEY_BF16
    assert int(consts["QSA_CKEY_FP8"]) == qsa.CKEY_FP8 == 2
    assert int(consts["QSA_KV_BF16"]) == qsa.KV_BF16 == 0 and int(consts["QSA_KV_FP8"]) == qsa.KV_FP8 == 1


@pytest.mark.parametrize("over,code", [
    (dict(k=None), qsa.QSA_ERR_INVALID_ARG),
    (dict(ckey=None), qsa.QSA_ERR_INVALID_ARG),
    (dict(block_table=None), qsa.QSA_ERR_INVALID_ARG),
    (dict(head_dim=128), qsa.QSA_ERR_UNSUPPORTED),
    (dict(page_size=48), qsa.QSA_ERR_INVALID_ARG),
    (dict(page_size=2), qsa.QSA_ERR_INVALID_ARG),
    (dict(max_seq_len=(1 << 20) + 1, max_pages_per_seq=20000), qsa.QSA_ERR_UNSUPPORTED),
    (dict(max_pages_per_seq=10), qsa.QSA_ERR_INVALID_ARG),      # 10 * 64 < 3200
    (dict(num_pages=1 << 24), qsa.QSA_ERR_UNSUPPORTED),          # 2^24 pages x 2 heads x 64 rows = 2^31
    (dict(k=P + 8), qsa.QSA_ERR_INVALID_ARG),                    # misaligned
    (dict(batch=-1), qsa.QSA_ERR_INVALID_ARG),
    (dict(ckey_dtype=3), qsa.QSA_ERR_INVALID_ARG),
    (dict(ckey_dtype=-1), qsa.QSA_ERR_INVALID_ARG),
    (dict(kv_dtype=2), qsa.QSA_ERR_INVALID_ARG),
    (dict(kv_dtype=-1), qsa.QSA_ERR_INVALID_ARG),
])
def test_compress_rejects(over, code):
    d = kv(**over)
    assert status("qsa_compress_keys", ctypes.byref(d), None, 0, None) == code
    assert qsa.qsa_last_error() != ""


def test_scores_rejects_null_q():
    d = kv()
    assert status("qsa_block_scores", ctypes.byref(d), None, 4096, None, None, 2, 8, P, 800, None) == \
        qsa.QSA_ERR_INVALID_ARG


def test_scores_head_and_stride_checks():
    d = kv()
    L = "qsa_block_scores"
    # Hq not a multiple of Hkv
    assert status(L, ctypes.byref(d), P, 2048, None, None, 2, 7, P, 800, None) == qsa.QSA_ERR_UNSUPPORTED
    # group of 18 > 16
    assert status(L, ctypes.byref(d), P, 36 * 256, None, None, 2, 36, P, 800, None) == qsa.QSA_ERR_UNSUPPORTED
    # row stride below Hq * 256, or not a multiple of 8
    assert status(L, ctypes.byref(d), P, 1000, None, None, 2, 8, P, 800, None) == qsa.QSA_ERR_INVALID_ARG
    assert status(L, ctypes.byref(d), P, 2052, None, None, 2, 8, P, 800, None) == qsa.QSA_ERR_INVALID_ARG
    # decode mode needs R == batch
    assert status(L, ctypes.byref(d), P, 2048, None, None, 3, 8, P, 800, None) == qsa.QSA_ERR_INVALID_ARG
    # q_seq without q_pos
    assert status(L, ctypes.byref(d), P, 2048, P, None, 2, 8, P, 800, None) == qsa.QSA_ERR_INVALID_ARG
    # score_stride out of range
    assert status(L, ctypes.byref(d), P, 2048, None, None, 2, 8, P, 0, None) == qsa.QSA_ERR_INVALID_ARG
    assert status(L, ctypes.byref(d), P, 2048, None, None, 2, 8, P, (1 << 18) + 1, None) == qsa.QSA_ERR_INVALID_ARG


def test_decode_scores_refresh_rejects():
    f = qsa.lib().qsa_decode_scores_refresh
    d = kv()
    assert f(ctypes.byref(d), None, 4096, 16, P, 800, None) == qsa.QSA_ERR_INVALID_ARG     # q
    assert f(ctypes.byref(d), P, 4096, 16, None, 800, None) == qsa.QSA_ERR_INVALID_ARG     # scores
    assert f(ctypes.byref(d), P, 4096, 16, P, 0, None) == qsa.QSA_ERR_INVALID_ARG         # stride
    assert f(ctypes.byref(d), P, 4096, 15, P, 800, None) == qsa.QSA_ERR_UNSUPPORTED       # Hq % Hkv
    dk = kv(k=None)                                                                       # K is read
    assert f(ctypes.byref(dk), P, 4096, 16, P, 800, None) == qsa.QSA_ERR_INVALID_ARG
    dc = kv(ckey=None)
    assert f(ctypes.byref(dc), P, 4096, 16, P, 800, None) == qsa.QSA_ERR_INVALID_ARG


def test_topk_rejects():
    L = "qsa_topk_blocks"
    assert status(L, None, 100, None, 2, 2, 16, P, P, None) == qsa.QSA_ERR_INVALID_ARG
    assert status(L, P, 100, None, 2, 2, 2049, P, P, None) == qsa.QSA_ERR_INVALID_ARG
    assert status(L, P, 100, None, 2, 2, -1, P, P, None) == qsa.QSA_ERR_INVALID_ARG
    assert status(L, P, 100, None, 2, 2, 16, None, P, None) == qsa.QSA_ERR_INVALID_ARG
    assert status(L, P, 100, None, 2, 2, 16, P, None, None) == qsa.QSA_ERR_INVALID_ARG
    assert status(L, P, 100, None, 2, 0, 16, P, P, None) == qsa.QSA_ERR_INVALID_ARG


def test_last_error_is_per_thread():
    """qsa_last_error() belongs to the calling thread: another thread's failure
    does not show in it, and a thread that made no failed call reads ""."""
    import threading
    L = qsa.lib()
    seen = {}

    def fail_here():
        seen["rc"] = L.qsa_topk_blocks(P, 100, None, 2, 2, 2049, P, P, None)
        seen["msg"] = L.qsa_last_error().decode()

    def look_only():
        seen["other"] = L.qsa_last_error().decode()

    t = threading.Thread(target=fail_here)
    t.start()
    t.join()
    t = threading.Thread(target=look_only)
    t.start()
    t.join()
    assert seen["rc"] == qsa.QSA_ERR_INVALID_ARG and "2049" in seen["msg"]
    assert seen["other"] == ""


def test_topk_ws_rejects_and_sizes():
    """The two-stage select: same argument checks as the one-stage call, plus the
    candidate workspace (two arrays of ceil(stride / 8192) * k entries per row and
    KV head, each rounded up to 256 bytes); rows of up to 16,384 blocks need none."""
    W = qsa.qsa_topk_workspace_bytes
    assert W(4, 2, 512, 16384) == 0
    assert W(4, 2, 0, 65536) == 0
    assert W(0, 2, 512, 65536) == 0
    assert W(4, 2, 2049, 65536) == 0 and W(4, 2, 512, (1 << 18) + 1) == 0
    assert W(1, 1, 512, 16385) == 2 * 6144
    assert W(8, 2, 512, 65536) == 2 * 16 * 8 * 512 * 4
    assert W(3, 1, 17, 20001) == 2 * ((3 * 3 * 17 * 4 + 255) // 256 * 256)
    L = "qsa_topk_blocks_ws"
    need = W(2, 2, 512, 65536)
    assert status(L, P, 65536, None, 2, 2, 512, P, P, None, need, None) == qsa.QSA_ERR_INVALID_ARG
    assert status(L, P, 65536, None, 2, 2, 512, P, P, P, need - 1, None) == qsa.QSA_ERR_INVALID_ARG
    assert status(L, P, 65536, None, 2, 2, 512, P, P, P + 4, need, None) == qsa.QSA_ERR_INVALID_ARG
    assert status(L, None, 65536, None, 2, 2, 512, P, P, P, need, None) == qsa.QSA_ERR_INVALID_ARG
    assert status(L, P, 65536, None, 2, 2, 2049, P, P, P, need, None) == qsa.QSA_ERR_INVALID_ARG
    assert status(L, P, 65536, None, 2, 0, 512, P, P, P, need, None) == qsa.QSA_ERR_INVALID_ARG
    assert status(L, P, 65536, None, 2, 2, 512, None, P, P, need, None) == qsa.QSA_ERR_INVALID_ARG


def test_decode_rejects():
    d = kv()
    f = qsa.lib().qsa_sparse_attn_decode
    base = [ctypes.byref(d), P, 4096, 16, P, P, 512, 0.0, 0, P, 4096, P, None, None, P, 1 << 30, None]

    def call(**ch):
        a = list(base)
        names = ["kv", "q", "qs", "Hq", "sel", "cnt", "k", "scale", "S", "out", "os", "lse", "po", "pl", "ws", "wb", "st"]
        for n, v in ch.items():
            a[names.index(n)] = v
        return f(*a)

    assert call(k=4096) == qsa.QSA_ERR_INVALID_ARG
    assert call(S=65) == qsa.QSA_ERR_INVALID_ARG
    assert call(cnt=None) == qsa.QSA_ERR_INVALID_ARG
    assert call(out=None) == qsa.QSA_ERR_INVALID_ARG
    assert call(os=100) == qsa.QSA_ERR_INVALID_ARG
    assert call(po=P, S=0) == qsa.QSA_ERR_INVALID_ARG          # partials need S >= 1
    assert call(po=P, pl=None, S=4) == qsa.QSA_ERR_INVALID_ARG
    assert call(ws=None, S=4) == qsa.QSA_ERR_INVALID_ARG        # split merge needs a workspace
    assert call(wb=16, S=4) == qsa.QSA_ERR_INVALID_ARG
    assert call(os=8192, S=4) == qsa.QSA_ERR_UNSUPPORTED        # split merge writes dense rows
    dv = kv(v=None)
    assert f(ctypes.byref(dv), *base[1:]) == qsa.QSA_ERR_INVALID_ARG


def test_extend_and_merge_reject():
    d = kv()
    f = qsa.lib().qsa_sparse_attn_extend
    assert f(ctypes.byref(d), P, 4096, None, P, 10, 16, P, P, 512, 0.0, P, 4096, None, None) == qsa.QSA_ERR_INVALID_ARG
    assert f(ctypes.byref(d), P, 4096, P, P, -1, 16, P, P, 512, 0.0, P, 4096, None, None) == qsa.QSA_ERR_INVALID_ARG
    assert f(ctypes.byref(d), P, 4096, P, P, 10, 48, P, P, 512, 0.0, P, 48 * 256, None, None) == qsa.QSA_ERR_UNSUPPORTED
    u = qsa.lib().qsa_sparse_attn_extend_union  # same argument checks, all before any launch
    assert u(ctypes.byref(d), P, 4096, None, P, 10, 16, P, P, 512, 0.0, P, 4096, None, None) == qsa.QSA_ERR_INVALID_ARG
    assert u(ctypes.byref(d), P, 4096, P, P, -1, 16, P, P, 512, 0.0, P, 4096, None, None) == qsa.QSA_ERR_INVALID_ARG
    assert u(ctypes.byref(d), P, 4096, P, P, 10, 48, P, P, 512, 0.0, P, 48 * 256, None, None) == qsa.QSA_ERR_UNSUPPORTED
    assert u(ctypes.byref(d), P, 4096, P, P, 10, 16, P, P, 4096, 0.0, P, 4096, None, None) == qsa.QSA_ERR_INVALID_ARG
    assert u(ctypes.byref(d), P, 4096, P, P, 10, 16, P, P, 512, 0.0, None, 4096, None, None) == qsa.QSA_ERR_INVALID_ARG
    assert u(ctypes.byref(d), P, 4096, P, P, 10, 16, P, P, 512, 0.0, P, 1024, None, None) == qsa.QSA_ERR_INVALID_ARG
    assert "out_row_stride" in qsa.qsa_last_error()
    m = qsa.lib().qsa_merge_lse
    assert m(P, P, 0, 10, 256, P, None, None) == qsa.QSA_ERR_INVALID_ARG
    assert m(P, P, 65, 10, 256, P, None, None) == qsa.QSA_ERR_INVALID_ARG
    assert m(P, P, 4, 10, 250, P, None, None) == qsa.QSA_ERR_UNSUPPORTED
    assert m(P, P, 4, 10, 2048, P, None, None) == qsa.QSA_ERR_UNSUPPORTED
    assert m(None, P, 4, 10, 256, P, None, None) == qsa.QSA_ERR_INVALID_ARG


def test_extend_split_rejects():
    d = kv()
    f = qsa.lib().qsa_sparse_attn_extend_split
    R, Hq = 10, 16
    wsb = qsa.qsa_extend_workspace_bytes(R, Hq, 4)
    assert wsb == qsa.qsa_decode_workspace_bytes(R, Hq, 4) > 0
    base = [ctypes.byref(d), P, 4096, P, P, R, Hq, P, P, 512, 0.0, 4, P, Hq * 256, None, P, wsb, None]
    names = ["kv", "q", "qs", "qseq", "qpos", "R", "Hq", "sel", "cnt", "k", "scale", "S", "out", "os", "lse", "ws",
             "wb", "st"]

    def call(**ch):
        a = list(base)
        for n, v in ch.items():
            a[names.index(n)] = v
        return f(*a)

    assert call(qseq=None) == qsa.QSA_ERR_INVALID_ARG
    assert call(qpos=None) == qsa.QSA_ERR_INVALID_ARG
    assert call(R=-1) == qsa.QSA_ERR_INVALID_ARG
    assert call(Hq=48, os=48 * 256) == qsa.QSA_ERR_UNSUPPORTED     # g = 24 > 16
    assert call(k=2049) == qsa.QSA_ERR_INVALID_ARG
    assert call(cnt=None) == qsa.QSA_ERR_INVALID_ARG
    assert call(S=-1) == qsa.QSA_ERR_INVALID_ARG
    assert call(S=65) == qsa.QSA_ERR_INVALID_ARG
    assert call(out=None) == qsa.QSA_ERR_INVALID_ARG
    assert call(os=100) == qsa.QSA_ERR_INVALID_ARG
    assert call(ws=None) == qsa.QSA_ERR_INVALID_ARG                 # a split read needs a workspace
    assert call(wb=wsb - 1) == qsa.QSA_ERR_INVALID_ARG
    assert call(ws=P + 16) == qsa.QSA_ERR_INVALID_ARG               # 256-byte aligned
    assert call(os=Hq * 256 + 8) == qsa.QSA_ERR_UNSUPPORTED         # a split read writes dense rows
    assert call(S=0, ws=None) == qsa.QSA_ERR_INVALID_ARG            # 20 (row, KV head) units: the library splits
    assert "workspace" in qsa.qsa_last_error()
    big = 1 << 27                                                   # 2^27 rows x 16 heads: 2^31 merged rows
    assert call(R=big, S=2, wb=1 << 62) == qsa.QSA_ERR_UNSUPPORTED
    assert "merged rows" in qsa.qsa_last_error()
    dv = kv(v=None)
    assert f(ctypes.byref(dv), *base[1:]) == qsa.QSA_ERR_INVALID_ARG
    # sizes: none for one split or bad arguments; num_splits = 0 covers any split count the library picks
    assert qsa.qsa_extend_workspace_bytes(R, Hq, 1) == 0
    assert qsa.qsa_extend_workspace_bytes(R, Hq, 65) == 0
    assert qsa.qsa_extend_workspace_bytes(0, Hq, 4) == 0
    assert qsa.qsa_extend_workspace_bytes(R, Hq, 0) == qsa.qsa_extend_workspace_bytes(R, Hq, 16)


def test_workspace_size_formula():
    # S partials of [B][Hq][256] fp32 plus [B][Hq] lse, each rounded up to 256 bytes
    S, B, Hq = 4, 3, 6
    n = S * B * Hq
    want = ((n * 256 * 4 + 255) // 256) * 256 + ((n * 4 + 255) // 256) * 256
    assert qsa.qsa_decode_workspace_bytes(B, Hq, S) == want
    assert qsa.qsa_decode_workspace_bytes(B, Hq, 1) == 0
    assert qsa.qsa_decode_workspace_bytes(B, Hq, 0) >= qsa.qsa_decode_workspace_bytes(B, Hq, 16)


def test_fused_rejects():
    d = kv()
    f = qsa.lib().qsa_decode_fused
    wsb = qsa.qsa_decode_fused_workspace_bytes(d, 16, 512, 0)
    assert wsb > 0
    base = [ctypes.byref(d), P, 4096, 16, 512, 0.0, 0, P, P, P, 4096, P, P, wsb, None]
    names = ["kv", "q", "qs", "Hq", "k", "scale", "S", "sel", "cnt", "out", "os", "lse", "ws", "wb", "st"]

    def call(**ch):
        a = list(base)
        for n, v in ch.items():
            a[names.index(n)] = v
        return f(*a)

    assert call(k=2049) == qsa.QSA_ERR_INVALID_ARG
    assert call(k=-1) == qsa.QSA_ERR_INVALID_ARG
    assert call(S=65) == qsa.QSA_ERR_INVALID_ARG
    assert call(S=-1) == qsa.QSA_ERR_INVALID_ARG
    assert call(sel=None) == qsa.QSA_ERR_INVALID_ARG
    assert call(cnt=None) == qsa.QSA_ERR_INVALID_ARG
    assert call(out=None) == qsa.QSA_ERR_INVALID_ARG
    assert call(out=P + 2) == qsa.QSA_ERR_INVALID_ARG           # out must be 8-byte aligned
    assert call(os=100) == qsa.QSA_ERR_INVALID_ARG
    assert call(os=4098) == qsa.QSA_ERR_INVALID_ARG              # row stride not a multiple of 4
    assert call(q=None) == qsa.QSA_ERR_INVALID_ARG
    assert call(ws=None) == qsa.QSA_ERR_INVALID_ARG
    assert call(wb=wsb - 1) == qsa.QSA_ERR_INVALID_ARG
    assert call(ws=P + 16) == qsa.QSA_ERR_INVALID_ARG            # workspace must be 256-byte aligned
    assert call(Hq=7) == qsa.QSA_ERR_UNSUPPORTED
    for over in (dict(v=None), dict(ckey=None), dict(k=None)):
        dv = kv(**over)
        assert f(ctypes.byref(dv), *base[1:]) == qsa.QSA_ERR_INVALID_ARG
    assert qsa.qsa_last_error() != ""


def test_fused_workspace_bytes():
    d = kv()
    B, Hq = 2, 16
    auto = qsa.qsa_decode_fused_workspace_bytes(d, Hq, 512, 0)
    s4 = qsa.qsa_decode_fused_workspace_bytes(d, Hq, 512, 4)
    s16 = qsa.qsa_decode_fused_workspace_bytes(d, Hq, 512, 16)
    # the partials grow with the split count: S x B x Hq x (1 KiB + 4 B)
    assert s16 - s4 >= 12 * B * Hq * 1024
    assert auto in (s4, s16) or auto > 0
    assert auto % 256 == 0 and s4 % 256 == 0
    # the scores (4 B per block of every (sequence, KV head), the row rounded up to
    # 64 blocks) are part of it: 800 more blocks in each of the 4 rows
    longer = qsa.qsa_decode_fused_workspace_bytes(kv(max_seq_len=6400, max_pages_per_seq=100), Hq, 512, 4)
    assert longer - s4 >= 4 * (800 - 64) * 4
    for args in ((Hq, -1, 0), (Hq, 2049, 0), (Hq, 512, 65), (0, 512, 0)):
        assert qsa.qsa_decode_fused_workspace_bytes(d, *args) == 0
    assert qsa.qsa_decode_fused_workspace_bytes(kv(batch=-1), Hq, 512, 0) == 0


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(qsa, "_lib", None)
    monkeypatch.setattr(qsa, "LIB_PATH", str(tmp_path / "libqsa.so"))
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        qsa.lib()


def test_noalloc_decode_rejects_partials_beyond_the_scratch_on_the_host():
    """qsa_sparse_attn_decode_noalloc: partials beyond QSA_NOALLOC_SCRATCH_BYTES are
    rejected before any HIP call (64 splits x 1000 rows x 16 heads)."""
    d = kv(batch=1000)
    rc = status("qsa_sparse_attn_decode_noalloc", ctypes.byref(d), P, 16 * 256, 16, P, P, 512, ctypes.c_float(0.0),
                64, P, 16 * 256, P, None)
    assert rc == qsa.QSA_ERR_UNSUPPORTED
    assert "scratch" in qsa.qsa_last_error()
    text = open(HEADER).read()
    assert re.search(r"#define QSA_NOALLOC_SCRATCH_BYTES \(8u << 20\)", text)
