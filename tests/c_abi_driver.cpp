// A decode step or an extend chunk driven through the C ABI alone: this program
// uses include/qsa.h and the HIP runtime, with no Python and no torch.  It reads a
// case from the directory given as argv[1] (sizes in meta.txt, arrays as raw
// little-endian files), allocates every device buffer itself, and runs on one
// stream of its own either (argv[2] = decode)
//   qsa_compress_keys -> qsa_decode_scores_refresh -> qsa_topk_blocks_ws ->
//   qsa_sparse_attn_decode (library-chosen splits, internal merge)
// or (argv[2] = extend, R query rows at their own positions)
//   qsa_compress_keys -> qsa_block_scores -> qsa_topk_blocks ->
//   qsa_sparse_attn_extend
// then writes the block keys, scores, selection, outputs and lse back to the
// directory.  It also checks that a call with an out-of-range argument is
// rejected, with a message, before anything runs.
//
// meta.txt: batch Hq Hkv page_size num_pages max_pages_per_seq max_seq_len k
//           score_stride kv_dtype ckey_dtype R
// inputs:   k.bin v.bin (the paged pool as the cache stores it), table.bin
//           (int32 [batch][max_pages_per_seq]), lens.bin (int32 [batch]),
//           q.bin (bf16 [R][Hq][256]); extend also q_seq.bin, q_pos.bin (int32 [R])
// outputs:  ckey.bin scores.bin sel.bin cnt.bin out.bin lse.bin
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "qsa.h"

namespace {

void hip_check(hipError_t e, const char* what) {
    if (e != hipSuccess) {
        std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
        std::exit(2);
    }
}

void qsa_check(int rc, const char* what) {
    if (rc != QSA_OK) {
        std::fprintf(stderr, "%s failed (status %d): %s\n", what, rc, qsa_last_error());
        std::exit(3);
    }
}

std::vector<char> read_file(const std::string& path, size_t bytes) {
    FILE* f = std::fopen(path.c_str(), "rb");
    if (!f) {
        std::fprintf(stderr, "cannot open %s\n", path.c_str());
        std::exit(1);
    }
    std::vector<char> buf(bytes);
    const size_t n = bytes ? std::fread(buf.data(), 1, bytes, f) : 0;
    const bool extra = std::fgetc(f) != EOF;
    std::fclose(f);
    if (n != bytes || extra) {
        std::fprintf(stderr, "%s: expected exactly %zu bytes\n", path.c_str(), bytes);
        std::exit(1);
    }
    return buf;
}

void write_file(const std::string& path, const std::vector<char>& buf) {
    FILE* f = std::fopen(path.c_str(), "wb");
    if (!f || std::fwrite(buf.data(), 1, buf.size(), f) != buf.size()) {
        std::fprintf(stderr, "cannot write %s\n", path.c_str());
        std::exit(1);
    }
    std::fclose(f);
}

struct Device {
    std::vector<void*> owned;
    void* alloc(size_t bytes) {
        void* p = nullptr;
        hip_check(hipMalloc(&p, bytes ? bytes : 16), "hipMalloc");
        owned.push_back(p);
        return p;
    }
    void* upload(const std::vector<char>& h) {
        void* p = alloc(h.size());
        if (!h.empty()) hip_check(hipMemcpy(p, h.data(), h.size(), hipMemcpyHostToDevice), "upload");
        return p;
    }
    void* zeros(size_t bytes) {
        void* p = alloc(bytes);
        hip_check(hipMemset(p, 0, bytes ? bytes : 16), "hipMemset");
        return p;
    }
    ~Device() {
        for (void* p : owned) (void)hipFree(p);
    }
};

std::vector<char> download(const void* d, size_t bytes) {
    std::vector<char> h(bytes);
    if (bytes) hip_check(hipMemcpy(h.data(), d, bytes, hipMemcpyDeviceToHost), "download");
    return h;
}

}  // namespace

int main(int argc, char** argv) {
    const std::string mode = argc == 3 ? argv[2] : "";
    if (mode != "decode" && mode != "extend") {
        std::fprintf(stderr, "usage: %s <case directory> decode|extend\n", argv[0]);
        return 1;
    }
    const bool extend = mode == "extend";
    const std::string dir = argv[1];
    int B, Hq, Hkv, ps, num_pages, max_pages, max_len, k, stride, kv_dtype, ckey_dtype, R;
    {
        FILE* m = std::fopen((dir + "/meta.txt").c_str(), "r");
        const int got = m ? std::fscanf(m, "%d %d %d %d %d %d %d %d %d %d %d %d", &B, &Hq, &Hkv, &ps, &num_pages,
                                        &max_pages, &max_len, &k, &stride, &kv_dtype, &ckey_dtype, &R)
                          : 0;
        if (m) std::fclose(m);
        if (got != 12 || B < 1 || Hq < 1 || Hkv < 1 || ps < 4 || num_pages < 1 || max_pages < 1 || k < 0 ||
            stride < 1 || R < 1 || (!extend && R != B)) {
            std::fprintf(stderr, "bad meta.txt\n");
            return 1;
        }
    }
    const size_t D = QSA_HEAD_DIM;
    const size_t kv_bytes = kv_dtype == QSA_KV_FP8 ? 1 : 2;
    const size_t ckey_bytes = ckey_dtype == QSA_CKEY_FP32 ? 4 : (ckey_dtype == QSA_CKEY_BF16 ? 2 : 1);
    const size_t pool = (size_t)num_pages * Hkv * ps * D;
    const size_t ckey_size = (size_t)num_pages * Hkv * (ps / 4) * D * ckey_bytes;
    const size_t q_size = (size_t)R * Hq * D * 2;

    const std::vector<char> hk = read_file(dir + "/k.bin", pool * kv_bytes);
    const std::vector<char> hv = read_file(dir + "/v.bin", pool * kv_bytes);
    const std::vector<char> htable = read_file(dir + "/table.bin", (size_t)B * max_pages * 4);
    const std::vector<char> hlens = read_file(dir + "/lens.bin", (size_t)B * 4);
    const std::vector<char> hq = read_file(dir + "/q.bin", q_size);
    std::vector<char> hseq, hpos;
    if (extend) {
        hseq = read_file(dir + "/q_seq.bin", (size_t)R * 4);
        hpos = read_file(dir + "/q_pos.bin", (size_t)R * 4);
    } else {
        hpos.resize(hlens.size());  // decode rows sit at t = L - 1
        for (int i = 0; i < B; ++i) {
            int32_t L;
            std::memcpy(&L, hlens.data() + 4 * i, 4);
            const int32_t t = L - 1;
            std::memcpy(hpos.data() + 4 * i, &t, 4);
        }
    }

    Device dev;
    qsa_kv_t kv;
    kv.k = dev.upload(hk);
    kv.v = dev.upload(hv);
    kv.ckey = dev.zeros(ckey_size);
    kv.block_table = static_cast<const int32_t*>(dev.upload(htable));
    kv.seq_lens = static_cast<const int32_t*>(dev.upload(hlens));
    kv.batch = B;
    kv.num_kv_heads = Hkv;
    kv.head_dim = (int32_t)D;
    kv.page_size = ps;
    kv.num_pages = num_pages;
    kv.max_pages_per_seq = max_pages;
    kv.max_seq_len = max_len;
    kv.ckey_dtype = ckey_dtype;
    kv.kv_dtype = kv_dtype;
    const void* q = dev.upload(hq);
    const int32_t* q_pos = static_cast<const int32_t*>(dev.upload(hpos));
    const int32_t* q_seq = extend ? static_cast<const int32_t*>(dev.upload(hseq)) : nullptr;

    const size_t scores_size = (size_t)R * Hkv * stride * 4;
    const size_t sel_size = (size_t)R * Hkv * (k > 0 ? k : 1) * 4;
    float* scores = static_cast<float*>(dev.alloc(scores_size));
    int32_t* sel = static_cast<int32_t*>(dev.alloc(sel_size));
    int32_t* cnt = static_cast<int32_t*>(dev.alloc((size_t)R * Hkv * 4));
    void* out = dev.alloc(q_size);
    float* lse = static_cast<float*>(dev.alloc((size_t)R * Hq * 4));
    const size_t topk_ws = qsa_topk_workspace_bytes(B, Hkv, k, stride);
    void* topk_ws_ptr = topk_ws ? dev.alloc(topk_ws) : nullptr;
    const size_t attn_ws = qsa_decode_workspace_bytes(B, Hq, 0);
    void* attn_ws_ptr = attn_ws ? dev.alloc(attn_ws) : nullptr;

    hipStream_t st;
    hip_check(hipStreamCreate(&st), "hipStreamCreate");
    const int64_t row = (int64_t)Hq * D;
    qsa_check(qsa_compress_keys(&kv, nullptr, 0, st), "qsa_compress_keys");
    if (extend) {
        qsa_check(qsa_block_scores(&kv, q, row, q_seq, q_pos, R, Hq, scores, stride, st), "qsa_block_scores");
        qsa_check(qsa_topk_blocks(scores, stride, q_pos, R, Hkv, k, sel, cnt, st), "qsa_topk_blocks");
        qsa_check(qsa_sparse_attn_extend(&kv, q, row, q_seq, q_pos, R, Hq, sel, cnt, k, 0.0f, out, row, lse, st),
                  "qsa_sparse_attn_extend");
    } else {
        qsa_check(qsa_decode_scores_refresh(&kv, q, row, Hq, scores, stride, st), "qsa_decode_scores_refresh");
        qsa_check(qsa_topk_blocks_ws(scores, stride, q_pos, B, Hkv, k, sel, cnt, topk_ws_ptr, topk_ws, st),
                  "qsa_topk_blocks_ws");
        qsa_check(qsa_sparse_attn_decode(&kv, q, row, Hq, sel, cnt, k, 0.0f, 0, out, row, lse, nullptr, nullptr,
                                         attn_ws_ptr, attn_ws, st),
                  "qsa_sparse_attn_decode");
    }
    // argument checks run on the host, before any launch
    const int bad = qsa_topk_blocks(scores, stride, q_pos, R, Hkv, QSA_MAX_TOPK + 1, sel, cnt, st);
    const char* msg = qsa_last_error();
    if (bad != QSA_ERR_INVALID_ARG || !msg || !*msg) {
        std::fprintf(stderr, "k = %d was not rejected as an invalid argument (status %d)\n", QSA_MAX_TOPK + 1, bad);
        return 4;
    }
    std::printf("rejected as expected: %s\n", msg);
    hip_check(hipStreamSynchronize(st), "hipStreamSynchronize");
    hip_check(hipGetLastError(), "kernels");

    write_file(dir + "/ckey.bin", download(kv.ckey, ckey_size));
    write_file(dir + "/scores.bin", download(scores, scores_size));
    write_file(dir + "/sel.bin", download(sel, sel_size));
    write_file(dir + "/cnt.bin", download(cnt, (size_t)R * Hkv * 4));
    write_file(dir + "/out.bin", download(out, q_size));
    write_file(dir + "/lse.bin", download(lse, (size_t)R * Hq * 4));
    hip_check(hipStreamDestroy(st), "hipStreamDestroy");
    std::printf("libqsa version %d: %s of %d rows over %d sequences done\n", qsa_version(), mode.c_str(), R, B);
    return 0;
}
