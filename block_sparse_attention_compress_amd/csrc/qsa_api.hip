// C ABI of libqsa.so: host-side validation, then kernel launches.  Nothing here
// touches HIP before the arguments have been accepted, so a rejected call costs
// no device work and can be tested without a GPU.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "qsa.h"
#include "qsa_launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return QSA_OK;
}

int hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(QSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int log2_exact(int v) {
    if (v <= 0 || (v & (v - 1))) return -1;
    int l = 0;
    while ((1 << l) < v) ++l;
    return l;
}

// Checks the cache descriptor.  need_kv: K and V are read; need_ckey: block
// keys are read or written.
int check_kv(const qsa_kv_t* kv, bool need_k, bool need_v, bool need_ckey, qsa::PagedKV* out) {
    if (!kv) return fail(QSA_ERR_INVALID_ARG, "kv descriptor is NULL");
    if (need_k && !kv->k) return fail(QSA_ERR_INVALID_ARG, "kv->k is NULL");
    if (need_v && !kv->v) return fail(QSA_ERR_INVALID_ARG, "kv->v is NULL");
    if (need_ckey && !kv->ckey) return fail(QSA_ERR_INVALID_ARG, "kv->ckey is NULL");
    if (!kv->block_table || !kv->seq_lens) return fail(QSA_ERR_INVALID_ARG, "kv->block_table / seq_lens is NULL");
    if ((need_k && !aligned(kv->k, 16)) || (need_v && !aligned(kv->v, 16)) || (need_ckey && !aligned(kv->ckey, 16)))
        return fail(QSA_ERR_INVALID_ARG, "k, v and ckey must be 16-byte aligned");
    if (kv->head_dim != QSA_HEAD_DIM)
        return fail(QSA_ERR_UNSUPPORTED, "head_dim %d: only %d is supported", kv->head_dim, QSA_HEAD_DIM);
    if (kv->batch < 0 || kv->batch > 65535) return fail(QSA_ERR_INVALID_ARG, "batch %d out of [0, 65535]", kv->batch);
    if (kv->num_kv_heads < 1 || kv->num_kv_heads > 65535)
        return fail(QSA_ERR_INVALID_ARG, "num_kv_heads %d out of [1, 65535]", kv->num_kv_heads);
    const int lg = log2_exact(kv->page_size);
    if (lg < 2) return fail(QSA_ERR_INVALID_ARG, "page_size %d is not a power of two >= 4", kv->page_size);
    if (kv->num_pages < 1 || kv->max_pages_per_seq < 1)
        return fail(QSA_ERR_INVALID_ARG, "num_pages and max_pages_per_seq must be >= 1");
    if (kv->max_seq_len < 0) return fail(QSA_ERR_INVALID_ARG, "max_seq_len %d < 0", kv->max_seq_len);
    if (kv->ckey_dtype != QSA_CKEY_FP32 && kv->ckey_dtype != QSA_CKEY_BF16 && kv->ckey_dtype != QSA_CKEY_FP8)
        return fail(QSA_ERR_INVALID_ARG, "ckey_dtype %d is not QSA_CKEY_FP32, QSA_CKEY_BF16 or QSA_CKEY_FP8",
                    kv->ckey_dtype);
    if (kv->kv_dtype != QSA_KV_BF16 && kv->kv_dtype != QSA_KV_FP8)
        return fail(QSA_ERR_INVALID_ARG, "kv_dtype %d is neither QSA_KV_BF16 nor QSA_KV_FP8", kv->kv_dtype);
    if (kv->max_seq_len > QSA_MAX_SEQ_LEN)
        return fail(QSA_ERR_UNSUPPORTED, "max_seq_len %d exceeds %d", kv->max_seq_len, QSA_MAX_SEQ_LEN);
    if ((int64_t)kv->max_pages_per_seq * kv->page_size < kv->max_seq_len)
        return fail(QSA_ERR_INVALID_ARG, "max_pages_per_seq * page_size < max_seq_len");
    if ((int64_t)kv->num_pages * kv->num_kv_heads * kv->page_size >= (int64_t)1 << 31)
        return fail(QSA_ERR_UNSUPPORTED, "pool of %lld token rows exceeds 2^31",
                    (long long)kv->num_pages * kv->num_kv_heads * kv->page_size);
    out->k = static_cast<const uint16_t*>(kv->k);
    out->v = static_cast<const uint16_t*>(kv->v);
    out->ckey = kv->ckey;
    out->ckey_type = kv->ckey_dtype;  // QSA_CKEY_* values are the kernels' key types
    out->kv_fp8 = kv->kv_dtype == QSA_KV_FP8;
    out->block_table = kv->block_table;
    out->seq_lens = kv->seq_lens;
    out->batch = kv->batch;
    out->Hkv = kv->num_kv_heads;
    out->lg_ps = lg;
    out->num_pages = kv->num_pages;
    out->max_pages = kv->max_pages_per_seq;
    out->max_seq_len = kv->max_seq_len;
    return QSA_OK;
}

int check_heads(int Hq, int Hkv) {
    if (Hq < 1) return fail(QSA_ERR_INVALID_ARG, "Hq %d < 1", Hq);
    if (Hq % Hkv) return fail(QSA_ERR_UNSUPPORTED, "Hq %d is not a multiple of Hkv %d", Hq, Hkv);
    if (Hq / Hkv > QSA_MAX_GROUP)
        return fail(QSA_ERR_UNSUPPORTED, "group of %d query heads per KV head exceeds %d", Hq / Hkv, QSA_MAX_GROUP);
    return QSA_OK;
}

int check_q(const void* q, int64_t q_row_stride, int Hq) {
    if (!q) return fail(QSA_ERR_INVALID_ARG, "q is NULL");
    if (!aligned(q, 16)) return fail(QSA_ERR_INVALID_ARG, "q must be 16-byte aligned");
    if (q_row_stride < (int64_t)Hq * QSA_HEAD_DIM || q_row_stride % 8)
        return fail(QSA_ERR_INVALID_ARG, "q_row_stride %lld must be >= Hq * 256 and a multiple of 8",
                    (long long)q_row_stride);
    return QSA_OK;
}

int auto_splits(int64_t units, int k) {
    // aim at ~256 workgroups (one per CU) while keeping >= 16 blocks per split: a
    // split sweep over 2-16 put the best step there for 2, 16 and 64 (row, KV head)
    // units (64 units: S = 4 beat S = 8 by 3 %)
    int64_t s = (256 + units - 1) / (units > 0 ? units : 1);
    const int64_t cap = k / 16 > 1 ? k / 16 : 1;
    if (s > cap) s = cap;
    if (s > 16) s = 16;
    return s < 1 ? 1 : (int)s;
}

constexpr int kAutoSplitMax = 16;

// ---- static scratch of the no-allocation decode entry point
//
// The split partials of qsa_sparse_attn_decode_noalloc live in this array: one
// copy per GPU, loaded with the code object and held until the process ends.
// Host code never passes the array's name to a kernel (on the host it names a
// host-side stand-in): the device address is looked up once per device, with
// that device current, and kept in g_scratch_ptr.
constexpr size_t kScratchBytes = QSA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_for_current_device(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(QSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(QSA_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(QSA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return QSA_OK;
}

// Attention writing the final result (out, lse) of rows.R rows (decode: one per
// sequence; extend: rows.q_seq / rows.q_pos): one launch when the split count is
// 1, else blocked split partials and the merge.  The partials go to the caller's
// `workspace`, or with use_scratch to the static scratch (the no-allocation
// entry point; workspace is then ignored).
int attn_final(const qsa::PagedKV& p, const qsa::Rows& rows, const int32_t* sel_idx, const int32_t* sel_cnt,
               int32_t k, float sc, int32_t num_splits, void* out, int64_t out_row_stride, float* lse,
               void* workspace, size_t workspace_bytes, bool use_scratch, hipStream_t st, const char* what) {
    const int Hq = rows.Hq;
    if (!out) return fail(QSA_ERR_INVALID_ARG, "out is NULL");
    if (out_row_stride < (int64_t)Hq * QSA_HEAD_DIM)
        return fail(QSA_ERR_INVALID_ARG, "out_row_stride %lld < Hq * 256", (long long)out_row_stride);
    const int R = rows.R;
    const int S = num_splits == 0 ? auto_splits((int64_t)R * p.Hkv, k) : num_splits;
    if (S == 1) {
        qsa::AttnOut o{static_cast<uint16_t*>(out), out_row_stride, lse, nullptr, nullptr};
        return hip_status(qsa::launch_attn(p, rows, sel_idx, sel_cnt, k, sc, 1, false, o, st), what);
    }
    if (out_row_stride != (int64_t)Hq * QSA_HEAD_DIM || !aligned(out, 8))
        return fail(QSA_ERR_UNSUPPORTED, "a split attention writes a dense, 8-byte aligned out");
    if ((int64_t)R * Hq > 0x7fffffff)  // the merge indexes its rows with 32-bit integers
        return fail(QSA_ERR_UNSUPPORTED, "%d rows x %d heads exceed 2^31 - 1 merged rows", R, Hq);
    const size_t need = qsa_decode_workspace_bytes(R, Hq, S);
    if (use_scratch) {
        if (need > kScratchBytes)
            return fail(QSA_ERR_UNSUPPORTED,
                        "%d splits of %d rows x %d heads need %zu bytes of partials, more than the %zu bytes of "
                        "static scratch (use qsa_sparse_attn_decode with a workspace, or fewer splits)",
                        S, R, Hq, need, (size_t)kScratchBytes);
        if (int rc = scratch_for_current_device(&workspace)) return rc;
        workspace_bytes = kScratchBytes;
    } else if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) {
        return fail(QSA_ERR_INVALID_ARG, "workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                    workspace_bytes);
    }
    const int64_t n = (int64_t)S * R * Hq;
    float* wo = static_cast<float*>(workspace);
    float* wl = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                         (((size_t)n * QSA_HEAD_DIM * sizeof(float) + 255) & ~(size_t)255));
    qsa::AttnOut o{nullptr, 0, nullptr, wo, wl};
    if (int rc = hip_status(qsa::launch_attn(p, rows, sel_idx, sel_cnt, k, sc, S, true, o, st), what)) return rc;
    return hip_status(qsa::launch_merge(wo, wl, S, R * Hq, QSA_HEAD_DIM, static_cast<uint16_t*>(out), lse, st),
                      what);
}


}  // namespace

extern "C" {

int qsa_version(void) { return 100; }

const char* qsa_last_error(void) { return g_err; }

int qsa_compress_keys(const qsa_kv_t* kv, const int32_t* first_token, int32_t max_new_tokens, void* stream) {
    qsa::PagedKV p;
    if (int rc = check_kv(kv, true, false, true, &p)) return rc;
    const int span = (first_token && max_new_tokens > 0 && max_new_tokens < p.max_seq_len) ? max_new_tokens
                                                                                          : p.max_seq_len;
    return hip_status(qsa::launch_compress(p, first_token, span, static_cast<hipStream_t>(stream)),
                      "qsa_compress_keys");
}

int qsa_block_scores(const qsa_kv_t* kv, const void* q, int64_t q_row_stride, const int32_t* q_seq,
                     const int32_t* q_pos, int32_t R, int32_t Hq, float* scores, int32_t score_stride,
                     void* stream) {
    qsa::PagedKV p;
    if (int rc = check_kv(kv, false, false, true, &p)) return rc;
    if (int rc = check_heads(Hq, p.Hkv)) return rc;
    if (int rc = check_q(q, q_row_stride, Hq)) return rc;
    if (R < 0) return fail(QSA_ERR_INVALID_ARG, "R %d < 0", R);
    if (R > 65535) return fail(QSA_ERR_UNSUPPORTED, "R %d exceeds 65535 rows per call", R);
    if (!scores) return fail(QSA_ERR_INVALID_ARG, "scores is NULL");
    if (score_stride < 1 || score_stride > QSA_MAX_SEQ_LEN / QSA_MICROBLOCK)
        return fail(QSA_ERR_INVALID_ARG, "score_stride %d out of [1, %d]", score_stride,
                    QSA_MAX_SEQ_LEN / QSA_MICROBLOCK);
    if ((q_seq == nullptr) != (q_pos == nullptr))
        return fail(QSA_ERR_INVALID_ARG, "q_seq and q_pos must both be given or both be NULL");
    if (!q_seq && R != p.batch) return fail(QSA_ERR_INVALID_ARG, "decode scoring needs R == batch (%d != %d)", R, p.batch);
    qsa::Rows rows{static_cast<const uint16_t*>(q), q_row_stride, q_seq, q_pos, R, Hq};
    hipStream_t st = static_cast<hipStream_t>(stream);
    // more rows than sequences: rows share block keys, score them as a matrix product
    const bool tiled = q_seq && R > p.batch;
    hipError_t e = tiled ? qsa::launch_scores_tiled(p, rows, scores, score_stride, st)
                         : qsa::launch_scores_stream(p, rows, scores, score_stride, false, st);
    return hip_status(e, "qsa_block_scores");
}

int qsa_decode_scores_refresh(const qsa_kv_t* kv, const void* q, int64_t q_row_stride, int32_t Hq, float* scores,
                              int32_t score_stride, void* stream) {
    qsa::PagedKV p;
    if (int rc = check_kv(kv, true, false, true, &p)) return rc;
    if (int rc = check_heads(Hq, p.Hkv)) return rc;
    if (int rc = check_q(q, q_row_stride, Hq)) return rc;
    if (!scores) return fail(QSA_ERR_INVALID_ARG, "scores is NULL");
    if (score_stride < 1 || score_stride > QSA_MAX_SEQ_LEN / QSA_MICROBLOCK)
        return fail(QSA_ERR_INVALID_ARG, "score_stride %d out of [1, %d]", score_stride,
                    QSA_MAX_SEQ_LEN / QSA_MICROBLOCK);
    qsa::Rows rows{static_cast<const uint16_t*>(q), q_row_stride, nullptr, nullptr, p.batch, Hq};
    return hip_status(qsa::launch_scores_stream(p, rows, scores, score_stride, true, static_cast<hipStream_t>(stream)),
                      "qsa_decode_scores_refresh");
}

static int check_topk(const float* scores, int32_t score_stride, int32_t R, int32_t Hkv, int32_t k,
                      const int32_t* sel_idx, const int32_t* sel_cnt) {
    if (!scores) return fail(QSA_ERR_INVALID_ARG, "scores is NULL");
    if (score_stride < 1 || score_stride > QSA_MAX_SEQ_LEN / QSA_MICROBLOCK)
        return fail(QSA_ERR_INVALID_ARG, "score_stride %d out of [1, %d]", score_stride,
                    QSA_MAX_SEQ_LEN / QSA_MICROBLOCK);
    if (R < 0 || Hkv < 1) return fail(QSA_ERR_INVALID_ARG, "R %d / Hkv %d out of range", R, Hkv);
    if ((int64_t)R * Hkv > 0x7fffffff) return fail(QSA_ERR_UNSUPPORTED, "R * Hkv exceeds 2^31 - 1");
    if (k < 0 || k > QSA_MAX_TOPK) return fail(QSA_ERR_INVALID_ARG, "k %d out of [0, %d]", k, QSA_MAX_TOPK);
    if (!sel_cnt || (k > 0 && !sel_idx)) return fail(QSA_ERR_INVALID_ARG, "sel_idx / sel_cnt is NULL");
    return QSA_OK;
}

int qsa_topk_blocks(const float* scores, int32_t score_stride, const int32_t* q_pos, int32_t R, int32_t Hkv,
                    int32_t k, int32_t* sel_idx, int32_t* sel_cnt, void* stream) {
    if (int rc = check_topk(scores, score_stride, R, Hkv, k, sel_idx, sel_cnt)) return rc;
    return hip_status(qsa::launch_topk(scores, score_stride, q_pos, R, Hkv, k, sel_idx, sel_cnt,
                                       static_cast<hipStream_t>(stream)),
                      "qsa_topk_blocks");
}

size_t qsa_topk_workspace_bytes(int32_t R, int32_t Hkv, int32_t k, int32_t score_stride) {
    if (R <= 0 || Hkv <= 0 || k < 0 || k > QSA_MAX_TOPK || score_stride < 1 ||
        score_stride > QSA_MAX_SEQ_LEN / QSA_MICROBLOCK || (int64_t)R * Hkv > 0x7fffffff)
        return 0;
    return qsa::topk_workspace_bytes(R, Hkv, k, score_stride);
}

int qsa_topk_blocks_ws(const float* scores, int32_t score_stride, const int32_t* q_pos, int32_t R, int32_t Hkv,
                       int32_t k, int32_t* sel_idx, int32_t* sel_cnt, void* workspace, size_t workspace_bytes,
                       void* stream) {
    if (int rc = check_topk(scores, score_stride, R, Hkv, k, sel_idx, sel_cnt)) return rc;
    const size_t need = qsa::topk_workspace_bytes(R, Hkv, k, score_stride);
    if (need > 0) {
        if (!workspace) return fail(QSA_ERR_INVALID_ARG, "workspace is NULL (%zu bytes needed)", need);
        if (workspace_bytes < need)
            return fail(QSA_ERR_INVALID_ARG, "workspace_bytes %zu < %zu", workspace_bytes, need);
        if (!aligned(workspace, 16)) return fail(QSA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    }
    return hip_status(qsa::launch_topk_split(scores, score_stride, q_pos, R, Hkv, k, sel_idx, sel_cnt, workspace,
                                             static_cast<hipStream_t>(stream)),
                      "qsa_topk_blocks_ws");
}

size_t qsa_decode_workspace_bytes(int32_t batch, int32_t Hq, int32_t num_splits) {
    const int64_t S = num_splits == 0 ? kAutoSplitMax : num_splits;
    if (S <= 1 || batch <= 0 || Hq <= 0) return 0;
    const int64_t n = S * batch * Hq;
    const size_t out_bytes = (size_t)n * QSA_HEAD_DIM * sizeof(float);
    const size_t lse_bytes = (size_t)n * sizeof(float);
    return ((out_bytes + 255) & ~(size_t)255) + ((lse_bytes + 255) & ~(size_t)255);
}

int qsa_sparse_attn_decode(const qsa_kv_t* kv, const void* q, int64_t q_row_stride, int32_t Hq,
                           const int32_t* sel_idx, const int32_t* sel_cnt, int32_t k, float scale,
                           int32_t num_splits, void* out, int64_t out_row_stride, float* lse, float* part_out,
                           float* part_lse, void* workspace, size_t workspace_bytes, void* stream) {
    qsa::PagedKV p;
    if (int rc = check_kv(kv, true, true, false, &p)) return rc;
    if (int rc = check_heads(Hq, p.Hkv)) return rc;
    if (int rc = check_q(q, q_row_stride, Hq)) return rc;
    if (k < 0 || k > QSA_MAX_TOPK) return fail(QSA_ERR_INVALID_ARG, "k %d out of [0, %d]", k, QSA_MAX_TOPK);
    if (!sel_cnt || (k > 0 && !sel_idx)) return fail(QSA_ERR_INVALID_ARG, "sel_idx / sel_cnt is NULL");
    if (num_splits < 0 || num_splits > QSA_MAX_SPLITS)
        return fail(QSA_ERR_INVALID_ARG, "num_splits %d out of [0, %d]", num_splits, QSA_MAX_SPLITS);
    const float sc = scale > 0.f ? scale : 0.0625f;
    hipStream_t st = static_cast<hipStream_t>(stream);
    qsa::Rows rows{static_cast<const uint16_t*>(q), q_row_stride, nullptr, nullptr, p.batch, Hq};
    if ((int64_t)p.batch * p.Hkv * (num_splits > 0 ? num_splits : kAutoSplitMax) > 0x7fffffff)
        return fail(QSA_ERR_UNSUPPORTED, "too many work units");
    if (part_out) {
        if (num_splits < 1) return fail(QSA_ERR_INVALID_ARG, "partials need num_splits >= 1");
        if (!part_lse) return fail(QSA_ERR_INVALID_ARG, "part_lse is NULL");
        if (!aligned(part_out, 16)) return fail(QSA_ERR_INVALID_ARG, "part_out must be 16-byte aligned");
        qsa::AttnOut o{nullptr, 0, nullptr, part_out, part_lse};
        return hip_status(qsa::launch_attn(p, rows, sel_idx, sel_cnt, k, sc, num_splits, false, o, st),
                          "qsa_sparse_attn_decode");
    }
    return attn_final(p, rows, sel_idx, sel_cnt, k, sc, num_splits, out, out_row_stride, lse, workspace,
                      workspace_bytes, false, st, "qsa_sparse_attn_decode");
}

int qsa_sparse_attn_decode_noalloc(const qsa_kv_t* kv, const void* q, int64_t q_row_stride, int32_t Hq,
                                   const int32_t* sel_idx, const int32_t* sel_cnt, int32_t k, float scale,
                                   int32_t num_splits, void* out, int64_t out_row_stride, float* lse, void* stream) {
    qsa::PagedKV p;
    if (int rc = check_kv(kv, true, true, false, &p)) return rc;
    if (int rc = check_heads(Hq, p.Hkv)) return rc;
    if (int rc = check_q(q, q_row_stride, Hq)) return rc;
    if (k < 0 || k > QSA_MAX_TOPK) return fail(QSA_ERR_INVALID_ARG, "k %d out of [0, %d]", k, QSA_MAX_TOPK);
    if (!sel_cnt || (k > 0 && !sel_idx)) return fail(QSA_ERR_INVALID_ARG, "sel_idx / sel_cnt is NULL");
    if (num_splits < 0 || num_splits > QSA_MAX_SPLITS)
        return fail(QSA_ERR_INVALID_ARG, "num_splits %d out of [0, %d]", num_splits, QSA_MAX_SPLITS);
    if ((int64_t)p.batch * p.Hkv * (num_splits > 0 ? num_splits : kAutoSplitMax) > 0x7fffffff)
        return fail(QSA_ERR_UNSUPPORTED, "too many work units");
    const float sc = scale > 0.f ? scale : 0.0625f;
    qsa::Rows rows{static_cast<const uint16_t*>(q), q_row_stride, nullptr, nullptr, p.batch, Hq};
    return attn_final(p, rows, sel_idx, sel_cnt, k, sc, num_splits, out, out_row_stride, lse, nullptr, 0, true,
                      static_cast<hipStream_t>(stream), "qsa_sparse_attn_decode_noalloc");
}

size_t qsa_decode_fused_workspace_bytes(const qsa_kv_t* kv, int32_t Hq, int32_t k, int32_t num_splits) {
    if (!kv || kv->batch < 0 || kv->num_kv_heads < 1 || Hq < 1 || kv->max_seq_len < 0 ||
        kv->max_seq_len > QSA_MAX_SEQ_LEN || k < 0 || k > QSA_MAX_TOPK || num_splits < 0 ||
        num_splits > QSA_MAX_SPLITS)
        return 0;
    const int S = num_splits == 0 ? auto_splits((int64_t)kv->batch * kv->num_kv_heads, k) : num_splits;
    return qsa::fused_workspace_bytes(kv->batch, kv->num_kv_heads, Hq, kv->max_seq_len, S);
}

int qsa_decode_fused(const qsa_kv_t* kv, const void* q, int64_t q_row_stride, int32_t Hq, int32_t k, float scale,
                     int32_t num_splits, int32_t* sel_idx, int32_t* sel_cnt, void* out, int64_t out_row_stride,
                     float* lse, void* workspace, size_t workspace_bytes, void* stream) {
    qsa::PagedKV p;
    if (int rc = check_kv(kv, true, true, true, &p)) return rc;
    if (int rc = check_heads(Hq, p.Hkv)) return rc;
    if (int rc = check_q(q, q_row_stride, Hq)) return rc;
    if (k < 0 || k > QSA_MAX_TOPK) return fail(QSA_ERR_INVALID_ARG, "k %d out of [0, %d]", k, QSA_MAX_TOPK);
    if (!sel_cnt || (k > 0 && !sel_idx)) return fail(QSA_ERR_INVALID_ARG, "sel_idx / sel_cnt is NULL");
    if (num_splits < 0 || num_splits > QSA_MAX_SPLITS)
        return fail(QSA_ERR_INVALID_ARG, "num_splits %d out of [0, %d]", num_splits, QSA_MAX_SPLITS);
    if (!out) return fail(QSA_ERR_INVALID_ARG, "out is NULL");
    if (!aligned(out, 8) || out_row_stride < (int64_t)Hq * QSA_HEAD_DIM || out_row_stride % 4)
        return fail(QSA_ERR_INVALID_ARG, "out must be 8-byte aligned with a row stride >= Hq * 256, a multiple of 4");
    const int S = num_splits == 0 ? auto_splits((int64_t)p.batch * p.Hkv, k) : num_splits;
    const int64_t units = (int64_t)p.batch * p.Hkv;
    const int64_t chunks = ((int64_t)p.max_seq_len + 3) / 4 / 64 + 2;  // scan items of 64 blocks
    if (units * (chunks + S) > 0x7fffffff) return fail(QSA_ERR_UNSUPPORTED, "too many work items");
    const size_t need = qsa::fused_workspace_bytes(p.batch, p.Hkv, Hq, p.max_seq_len, S);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
        return fail(QSA_ERR_INVALID_ARG, "workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                    workspace_bytes);
    const float sc = scale > 0.f ? scale : 0.0625f;
    qsa::Rows rows{static_cast<const uint16_t*>(q), q_row_stride, nullptr, nullptr, p.batch, Hq};
    return hip_status(qsa::launch_fused_decode(p, rows, k, sc, S, sel_idx, sel_cnt, static_cast<uint16_t*>(out),
                                               out_row_stride, lse, workspace, static_cast<hipStream_t>(stream)),
                      "qsa_decode_fused");
}

int qsa_sparse_attn_extend(const qsa_kv_t* kv, const void* q, int64_t q_row_stride, const int32_t* q_seq,
                           const int32_t* q_pos, int32_t R, int32_t Hq, const int32_t* sel_idx,
                           const int32_t* sel_cnt, int32_t k, float scale, void* out, int64_t out_row_stride,
                           float* lse, void* stream) {
    qsa::PagedKV p;
    if (int rc = check_kv(kv, true, true, false, &p)) return rc;
    if (int rc = check_heads(Hq, p.Hkv)) return rc;
    if (int rc = check_q(q, q_row_stride, Hq)) return rc;
    if (!q_seq || !q_pos) return fail(QSA_ERR_INVALID_ARG, "q_seq / q_pos is NULL");
    if (R < 0) return fail(QSA_ERR_INVALID_ARG, "R %d < 0", R);
    if ((int64_t)R * p.Hkv > 0x7fffffff) return fail(QSA_ERR_UNSUPPORTED, "R * Hkv exceeds 2^31 - 1");
    if (k < 0 || k > QSA_MAX_TOPK) return fail(QSA_ERR_INVALID_ARG, "k %d out of [0, %d]", k, QSA_MAX_TOPK);
    if (!sel_cnt || (k > 0 && !sel_idx)) return fail(QSA_ERR_INVALID_ARG, "sel_idx / sel_cnt is NULL");
    if (!out) return fail(QSA_ERR_INVALID_ARG, "out is NULL");
    if (out_row_stride < (int64_t)Hq * QSA_HEAD_DIM)
        return fail(QSA_ERR_INVALID_ARG, "out_row_stride %lld < Hq * 256", (long long)out_row_stride);
    const float sc = scale > 0.f ? scale : 0.0625f;
    qsa::Rows rows{static_cast<const uint16_t*>(q), q_row_stride, q_seq, q_pos, R, Hq};
    qsa::AttnOut o{static_cast<uint16_t*>(out), out_row_stride, lse, nullptr, nullptr};
    return hip_status(qsa::launch_attn(p, rows, sel_idx, sel_cnt, k, sc, 1, false, o, static_cast<hipStream_t>(stream)),
                      "qsa_sparse_attn_extend");
}

size_t qsa_extend_workspace_bytes(int32_t R, int32_t Hq, int32_t num_splits) {
    if (num_splits < 0 || num_splits > QSA_MAX_SPLITS) return 0;
    return qsa_decode_workspace_bytes(R, Hq, num_splits);
}

int qsa_sparse_attn_extend_split(const qsa_kv_t* kv, const void* q, int64_t q_row_stride, const int32_t* q_seq,
                                 const int32_t* q_pos, int32_t R, int32_t Hq, const int32_t* sel_idx,
                                 const int32_t* sel_cnt, int32_t k, float scale, int32_t num_splits, void* out,
                                 int64_t out_row_stride, float* lse, void* workspace, size_t workspace_bytes,
                                 void* stream) {
    qsa::PagedKV p;
    if (int rc = check_kv(kv, true, true, false, &p)) return rc;
    if (int rc = check_heads(Hq, p.Hkv)) return rc;
    if (int rc = check_q(q, q_row_stride, Hq)) return rc;
    if (!q_seq || !q_pos) return fail(QSA_ERR_INVALID_ARG, "q_seq / q_pos is NULL");
    if (R < 0) return fail(QSA_ERR_INVALID_ARG, "R %d < 0", R);
    if (k < 0 || k > QSA_MAX_TOPK) return fail(QSA_ERR_INVALID_ARG, "k %d out of [0, %d]", k, QSA_MAX_TOPK);
    if (!sel_cnt || (k > 0 && !sel_idx)) return fail(QSA_ERR_INVALID_ARG, "sel_idx / sel_cnt is NULL");
    if (num_splits < 0 || num_splits > QSA_MAX_SPLITS)
        return fail(QSA_ERR_INVALID_ARG, "num_splits %d out of [0, %d]", num_splits, QSA_MAX_SPLITS);
    if ((int64_t)R * p.Hkv * (num_splits > 0 ? num_splits : kAutoSplitMax) > 0x7fffffff)
        return fail(QSA_ERR_UNSUPPORTED, "too many work units");
    if (!out) return fail(QSA_ERR_INVALID_ARG, "out is NULL");
    const float sc = scale > 0.f ? scale : 0.0625f;
    qsa::Rows rows{static_cast<const uint16_t*>(q), q_row_stride, q_seq, q_pos, R, Hq};
    if (R == 0) return QSA_OK;
    return attn_final(p, rows, sel_idx, sel_cnt, k, sc, num_splits, out, out_row_stride, lse, workspace,
                      workspace_bytes, false, static_cast<hipStream_t>(stream), "qsa_sparse_attn_extend_split");
}

int qsa_sparse_attn_extend_union(const qsa_kv_t* kv, const void* q, int64_t q_row_stride, const int32_t* q_seq,
                                 const int32_t* q_pos, int32_t R, int32_t Hq, const int32_t* sel_idx,
                                 const int32_t* sel_cnt, int32_t k, float scale, void* out, int64_t out_row_stride,
                                 float* lse, void* stream) {
    qsa::PagedKV p;
    if (int rc = check_kv(kv, true, true, false, &p)) return rc;
    if (int rc = check_heads(Hq, p.Hkv)) return rc;
    if (int rc = check_q(q, q_row_stride, Hq)) return rc;
    if (!q_seq || !q_pos) return fail(QSA_ERR_INVALID_ARG, "q_seq / q_pos is NULL");
    if (R < 0) return fail(QSA_ERR_INVALID_ARG, "R %d < 0", R);
    if ((int64_t)R * p.Hkv > 0x7fffffff) return fail(QSA_ERR_UNSUPPORTED, "R * Hkv exceeds 2^31 - 1");
    if (k < 0 || k > QSA_MAX_TOPK) return fail(QSA_ERR_INVALID_ARG, "k %d out of [0, %d]", k, QSA_MAX_TOPK);
    if (!sel_cnt || (k > 0 && !sel_idx)) return fail(QSA_ERR_INVALID_ARG, "sel_idx / sel_cnt is NULL");
    if (!out) return fail(QSA_ERR_INVALID_ARG, "out is NULL");
    if (out_row_stride < (int64_t)Hq * QSA_HEAD_DIM)
        return fail(QSA_ERR_INVALID_ARG, "out_row_stride %lld < Hq * 256", (long long)out_row_stride);
    const float sc = scale > 0.f ? scale : 0.0625f;
    qsa::Rows rows{static_cast<const uint16_t*>(q), q_row_stride, q_seq, q_pos, R, Hq};
    return hip_status(qsa::launch_attn_union(p, rows, sel_idx, sel_cnt, k, sc, static_cast<uint16_t*>(out),
                                             out_row_stride, lse, static_cast<hipStream_t>(stream)),
                      "qsa_sparse_attn_extend_union");
}

int qsa_merge_lse(const float* part_out, const float* part_lse, int32_t S, int32_t N, int32_t D, void* out_bf16,
                  float* out_lse, void* stream) {
    if (!part_out || !part_lse || !out_bf16) return fail(QSA_ERR_INVALID_ARG, "part_out / part_lse / out is NULL");
    if (S < 1 || S > QSA_MAX_SPLITS) return fail(QSA_ERR_INVALID_ARG, "S %d out of [1, %d]", S, QSA_MAX_SPLITS);
    if (N < 0) return fail(QSA_ERR_INVALID_ARG, "N %d < 0", N);
    if (D < 4 || D > 1024 || D % 4) return fail(QSA_ERR_UNSUPPORTED, "D %d must be a multiple of 4 in [4, 1024]", D);
    if (!aligned(part_out, 16) || !aligned(out_bf16, 8))
        return fail(QSA_ERR_INVALID_ARG, "part_out must be 16-byte and out 8-byte aligned");
    return hip_status(qsa::launch_merge(part_out, part_lse, S, N, D, static_cast<uint16_t*>(out_bf16), out_lse,
                                        static_cast<hipStream_t>(stream)),
                      "qsa_merge_lse");
}

}  // extern "C"
