// Host-side launchers of the QSA kernels.  Arguments are validated by the
// C ABI layer (qsa_api.hip) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qsa {

struct PagedKV {
    const uint16_t* k;        // bf16 rows, or fp8 E4M3 rows when kv_fp8 (the same address)
    const uint16_t* v;
    int kv_fp8;               // K and V hold fp8 E4M3 codes (256 B per row) instead of bf16
    void* ckey;               // block keys of type ckey_type
    int ckey_type;            // 0 fp32, 1 bf16, 2 fp8 E4M3 (kKeyF32 / kKeyBF16 / kKeyFP8)
    const int32_t* block_table;
    const int32_t* seq_lens;
    int batch, Hkv, lg_ps, num_pages, max_pages, max_seq_len;
};

struct Rows {
    const uint16_t* q;        // bf16 [R] rows of [Hq][256]
    int64_t q_stride;         // elements between rows
    const int32_t* q_seq;     // NULL: row r is sequence r
    const int32_t* q_pos;     // NULL: t = L - 1
    int R, Hq;
};

// span: host bound on the tokens per sequence from first_token on
hipError_t launch_compress(const PagedKV& kv, const int32_t* first_token, int span, hipStream_t st);

// refresh: decode rows only; also rebuilds the block key holding each sequence's newest token
hipError_t launch_scores_stream(const PagedKV& kv, const Rows& rows, float* scores, int score_stride, bool refresh,
                                hipStream_t st);
hipError_t launch_scores_tiled(const PagedKV& kv, const Rows& rows, float* scores, int score_stride,
                               hipStream_t st);

hipError_t launch_topk(const float* scores, int score_stride, const int32_t* q_pos, int R, int Hkv, int k,
                       int32_t* sel_idx, int32_t* sel_cnt, hipStream_t st);
// two-stage select for long rows through a candidate workspace of
// topk_workspace_bytes() bytes (0: one stage, same as launch_topk)
size_t topk_workspace_bytes(int R, int Hkv, int k, int score_stride);
hipError_t launch_topk_split(const float* scores, int score_stride, const int32_t* q_pos, int R, int Hkv, int k,
                             int32_t* sel_idx, int32_t* sel_cnt, void* workspace, hipStream_t st);

struct AttnOut {
    uint16_t* out;            // bf16, final result (num_splits == 1 and part_out == NULL)
    int64_t out_stride;
    float* lse;               // [R][Hq] or NULL
    float* part_out;          // fp32 [S][R][Hq][256] (partials)
    float* part_lse;          // fp32 [S][R][Hq]
};

// num_splits work units per (row, KV head); blocked: split s takes the
// contiguous range [s, s+1) * ceil(k / S) of the k selection slots, else the
// token slots p with p mod S == s
hipError_t launch_attn(const PagedKV& kv, const Rows& rows, const int32_t* sel_idx, const int32_t* sel_cnt, int k,
                       float scale, int num_splits, bool blocked, const AttnOut& o, hipStream_t st);

// Extend attention over the union of each tile of consecutive rows' selections
// (same result set as launch_attn with one split; outputs bf16 out, lse)
hipError_t launch_attn_union(const PagedKV& kv, const Rows& rows, const int32_t* sel_idx, const int32_t* sel_cnt, int k,
                             float scale, uint16_t* out, int64_t out_stride, float* lse, hipStream_t st);

// Fused decode (scores, top-k, attention, merge in one persistent launch) with S
// attention splits per (row, KV head); workspace laid out by fused_workspace_bytes,
// its first fused_control_bytes zero before the call and zero after it.
size_t fused_workspace_bytes(int batch, int Hkv, int Hq, int max_seq_len, int S);
size_t fused_control_bytes(int batch, int Hkv);
hipError_t launch_fused_decode(const PagedKV& kv, const Rows& rows, int k, float scale, int S, int32_t* sel_idx,
                               int32_t* sel_cnt, uint16_t* out, int64_t out_stride, float* lse, void* workspace,
                               hipStream_t st);

hipError_t launch_merge(const float* part_out, const float* part_lse, int S, int N, int D, uint16_t* out,
                        float* out_lse, hipStream_t st);

}  // namespace qsa
