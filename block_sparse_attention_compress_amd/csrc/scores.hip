// a2 -- block scores for decode: s[r][h][b] = (sum of the group's query heads) . ckey[b].
//
// The indexer scores the compressed blocks against the query ("Qwen 4 QSA
// krijgt decode-contextparallellisme", section "Wat de pull request
// daadwerkelijk verandert"); the pages do not say how the query heads of a KV
// group are combined, and the library scores with their sum (one selection per
// KV head).  Scores are left unscaled: the softmax scale does not change the
// order.
//
// scores_stream_kernel: one row reads its whole block-key list once.  This is
// the dominant HBM stream of a decode step.  A wave takes 16 blocks (16 KiB of
// fp32 keys; 8 KiB bf16, 4 KiB fp8) at a time, each lane 4 dims of each block,
// and folds the 16 dot products with a reduce-scatter butterfly (17 lane
// exchanges for 16 blocks instead of 16 x 6).  Its REFRESH form also rebuilds
// the block key of each sequence's newest token from K (bf16 or fp8 rows) and
// scores that block with it, replacing a separate compress launch.  Extend
// rows are scored by scores_tiled_kernel (scores_tiled.hip).
#include "qsa_device.h"
#include "qsa_launch.h"
#include "scan_body.h"

namespace qsa {

template <bool PAGE16, int KT, bool REFRESH>
__global__ __launch_bounds__(256) void scores_stream_kernel(
    const uint16_t* __restrict__ q, int64_t q_stride, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_pos, int g, const void* ckey, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, int Hkv, int lg_ps, int max_pages, float* __restrict__ scores,
    int score_stride, const void* __restrict__ kcache, int kv8) {
    const int row = blockIdx.z;
    const int h = blockIdx.y;
    const int seq = q_seq ? q_seq[row] : row;
    const int L = seq_lens[seq];
    const int t = q_pos ? q_pos[row] : L - 1;
    if (t < 0) return;
    const int n_elig = min(t / 4 + 1, score_stride);
    constexpr int kStreamChunk = stream_chunk(KT);
    const int chunk0 = blockIdx.x * kStreamChunk;
    if (chunk0 >= n_elig) return;
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int wb0 = chunk0 + wave * (kStreamChunk / 4);  // this wave's first block
    if (wb0 >= n_elig) return;
    __shared__ float4 stash[REFRESH ? 4 * 64 : 1];
    Refresh rf;
    if (REFRESH) {
        // decode rows (t = L - 1): the newest token's block is rebuilt by the wave
        // that scores it, or by the row's first wave when the row is cut short
        const int b = t >> 2;
        const bool scored = b < n_elig;
        if (scored ? (wb0 <= b && b < wb0 + kStreamChunk / 4) : wb0 == 0) {
            rf.k = kcache;
            rf.kv8 = kv8 != 0;
            rf.ckey = const_cast<void*>(ckey);
            rf.b = b;
            rf.n = L - 4 * b;
            rf.score = scored;
            rf.stash = stash + wave * 64;
        }
    }
    scan_wave<PAGE16, false, KT, REFRESH>(q + (int64_t)row * q_stride + (int64_t)h * g * kHeadDim, g, ckey,
                                            block_table + (int64_t)seq * max_pages, Hkv, h, lg_ps, n_elig, wb0, lane,
                                            scores + ((int64_t)row * Hkv + h) * score_stride, rf);
}

hipError_t launch_scores_stream(const PagedKV& kv, const Rows& rows, float* scores, int score_stride, bool refresh,
                                hipStream_t st) {
    if (rows.R == 0) return hipSuccess;
    const int chunk = stream_chunk(kv.ckey_type);
    dim3 grid((score_stride + chunk - 1) / chunk, kv.Hkv, rows.R);
    const bool page16 = kv.lg_ps >= 6;
#define QSA_SCAN(P16, KT, RF)                                                                                      \
    hipLaunchKernelGGL((scores_stream_kernel<P16, KT, RF>), grid, dim3(256), 0, st, rows.q, rows.q_stride,          \
                       rows.q_seq, rows.q_pos, rows.Hq / kv.Hkv, kv.ckey, kv.block_table, kv.seq_lens, kv.Hkv,      \
                       kv.lg_ps, kv.max_pages, scores, score_stride, kv.k, kv.kv_fp8)
#define QSA_SCAN_RF(P16, KT)          \
    do {                              \
        if (refresh)                  \
            QSA_SCAN(P16, KT, true);  \
        else                          \
            QSA_SCAN(P16, KT, false); \
    } while (0)
#define QSA_SCAN_KT(P16)                   \
    do {                                   \
        if (kv.ckey_type == kKeyFP8)       \
            QSA_SCAN_RF(P16, kKeyFP8);     \
        else if (kv.ckey_type == kKeyBF16) \
            QSA_SCAN_RF(P16, kKeyBF16);    \
        else                               \
            QSA_SCAN_RF(P16, kKeyF32);     \
    } while (0)
    if (page16)
        QSA_SCAN_KT(true);
    else
        QSA_SCAN_KT(false);
#undef QSA_SCAN_KT
#undef QSA_SCAN_RF
#undef QSA_SCAN
    return hipGetLastError();
}

}  // namespace qsa
