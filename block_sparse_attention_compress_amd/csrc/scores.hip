// a2 -- block scores: s[r][h][b] = (sum of the group's query heads) . ckey[b].
//
// The indexer scores the compressed blocks against the query ("Qwen 4 QSA
// krijgt decode-contextparallellisme", section "Wat de pull request
// daadwerkelijk verandert"); the pages do not say how the query heads of a KV
// group are combined, and the library scores with their sum (one selection per
// KV head).  Scores are left unscaled: the softmax scale does not change the
// order.
//
// Two kernels, both fp32:
//  * scores_stream_kernel (decode): one row reads its whole block-key list once.
//    This is the dominant HBM stream of a decode step.  A wave takes 16 blocks
//    (16 KiB of fp32 keys; 8 KiB bf16, 4 KiB fp8) at a time, each lane 4 dims of
//    each block, and folds the 16 dot products with a reduce-scatter butterfly
//    (17 lane exchanges for 16 blocks instead of 16 x 6).  Its REFRESH form also
//    rebuilds the block key of each sequence's newest token from K (bf16 or fp8
//    rows) and scores that block with it, replacing a separate compress launch.
//  * scores_tiled_kernel (extend): many query rows share one sequence, so the
//    scores are a dense [rows x 256] . [256 x blocks] product; 16x16x4 fp32
//    matrix-core tiles, 16 rows per wave.
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

// Extend: 16 rows per wave, kTiledWaves waves (64 rows) per workgroup, and
// kTiledChunk blocks per workgroup (grid z), so a chunk of new tokens spreads
// over every CU.  Lane
// (c = lane & 15, kq = lane >> 4) holds, at k-step m, qsum[row c][64 kq + m] (A
// operand) and ckey[block c][64 kq + m] (B operand): the same dim for A and B, so
// the 64 steps of the 16x16x4 matrix-core op cover all 256 dims.  Output element
// i of the lane is row 4 kq + i, block c of the tile.
//
// When the workgroup's rows belong to one sequence (the usual extend chunk), its
// waves share each 16-block tile of keys: the threads load it together, it is
// staged in LDS (fp32, rows padded against bank conflicts), and two tiles are in
// flight while one is multiplied.  Otherwise each wave streams its own tiles, a
// quarter (16 dims) at a time so that this path needs few registers, and rows of
// one wave that belong to different sequences are scored in separate passes.
constexpr int kTiledChunk = 512;
constexpr int kTiledWaves = 4;  // waves (16 query rows each) per workgroup (8: slower)
constexpr int kTRow = kHeadDim + 4;  // padded key row of an LDS tile (floats)

template <int KT, int NW>
__global__ __launch_bounds__(64 * NW) void scores_tiled_kernel(
    const uint16_t* __restrict__ q, int64_t q_stride, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_pos, int R, int g, const void* __restrict__ ckey,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens, int Hkv, int lg_ps, int max_pages,
    float* __restrict__ scores, int score_stride) {
    __shared__ float ktile[2][16 * kTRow];
    __shared__ int w_smin[NW], w_smax[NW], w_nend[NW];
    constexpr int TPB = 4 * NW;        // threads per block key of a staged tile
    constexpr int FPT = 64 / TPB;      // float4 (Raw) pieces per thread
    typedef typename KeyRaw<KT>::type Raw;
    const Raw* keys = reinterpret_cast<const Raw*>(ckey);  // a block key is 64 Raw
    const int h = blockIdx.y;
    const int bc0 = blockIdx.z * kTiledChunk;  // this workgroup's first block
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = wave_id();
    const int r0 = blockIdx.x * (16 * NW) + wave * 16;
    const int c = lane & 15, kq = lane >> 4;
    const int row = r0 + c;
    const bool valid = row < R;
    const int seq_r = valid ? q_seq[row] : -1;
    const int t_r = valid ? q_pos[row] : -1;
    // rows whose eligible blocks all lie before this chunk take no part
    const int ne_row = valid && t_r >= 0 ? min(t_r / 4 + 1, score_stride) : 0;
    const bool live = ne_row > bc0;
    const int lg_bpp = lg_ps - 2;

    // ---- one sequence for the whole workgroup?  (decided before any wave leaves)
    {
        int smin = live ? seq_r : 0x7fffffff, smax = live ? seq_r : -1;
        int nend = live ? min(ne_row, bc0 + kTiledChunk) : 0;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            smin = min(smin, __shfl_xor(smin, o));
            smax = max(smax, __shfl_xor(smax, o));
            nend = max(nend, __shfl_xor(nend, o));
        }
        if (lane == 0) {
            w_smin[wave] = smin;
            w_smax[wave] = smax;
            w_nend[wave] = nend;
        }
    }
    __syncthreads();
    int smin = w_smin[0], smax = w_smax[0], wg_end = w_nend[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
        smin = min(smin, w_smin[w]);
        smax = max(smax, w_smax[w]);
        wg_end = max(wg_end, w_nend[w]);
    }
    if (smax < 0) return;  // no live row in the workgroup (uniform)

    float a[64];
#pragma unroll
    for (int m = 0; m < 64; ++m) a[m] = 0.f;
    if (live) {
        const uint16_t* qrow = q + (int64_t)row * q_stride + (int64_t)h * g * kHeadDim + 64 * kq;
        for (int j = 0; j < g; ++j) {
            const uint4* p = reinterpret_cast<const uint4*>(qrow + j * kHeadDim);
            uint4 ws[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) ws[i] = p[i];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint4 w = ws[i];
                a[8 * i + 0] += bf16_lo(w.x);
                a[8 * i + 1] += bf16_hi(w.x);
                a[8 * i + 2] += bf16_lo(w.y);
                a[8 * i + 3] += bf16_hi(w.y);
                a[8 * i + 4] += bf16_lo(w.z);
                a[8 * i + 5] += bf16_hi(w.z);
                a[8 * i + 6] += bf16_lo(w.w);
                a[8 * i + 7] += bf16_hi(w.w);
            }
        }
    }

    if (smin == smax) {
        // ---- shared tiles through LDS; every wave stays to the end (barriers)
        const int s = smin;
        const int nb_seq = (seq_lens[s] + 3) >> 2;
        const int ne_c = live ? ne_row : 0;
        int ne_out[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ne_out[i] = __shfl(ne_c, 4 * kq + i);
        const int wave_end = min(wave_max_int(ne_c), bc0 + kTiledChunk);
        const int ntiles = (wg_end - bc0 + 15) / 16;
        // this thread's share of a tile: block bl, float4 slots f0 + 16 j of its key
        const int bl = tid / TPB, f0 = tid % TPB;
        auto load = [&](int t, Raw* gr) {
            const int b = bc0 + 16 * t + bl;
            if (b < nb_seq) {
                const int64_t page = block_table[(int64_t)s * max_pages + (b >> lg_bpp)];
                const int64_t brow = ((page * Hkv + h) << lg_bpp) + (b & ((1 << lg_bpp) - 1));
                const Raw* src = keys + brow * (kHeadDim / 4) + f0;
#pragma unroll
                for (int j = 0; j < FPT; ++j) gr[j] = src[TPB * j];
            } else {
#pragma unroll
                for (int j = 0; j < FPT; ++j) gr[j] = Raw{};
            }
        };
        auto stage = [&](int slot, const Raw* gr) {
            float* dst = ktile[slot] + bl * kTRow + 4 * f0;
#pragma unroll
            for (int j = 0; j < FPT; ++j) *reinterpret_cast<float4*>(dst + 4 * TPB * j) = key4(gr[j]);
        };
        auto compute = [&](int t, int slot) {
            const int bt0 = bc0 + 16 * t;
            if (bt0 >= wave_end) return;  // this wave's rows are done (uniform per wave)
            const float* src = ktile[slot] + c * kTRow + 64 * kq;
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float4 kv = *reinterpret_cast<const float4*>(src + 4 * i);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[4 * i + 0], kv.x, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[4 * i + 1], kv.y, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[4 * i + 2], kv.z, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[4 * i + 3], kv.w, acc, 0, 0, 0);
            }
            const int b = bt0 + c;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (b < ne_out[i]) scores[((int64_t)(r0 + 4 * kq + i) * Hkv + h) * score_stride + b] = acc[i];
        };
        // two register sets (named, so nothing is indexed across iterations) and two
        // LDS slots: tile t is multiplied from slot t % 2 while tiles t + 1 and t + 2
        // are in flight
        Raw g0[FPT], g1[FPT];
        load(0, g0);
        if (ntiles > 1) load(1, g1);
        stage(0, g0);
        __syncthreads();
        for (int t = 0; t < ntiles; t += 2) {
            if (t + 2 < ntiles) load(t + 2, g0);
            compute(t, 0);
            if (t + 1 < ntiles) stage(1, g1);
            __syncthreads();
            if (t + 1 >= ntiles) break;
            if (t + 3 < ntiles) load(t + 3, g1);
            compute(t + 1, 1);
            if (t + 2 < ntiles) stage(0, g0);
            __syncthreads();
        }
        return;
    }

    // ---- rows of several sequences: each wave streams its own tiles
    if (r0 >= R || !__ballot(live)) return;
    uint64_t pending = __ballot(live && kq == 0) & 0xffffull;
    while (pending) {
        const int first = __builtin_ctzll(pending);
        const int s = __shfl(seq_r, first);
        const uint64_t active = __ballot(kq == 0 && live && seq_r == s) & 0xffffull;
        pending &= ~active;
        const int nb_seq = (seq_lens[s] + 3) >> 2;
        const int ne_c = ((active >> c) & 1) ? ne_row : 0;
        const int n_end = min(wave_max_int(ne_c), bc0 + kTiledChunk);
        int ne_out[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ne_out[i] = __shfl(ne_c, 4 * kq + i);
        // a quarter of the keys of the tile at bt0 (dims 64 kq + 16 qt .. + 15 of
        // block bt0 + c) into v, raw (zeros past the sequence).  One quarter is in
        // flight while the previous one is multiplied, which keeps this path's
        // registers (and so the kernel's) low.
        auto load_q = [&](int bt0, int qt, Raw* v) {
            const int b = bt0 + c;
            if (b < nb_seq) {
                const int64_t page = block_table[(int64_t)s * max_pages + (b >> lg_bpp)];
                const int64_t brow = ((page * Hkv + h) << lg_bpp) + (b & ((1 << lg_bpp) - 1));
                const Raw* src = keys + brow * (kHeadDim / 4) + 16 * kq + 4 * qt;
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = src[i];
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = Raw{};
            }
        };
        // k-steps 16 qt .. 16 qt + 15 of the 16x16x4 product
        auto mma_q = [&](int qt, const Raw* v, floatx4& acc) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 kv = key4(v[i]);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[16 * qt + 4 * i + 0], kv.x, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[16 * qt + 4 * i + 1], kv.y, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[16 * qt + 4 * i + 2], kv.z, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[16 * qt + 4 * i + 3], kv.w, acc, 0, 0, 0);
            }
        };
        Raw qa[4], qb[4];
        if (bc0 < n_end) load_q(bc0, 0, qa);
        for (int bt0 = bc0; bt0 < n_end; bt0 += 16) {
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
            load_q(bt0, 1, qb);
            mma_q(0, qa, acc);
            load_q(bt0, 2, qa);
            mma_q(1, qb, acc);
            load_q(bt0, 3, qb);
            mma_q(2, qa, acc);
            if (bt0 + 16 < n_end) load_q(bt0 + 16, 0, qa);
            mma_q(3, qb, acc);
            const int b = bt0 + c;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rr = 4 * kq + i;
                if (b < ne_out[i]) scores[((int64_t)(r0 + rr) * Hkv + h) * score_stride + b] = acc[i];
            }
        }
    }
}

hipError_t launch_scores_stream(const PagedKV& kv, const Rows& rows, float* scores, int score_stride, bool refresh,
                                hipStream_t st) {
    if (rows.R == 0) return hipSuccess;
    dim3 grid((score_stride + kStreamChunk - 1) / kStreamChunk, kv.Hkv, rows.R);
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

hipError_t launch_scores_tiled(const PagedKV& kv, const Rows& rows, float* scores, int score_stride,
                               hipStream_t st) {
    if (rows.R == 0) return hipSuccess;
    dim3 grid((rows.R + 16 * kTiledWaves - 1) / (16 * kTiledWaves), kv.Hkv, (score_stride + kTiledChunk - 1) / kTiledChunk);
#define QSA_TILED(KT)                                                                                            \
    hipLaunchKernelGGL((scores_tiled_kernel<KT, kTiledWaves>), grid, dim3(64 * kTiledWaves), 0, st, rows.q,       \
                       rows.q_stride, rows.q_seq,                                                                \
                       rows.q_pos, rows.R, rows.Hq / kv.Hkv, kv.ckey, kv.block_table, kv.seq_lens, kv.Hkv, kv.lg_ps, \
                       kv.max_pages, scores, score_stride)
    if (kv.ckey_type == kKeyFP8)
        QSA_TILED(kKeyFP8);
    else if (kv.ckey_type == kKeyBF16)
        QSA_TILED(kKeyBF16);
    else
        QSA_TILED(kKeyF32);
#undef QSA_TILED
    return hipGetLastError();
}

}  // namespace qsa
