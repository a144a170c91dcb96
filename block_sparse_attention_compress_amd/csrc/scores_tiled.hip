// a2 -- block scores for extend rows: s[r][h][b] = (sum of the group's query
// heads) . ckey[b], for many query rows of one sequence at once.
//
// The indexer scores the compressed blocks against the query ("Qwen 4 QSA
// krijgt decode-contextparallellisme", section "Wat de pull request
// daadwerkelijk verandert"); with many query rows per sequence (an extend
// chunk) the scores are a dense [rows x 256] . [256 x blocks] product, so they
// run on matrix cores.  Results are fp32, as the decode scan's.
#include "qsa_device.h"
#include "qsa_launch.h"
#include "scan_body.h"

namespace qsa {

// 16 rows per wave, kTiledWaves waves (64 rows) per workgroup, and `chunk`
// blocks per workgroup (grid z), so a chunk of new tokens spreads over every CU:
// kTiledChunk, or fewer when the grid would otherwise be small (few rows, or
// short contexts), where each workgroup's chain of tiles and not the matrix
// cores sets the time.  The chunk halves while the grid holds fewer than 512
// workgroups, down to 256 blocks, then while it holds fewer than 256, down to
// 32.  Measured on one 32,768-token sequence, (12,1) heads (us, before -> after
// the second step): 16 rows 22.7 -> 15.3, 64 rows 28.1 -> 21.1, 128 rows
// 29.0 -> 24.2, 512 rows 47.3 -> 42.6; one target of 256 workgroups for every
// row count made 2,048 rows slower (94 -> 110), one of 512 with 32-block
// chunks made 128-256 rows slower (31 -> 40 at 256).
//
// When the workgroup's rows belong to one sequence (the usual extend chunk), its
// waves share each 16-block tile of keys: the threads load it together, it is
// staged in LDS, and two tiles are in flight while one is multiplied.  The
// product runs on bf16 matrix cores (v_mfma_f32_16x16x32_bf16) with fp32
// accuracy: every fp32 operand x is split exactly into three bf16 pieces
// x = x1 + x2 + x3 (x1 = bf16(x), x2 = bf16(x - x1), x3 = x - x1 - x2, each step
// exact), the products of two bf16 values are exact in fp32, and
//   q . k = q1.k1 + (q1.k2 + q2.k1 + q1.k3 + q2.k2 + q3.k1) + (terms below 2^-24 |q||k|)
// with the first dot product in one fp32 accumulator and the five smaller ones
// in another, so the rounding error is that of an fp32 dot product of the same
// length.  bf16 and fp8 block keys are exact bf16 values: one key piece, three
// products.  Lane (c = lane & 15, kq = lane >> 4) holds, for k-slice m, dims
// 32 m + 8 kq .. + 7 of query row c (A) and of block c of the tile (B); output
// element i of the lane is row 4 kq + i, block c.
//
// Otherwise (rows of several sequences in one workgroup) each wave streams its
// own tiles in fp32 on 16x16x4 fp32 matrix cores, a quarter (16 dims) at a time
// so that this path needs few registers; there lane (c, kq) holds, at k-step m,
// dims 64 kq + m of row c (A) and of block c (B).  Rows of one wave that belong
// to different sequences are scored in separate passes.
constexpr int kTiledChunk = 1024;  // blocks per workgroup (at most)
constexpr int kTiledMidChunk = 256;  // the chunk's floor while the grid is below kTiledMinGrid
constexpr int kTiledMinGrid = 512;
constexpr int kTiledMinChunk = 32;   // the chunk's floor while the grid is below kTiledFewGrid
constexpr int kTiledFewGrid = 256;
constexpr int kTiledWaves = 4;  // waves (16 query rows each) per workgroup (8: slower)
constexpr int kSRow = kHeadDim + 8;  // padded key row of an LDS tile plane (bf16 elements)
// pages of one sequence that a chunk's blocks can span (4-token pages: one per block)
constexpr int kTiledPages = kTiledChunk + 1;

// (a, b) -> their first N bf16 pieces, packed (a in the low half of each word):
// piece 1 = bf16(x), piece 2 = bf16(x - piece 1), piece 3 = bf16(x - piece 1 -
// piece 2).  Each difference is exact in fp32, and for N = 3 the pieces sum to x
// exactly (an fp32 significand has 24 bits, a bf16 one 8); N = 1 is the plain
// rounding.  Piece p of both values comes from one hardware conversion (round to
// nearest even, as f32_to_bf16_rne for finite values) and the remainders from the
// packed word: about 5.5 vector instructions per value for three pieces, against
// 14.5 with the integer rounding (fp32-key C4 scores 162 -> 150 us, the 7,810-row
// prefill 1.107 -> 1.012 ms, scores bit-equal).
template <int N>
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t* w) {
#pragma unroll
    for (int p = 0; p < N; ++p) {
        w[p] = pack_bf16x2_hw(a, b);
        if (p + 1 < N) {
            a -= __uint_as_float(w[p] << 16);
            b -= __uint_as_float(w[p] & 0xffff0000u);
        }
    }
}

template <int KT, int NW>
__global__ __launch_bounds__(64 * NW) void scores_tiled_kernel(
    const uint16_t* __restrict__ q, int64_t q_stride, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_pos, int R, int g, const void* __restrict__ ckey,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens, int Hkv, int lg_ps, int max_pages,
    float* __restrict__ scores, int score_stride, int chunk) {
    constexpr int NP = KT == kKeyF32 ? 3 : 1;  // bf16 pieces of a key element
    __shared__ __attribute__((aligned(16))) uint16_t ktile[2][NP][16 * kSRow];
    __shared__ int64_t ptab[kTiledPages];  // block-table entries of the chunk (one-sequence path)
    __shared__ int w_smin[NW], w_smax[NW], w_nend[NW];
    constexpr int TPB = 4 * NW;        // threads per block key of a staged tile
    constexpr int FPT = 64 / TPB;      // float4 (Raw) pieces per thread
    typedef typename KeyRaw<KT>::type Raw;
    const Raw* keys = reinterpret_cast<const Raw*>(ckey);  // a block key is 64 Raw
    const int h = blockIdx.y;
    const int bc0 = blockIdx.z * chunk;  // this workgroup's first block
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
        int nend = live ? min(ne_row, bc0 + chunk) : 0;
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
    // the group sum in head order; two heads' loads are in flight at a time
    // SLICED: lane dims 32 m + 8 kq + i at a[8 m + i] (the bf16 path), else dims
    // 64 kq + i at a[i] (the fp32 path)
    auto sum_query = [&](bool sliced) {
        if (!live) return;
        const uint16_t* qrow = q + (int64_t)row * q_stride + (int64_t)h * g * kHeadDim + (sliced ? 8 : 64) * kq;
        const int step = sliced ? 32 : 8;  // elements between the lane's 8-element pieces
        auto add_head = [&](const uint4* ws) {
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
        };
        for (int j = 0; j < g; j += 2) {
            const uint16_t* p0 = qrow + j * kHeadDim;
            const uint16_t* p1 = qrow + min(j + 1, g - 1) * kHeadDim;
            uint4 w0[8], w1[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) w0[i] = *reinterpret_cast<const uint4*>(p0 + step * i);
#pragma unroll
            for (int i = 0; i < 8; ++i) w1[i] = *reinterpret_cast<const uint4*>(p1 + step * i);
            add_head(w0);
            if (j + 1 < g) add_head(w1);
        }
    };

    if (smin == smax) {
        // ---- shared tiles through LDS; every wave stays to the end (barriers)
        const int s = smin;
        const int nb_seq = (seq_lens[s] + 3) >> 2;
        const int ne_c = live ? ne_row : 0;
        int ne_out[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ne_out[i] = __shfl(ne_c, 4 * kq + i);
        const int wave_end = min(wave_max_int(ne_c), bc0 + chunk);
        const int ntiles = (wg_end - bc0 + 15) / 16;
        // the block-table entries of the chunk's blocks [bc0, min(wg_end, nb_seq)) go to
        // LDS first, so that no key load waits on a dependent table load in the loop
        if (nb_seq <= bc0) return;  // (uniform) only with a position past its sequence's end
        const int bmax = min(wg_end, nb_seq) - 1;  // >= bc0; pages past the sequence are never read
        const int p0 = bc0 >> lg_bpp;
        for (int i = tid; i <= (bmax >> lg_bpp) - p0; i += 64 * NW)
            ptab[i] = block_table[(int64_t)s * max_pages + p0 + i];
        __syncthreads();
        // this thread's share of a tile: block bl, float4 slots f0 + 16 j of its key.
        // Blocks past the sequence load its last block instead: their scores are
        // never stored (every row's eligible blocks end inside the sequence).
        const int bl = tid / TPB, f0 = tid % TPB;
        auto load = [&](int t, Raw* gr) {
            const int b = min(bc0 + 16 * t + bl, bmax);
            const int64_t page = ptab[(b >> lg_bpp) - p0];
            const int64_t brow = ((page * Hkv + h) << lg_bpp) + (b & ((1 << lg_bpp) - 1));
            const Raw* src = keys + brow * (kHeadDim / 4) + f0;
#pragma unroll
            for (int j = 0; j < FPT; ++j) gr[j] = src[TPB * j];
        };
        bf16x8 qp[3][8];  // the query's three bf16 pieces, k-slice m at qp[piece][m]
        // staging: the key elements as bf16 pieces, plane p holding piece p + 1
        auto stage = [&](int slot, const Raw* gr) {
#pragma unroll
            for (int j = 0; j < FPT; ++j) {
                const int off = bl * kSRow + 4 * (f0 + TPB * j);
                if (KT == kKeyBF16) {
                    *reinterpret_cast<Raw*>(&ktile[slot][0][off]) = gr[j];  // already bf16
                } else {
                    const float4 x = key4(gr[j]);
                    const float e[4] = {x.x, x.y, x.z, x.w};
                    uint32_t w[NP][2];
#pragma unroll
                    for (int u = 0; u < 4; u += 2) {
                        uint32_t pw[NP];
                        split_bf16x2<NP>(e[u], e[u + 1], pw);
#pragma unroll
                        for (int pl = 0; pl < NP; ++pl) w[pl][u / 2] = pw[pl];
                    }
#pragma unroll
                    for (int pl = 0; pl < NP; ++pl)
                        *reinterpret_cast<uint2*>(&ktile[slot][pl][off]) = make_uint2(w[pl][0], w[pl][1]);
                }
            }
        };
        auto compute = [&](int t, int slot) {
            const int bt0 = bc0 + 16 * t;
            if (bt0 >= wave_end) return;  // this wave's rows are done (uniform per wave)
            floatx4 hi = {0.f, 0.f, 0.f, 0.f}, lo = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                bf16x8 kb[NP];
#pragma unroll
                for (int pl = 0; pl < NP; ++pl)
                    kb[pl] = *reinterpret_cast<const bf16x8*>(&ktile[slot][pl][c * kSRow + 32 * m + 8 * kq]);
                hi = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qp[0][m], kb[0], hi, 0, 0, 0);
                lo = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qp[1][m], kb[0], lo, 0, 0, 0);
                lo = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qp[2][m], kb[0], lo, 0, 0, 0);
                if (NP == 3) {
                    lo = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qp[0][m], kb[NP > 1 ? 1 : 0], lo, 0, 0, 0);
                    lo = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qp[1][m], kb[NP > 1 ? 1 : 0], lo, 0, 0, 0);
                    lo = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qp[0][m], kb[NP > 2 ? 2 : 0], lo, 0, 0, 0);
                }
            }
            const int b = bt0 + c;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (b < ne_out[i]) scores[((int64_t)(r0 + 4 * kq + i) * Hkv + h) * score_stride + b] = hi[i] + lo[i];
        };
        // two register sets (named, so nothing is indexed across iterations) and two
        // LDS slots: tile t is multiplied from slot t % 2 while tiles t + 1 and t + 2
        // are in flight
        Raw g0[FPT], g1[FPT];
        load(0, g0);  // the first key tiles fly while the group-summed query is formed
        if (ntiles > 1) load(1, g1);
        sum_query(true);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            uint32_t w[3][4];
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
                uint32_t pw[3];
                split_bf16x2<3>(a[8 * m + i], a[8 * m + i + 1], pw);
#pragma unroll
                for (int pl = 0; pl < 3; ++pl) w[pl][i / 2] = pw[pl];
            }
#pragma unroll
            for (int pl = 0; pl < 3; ++pl) qp[pl][m] = __builtin_bit_cast(bf16x8, make_uint4(w[pl][0], w[pl][1], w[pl][2], w[pl][3]));
        }
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
    sum_query(false);
    uint64_t pending = __ballot(live && kq == 0) & 0xffffull;
    while (pending) {
        const int first = __builtin_ctzll(pending);
        const int s = __shfl(seq_r, first);
        const uint64_t active = __ballot(kq == 0 && live && seq_r == s) & 0xffffull;
        pending &= ~active;
        const int nb_seq = (seq_lens[s] + 3) >> 2;
        const int ne_c = ((active >> c) & 1) ? ne_row : 0;
        const int n_end = min(wave_max_int(ne_c), bc0 + chunk);
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

hipError_t launch_scores_tiled(const PagedKV& kv, const Rows& rows, float* scores, int score_stride,
                               hipStream_t st) {
    if (rows.R == 0) return hipSuccess;
    const int64_t row_tiles = (rows.R + 16 * kTiledWaves - 1) / (16 * kTiledWaves);
    auto grid_of = [&](int ch) { return row_tiles * kv.Hkv * ((score_stride + ch - 1) / ch); };
    int chunk = kTiledChunk;
    while (chunk > kTiledMidChunk && grid_of(chunk) < kTiledMinGrid) chunk /= 2;
    while (chunk > kTiledMinChunk && grid_of(chunk) < kTiledFewGrid) chunk /= 2;
    dim3 grid((unsigned)row_tiles, kv.Hkv, (score_stride + chunk - 1) / chunk);
#define QSA_TILED(KT)                                                                                            \
    hipLaunchKernelGGL((scores_tiled_kernel<KT, kTiledWaves>), grid, dim3(64 * kTiledWaves), 0, st, rows.q,       \
                       rows.q_stride, rows.q_seq,                                                                \
                       rows.q_pos, rows.R, rows.Hq / kv.Hkv, kv.ckey, kv.block_table, kv.seq_lens, kv.Hkv, kv.lg_ps, \
                       kv.max_pages, scores, score_stride, chunk)
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
