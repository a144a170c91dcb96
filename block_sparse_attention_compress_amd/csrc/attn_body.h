// Exact softmax attention of one (row, KV head, split) work unit over the tokens
// of its selected blocks.  Used by attn_kernel (decode and extend) and by the
// fused decode kernel.  The design (matrix-core tiles, lazy-rescaled online
// softmax, LDS staging) is described at the top of attn.hip.
#pragma once

#include "qsa_device.h"

namespace qsa {

constexpr int kAttnWaves = 4;
// Slot-table entries past a work unit's last token, all -1: the tile pipeline
// reads the slots of each wave's next tile unclamped, up to 16 kAttnWaves + 15
// past the last one.
constexpr int kSlotPad = 16 * kAttnWaves + 16;
constexpr int kMaxSel = 2048;
constexpr float kLazy = 8.0f;  // log2 of the largest unnormalised weight
constexpr int kKRow = kHeadDim + 8;   // padded K row in the LDS tile (elements): spreads rows over banks
constexpr int kKRow8 = kHeadDim + 8;  // padded fp8 row in the LDS tile (bytes)
// bytes of one staged row: bf16 rows for a bf16 cache, raw codes for an fp8 cache
template <bool KV8>
constexpr int kTileRowBytes = KV8 ? kKRow8 : 2 * kKRow;
// LDS bytes of the 4 waves' K and V staging tiles
__host__ __device__ constexpr size_t attn_tile_bytes(bool kv8) {
    return (size_t)kAttnWaves * 2 * 16 * (kv8 ? kTileRowBytes<true> : kTileRowBytes<false>);
}
// An fp8 cache's kernel keeps the query operand in LDS (16 padded bf16 rows after
// the tiles) rather than in 32 registers, which fits it in 168 registers: 3 waves
// per SIMD, and 3 workgroups per CU within the LDS.  A bf16 cache's loop is bound
// by its L2 gathers, not by latency, and keeps the query in registers.
constexpr int kQRow = kHeadDim + 8;  // padded query row in LDS (elements)
__host__ __device__ constexpr size_t attn_q_bytes(bool kv8) { return kv8 ? (size_t)16 * kQRow * 2 : 0; }
// LDS bytes of the loop: slot table, staging tiles, query rows (fp8 cache)
__host__ __device__ constexpr size_t attn_loop_bytes(int table_words, bool kv8) {
    return (size_t)table_words * 4 + attn_tile_bytes(kv8) + attn_q_bytes(kv8);
}

typedef short bf16x4s __attribute__((ext_vector_type(4)));

struct AttnParams {
    const uint16_t* k;
    const uint16_t* v;
    const int32_t* block_table;
    const int32_t* seq_lens;
    int Hkv, lg_ps, max_pages;
    const uint16_t* q;
    int64_t q_stride;
    const int32_t* q_seq;
    const int32_t* q_pos;
    int R, Hq, g;
    const int32_t* sel;
    const int32_t* cnt;
    int kstride;
    float scale_log2;
    int S;
    int blocked;  // 1: split s takes a contiguous range of selected blocks; 0: token slots p mod S
    int table_words;  // int32 words of LDS reserved for the slot table
    uint16_t* out;
    int64_t out_stride;
    float* lse;
    float* part_out;
    float* part_lse;
};

__device__ __forceinline__ uint32_t u4_word(const uint4& a, int w) {
    return w == 0 ? a.x : (w == 1 ? a.y : (w == 2 ? a.z : a.w));
}

// Raw K / V tile registers: 8 bf16 (or 8 fp8 E4M3 codes) of one row per lane.
template <bool KV8>
struct KVRaw {
    typedef uint4 type;
};
template <>
struct KVRaw<true> {
    typedef uint2 type;
};

// 8 elements as bf16.  fp8 codes are widened exactly (every E4M3 value is a bf16
// value), two per instruction: the scaled fp8 -> bf16 conversion with a scale of
// 1 takes the two codes of one 16-bit half of a word (low half: first code in
// the low bf16).
__device__ __forceinline__ uint4 kv_bf16x8(const uint4& x) { return x; }
__device__ __forceinline__ uint4 kv_bf16x8(const uint2& x) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.x, 1.0f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.x, 1.0f, true);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.y, 1.0f, false);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.y, 1.0f, true);
    return make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, c),
                      __builtin_bit_cast(uint32_t, d));
}

// LDS: `smem` is dynamic shared memory of the launch: the slot table (16 B per
// selected block of this work unit and kSlotPad entries of -1, P.table_words
// int32) and the 4 waves' K and V
// staging tiles, later reused for the waves' O exchange (4 waves x g heads x
// 1 KiB); the launch sizes it to the larger need.  Ends with a barrier-free
// write of the result; the caller separates work units sharing `smem` with a
// barrier.
template <bool KV8>
__device__ __forceinline__ void attend_split(const AttnParams& P, int row, int h, int s, float* smem) {
    __shared__ float wm[kAttnWaves][16], wl[kAttnWaves][16], h_inv[16], h_lse[16];
    int32_t* slot_row = reinterpret_cast<int32_t*>(smem);
    const int S = P.S;
    const int seq = P.q_seq ? P.q_seq[row] : row;
    const int L = P.seq_lens[seq];
    const int t = P.q_pos ? P.q_pos[row] : L - 1;
    const int64_t lim = min((int64_t)L, (int64_t)t + 1);  // tokens at positions < lim are visible
    const int g = P.g;
    const int tid = threadIdx.x;

    const int lane = tid & 63;
    const int wave = wave_id();
    const int c = lane & 15;
    const int qq = lane >> 4;

    // The query, the count and the selection are independent reads: issue them
    // together.  Blocked splits cut the k selection slots (not the count), so the
    // selection reads need not wait for the count.
    bf16x8 qb[8];
    uint16_t* qlds = reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(smem + P.table_words) + attn_tile_bytes(KV8));
    if constexpr (KV8) {
        // 16 rows of 256 dims (rows g..15 zero), 16 bytes per thread and pass;
        // read back by the loop after the slot table's barrier
        const uint16_t* qp = P.q + (int64_t)row * P.q_stride + (int64_t)h * g * kHeadDim;
#pragma unroll
        for (int e = tid; e < 16 * (kHeadDim / 8); e += 256) {
            const int hh = e / (kHeadDim / 8), d = 8 * (e % (kHeadDim / 8));
            const bf16x8 x = hh < g ? *reinterpret_cast<const bf16x8*>(qp + hh * kHeadDim + d) : bf16x8{};
            *reinterpret_cast<bf16x8*>(qlds + hh * kQRow + d) = x;
        }
    } else {
        const uint16_t* qp = P.q + (int64_t)row * P.q_stride + (int64_t)(h * g + min(c, g - 1)) * kHeadDim + 8 * qq;
#pragma unroll
        for (int m = 0; m < 8; ++m) qb[m] = *reinterpret_cast<const bf16x8*>(qp + 32 * m);
        if (c >= g) {
#pragma unroll
            for (int m = 0; m < 8; ++m) qb[m] = bf16x8{};
        }
    }
    const int cnt_raw = P.cnt[(int64_t)row * P.Hkv + h];
    int jb = 0, jcap = P.kstride;
    if (P.blocked) {
        const int per = (P.kstride + S - 1) / S;
        jb = min(P.kstride, s * per);
        jcap = min(P.kstride, jb + per);
    }
    const int32_t* sel_row = P.sel + ((int64_t)row * P.Hkv + h) * P.kstride;
    constexpr int kIt = kMaxSel / 256;
    int bsel[kIt];
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
        const int j = jb + tid + 256 * it;
        bsel[it] = j < jcap ? sel_row[j] : -1;
    }
    // selected blocks [jb, je) feed this workgroup; the table holds their slots
    const int nsel = max(0, min(cnt_raw, P.kstride));
    const int je = max(jb, min(nsel, jcap));
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
        const int j = jb + tid + 256 * it;
        if (j >= je) break;
        const int b = bsel[it];
        const int64_t pos0 = 4 * (int64_t)b;
        int32_t base = 0;
        int nv = 0;
        if (b >= 0 && pos0 < lim) {
            base = (int32_t)token_row(P.block_table, seq, P.max_pages, P.Hkv, h, P.lg_ps, pos0);
            nv = (int)min(lim - pos0, (int64_t)4);
        }
        *reinterpret_cast<int4*>(slot_row + 4 * (j - jb)) = make_int4(
            nv > 0 ? base : -1, nv > 1 ? base + 1 : -1, nv > 2 ? base + 2 : -1, nv > 3 ? base + 3 : -1);
    }
    for (int i = tid; i < kSlotPad; i += 256) slot_row[4 * (je - jb) + i] = -1;
    __syncthreads();

    // split-local slot n lives at table entry slot0 + sstep * n
    const int ntok = 4 * (je - jb);
    int n_s, slot0, sstep;
    if (P.blocked) {
        n_s = ntok;
        slot0 = 0;
        sstep = 1;
    } else {
        n_s = ntok > s ? (ntok - s + S - 1) / S : 0;
        slot0 = s;
        sstep = S;
    }
    const int ntiles = (n_s + 15) / 16;
    typedef typename KVRaw<KV8>::type Raw;  // 8 elements of a row, as loaded and as staged
    // this wave's K and V staging tiles: 16 rows of RB bytes each
    constexpr int RB = kTileRowBytes<KV8>;
    constexpr int EB = KV8 ? 1 : 2;  // bytes per element
    uint8_t* ktile = reinterpret_cast<uint8_t*>(smem + P.table_words) + wave * 2 * 16 * RB;
    uint8_t* vtile = ktile + 16 * RB;

    float m_run = -INFINITY;  // reference max of head c (log2 units), same in every qq group
    float l_run = 0.f;        // this lane's share of the head's normaliser
    floatx4 O[16];
#pragma unroll
    for (int nt = 0; nt < 16; ++nt) O[nt] = floatx4{0.f, 0.f, 0.f, 0.f};

    // One 16-token tile, staged in this wave's LDS tiles: S^T = K Q^T, the online
    // softmax, O += P V.  Bit i of `live` clear masks token 4 qq + i (its staged
    // bytes may be anything: its weight and its V slice are zeroed).
    auto compute_tile = [&](int live) {
        auto k_operand = [&](int m) {
            const uint4 x = kv_bf16x8(*reinterpret_cast<const Raw*>(ktile + c * RB + EB * (32 * m + 8 * qq)));
            return __builtin_bit_cast(bf16x8, x);
        };
        // ---- S^T = K . Q^T: st[i] = S[head c][token n0 + 4 qq + i]
        floatx4 st = {0.f, 0.f, 0.f, 0.f};
        {
            bf16x8 kb[8];
#pragma unroll
            for (int m = 0; m < 8; ++m) kb[m] = k_operand(m);
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const bf16x8 qm = KV8 ? *reinterpret_cast<const bf16x8*>(qlds + c * kQRow + 32 * m + 8 * qq) : qb[m];
                st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[m], qm, st, 0, 0, 0);
            }
        }
        uint4 vv[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint8_t* vr = vtile + (4 * qq + i) * RB + EB * 8 * c;
            vv[i][0] = kv_bf16x8(*reinterpret_cast<const Raw*>(vr));
            vv[i][1] = kv_bf16x8(*reinterpret_cast<const Raw*>(vr + EB * 128));
        }
        float x[4];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = (live >> i) & 1 ? st[i] * P.scale_log2 : -INFINITY;
            mx = fmaxf(mx, x[i]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        // ---- lazy rescale: only when some head's max passes its reference by 2^8
        if (__ballot(mx > m_run + kLazy)) {
            const float m_new = mx > m_run + kLazy ? fmaxf(m_run, mx) : m_run;
            const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float a_i = __shfl(alpha, 4 * qq + i);
#pragma unroll
                for (int nt = 0; nt < 16; ++nt) O[nt][i] *= a_i;
            }
        }
        const float m_use = m_run == -INFINITY ? 0.f : m_run;
        uint32_t pw[2];
        float psum = 0.f;
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            pw[w] = pack_bf16x2_hw(__builtin_amdgcn_exp2f(x[2 * w] - m_use),
                                   __builtin_amdgcn_exp2f(x[2 * w + 1] - m_use));
            psum += bf16_lo(pw[w]) + bf16_hi(pw[w]);
        }
        l_run += psum;
        // ---- zero the V of masked slots (their weight is 0, their bytes may be anything)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (!((live >> i) & 1)) {
                vv[i][0] = make_uint4(0, 0, 0, 0);
                vv[i][1] = make_uint4(0, 0, 0, 0);
            }
        // ---- O += P . V; k-slot i of lane (., qq) is token n0 + 4 qq + i
        bf16x4s pa;
        {
            uint32_t* p32 = reinterpret_cast<uint32_t*>(&pa);
            p32[0] = pw[0];
            p32[1] = pw[1];
        }
#pragma unroll
        for (int nt = 0; nt < 16; ++nt) {
            const int hf = nt >> 3, e = (nt & 7) >> 1;  // dim 128 hf + 8c + (nt & 7): dword e of half hf
            const uint32_t d0 = u4_word(vv[0][hf], e), d1 = u4_word(vv[1][hf], e);
            const uint32_t d2 = u4_word(vv[2][hf], e), d3 = u4_word(vv[3][hf], e);
            bf16x4s vb;
            uint32_t* v32 = reinterpret_cast<uint32_t*>(&vb);
            // one byte permute per word: the low (even nt) or high (odd nt) bf16 of
            // each of two tokens' dwords
            constexpr uint32_t kLo = 0x05040100u, kHi = 0x07060302u;
            v32[0] = __builtin_amdgcn_perm(d1, d0, (nt & 1) ? kHi : kLo);
            v32[1] = __builtin_amdgcn_perm(d3, d2, (nt & 1) ? kHi : kLo);
            O[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, O[nt], 0, 0, 0);
        }
    };

    // Raw tile loads are coalesced -- instruction j covers tile rows 2j and 2j+1
    // (1 KiB of bf16, 512 B of fp8) -- and land in this wave's LDS tiles, from
    // which the MFMA layouts are read.  The loads of tile i+1 are issued before
    // tile i is computed, so a wave always has a tile in flight.  fp8 rows are
    // staged as codes and widened to bf16 as the MFMA operands are read, which
    // halves their LDS traffic.
    // (the raw tile is 16 named registers, not an array: an array indexed in a
    // loop across the tile pipeline was kept in scratch memory)
    Raw k0, k1, k2, k3, k4, k5, k6, k7, v0, v1, v2, v3, v4, v5, v6, v7;
    // The slot reads are unconditional, so that a tile's LDS reads issue back to
    // back rather than one round trip per load, and the next tile's are issued
    // before this tile's staging writes.  The index is clamped to the last slot,
    // and a slot past the split's end loads row 0 (bf16 rows: one cached line);
    // `live` masks those tokens (their weight and V slice are zeroed).
    // fp8 rows, whose loop is bound by its vector-ALU work and its loads in flight
    // rather than by the gathers, use a leaner form (C4 extend attention 380-431
    // -> 360-368 us; with bf16 rows the same form measured 2-3 % slower): with a slot
    // step of 1 (the split's slots are consecutive table entries from 0) the
    // table is read directly -- the kSlotPad entries after the last slot are -1 --
    // from two addresses with immediate offsets, and no load tests its slot
    // against the split's end: a slot past it reads -1 or the last slot's cache
    // row, both inside the cache (-1 reads row 0).  With no slot at all
    // (n_s == 0) nothing is loaded.
    const int last_slot = max(n_s - 1, 0);
    // this lane's bytes of a row, folded into the K and V bases (fp8 rows)
    const uint8_t* kb_lane = reinterpret_cast<const uint8_t*>(P.k) + sizeof(Raw) * (lane & 31);
    const uint8_t* vb_lane = reinterpret_cast<const uint8_t*>(P.v) + sizeof(Raw) * (lane & 31);
    int n0_, rr_[8], lv_[4];
#define QSA_SLOT(N) slot_row[slot0 + sstep * min((N), last_slot)]
#define QSA_SLOTS(TILE, DIRECT)                                                             \
    do {                                                                                    \
        n0_ = (TILE) * 16;                                                                  \
        if constexpr (DIRECT) {                                                             \
            const int32_t* sr_ = slot_row + n0_ + (lane >> 5);                              \
            _Pragma("unroll") for (int j_ = 0; j_ < 8; ++j_) rr_[j_] = sr_[2 * j_];         \
            const int4 l4_ = *reinterpret_cast<const int4*>(slot_row + n0_ + 4 * qq);      \
            lv_[0] = l4_.x;                                                                 \
            lv_[1] = l4_.y;                                                                 \
            lv_[2] = l4_.z;                                                                 \
            lv_[3] = l4_.w;                                                                 \
        } else {                                                                            \
            _Pragma("unroll") for (int j_ = 0; j_ < 8; ++j_) rr_[j_] = QSA_SLOT(n0_ + 2 * j_ + (lane >> 5)); \
            _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_) lv_[i_] = QSA_SLOT(n0_ + 4 * qq + i_); \
        }                                                                                   \
    } while (0)
#define QSA_LOAD_J(J, KX, VX)                                                               \
    do {                                                                                    \
        if constexpr (KV8) {                                                                \
            const int64_t off = (int64_t)max(rr_[J], 0) * (kHeadDim * EB);                  \
            KX = *reinterpret_cast<const Raw*>(kb_lane + off);                              \
            VX = *reinterpret_cast<const Raw*>(vb_lane + off);                              \
        } else {                                                                            \
            const int rr = n0_ + 2 * (J) + (lane >> 5) < n_s ? rr_[J] : -1;                 \
            const int64_t off = (int64_t)max(rr, 0) * kHeadDim * EB + sizeof(Raw) * (lane & 31); \
            KX = *reinterpret_cast<const Raw*>(reinterpret_cast<const uint8_t*>(P.k) + off); \
            VX = *reinterpret_cast<const Raw*>(reinterpret_cast<const uint8_t*>(P.v) + off); \
        }                                                                                   \
    } while (0)
#define QSA_LOAD_RAW(LIVE)                                                                  \
    do {                                                                                    \
        QSA_LOAD_J(0, k0, v0);                                                              \
        QSA_LOAD_J(1, k1, v1);                                                              \
        QSA_LOAD_J(2, k2, v2);                                                              \
        QSA_LOAD_J(3, k3, v3);                                                              \
        QSA_LOAD_J(4, k4, v4);                                                              \
        QSA_LOAD_J(5, k5, v5);                                                              \
        QSA_LOAD_J(6, k6, v6);                                                              \
        QSA_LOAD_J(7, k7, v7);                                                              \
        /* which of the tokens 4 qq + i, whose scores / weights this lane owns, are live */ \
        LIVE = 0;                                                                           \
        _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_)                                    \
            LIVE |= (n0_ + 4 * qq + i_ < n_s && lv_[i_] >= 0) << i_;                         \
    } while (0)
#define QSA_STAGE_J(J, KX, VX)                                                              \
    do {                                                                                    \
        const int r = 2 * (J) + (lane >> 5);                                                \
        *reinterpret_cast<Raw*>(ktile + r * RB + sizeof(Raw) * (lane & 31)) = KX;           \
        *reinterpret_cast<Raw*>(vtile + r * RB + sizeof(Raw) * (lane & 31)) = VX;           \
    } while (0)
// The tile pipeline.  DIRECT: the split's slots are table entries 0, 1, 2, ...
// (slot step 1), read without a clamp (fp8 rows).
#define QSA_TILE_LOOP(DIRECT)                                                               \
    do {                                                                                    \
        if (!KV8 || n_s > 0) { /* bf16 rows test each load's slot against n_s */           \
            QSA_SLOTS(wave, DIRECT);                                                        \
            QSA_LOAD_RAW(live_next);                                                        \
        }                                                                                   \
        for (int tile = wave; tile < ntiles; tile += kAttnWaves) {                          \
            QSA_SLOTS(tile + kAttnWaves, DIRECT);                                           \
            QSA_STAGE_J(0, k0, v0);                                                         \
            QSA_STAGE_J(1, k1, v1);                                                         \
            QSA_STAGE_J(2, k2, v2);                                                         \
            QSA_STAGE_J(3, k3, v3);                                                         \
            QSA_STAGE_J(4, k4, v4);                                                         \
            QSA_STAGE_J(5, k5, v5);                                                         \
            QSA_STAGE_J(6, k6, v6);                                                         \
            QSA_STAGE_J(7, k7, v7);                                                         \
            const int live = live_next;                                                     \
            QSA_LOAD_RAW(live_next);                                                        \
            compute_tile(live);                                                             \
        }                                                                                   \
    } while (0)
    int live_next;
    if constexpr (KV8) {
        if (sstep == 1)
            QSA_TILE_LOOP(true);
        else
            QSA_TILE_LOOP(false);
    } else {
        QSA_TILE_LOOP(false);
    }
#undef QSA_TILE_LOOP
#undef QSA_LOAD_RAW
#undef QSA_LOAD_J
#undef QSA_SLOT
#undef QSA_SLOTS
#undef QSA_STAGE_J

    // ---- merge the 4 waves in LDS.  Per head: M = the largest reference max of
    // the waves that saw a token; wave w's O and l are scaled by 2^(m_w - M)
    // before the exchange, so the final pass only adds the 4 slots and
    // multiplies by 1 / sum(l).
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    __syncthreads();  // the slot table is dead; smem becomes the O exchange
    if (qq == 0) {
        wm[wave][c] = m_run;
        wl[wave][c] = l_tot;
    }
    __syncthreads();
    const float kLn2 = 0.6931471805599453f;
    auto head_max = [&](int hh) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, wl[w][hh] > 0.f ? wm[w][hh] : -INFINITY);
        return M;
    };
    if (wave == 0 && qq == 0 && c < g) {  // one lane per head: 1 / sum(l) and the lse
        const float M = head_max(c);
        float den = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < kAttnWaves; ++w)
                if (wl[w][c] > 0.f) den += __builtin_amdgcn_exp2f(wm[w][c] - M) * wl[w][c];
        }
        h_inv[c] = M != -INFINITY ? 1.0f / den : 0.f;
        h_lse[c] = M != -INFINITY ? (M + __log2f(den)) * kLn2 : -INFINITY;
    }
    // this lane's O: heads 4 qq + i, dims 128 hf + 8 c + j at O[8 hf + j][i]
    float* ow = smem + wave * g * kHeadDim;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int hh = 4 * qq + i;
        if (hh < g) {
            const float M = head_max(hh);
            const float f = wl[wave][hh] > 0.f ? __builtin_amdgcn_exp2f(wm[wave][hh] - M) : 0.f;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                float4* dst = reinterpret_cast<float4*>(ow + hh * kHeadDim + 128 * hf + 8 * c);
                dst[0] = make_float4(O[8 * hf + 0][i] * f, O[8 * hf + 1][i] * f, O[8 * hf + 2][i] * f,
                                     O[8 * hf + 3][i] * f);
                dst[1] = make_float4(O[8 * hf + 4][i] * f, O[8 * hf + 5][i] * f, O[8 * hf + 6][i] * f,
                                     O[8 * hf + 7][i] * f);
            }
        }
    }
    __syncthreads();

    // thread: 4 consecutive dims of one head per pass
    const float4* o4 = reinterpret_cast<const float4*>(smem);
    const bool out8 = ((reinterpret_cast<uintptr_t>(P.out) | (uintptr_t)(P.out_stride * 2)) & 7) == 0;
    for (int e = tid; e < g * (kHeadDim / 4); e += 256) {
        const int hh = e >> 6;
        const int d = 4 * (e & 63);
        float4 acc = o4[hh * 64 + (e & 63)];
#pragma unroll
        for (int w = 1; w < kAttnWaves; ++w) {
            const float4 x = o4[(w * g + hh) * 64 + (e & 63)];
            acc.x += x.x;
            acc.y += x.y;
            acc.z += x.z;
            acc.w += x.w;
        }
        const float inv = h_inv[hh];
        const float4 o = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
        const int head = h * g + hh;
        if (P.part_out) {
            const int64_t prow = ((int64_t)s * P.R + row) * P.Hq + head;
            *reinterpret_cast<float4*>(P.part_out + prow * kHeadDim + d) = o;
            if (d == 0) P.part_lse[prow] = h_lse[hh];
        } else {
            uint16_t* dst = P.out + (int64_t)row * P.out_stride + (int64_t)head * kHeadDim + d;
            if (out8) {
                *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2_hw(o.x, o.y), pack_bf16x2_hw(o.z, o.w));
            } else {
                dst[0] = (uint16_t)f32_to_bf16_rne(o.x);
                dst[1] = (uint16_t)f32_to_bf16_rne(o.y);
                dst[2] = (uint16_t)f32_to_bf16_rne(o.z);
                dst[3] = (uint16_t)f32_to_bf16_rne(o.w);
            }
            if (d == 0 && P.lse) P.lse[(int64_t)row * P.Hq + head] = h_lse[hh];
        }
    }
}

}  // namespace qsa
