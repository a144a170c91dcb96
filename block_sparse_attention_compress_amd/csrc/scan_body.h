// One wave's share of the decode block-score scan: 16 blocks at a time, each
// lane one float4 of each block key, 16 dot products folded by a reduce-scatter
// butterfly.  Used by scores_stream_kernel and by the fused decode kernel.
// The keys are read once per step: their loads carry the nontemporal hint
// (measured at 32 sequences of 32K-64K tokens: 140 -> 122 us).
#pragma once

#include "qsa_device.h"

namespace qsa {

// Blocks per workgroup (4 waves, each a run of 16-block groups), by block-key
// type.  fp32 keys: 64 (a 16-block group is 16 KiB; with nontemporal key loads,
// 32 rows of 32K-64K tokens, (16,2) heads: 256 / 128 / 64 blocks took
// 127.8 / 124.5 / 122.5 us, and 8 rows of 256K tokens 167.2 / 164.1 / 163.4 us).
// bf16 and fp8 keys make a group 8 KiB and 4 KiB, and want more of them per
// wave: 128 blocks (same workloads, 64 / 128 / 256 blocks: bf16 keys at 32 rows
// 67.8 / 67.8 / 71.1 us, at 8 rows 94.3 / 86.1 / 85.9 us; fp8 keys at 32 rows
// 41.9 / 36.8 / 38.2 us, at 8 rows 55.0 / 46.5 / 46.3 us).
__host__ __device__ constexpr int stream_chunk(int kt) { return kt == kKeyF32 ? 64 : 128; }

// Scores of blocks [wb0, wb0 + 16 kGroups) ∩ [0, n_elig) of one (row, KV head):
//   srow[b] = (sum of the g query heads at qrow) . ckey[b]
// qrow: the row's first query head of the group (bf16 [g][256]); bt: the
// sequence's block-table row.  Requires wb0 < n_elig.
// PAGE16: a page holds >= 16 blocks (page_size >= 64).  A wave's group of 16
// blocks starts 16-aligned, so it lies in one page: one block-table lookup gives
// 16 KiB of contiguous block keys, and the loads need no per-block branch (slots
// past the row end are still inside the page; their sums are never written).
// COHERENT: scores are stored at device scope (written through to where every
// CU reads them), for a reader in another workgroup of the same launch.
// KT: block-key type.  bf16 keys are 8 bytes per lane and block, fp8 E4M3 keys
// 4 bytes (16 for fp32); they are kept raw until the dot product, so the next
// group's loads still fly while a group is reduced.
// REFRESH: the wave named by `rf` first rebuilds one block key from the K cache
// (the block holding a sequence's newest token), stores it, and scores that
// block with it in place of the stored, stale key.
template <int KT>
struct KeyRaw {
    typedef float4 type;
    static __device__ __forceinline__ float4 from(const float4& m) { return m; }
};
template <>
struct KeyRaw<kKeyBF16> {
    typedef uint2 type;
    static __device__ __forceinline__ uint2 from(const float4& m) {
        return make_uint2(pack_bf16x2(m.x, m.y), pack_bf16x2(m.z, m.w));
    }
};
template <>
struct KeyRaw<kKeyFP8> {
    typedef uint32_t type;
    static __device__ __forceinline__ uint32_t from(const float4& m) { return pack_fp8x4(m.x, m.y, m.z, m.w); }
};

struct Refresh {
    const void* k = nullptr;      // K cache [num_pages][Hkv][page_size][256], bf16 or fp8 E4M3 (kv8)
    bool kv8 = false;
    void* ckey = nullptr;         // block keys, written
    int b = -1;                   // block to rebuild (-1: none in this wave)
    int n = 0;                    // its tokens, 1..4
    bool score = false;           // b is one of the blocks this wave scores
    float4* stash = nullptr;      // this wave's 64 x 16 bytes of LDS: the rebuilt key until it is scored
};
__device__ __forceinline__ float4 key4(const float4& x) { return x; }
__device__ __forceinline__ float4 key4(const uint2& x) {
    return make_float4(bf16_lo(x.x), bf16_hi(x.x), bf16_lo(x.y), bf16_hi(x.y));
}
__device__ __forceinline__ float4 key4(const uint32_t& x) { return unpack_fp8x4(x); }

template <bool PAGE16, bool COHERENT = false, int KT = kKeyF32, bool REFRESH = false>
__device__ __forceinline__ void scan_wave(const uint16_t* __restrict__ qrow, int g, const void* ckey,
                                          const int32_t* __restrict__ bt, int Hkv, int h, int lg_ps, int n_elig,
                                          int wb0, int lane, float* __restrict__ srow, const Refresh& rf = Refresh{}) {
    typedef typename KeyRaw<KT>::type Raw;
    const Raw* keys = reinterpret_cast<const Raw*>(ckey);  // a block key is 64 Raw
    const int lg_bpp = lg_ps - 2;  // blocks per page = page_size / 4
    // block-key rows of the wave's groups (PAGE16), looked up before any wait
    constexpr int kGroups = stream_chunk(KT) / 64;  // 16-block groups per wave
    int64_t gbase[kGroups];
    if (PAGE16) {
#pragma unroll
        for (int grp = 0; grp < kGroups; ++grp) {
            const int b0 = min(wb0 + grp * 16, n_elig - 1) & ~15;
            gbase[grp] = (((int64_t)bt[b0 >> lg_bpp] * Hkv + h) << lg_bpp) + (b0 & ((1 << lg_bpp) - 1));
        }
    }

    auto load_group = [&](int grp, Raw* v) {
        const int b0 = wb0 + grp * 16;
        if (PAGE16) {
            const Raw* src = keys + gbase[grp] * (kHeadDim / 4) + lane;
#pragma unroll
            for (int j = 0; j < 16; ++j) v[j] = load_stream(&src[j * (kHeadDim / 4)]);
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int b = min(b0 + j, n_elig - 1);
                const int64_t page = bt[b >> lg_bpp];
                const int64_t brow = ((page * Hkv + h) << lg_bpp) + (b & ((1 << lg_bpp) - 1));
                v[j] = load_stream(&keys[brow * (kHeadDim / 4) + lane]);
            }
        }
    };
    // the first group's block keys are requested before the query
    Raw v[16];
    load_group(0, v);

    if (REFRESH && rf.b >= 0) {
        // the block's tokens are consecutive rows of one page; lane: dims 4 lane .. 4 lane + 3
        const int64_t pos0 = 4 * (int64_t)rf.b;
        const int64_t row = (((int64_t)bt[pos0 >> lg_ps] * Hkv + h) << lg_ps) + (pos0 & ((1 << lg_ps) - 1));
        float4 kt[4];  // the lane's 4 dims of each token, exact
        if (rf.kv8) {
            const uint32_t* src = reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(rf.k) + row * kHeadDim) + lane;
            uint32_t a[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) a[u] = u < rf.n ? src[u * (kHeadDim / 4)] : 0u;
#pragma unroll
            for (int u = 0; u < 4; ++u) kt[u] = unpack_fp8x4(a[u]);
        } else {
            const uint2* src = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(rf.k) + row * kHeadDim) + lane;
            uint2 a[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) a[u] = u < rf.n ? src[u * (kHeadDim / 4)] : make_uint2(0, 0);
#pragma unroll
            for (int u = 0; u < 4; ++u) kt[u] = make_float4(bf16_lo(a[u].x), bf16_hi(a[u].x), bf16_lo(a[u].y), bf16_hi(a[u].y));
        }
        float4 m;
        m.x = block_mean(kt[0].x, kt[1].x, kt[2].x, kt[3].x, rf.n);
        m.y = block_mean(kt[0].y, kt[1].y, kt[2].y, kt[3].y, rf.n);
        m.z = block_mean(kt[0].z, kt[1].z, kt[2].z, kt[3].z, rf.n);
        m.w = block_mean(kt[0].w, kt[1].w, kt[2].w, kt[3].w, rf.n);
        const Raw fresh = KeyRaw<KT>::from(m);
        // block-key row in [num_pages][Hkv][page_size / 4][256]
        const int64_t brow = ((row >> lg_ps) << (lg_ps - 2)) + ((row & ((1 << lg_ps) - 1)) >> 2);
        reinterpret_cast<Raw*>(rf.ckey)[brow * (kHeadDim / 4) + lane] = fresh;
        // parked in LDS rather than held in registers through the loop
        if (rf.score) reinterpret_cast<Raw*>(rf.stash)[lane] = fresh;
    }

    // group-summed query: lane holds dims 4*lane .. 4*lane+3; the g loads are
    // issued together (one wait), summed in head order
    float4 qs = make_float4(0.f, 0.f, 0.f, 0.f);
    {
        const uint16_t* qp = qrow + 4 * lane;
        uint2 qw[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) qw[j] = j < g ? *reinterpret_cast<const uint2*>(qp + j * kHeadDim) : make_uint2(0, 0);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            qs.x += bf16_lo(qw[j].x);
            qs.y += bf16_hi(qw[j].x);
            qs.z += bf16_lo(qw[j].y);
            qs.w += bf16_hi(qw[j].y);
        }
    }

    for (int grp = 0; grp < kGroups; ++grp) {
        const int b0 = wb0 + grp * 16;
        if (b0 >= n_elig) break;
        if (REFRESH && rf.score && ((rf.b - wb0) >> 4) == grp) {
            const int jf = (rf.b - wb0) & 15;
            const Raw fresh = reinterpret_cast<const Raw*>(rf.stash)[lane];
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (j == jf) v[j] = fresh;
        }
        // explicit fused multiply-adds: every instantiation rounds the same way
        float p[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float4 kv = key4(v[j]);
            p[j] = fmaf(qs.w, kv.w, fmaf(qs.z, kv.z, fmaf(qs.y, kv.y, qs.x * kv.x)));
        }
        // the next group's loads fly while this group is reduced
        if (grp < kGroups - 1 && b0 + 16 < n_elig) load_group(grp + 1, v);
        // reduce-scatter: after the step across lane bit m (m = 5, 4, 3, 2) a lane
        // keeps the half of its blocks selected by that bit; finally lane l holds
        // the full sum of block l >> 2 (lanes differing in bits 0, 1 agree).  Each
        // block's partial sums only ever meet each other.
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const bool up = lane & 32;
            const float keep = up ? p[i + 8] : p[i], send = up ? p[i] : p[i + 8];
            p[i] = keep + __shfl_xor(send, 32);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool up = lane & 16;
            const float keep = up ? p[i + 4] : p[i], send = up ? p[i] : p[i + 4];
            p[i] = keep + __shfl_xor(send, 16);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const bool up = lane & 8;
            const float keep = up ? p[i + 2] : p[i], send = up ? p[i] : p[i + 2];
            p[i] = keep + __shfl_xor(send, 8);
        }
        {
            const bool up = lane & 4;
            const float keep = up ? p[1] : p[0], send = up ? p[0] : p[1];
            p[0] = keep + __shfl_xor(send, 4);
        }
        p[0] += __shfl_xor(p[0], 2);
        p[0] += __shfl_xor(p[0], 1);
        const int b = b0 + (lane >> 2);
        if ((lane & 3) == 0 && b < n_elig) {
            if (COHERENT)
                __hip_atomic_store(srow + b, p[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else
                srow[b] = p[0];
        }
    }
}

}  // namespace qsa
