// Fused decode: block scores, top-k selection, sparse attention and the
// log-sum-exp merge of one decode step in a single persistent launch.
//
// The method's steps are those of the separate entry points (the indexer scores
// 4-token microblocks, the best 512 are kept, exact attention runs over their
// uncompressed K/V, split partials are combined at the end: "Qwen 4 QSA krijgt
// decode-contextparallellisme", section "Wat de pull request daadwerkelijk
// verandert").  What the fusion removes is the idle time between them: with one
// launch per step, the chip waits at every boundary for the slowest (row, KV
// head), the top-k (a few workgroups, latency-bound) runs on an otherwise empty
// GPU, and every attention workgroup starts with the same dependent loads at the
// same moment.  Here the top-k of a unit overlaps the scoring of the others.
//
// Work items, in ticket order (a global counter hands them out, so an item is
// only ever taken after every item before it):
//   scan item (u, c)   the block scores of chunk c (stream_chunk blocks) of unit u, the
//                      code of scores_stream_kernel, stored at device scope.
//                      The last chunk of u to finish (arrival counter) runs the
//                      top-k of u and raises u's ready flag.
//   attention (u, s)   waits for u's ready flag, then split s of u's selected
//                      blocks (contiguous range) as in attn_kernel, written as a
//                      partial (o, lse).  The last split to finish merges u's
//                      partials into the bf16 output and lse.
// All scan items precede all attention items: an attention item taken while its
// unit is still being scored holds a workgroup slot idle, and interleaving them
// (attention of unit u after the scans of unit u + D) measured slower for every
// lag D tried.  A waiting item only waits for items with lower tickets, which
// running workgroups hold, so the wait always ends.  It is still bounded: an item
// whose wait times out counts it in the workspace and writes a NaN partial in
// place of its split, so the unit's output and lse come out NaN rather than
// computed from a selection that may not be there yet.
//
// Flags carry the call's epoch instead of 0 / 1: the workspace holds a call
// counter E, a unit's selection raises its ready word to E + 1, and attention
// items wait for exactly that value.  A ready word left by an earlier call (even
// one raised late, after a time-out) holds at most E and never satisfies a later
// wait.  The arrival counters and the ticket counters are returned to zero by
// their last user, and the last workgroup out advances E, so the workspace needs
// no clearing between calls.
//
// Top-k of a unit (256 threads, scores read back from memory): an LDS histogram
// of the top 12 bits of the order-preserving keys gives the bin B holding the
// k-th largest; the blocks of the bins above B (all selected) and B's candidates
// are compacted in index order; a candidate is taken by its rank in (score
// descending, block index ascending) -- the order of qsa_topk_blocks -- and the
// two index lists are merged into the output by binary search.  A bin of more
// than 1,024 candidates (heavy ties) takes a pass-based path instead.
//
// Measured on MI355X (32 sequences of 32K-64K tokens, (16,2) heads) this path is
// slower than the separate calls, about 0.35 against 0.20 ms per step: a scan
// item in the persistent loop costs more than a scan workgroup of
// scores_stream_kernel, one 256-thread top-k takes some 30 us, and the last
// unit's top-k, attention and merge form a tail that the separate calls do not
// have.  It is kept as a correct single-launch alternative.
#include <stdlib.h>

#include "attn_body.h"
#include "block_ops.h"
#include "qsa_device.h"
#include "qsa_launch.h"
#include "scan_body.h"

namespace qsa {

constexpr int kFusedThreads = 256;
constexpr int kSelBins = 4096;     // top 12 bits of the order key
constexpr int kSelCap = 4096;      // threshold-bin keys kept in LDS (pass-based path)
constexpr int kSelRound = 8192;    // scores per register round: 32 per thread
constexpr int kSelRankCap = 1024;  // threshold-bin candidates ranked directly
// LDS of a selection: the histogram, then the candidates (64-bit), the two index
// lists (kMaxSel ints each) and scalars; the pass-based path needs 2 kSelBins + 32
constexpr int kSelLdsInts = (kSelBins > 2 * kSelRankCap ? kSelBins : 2 * kSelRankCap) + 2 * kMaxSel + 32;
static_assert(kSelLdsInts >= 2 * kSelBins + 32, "LDS of the pass-based selection");
constexpr int kSpinLimit = 1 << 20;  // polls of a ready flag (about a second) before a wait is abandoned

struct FusedParams {
    AttnParams A;  // blocked splits; partials into the workspace
    const uint16_t* q;
    int64_t q_stride;
    int g;
    const void* ckey;  // fp32 or bf16 block keys
    const int32_t* block_table;
    const int32_t* seq_lens;
    int Hkv, lg_ps, max_pages;
    float* scores;  // workspace [U][score_stride]
    int score_stride;
    int k;
    int32_t* sel_idx;
    int32_t* sel_cnt;
    uint16_t* out;
    int64_t out_stride;
    float* lse;
    int* ctl;  // [0] ticket, [1] workgroups finished, [2] abandoned waits, [3] call epoch
    int* unit_ctl;  // per unit, 4 ints: scan arrivals, ready word (epoch + 1), attention arrivals, unused
    int U, C, S, n_items;
    int spin_limit;  // polls of a ready word before the wait is abandoned
};

// Item i -> (scan?, unit, chunk or split): the U C scan items first, unit by
// unit, then the U S attention items.
__device__ __forceinline__ void decode_item(const FusedParams& F, int i, bool& scan, int& u, int& j) {
    const int sc = F.U * F.C;
    scan = i < sc;
    if (scan) {
        u = i / F.C;
        j = i % F.C;
    } else {
        u = (i - sc) / F.S;
        j = (i - sc) % F.S;
    }
}

// ---------------------------------------------------------------- selection

// The pass-based selection (any n, any crowding): every step re-reads the scores.
// Same contract as select_unit.
__device__ __forceinline__ void select_unit_passes(const float* __restrict__ s, int n, int k, int32_t* __restrict__ out,
                                   int32_t* __restrict__ cnt_out, int* lds) {
    const int tid = threadIdx.x;
    if (n <= k || k == 0) {  // all eligible blocks, or none
        const int c = min(n, k);
        for (int j = tid; j < k; j += kFusedThreads) out[j] = j < c ? j : -1;
        if (tid == 0) *cnt_out = c;
        return;
    }
    int* hist = lds;
    uint32_t* cand = reinterpret_cast<uint32_t*>(lds + kSelBins);
    int* misc = lds + kSelBins + kSelCap;  // [0..3] results, [8..15] block-scan scratch
    int* itmp = misc + 8;
    const float4* s4 = reinterpret_cast<const float4*>(s);
    const int n4 = (n + 3) / 4;  // float4 slots; elements past n are skipped

    // ---- histogram of the top 12 key bits
    for (int i = tid; i < kSelBins; i += kFusedThreads) hist[i] = 0;
    __syncthreads();
#pragma unroll 4
    for (int i4 = tid; i4 < n4; i4 += kFusedThreads) {
        const float4 x = s4[i4];
        const int b = 4 * i4;
        atomicAdd(&hist[order_key(x.x) >> 20], 1);
        if (b + 1 < n) atomicAdd(&hist[order_key(x.y) >> 20], 1);
        if (b + 2 < n) atomicAdd(&hist[order_key(x.z) >> 20], 1);
        if (b + 3 < n) atomicAdd(&hist[order_key(x.w) >> 20], 1);
    }
    __syncthreads();
    {
        // thread t owns bins [16 t, 16 t + 16)
        int local = 0;
#pragma unroll
        for (int b = 0; b < 16; ++b) local += hist[16 * tid + b];
        const int incl = block_suffix_sum<kFusedThreads / 64>(local, itmp);
        const int above = incl - local;
        if (above < k && k <= incl) {
            int cum = above;
            for (int b = 16 * tid + 15; b >= 16 * tid; --b) {
                if (cum + hist[b] >= k) {
                    misc[0] = b;
                    misc[1] = cum;
                    break;
                }
                cum += hist[b];
            }
        }
        if (tid == 0) misc[2] = 0;
        __syncthreads();
    }
    const int B = misc[0];
    const int m = hist[B];
    int need = k - misc[1];  // keys of bin B taken, >= 1
    uint32_t prefix = (uint32_t)B << 20;
    const bool in_lds = m <= kSelCap;
    if (in_lds) {
#pragma unroll 4
        for (int i4 = tid; i4 < n4; i4 += kFusedThreads) {
            const float4 x = s4[i4];
            const float e[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t key = order_key(e[c]);
                if (4 * i4 + c < n && (key >> 20) == (uint32_t)B) cand[atomicAdd(&misc[2], 1)] = key;
            }
        }
    }
    __syncthreads();  // hist[B] read by everyone; hist becomes the 1024-bin sub-histogram

    // ---- the low 20 bits of the k-th key: two 10-bit radix passes within bin B
    int* sub = hist;
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
        const int shift = pass == 0 ? 10 : 0;
        const uint32_t fixed = pass == 0 ? 0xFFF00000u : 0xFFFFFC00u;
        for (int i = tid; i < 1024; i += kFusedThreads) sub[i] = 0;
        __syncthreads();
        if (in_lds) {
            for (int i = tid; i < m; i += kFusedThreads) {
                const uint32_t key = cand[i];
                if ((key & fixed) == prefix) atomicAdd(&sub[(key >> shift) & 1023], 1);
            }
        } else {
            for (int i4 = tid; i4 < n4; i4 += kFusedThreads) {
                const float4 x = s4[i4];
                const float e[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint32_t key = order_key(e[c]);
                    if (4 * i4 + c < n && (key & fixed) == prefix) atomicAdd(&sub[(key >> shift) & 1023], 1);
                }
            }
        }
        __syncthreads();
        int local = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) local += sub[4 * tid + b];
        const int incl = block_suffix_sum<kFusedThreads / 64>(local, itmp);
        const int above = incl - local;
        if (above < need && need <= incl) {
            int cum = above;
            for (int b = 4 * tid + 3; b >= 4 * tid; --b) {
                if (cum + sub[b] >= need) {
                    misc[0] = b;
                    misc[1] = cum;
                    break;
                }
                cum += sub[b];
            }
        }
        __syncthreads();
        need -= misc[1];
        prefix |= (uint32_t)misc[0] << shift;
        __syncthreads();  // misc and sub are rewritten by the next pass
    }
    const uint32_t T = prefix;  // the k-th largest key
    const int need_eq = need;   // keys equal to T that are taken, lowest indices first

    // ---- ordered compaction: thread t owns indices [lo, hi), a multiple of 4 wide
    const int seg = (((n + kFusedThreads - 1) / kFusedThreads) + 3) & ~3;
    const int lo = min(n, tid * seg), hi = min(n, lo + seg);
    int gt = 0, eq = 0;
    for (int i = lo; i < hi; i += 4) {
        const float4 x = s4[i >> 2];
        const float e[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t key = order_key(e[c]);
            if (i + c < hi) {
                gt += key > T;
                eq += key == T;
            }
        }
    }
    block_exclusive_scan2<kFusedThreads / 64>(gt, eq, itmp);
    for (int i = lo; i < hi; i += 4) {
        const float4 x = s4[i >> 2];
        const float e[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t key = order_key(e[c]);
            if (i + c >= hi) continue;
            if (key > T) {
                out[gt + min(eq, need_eq)] = i + c;
                ++gt;
            } else if (key == T) {
                if (eq < need_eq) out[gt + eq] = i + c;
                ++eq;
            }
        }
    }
    if (tid == 0) *cnt_out = k;
}

// Index of the first element of a[0, n) (ascending) that is >= x.
__device__ __forceinline__ int lower_bound_lds(const int* a, int n, int x) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (a[mid] < x)
            lo = mid + 1;
        else
            hi = mid;
    }
    return lo;
}

// The (k, -1 padded) ascending selection of scores s[0, n) into out, count into
// *cnt_out.  lds: kSelLdsInts ints.  Thread t owns 32 consecutive scores of each
// round of 8,192 (8 float4 loads, all in flight together; a row of one round
// stays in registers).  Pass 1 histograms the top 12 key bits and finds the bin B
// holding the k-th key.  Pass 2 compacts, in index order (per-thread counts and a
// prefix sum), the blocks of bins above B -- all selected -- and B's (key, index)
// candidates; a candidate is taken iff fewer than k - |above| candidates precede
// it in (key descending, index ascending).  The two index-ordered lists are then
// merged by binary search straight into the output.  A bin of more than 1,024
// candidates goes to the pass-based path.
__device__ __forceinline__ void select_unit(const float* __restrict__ s, int n, int k, int32_t* __restrict__ out,
                            int32_t* __restrict__ cnt_out, int* lds) {
    const int tid = threadIdx.x;
    if (n <= k || k == 0) {  // all eligible blocks, or none
        const int c = min(n, k);
        for (int j = tid; j < k; j += kFusedThreads) out[j] = j < c ? j : -1;
        if (tid == 0) *cnt_out = c;
        return;
    }
    int* hist = lds;                                        // pass 1
    uint64_t* cand = reinterpret_cast<uint64_t*>(lds);      // pass 2 on: (~key << 32) | index
    int* above_list = lds + 2 * kSelRankCap;                // blocks of bins above B, ascending
    int* taken = above_list + kMaxSel;                      // taken candidates, ascending
    int* misc = taken + kMaxSel;                            // [0..7] scalars, [8..15] block-scan scratch
    int* itmp = misc + 8;
    const float4* s4 = reinterpret_cast<const float4*>(s);
    const int n4 = (n + 3) / 4;
    const int rounds = (n + kSelRound - 1) / kSelRound;
    constexpr int kPer = kSelRound / kFusedThreads;  // scores per thread and round
    uint32_t key[kPer];
    auto load = [&](int r) {
#pragma unroll
        for (int j = 0; j < kPer / 4; ++j) {
            // clamped, unconditional: all loads of the round are in flight at once
            const float4 x = s4[min(r * (kSelRound / 4) + (kPer / 4) * tid + j, n4 - 1)];
            key[4 * j + 0] = order_key(x.x);
            key[4 * j + 1] = order_key(x.y);
            key[4 * j + 2] = order_key(x.z);
            key[4 * j + 3] = order_key(x.w);
        }
    };
    const int base0 = kPer * tid;  // first index of this thread within a round

    // ---- pass 1: histogram of the top 12 key bits
    for (int i = tid; i < kSelBins; i += kFusedThreads) hist[i] = 0;
    __syncthreads();
    for (int r = 0; r < rounds; ++r) {
        load(r);
        const int i0 = r * kSelRound + base0;
#pragma unroll
        for (int e = 0; e < kPer; ++e)
            if (i0 + e < n) atomicAdd(&hist[key[e] >> 20], 1);
    }
    __syncthreads();
    {
        int local = 0;
#pragma unroll
        for (int b = 0; b < 16; ++b) local += hist[16 * tid + b];
        const int incl = block_suffix_sum<kFusedThreads / 64>(local, itmp);
        const int above = incl - local;
        if (above < k && k <= incl) {
            int cum = above;
            for (int b = 16 * tid + 15; b >= 16 * tid; --b) {
                if (cum + hist[b] >= k) {
                    misc[0] = b;
                    misc[1] = cum;
                    break;
                }
                cum += hist[b];
            }
        }
        __syncthreads();
    }
    const uint32_t B = (uint32_t)misc[0];
    const int above = misc[1];   // keys in bins above B: all selected
    const int m = hist[B];       // candidates
    const int need = k - above;  // candidates taken, >= 1
    __syncthreads();             // hist is read; cand overwrites it
    if (m > kSelRankCap) {
        select_unit_passes(s, n, k, out, cnt_out, lds);
        return;
    }

    // ---- pass 2: index-ordered compaction of the blocks above B and of B's candidates
    int a_base = 0, c_base = 0;
    for (int r = 0; r < rounds; ++r) {
        if (rounds > 1) load(r);
        const int i0 = r * kSelRound + base0;
        int na = 0, nc = 0;
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const uint32_t b = key[e] >> 20;
            na += (i0 + e < n) & (b > B);
            nc += (i0 + e < n) & (b == B);
        }
        int ao = na, co = nc;
        block_exclusive_scan2<kFusedThreads / 64>(ao, co, itmp);
        if (tid == kFusedThreads - 1) {
            misc[2] = ao + na;
            misc[3] = co + nc;
        }
        ao += a_base;
        co += c_base;
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const uint32_t b = key[e] >> 20;
            if (i0 + e < n && b > B) above_list[ao++] = i0 + e;
            if (i0 + e < n && b == B) cand[co++] = ((uint64_t)~key[e] << 32) | (uint32_t)(i0 + e);
        }
        __syncthreads();
        a_base += misc[2];
        c_base += misc[3];
        __syncthreads();  // misc is rewritten by the next round
    }

    // ---- candidate c is taken iff fewer than `need` candidates order before it;
    // thread t decides candidates [cpt t, cpt (t + 1)), then compacts them in order
    const int cpt = (m + kFusedThreads - 1) / kFusedThreads;
    const int c_lo = min(m, cpt * tid), c_hi = min(m, c_lo + cpt);
    uint32_t take_bits = 0;  // cpt <= 4
    int nt = 0;
    for (int c = c_lo; c < c_hi; ++c) {
        const uint64_t x = cand[c];
        int rank = 0;
        for (int j = 0; j < m; ++j) rank += cand[j] < x;
        if (rank < need) {
            take_bits |= 1u << (c - c_lo);
            ++nt;
        }
    }
    int to = nt, unused = 0;
    block_exclusive_scan2<kFusedThreads / 64>(to, unused, itmp);
    for (int c = c_lo; c < c_hi; ++c)
        if (take_bits >> (c - c_lo) & 1u) taken[to++] = (int)(uint32_t)cand[c];
    __syncthreads();

    // ---- merge the two ascending lists into the output
    for (int i = tid; i < above; i += kFusedThreads) {
        const int x = above_list[i];
        out[i + lower_bound_lds(taken, need, x)] = x;
    }
    for (int i = tid; i < need; i += kFusedThreads) {
        const int x = taken[i];
        out[i + lower_bound_lds(above_list, above, x)] = x;
    }
    if (tid == 0) *cnt_out = k;
}

// ---------------------------------------------------------------- merge

// out / lse of the g heads of (row, KV head h) from the S partials (natural-log
// lse; all -inf gives 0 and -inf; a NaN partial, left by an abandoned wait, makes
// the result NaN).  lds: at least S * g + g floats.  The S x g partial lse are
// read in one round (one per thread), the weights are formed in LDS, and every
// thread then accumulates 4 dims of one head with up to 16 partial loads in
// flight, so a merge costs about two memory round trips whatever S is.
__device__ __forceinline__ void merge_unit(const FusedParams& F, int row, int h, float* lds) {
    const AttnParams& A = F.A;
    const int g = A.g, S = A.S;
    float* w = lds;           // [S][g] partial lse, then weights
    float* hlse = lds + S * g;  // [g] merged lse
    for (int e = threadIdx.x; e < S * g; e += kFusedThreads)
        w[e] = A.part_lse[((int64_t)(e / g) * A.R + row) * A.Hq + h * g + e % g];
    __syncthreads();
    if (threadIdx.x < g) {
        const int hh = threadIdx.x;
        float M = -INFINITY;
        for (int sp = 0; sp < S; ++sp) {
            const float x = w[sp * g + hh];
            M = (x != x || M != M) ? __builtin_nanf("") : fmaxf(M, x);
        }
        float z = 0.f;
        if (M != -INFINITY)
            for (int sp = 0; sp < S; ++sp) z += expf(w[sp * g + hh] - M);  // NaN M: z NaN
        for (int sp = 0; sp < S; ++sp)
            w[sp * g + hh] = M == -INFINITY ? 0.f : expf(w[sp * g + hh] - M) / z;
        hlse[hh] = M == -INFINITY ? -INFINITY : M + logf(z);
    }
    __syncthreads();
    constexpr int kBatch = 16;
    for (int e = threadIdx.x; e < g * 64; e += kFusedThreads) {
        const int hh = e >> 6;
        const int head = h * g + hh;
        const int d = 4 * (e & 63);
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int sp0 = 0; sp0 < S; sp0 += kBatch) {
            float4 x[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                x[j] = sp0 + j < S ? *reinterpret_cast<const float4*>(
                                         A.part_out + (((int64_t)(sp0 + j) * A.R + row) * A.Hq + head) * kHeadDim + d)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                if (sp0 + j >= S) break;
                const float ws = w[(sp0 + j) * g + hh];
                acc.x += ws * x[j].x;
                acc.y += ws * x[j].y;
                acc.z += ws * x[j].z;
                acc.w += ws * x[j].w;
            }
        }
        if (hlse[hh] == -INFINITY) acc = make_float4(0.f, 0.f, 0.f, 0.f);
        uint16_t* o = F.out + (int64_t)row * F.out_stride + (int64_t)head * kHeadDim + d;
        *reinterpret_cast<uint2*>(o) = make_uint2(pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w));
        if (d == 0 && F.lse) F.lse[(int64_t)row * A.Hq + head] = hlse[hh];
    }
}

// ---------------------------------------------------------------- kernel

template <bool PAGE16, int KT, bool KV8>
__global__ __launch_bounds__(kFusedThreads) __attribute__((amdgpu_waves_per_eu(2, 8))) void fused_decode_kernel(
    const FusedParams F) {
    extern __shared__ float smem[];
    __shared__ int sh_item, sh_last;
    __shared__ float4 stash[4 * 64];  // each wave's rebuilt newest block key until it is scored
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = wave_id();

    // the call's epoch: only the last workgroup out changes it, after every
    // workgroup of the launch has passed this read
    const int epoch = F.ctl[3];
    const int raised = (int)((unsigned)epoch + 1u);  // a unit's ready word once its selection is written
    int next = 0;  // thread 0: the ticket claimed for the following item
    if (tid == 0) next = atomicAdd(&F.ctl[0], 1);
    for (;;) {
        if (tid == 0) sh_item = next;
        __syncthreads();
        const int item = sh_item;
        __syncthreads();
        if (item >= F.n_items) break;
        if (tid == 0) next = atomicAdd(&F.ctl[0], 1);  // in flight while this item runs

        bool scan;
        int u, j;
        decode_item(F, item, scan, u, j);
        const int row = u / F.Hkv, h = u % F.Hkv;
        const int L = F.seq_lens[row];
        const int n_elig = L <= 0 ? 0 : min((L - 1) / 4 + 1, F.score_stride);
        float* srow = F.scores + (int64_t)u * F.score_stride;
        int* uc = F.unit_ctl + 4 * (int64_t)u;  // scan arrivals, ready word, attention arrivals

        if (scan) {
            constexpr int kStreamChunk = stream_chunk(KT);
            const int nch = max(1, (n_elig + kStreamChunk - 1) / kStreamChunk);
            if (j >= nch) continue;  // past the row: not counted
            const int wb0 = j * kStreamChunk + wave * (kStreamChunk / 4);
            // the block holding the newest token (t = L - 1) is rebuilt from K and
            // stored by the wave that scores it, or by the row's first wave when
            // the score stride cuts the row short (as scores_stream_kernel does)
            Refresh rf;
            {
                const int b = (L - 1) >> 2;
                const bool scored = b < n_elig;
                if (L > 0 && (scored ? (wb0 <= b && b < wb0 + kStreamChunk / 4) : wb0 == 0)) {
                    rf.k = F.A.k;
                    rf.kv8 = KV8;
                    rf.ckey = const_cast<void*>(F.ckey);
                    rf.b = b;
                    rf.n = L - 4 * b;
                    rf.score = scored;
                    rf.stash = stash + wave * 64;
                }
            }
            if (wb0 < n_elig)
                scan_wave<PAGE16, true, KT, true>(F.q + (int64_t)row * F.q_stride + (int64_t)h * F.g * kHeadDim,
                                                  F.g, F.ckey, F.block_table + (int64_t)row * F.max_pages, F.Hkv, h,
                                                  F.lg_ps, n_elig, wb0, lane, srow, rf);
            // The scores went out as device-scope stores: once every wave has seen
            // its own stores complete (the wait) and the barrier has passed, they are
            // visible device-wide, so the arrival needs no release (a release would
            // write back the whole L2 once per item).  Only the last arrival
            // acquires: it reads every chunk's scores.
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (tid == 0) {
                const bool last = __hip_atomic_fetch_add(&uc[0], 1, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT) == nch - 1;
                if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                sh_last = last;
            }
            __syncthreads();
            if (!sh_last) continue;
            if (tid == 0) uc[0] = 0;
            select_unit(srow, n_elig, F.k, F.sel_idx + (int64_t)u * F.k, F.sel_cnt + u, reinterpret_cast<int*>(smem));
            __syncthreads();
            if (tid == 0) __hip_atomic_store(&uc[1], raised, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            if (tid == 0) {
                int polls = 0;
                bool ok = true;
                while (__hip_atomic_load(&uc[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != raised) {
                    __builtin_amdgcn_s_sleep(8);
                    if (++polls >= F.spin_limit) {
                        atomicAdd(&F.ctl[2], 1);
                        ok = false;
                        break;
                    }
                }
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                sh_last = ok;
            }
            __syncthreads();
            if (sh_last) {
                attend_split<KV8>(F.A, row, h, j, smem);
            } else {
                // abandoned wait: the selection may not be written yet, so this split
                // reports NaN, which the merge carries into the unit's output and lse
                const AttnParams& A = F.A;
                for (int e = tid; e < A.g * 64; e += kFusedThreads) {
                    const int64_t prow = ((int64_t)j * A.R + row) * A.Hq + h * A.g + (e >> 6);
                    const float nan = __builtin_nanf("");
                    *reinterpret_cast<float4*>(A.part_out + prow * kHeadDim + 4 * (e & 63)) =
                        make_float4(nan, nan, nan, nan);
                    if ((e & 63) == 0) A.part_lse[prow] = nan;
                }
            }
            __syncthreads();
            if (tid == 0) {
                const bool last = __hip_atomic_fetch_add(&uc[2], 1, __ATOMIC_RELEASE,
                                                         __HIP_MEMORY_SCOPE_AGENT) == F.S - 1;
                if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                sh_last = last;
            }
            __syncthreads();
            if (!sh_last) continue;
            if (tid == 0) uc[2] = 0;
            merge_unit(F, row, h, smem);
        }
    }
    // the last workgroup out returns the ticket counters to zero and advances the
    // epoch for the next call
    if (tid == 0 && atomicAdd(&F.ctl[1], 1) == (int)gridDim.x - 1) {
        F.ctl[0] = 0;
        F.ctl[1] = 0;
        F.ctl[3] = raised;
    }
}

// ---------------------------------------------------------------- host

namespace {

struct FusedLayout {
    size_t ctl, arrive, scores, part_out, part_lse, total;
    int score_stride;
};

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

FusedLayout fused_layout(int batch, int Hkv, int Hq, int max_seq_len, int S) {
    FusedLayout l;
    const int64_t U = (int64_t)batch * Hkv;
    l.score_stride = (int)((((int64_t)max_seq_len + 3) / 4 + 63) & ~(int64_t)63);
    if (l.score_stride == 0) l.score_stride = 64;
    l.ctl = 0;
    l.arrive = 256;
    l.scores = align256(l.arrive + (size_t)4 * U * sizeof(int));
    l.part_out = align256(l.scores + (size_t)U * l.score_stride * sizeof(float));
    l.part_lse = align256(l.part_out + (size_t)S * batch * Hq * kHeadDim * sizeof(float));
    l.total = align256(l.part_lse + (size_t)S * batch * Hq * sizeof(float));
    return l;
}

// Workgroups of the fused kernel resident on the device at once.
int fused_capacity(size_t lds) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fused_decode_kernel<true, kKeyF32, false>, kFusedThreads, lds) !=
        hipSuccess)
        return 0;
    return cus * (per_cu > 0 ? per_cu : 1);
}

}  // namespace

size_t fused_workspace_bytes(int batch, int Hkv, int Hq, int max_seq_len, int S) {
    return fused_layout(batch, Hkv, Hq, max_seq_len, S).total;
}

size_t fused_control_bytes(int batch, int Hkv) { return align256(256 + (size_t)4 * batch * Hkv * sizeof(int)); }

hipError_t launch_fused_decode(const PagedKV& kv, const Rows& rows, int k, float scale, int S, int32_t* sel_idx,
                               int32_t* sel_cnt, uint16_t* out, int64_t out_stride, float* lse, void* workspace,
                               hipStream_t st) {
    const int U = kv.batch * kv.Hkv;
    if (U == 0) return hipSuccess;
    const FusedLayout l = fused_layout(kv.batch, kv.Hkv, rows.Hq, kv.max_seq_len, S);
    char* ws = static_cast<char*>(workspace);
    FusedParams F;
    AttnParams& A = F.A;
    A.k = kv.k;
    A.v = kv.v;
    A.block_table = kv.block_table;
    A.seq_lens = kv.seq_lens;
    A.Hkv = kv.Hkv;
    A.lg_ps = kv.lg_ps;
    A.max_pages = kv.max_pages;
    A.q = rows.q;
    A.q_stride = rows.q_stride;
    A.q_seq = nullptr;
    A.q_pos = nullptr;
    A.R = kv.batch;
    A.Hq = rows.Hq;
    A.g = rows.Hq / kv.Hkv;
    A.sel = sel_idx;
    A.cnt = sel_cnt;
    A.kstride = k;
    A.scale_log2 = scale * 1.4426950408889634f;
    A.S = S;
    A.blocked = 1;
    const int blocks_per_split = (k + S - 1) / S;
    A.table_words = 4 * ((blocks_per_split + 3) & ~3) + kSlotPad;
    A.out = nullptr;
    A.out_stride = 0;
    A.lse = nullptr;
    A.part_out = reinterpret_cast<float*>(ws + l.part_out);
    A.part_lse = reinterpret_cast<float*>(ws + l.part_lse);
    F.q = rows.q;
    F.q_stride = rows.q_stride;
    F.g = A.g;
    F.ckey = kv.ckey;
    F.block_table = kv.block_table;
    F.seq_lens = kv.seq_lens;
    F.Hkv = kv.Hkv;
    F.lg_ps = kv.lg_ps;
    F.max_pages = kv.max_pages;
    F.scores = reinterpret_cast<float*>(ws + l.scores);
    F.score_stride = l.score_stride;
    F.k = k;
    F.sel_idx = sel_idx;
    F.sel_cnt = sel_cnt;
    F.out = out;
    F.out_stride = out_stride;
    F.lse = lse;
    F.ctl = reinterpret_cast<int*>(ws + l.ctl);
    F.unit_ctl = reinterpret_cast<int*>(ws + l.arrive);
    F.U = U;
    F.C = (l.score_stride + stream_chunk(kv.ckey_type) - 1) / stream_chunk(kv.ckey_type);
    F.S = S;
    F.n_items = U * (F.C + S);
    // QSA_FUSED_SPIN_LIMIT (tests of the time-out path only) shortens the bounded
    // wait so that abandoned waits can be provoked without a stalled device
    F.spin_limit = kSpinLimit;
    if (const char* env = getenv("QSA_FUSED_SPIN_LIMIT")) {
        const long v = strtol(env, nullptr, 10);
        if (v >= 1 && v < kSpinLimit) F.spin_limit = (int)v;
    }

    const size_t attn_loop = attn_loop_bytes(A.table_words, kv.kv_fp8 != 0);
    const size_t attn_xchg = (size_t)kAttnWaves * A.g * kHeadDim * sizeof(float);
    size_t lds = attn_loop > attn_xchg ? attn_loop : attn_xchg;
    if (lds < (size_t)kSelLdsInts * 4) lds = (size_t)kSelLdsInts * 4;

    static thread_local int cap_dev = -1, cap = 0;
    static thread_local size_t cap_lds = 0;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev != cap_dev || lds != cap_lds) {
        cap = fused_capacity(lds);
        cap_dev = dev;
        cap_lds = lds;
    }
    const int resident = cap > 0 ? cap : 512;
    const int grid = F.n_items < resident ? F.n_items : resident;
    const bool page16 = kv.lg_ps >= 6;
#define QSA_FUSED(P16, KT)                                                                                      \
    do {                                                                                                        \
        if (kv.kv_fp8)                                                                                          \
            hipLaunchKernelGGL((fused_decode_kernel<P16, KT, true>), dim3(grid), dim3(kFusedThreads), lds, st, F); \
        else                                                                                                    \
            hipLaunchKernelGGL((fused_decode_kernel<P16, KT, false>), dim3(grid), dim3(kFusedThreads), lds, st, F); \
    } while (0)
#define QSA_FUSED_KT(P16)                  \
    do {                                   \
        if (kv.ckey_type == kKeyFP8)       \
            QSA_FUSED(P16, kKeyFP8);       \
        else if (kv.ckey_type == kKeyBF16) \
            QSA_FUSED(P16, kKeyBF16);      \
        else                               \
            QSA_FUSED(P16, kKeyF32);       \
    } while (0)
    if (page16)
        QSA_FUSED_KT(true);
    else
        QSA_FUSED_KT(false);
#undef QSA_FUSED_KT
#undef QSA_FUSED
    return hipGetLastError();
}

}  // namespace qsa
