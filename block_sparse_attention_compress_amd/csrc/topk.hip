// a3 -- top-k block selection per (query row, KV head).
//
// QSA keeps the 512 best-scoring microblocks ("Qwen 4 QSA krijgt
// decode-contextparallellisme", section "Wat de pull request daadwerkelijk
// verandert").  Ties are not discussed on the pages; the order used here is
// (score descending, block index ascending), with -0 equal to +0.
//
// Both kernels find the exact k-th largest key T (order-preserving uint32 map of
// the fp32 score) and how many keys equal to T are needed, then write, in
// ascending block order, every block with key > T and the lowest-indexed blocks
// with key == T.  The result does not depend on thread timing.
//
// topk_reg_kernel (rows of up to 65,536 blocks): one workgroup per (row, KV
// head) -- 1024 threads, or 512 when a launch has many rows -- with the row in
// registers (KPT scores per thread, thread t holding blocks t KPT .. t KPT +
// KPT - 1, so thread order is block order and one prefix sum of per-thread
// counts places the output).  Radix digits of raw float keys crowd into a few
// exponent bins, and LDS atomics on one address serialise, so the first pass
// bins uniformly between the row's min and max instead: any monotonic binning
// keeps the selection exact.  The bin holding the k-th value is then resolved
// exactly -- by ranking its candidates directly when there are at most as many
// as threads, else by exact radix passes restricted to that bin.  The same
// kernel runs the two stages of the long-row select (below).
//
// topk_global_kernel (longer rows, one stage): the same select with exact radix
// passes (11, 11, 10 bits) re-reading the row from L2.
#include <float.h>

#include "block_ops.h"
#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

// Workgroup min and max (returns max - min).  One barrier; tmp must not be
// written again by this workgroup.
__device__ __forceinline__ float block_min_max(float& mn, float& mx, float* tmp) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    mn = wave_prefix_min(mn);
    mx = wave_prefix_max(mx);
    if (lane == 63) {
        tmp[wave] = mn;
        tmp[32 + wave] = mx;
    }
    __syncthreads();
    mn = tmp[0];
    mx = tmp[32];
    for (int w = 1; w < nw; ++w) {
        mn = fminf(mn, tmp[w]);
        mx = fmaxf(mx, tmp[32 + w]);
    }
    return mx - mn;
}

// Trivial rows: everything eligible selected (n <= k), or nothing (k == 0).
__device__ __forceinline__ bool topk_trivial(int n, int k, int32_t* out, int32_t* cnt_out) {
    if (n <= k) {
        for (int j = threadIdx.x; j < k; j += blockDim.x) out[j] = j < n ? j : -1;
        if (threadIdx.x == 0) *cnt_out = n;
        return true;
    }
    if (k == 0) {
        if (threadIdx.x == 0) *cnt_out = 0;
        return true;
    }
    return false;
}

__device__ __forceinline__ int eligible(const int32_t* q_pos, int row, int score_stride) {
    if (!q_pos) return score_stride;
    const int t = q_pos[row];
    return t < 0 ? 0 : min(t / 4 + 1, score_stride);
}

// ------------------------------------------------------------------ registers

constexpr int kRegThreads = 1024;  // threads per row, unless many rows share the launch
constexpr int kManyThreads = 512;  // threads per row when rows are many (extend chunks)
constexpr int kManyThreadsShort = 256;  // ... and at most 16 x 256 = 4,096 blocks long
constexpr int kBins = 2048;

// Candidate workspace of the two-stage select for long rows: per (row, KV head),
// nslices x k (value, block index) pairs, slice j's top k in ascending index order.
struct SplitWs {
    float* val;
    int32_t* idx;
    int slice;    // blocks per slice (a multiple of 1024, >= 4 QSA_MAX_TOPK)
    int nslices;  // ceil(score_stride / slice)
};

// NT threads per row, KPT scores per thread: the first KR in registers, the rest
// in LDS (a 65,536-block row would not fit 1024 threads x 128 registers).  Thread
// t owns histogram bins [BPT t, BPT t + BPT).
// Many-row launches (NT = 512 or 256) ask for 8 waves per SIMD (at most 64
// registers), so that 4 of their 8-wave workgroups (8 of the 4-wave ones) share a
// CU instead of 3: the 7,810-row prefill
// (32 scores per thread, a few registers spilled) 508 -> 391-402 us, rows of
// 4,096 blocks 40.2 -> 36.4 us, C4 58.4 -> 57.6 us, selections bit-equal.
template <int NT, int KPT, int KR, int MODE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(NT <= 512 ? 8 : 1, 8))) void topk_reg_kernel(
    const float* __restrict__ scores, int score_stride, const int32_t* __restrict__ q_pos, int Hkv, int k,
    int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_cnt, SplitWs ws) {
    constexpr int NW = NT / 64;
    constexpr int BPT = kBins / NT;
    __shared__ int hist[kBins];
    __shared__ float cand_val[NT];
    __shared__ int cand_idx[NT];
    __shared__ int itmp[2 * NW];
    __shared__ float ftmp[64];
    __shared__ int sh_bin, sh_above, sh_ncand, sh_need_eq, sh_m;
    __shared__ uint32_t sh_T;
    constexpr int KL = KPT - KR;
    __shared__ float vl[KL > 0 ? KL * NT : 1];

    const int unit = blockIdx.x;
    const int n_row = eligible(q_pos, unit / Hkv, score_stride);
    int32_t* out = sel_idx + (int64_t)unit * k;
    const float* s = scores + (int64_t)unit * score_stride;
    int n = n_row, row_len = score_stride;
    // MODE 1: slice blockIdx.y of the row.  A row that fits one slice is finished
    // here (final output); a longer one leaves the slice's top k as candidates.
    // MODE 2: the candidates of a row longer than one slice.
    bool final_out = true;
    int base = 0;  // block index of this slice's first score
    float* cv = nullptr;
    int32_t* ci = nullptr;
    if (MODE == 1) {
        base = blockIdx.y * ws.slice;
        if (n_row > ws.slice) {
            if (base >= n_row || k == 0) return;
            final_out = false;
            s += base;
            n = min(ws.slice, n_row - base);
            row_len = min(ws.slice, score_stride - base);
            cv = ws.val + ((int64_t)unit * ws.nslices + blockIdx.y) * k;
            ci = ws.idx + ((int64_t)unit * ws.nslices + blockIdx.y) * k;
            if (n <= k) {  // a short last slice: all of it
                for (int j = threadIdx.x; j < k; j += blockDim.x) {
                    cv[j] = j < n ? s[j] + 0.0f : -INFINITY;
                    ci[j] = j < n ? base + j : -1;
                }
                return;
            }
        } else if (blockIdx.y > 0) {
            return;
        }
    } else if (MODE == 2) {
        if (n_row <= ws.slice) return;
        row_len = ws.nslices * k;
        n = ((n_row + ws.slice - 1) / ws.slice) * k;  // slices holding eligible blocks
        s = ws.val + (int64_t)unit * row_len;
        ci = ws.idx + (int64_t)unit * row_len;
    }
    if (final_out && topk_trivial(n_row, k, out, sel_cnt + unit)) return;
    // emit(j, i): the j-th selected (ascending) is local position i
    auto emit = [&](int j, int i, float x) {
        if (MODE == 2) out[j] = ci[i];
        else if (MODE == 1 && !final_out) {
            cv[j] = x;
            ci[j] = base + i;
        } else
            out[j] = i;
    };

    const int tid = threadIdx.x;
    const int i0 = tid * KPT;  // this thread's first block
    // the histogram is cleared while the loads fly; block_min_max's barrier orders it
    for (int i = tid; i < kBins; i += NT) hist[i] = 0;
    // slots past n hold -inf (scores are finite): it is never selected, and
    // every test below stays a function of the value (no per-slot masks kept live)
    float v[KR];
    auto put = [&](int e, float raw) {
        const float x = i0 + e < n ? raw + 0.0f : -INFINITY;  // + 0 turns -0 into +0
        if (e < KR) v[e < KR ? e : 0] = x;
        else vl[(e - KR) * NT + tid] = x;
    };
    if (KPT >= 4 && (row_len & 3) == 0 && (reinterpret_cast<uintptr_t>(s) & 15) == 0) {
        // float4 loads, clamped and unconditional, so all KPT / 4 are in flight at once
        // (a whole float4 lies inside the row: n4 <= row_len / 4)
        const float4* s4 = reinterpret_cast<const float4*>(s);
        const int n4 = (n + 3) / 4;
#pragma unroll
        for (int j = 0; j < (KPT >= 4 ? KPT / 4 : 1); ++j) {
            const float4 x = s4[min(i0 / 4 + j, n4 - 1)];
            put(4 * j + 0, x.x);
            put(4 * j + 1, x.y);
            put(4 * j + 2, x.z);
            put(4 * j + 3, x.w);
        }
    } else {
#pragma unroll
        for (int e = 0; e < KPT; ++e) put(e, s[min(i0 + e, n - 1)]);
    }
    auto V = [&](int e) -> float { return e < KR ? v[e < KR ? e : 0] : vl[(e - KR) * NT + tid]; };
    float mn = FLT_MAX, mx = -FLT_MAX;
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
        mn = fminf(mn, V(e) == -INFINITY ? FLT_MAX : V(e));
        mx = fmaxf(mx, V(e));
    }
    const float range = block_min_max(mn, mx, ftmp);
    if (range == 0.f) {  // every score equal: the k lowest indices (positions are in index order)
        for (int j = tid; j < k; j += NT) emit(j, j, mn);
        if (tid == 0 && final_out) sel_cnt[unit] = k;
        return;
    }
    float scale = (float)kBins / range;
    if (!(scale <= FLT_MAX)) scale = FLT_MAX;
    // monotonic in x; the -inf padding lands in bin 0 below every real score
    auto bin_of = [&](float x) { return (int)fminf(fmaxf((x - mn) * scale, 0.f), (float)(kBins - 1)); };
    // With at most 16 scores per thread, all in registers, each score's bin and
    // order key are computed once and kept (32 registers) rather than recomputed
    // by every pass that tests them; within the 64 registers of a many-row launch,
    // only up to 8 scores per thread (16 would spill).
    constexpr bool CACHE = KL == 0 && KPT <= (NT <= 512 ? 8 : 16);
    int bn[CACHE ? KPT : 1];
    uint32_t ky[CACHE ? KPT : 1];
    if constexpr (CACHE) {
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            bn[e] = bin_of(V(e));
            ky[e] = order_key(V(e));
        }
    }
    auto BIN = [&](int e) -> int {
        if constexpr (CACHE) return bn[CACHE ? e : 0];
        else return bin_of(V(e));
    };
    auto KEY = [&](int e) -> uint32_t {
        if constexpr (CACHE) return ky[CACHE ? e : 0];
        else return order_key(V(e));
    };

    // ---- pass 1: uniform bins over [mn, mx]
#pragma unroll
    for (int e = 0; e < KPT; ++e)
        if (V(e) != -INFINITY) atomicAdd(&hist[BIN(e)], 1);
    __syncthreads();
    // the thread whose bins hold the k-th largest names the bin (bins descend with
    // the score from the top one down)
    auto find_bin = [&](int want, bool keep_m) {
        int hb[BPT], local = 0;
#pragma unroll
        for (int b = 0; b < BPT; ++b) {
            hb[b] = hist[BPT * tid + b];
            local += hb[b];
        }
        const int incl = block_suffix_sum<NW, false>(local, itmp);
        int cum = incl - local;  // elements in higher bins
        if (cum < want && want <= incl) {
#pragma unroll
            for (int b = BPT - 1; b >= 0; --b) {
                if (cum < want && cum + hb[b] >= want) {
                    sh_bin = BPT * tid + b;
                    sh_above = cum;
                    if (keep_m) sh_m = hb[b];
                }
                cum += hb[b];
            }
        }
    };
    find_bin(k, true);
    if (tid == 0) sh_ncand = 0;
    __syncthreads();
    const int B = sh_bin;
    const int need = k - sh_above;  // how many of bin B's elements are taken (>= 1)
    // bin B's size, from a copy: the crowded path below clears hist with no barrier
    // between this read and the clear
    const int m = sh_m;

    if (m <= NT) {
        // ---- rank the bin's candidates directly
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            if (V(e) != -INFINITY && BIN(e) == B) {
                const int slot = atomicAdd(&sh_ncand, 1);
                cand_val[slot] = V(e);
                cand_idx[slot] = i0 + e;
            }
        }
        __syncthreads();
        if (tid < m) {
            const float x = cand_val[tid];
            const int xi = cand_idx[tid];
            int rank = 0, gt = 0;
            for (int u = 0; u < m; ++u) {
                const float y = cand_val[u];
                gt += y > x;
                rank += (y > x) || (y == x && cand_idx[u] < xi);
            }
            if (rank == need - 1) {  // the k-th element overall
                sh_T = order_key(x);
                sh_need_eq = need - gt;
            }
        }
        __syncthreads();
    } else {
        // ---- crowded bin: exact radix passes over the keys of bin B
        uint32_t prefix = 0, mask = 0;
        int remaining = need;
        const int shifts[3] = {21, 10, 0};
        const int widths[3] = {11, 11, 10};
        for (int pass = 0; pass < 3; ++pass) {
            const int shift = shifts[pass];
            const int nb = 1 << widths[pass];
            for (int i = tid; i < kBins; i += NT) hist[i] = 0;
            __syncthreads();
#pragma unroll
            for (int e = 0; e < KPT; ++e) {
                const uint32_t key = KEY(e);
                if (V(e) != -INFINITY && BIN(e) == B && (key & mask) == prefix)
                    atomicAdd(&hist[(key >> shift) & (nb - 1)], 1);
            }
            __syncthreads();
            find_bin(remaining, false);
            __syncthreads();
            remaining -= sh_above;
            prefix |= (uint32_t)sh_bin << shift;
            mask |= (uint32_t)(nb - 1) << shift;
            __syncthreads();
        }
        if (tid == 0) {
            sh_T = prefix;
            sh_need_eq = remaining;
        }
        __syncthreads();
    }
    const uint32_t T = sh_T;
    const int need_eq = sh_need_eq;

    // ---- ordered compaction: thread order is block order, so per-thread counts
    // and one prefix sum place every selected block
    int gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
        const uint32_t key = KEY(e);
        const bool real = V(e) != -INFINITY;
        gt += real && key > T;
        eq += real && key == T;
    }
    block_exclusive_scan2<NW, false>(gt, eq, itmp);  // last use of itmp
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
        if (V(e) == -INFINITY) continue;
        const uint32_t key = KEY(e);
        if (key > T) {
            emit(gt + min(eq, need_eq), i0 + e, V(e));
            ++gt;
        } else if (key == T) {
            if (eq < need_eq) emit(gt + eq, i0 + e, V(e));
            ++eq;
        }
    }
    if (tid == 0 && final_out) sel_cnt[unit] = k;
}

// --------------------------------------------------------------------- global

constexpr int kGlobThreads = 512;
constexpr int kGlobWaves = kGlobThreads / 64;

__global__ __launch_bounds__(kGlobThreads) void topk_global_kernel(const float* __restrict__ scores, int score_stride,
                                                                   const int32_t* __restrict__ q_pos, int Hkv, int k,
                                                                   int32_t* __restrict__ sel_idx,
                                                                   int32_t* __restrict__ sel_cnt) {
    __shared__ int hist[2048];
    __shared__ int tmp[kGlobWaves];
    __shared__ int found_bin, found_above;
    __shared__ int wave_gt[kGlobWaves], wave_eq[kGlobWaves];

    const int unit = blockIdx.x;
    const int n = eligible(q_pos, unit / Hkv, score_stride);
    const float* s = scores + (int64_t)unit * score_stride;
    int32_t* out = sel_idx + (int64_t)unit * k;
    const int tid = threadIdx.x;
    if (topk_trivial(n, k, out, sel_cnt + unit)) return;

    uint32_t prefix = 0, mask = 0;
    int remaining = k;
    const int shifts[3] = {21, 10, 0};
    const int widths[3] = {11, 11, 10};
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = shifts[pass];
        const int nbins = 1 << widths[pass];
        for (int i = tid; i < nbins; i += kGlobThreads) hist[i] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += kGlobThreads) {
            const uint32_t key = order_key(s[i]);
            if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & (nbins - 1)], 1);
        }
        __syncthreads();
        const int per = nbins / kGlobThreads;
        int local = 0;
        for (int i = 0; i < per; ++i) local += hist[tid * per + i];
        const int incl = block_suffix_sum<kGlobWaves>(local, tmp);
        const int above = incl - local;
        if (above < remaining && remaining <= incl) {
            int cum = above;
            for (int b = tid * per + per - 1; b >= tid * per; --b) {
                if (cum + hist[b] >= remaining) {
                    found_bin = b;
                    found_above = cum;
                    break;
                }
                cum += hist[b];
            }
        }
        __syncthreads();
        remaining -= found_above;
        prefix |= (uint32_t)found_bin << shift;
        mask |= (uint32_t)(nbins - 1) << shift;
        __syncthreads();
    }
    const uint32_t T = prefix;
    const int need_eq = remaining;

    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int seg = ((n + kGlobWaves * 64 - 1) / (kGlobWaves * 64)) * 64;
    const int lo = wave * seg, hi = min(n, lo + seg);
    int gt = 0, eq = 0;
    for (int base = lo; base < hi; base += 64) {
        const int i = base + lane;
        const uint32_t key = i < hi ? order_key(s[i]) : 0u;
        gt += __popcll(__ballot(i < hi && key > T));
        eq += __popcll(__ballot(i < hi && key == T));
    }
    if (lane == 0) {
        wave_gt[wave] = gt;
        wave_eq[wave] = eq;
    }
    __syncthreads();
    int eq_before = 0, sel_before = 0;
    for (int w = 0; w < wave; ++w) {
        const int take_eq = min(max(need_eq - eq_before, 0), wave_eq[w]);
        sel_before += wave_gt[w] + take_eq;
        eq_before += wave_eq[w];
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int base = lo; base < hi; base += 64) {
        const int i = base + lane;
        const uint32_t key = i < hi ? order_key(s[i]) : 0u;
        const bool is_gt = i < hi && key > T;
        const bool is_eq = i < hi && key == T;
        const uint64_t eq_mask = __ballot(is_eq);
        const int eq_rank = eq_before + __popcll(eq_mask & below);
        const bool take = is_gt || (is_eq && eq_rank < need_eq);
        const uint64_t take_mask = __ballot(take);
        const int pos = sel_before + __popcll(take_mask & below);
        if (take && pos < k) out[pos] = i;
        eq_before += __popcll(eq_mask);
        sel_before += __popcll(take_mask);
    }
    if (tid == 0) sel_cnt[unit] = k;
}

template <int MODE, int NT = kRegThreads>
static void launch_reg(int per, dim3 grid, const float* scores, int score_stride, const int32_t* q_pos, int Hkv, int k,
                       int32_t* sel_idx, int32_t* sel_cnt, SplitWs ws, hipStream_t st) {
#define QSA_TOPK_REG(KPT, KR)                                                                                   \
    hipLaunchKernelGGL((topk_reg_kernel<NT, KPT, KR, MODE>), grid, dim3(NT), 0, st, scores, score_stride, q_pos, \
                       Hkv, k, sel_idx, sel_cnt, ws)
    if (per <= 1) QSA_TOPK_REG(1, 1);
    else if (per <= 2) QSA_TOPK_REG(2, 2);
    else if (per <= 4) QSA_TOPK_REG(4, 4);
    else if (per <= 8) QSA_TOPK_REG(8, 8);
    else if (per <= 16) QSA_TOPK_REG(16, 16);
    else if (per <= 32) QSA_TOPK_REG(32, 32);
    else QSA_TOPK_REG(64, 32);
#undef QSA_TOPK_REG
}

// With many rows per launch (an extend chunk), 512-thread workgroups let several
// rows share a CU and hide each other's latency (256 and 128 threads were slower
// on rows of 8,192 blocks and more); rows of at most 4,096 blocks take 256 threads,
// 8 rows to a CU (4,096 rows of 1,024 blocks 24.0 -> 16.0 us, 2,048 rows of 4,096
// blocks 37.1 -> 32.7 us; selections bit-equal).  With few rows, 1024 threads
// shorten each row.
constexpr int kManyRows = 1024;

hipError_t launch_topk(const float* scores, int score_stride, const int32_t* q_pos, int R, int Hkv, int k,
                       int32_t* sel_idx, int32_t* sel_cnt, hipStream_t st) {
    if (R == 0) return hipSuccess;
    const int units = R * Hkv;
    const int per = (score_stride + kRegThreads - 1) / kRegThreads;  // scores per thread
    const int per_many = (score_stride + kManyThreads - 1) / kManyThreads;
    if (units >= kManyRows && score_stride <= 16 * kManyThreadsShort)
        launch_reg<0, kManyThreadsShort>((score_stride + kManyThreadsShort - 1) / kManyThreadsShort, dim3(units),
                                         scores, score_stride, q_pos, Hkv, k, sel_idx, sel_cnt, SplitWs{}, st);
    else if (units >= kManyRows && per_many <= 64)
        launch_reg<0, kManyThreads>(per_many, dim3(units), scores, score_stride, q_pos, Hkv, k, sel_idx, sel_cnt,
                                    SplitWs{}, st);
    else if (per <= 64)
        launch_reg<0>(per, dim3(units), scores, score_stride, q_pos, Hkv, k, sel_idx, sel_cnt, SplitWs{}, st);
    else
        hipLaunchKernelGGL(topk_global_kernel, dim3(units), dim3(kGlobThreads), 0, st, scores, score_stride, q_pos,
                           Hkv, k, sel_idx, sel_cnt);
    return hipGetLastError();
}

// Rows longer than kSplitMin blocks are selected in two stages: every slice of
// kSlice blocks keeps its own top k (one workgroup per slice, so a row spreads
// over many CUs), then one workgroup per row selects the top k of the slices'
// candidates.  A block in the row's top k is in its slice's top k (fewer than k
// blocks of the slice precede it in the order), and the candidates sit in block
// order, so the second stage, breaking ties by position, gives exactly the
// one-stage result.
constexpr int kSlice = 8192;
constexpr int kSplitMin = 16384;

static bool split_applies(int score_stride, int k) { return k >= 1 && score_stride > kSplitMin; }

size_t topk_workspace_bytes(int R, int Hkv, int k, int score_stride) {
    if (R <= 0 || Hkv <= 0 || !split_applies(score_stride, k)) return 0;
    const int64_t per_unit = (int64_t)((score_stride + kSlice - 1) / kSlice) * k;
    const size_t half = ((size_t)R * Hkv * per_unit * 4 + 255) & ~(size_t)255;
    return 2 * half;
}

hipError_t launch_topk_split(const float* scores, int score_stride, const int32_t* q_pos, int R, int Hkv, int k,
                             int32_t* sel_idx, int32_t* sel_cnt, void* workspace, hipStream_t st) {
    if (!split_applies(score_stride, k))
        return launch_topk(scores, score_stride, q_pos, R, Hkv, k, sel_idx, sel_cnt, st);
    if (R == 0) return hipSuccess;
    const int units = R * Hkv;
    const int nslices = (score_stride + kSlice - 1) / kSlice;
    const size_t half = topk_workspace_bytes(R, Hkv, k, score_stride) / 2;
    SplitWs ws{static_cast<float*>(workspace),
               reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + half), kSlice, nslices};
    launch_reg<1>(kSlice / kRegThreads, dim3(units, nslices), scores, score_stride, q_pos, Hkv, k, sel_idx, sel_cnt,
                  ws, st);
    const int per2 = (nslices * k + kRegThreads - 1) / kRegThreads;  // <= 32 * 2048 / 1024
    launch_reg<2>(per2, dim3(units), scores, score_stride, q_pos, Hkv, k, sel_idx, sel_cnt, ws, st);
    return hipGetLastError();
}

}  // namespace qsa
