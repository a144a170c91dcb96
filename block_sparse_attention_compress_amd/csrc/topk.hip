// a3 -- top-k block selection per (query row, KV head).
//
// QSA keeps the 512 best-scoring microblocks ("Qwen 4 QSA krijgt
// decode-contextparallellisme", section "Wat de pull request daadwerkelijk
// verandert").  Ties are not discussed on the pages; the order used here is
// (score descending, block index ascending), with -0 equal to +0.
//
// One 512-thread workgroup per (row, KV head).  Scores are mapped to
// order-preserving uint32 keys; three radix passes (11, 11 and 10 bits) with
// LDS histograms find the exact k-th key T and how many of the keys equal to T
// are needed.  A final ordered pass writes the blocks with key > T and the
// lowest-indexed blocks with key == T, in ascending block order (so the output is
// the same whatever the thread timing).  The row is re-read from L2 per pass.
#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

constexpr int kTopkThreads = 512;
constexpr int kTopkWaves = kTopkThreads / 64;

// Inclusive scan over the block of one int per thread, in reverse thread order
// (thread t gets the sum over threads >= t).  Uses `tmp` [kTopkWaves].
__device__ __forceinline__ int block_suffix_sum(int v, int* tmp) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    // within a wave: suffix over lanes >= lane
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int other = __shfl_down(v, o);
        if (lane + o < 64) v += other;
    }
    if (lane == 0) tmp[wave] = v;  // wave total
    __syncthreads();
    int after = 0;
    for (int w = wave + 1; w < kTopkWaves; ++w) after += tmp[w];
    __syncthreads();
    return v + after;
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ scores, int score_stride,
                                                            const int32_t* __restrict__ q_pos, int Hkv, int k,
                                                            int32_t* __restrict__ sel_idx,
                                                            int32_t* __restrict__ sel_cnt) {
    __shared__ int hist[2048];
    __shared__ int tmp[kTopkWaves];
    __shared__ int found_bin, found_above;
    __shared__ int wave_gt[kTopkWaves], wave_eq[kTopkWaves];

    const int unit = blockIdx.x;
    const int row = unit / Hkv;
    int n = score_stride;
    if (q_pos) {
        const int t = q_pos[row];
        n = t < 0 ? 0 : min(t / 4 + 1, score_stride);
    }
    const float* s = scores + (int64_t)unit * score_stride;
    int32_t* out = sel_idx + (int64_t)unit * k;
    const int tid = threadIdx.x;

    if (n <= k) {  // everything eligible is selected
        for (int j = tid; j < k; j += kTopkThreads) out[j] = j < n ? j : -1;
        if (tid == 0) sel_cnt[unit] = n;
        return;
    }
    if (k == 0) {
        if (tid == 0) sel_cnt[unit] = 0;
        return;
    }

    // ---- radix select of the k-th largest key
    uint32_t prefix = 0, mask = 0;
    int remaining = k;  // how many still to take among keys matching prefix
    const int shifts[3] = {21, 10, 0};
    const int widths[3] = {11, 11, 10};
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = shifts[pass];
        const int nbins = 1 << widths[pass];
        for (int i = tid; i < nbins; i += kTopkThreads) hist[i] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += kTopkThreads) {
            const uint32_t key = order_key(s[i]);
            if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & (nbins - 1)], 1);
        }
        __syncthreads();
        // thread t owns bins [t*per, (t+1)*per); find the bin holding the
        // remaining-th largest matching key
        const int per = nbins / kTopkThreads;  // 4, 4, 2
        int local = 0;
        for (int i = 0; i < per; ++i) local += hist[tid * per + i];
        const int incl = block_suffix_sum(local, tmp);  // keys in bins >= tid*per
        const int above = incl - local;                 // keys in bins > my range
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
    const int need_eq = remaining;  // >= 1

    // ---- ordered compaction: wave w owns a contiguous segment of the row
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int seg = ((n + kTopkWaves * 64 - 1) / (kTopkWaves * 64)) * 64;
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

hipError_t launch_topk(const float* scores, int score_stride, const int32_t* q_pos, int R, int Hkv, int k,
                       int32_t* sel_idx, int32_t* sel_cnt, hipStream_t st) {
    if (R == 0) return hipSuccess;
    hipLaunchKernelGGL(topk_kernel, dim3(R * Hkv), dim3(kTopkThreads), 0, st, scores, score_stride, q_pos, Hkv, k,
                       sel_idx, sel_cnt);
    return hipGetLastError();
}

}  // namespace qsa
