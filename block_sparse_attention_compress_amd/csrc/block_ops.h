// Workgroup-wide prefix sums (DPP lane moves within a wave, then one LDS
// exchange), shared by the top-k selection kernels.
#pragma once

#include "qsa_device.h"

namespace qsa {

// DPP move: lane i reads v from the lane CTRL names; lanes of rows outside
// ROW_MASK, and (BOUND_ZERO false) lanes whose source is outside the row, get old.
template <int CTRL, int ROW_MASK, bool BOUND_ZERO>
__device__ __forceinline__ int dpp_move(int old, int v) {
    return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xF, BOUND_ZERO);
}

// Inclusive prefix sum over the 64 lanes: shifts by 1, 2, 4, 8 inside each
// 16-lane row, then lane 15 of each row is added to the next row and lane 31 to
// the upper two rows.
__device__ __forceinline__ int wave_prefix_sum(int v) {
    v += dpp_move<0x111, 0xF, true>(0, v);   // row_shr:1
    v += dpp_move<0x112, 0xF, true>(0, v);   // row_shr:2
    v += dpp_move<0x114, 0xF, true>(0, v);   // row_shr:4
    v += dpp_move<0x118, 0xF, true>(0, v);   // row_shr:8
    v += dpp_move<0x142, 0xA, false>(0, v);  // row_bcast:15 into rows 1, 3
    v += dpp_move<0x143, 0xC, false>(0, v);  // row_bcast:31 into rows 2, 3
    return v;
}

// Running max / min over lanes 0..i (lane 63 holds the wave's).
__device__ __forceinline__ float wave_prefix_max(float v) {
    const int lo = __float_as_int(-INFINITY);
    v = fmaxf(v, __int_as_float(dpp_move<0x111, 0xF, false>(lo, __float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_move<0x112, 0xF, false>(lo, __float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_move<0x114, 0xF, false>(lo, __float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_move<0x118, 0xF, false>(lo, __float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_move<0x142, 0xA, false>(lo, __float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_move<0x143, 0xC, false>(lo, __float_as_int(v))));
    return v;
}
__device__ __forceinline__ float wave_prefix_min(float v) {
    const int hi = __float_as_int(INFINITY);
    v = fminf(v, __int_as_float(dpp_move<0x111, 0xF, false>(hi, __float_as_int(v))));
    v = fminf(v, __int_as_float(dpp_move<0x112, 0xF, false>(hi, __float_as_int(v))));
    v = fminf(v, __int_as_float(dpp_move<0x114, 0xF, false>(hi, __float_as_int(v))));
    v = fminf(v, __int_as_float(dpp_move<0x118, 0xF, false>(hi, __float_as_int(v))));
    v = fminf(v, __int_as_float(dpp_move<0x142, 0xA, false>(hi, __float_as_int(v))));
    v = fminf(v, __int_as_float(dpp_move<0x143, 0xC, false>(hi, __float_as_int(v))));
    return v;
}

// Suffix sum over the block (thread t gets the sum over threads >= t) of one
// int per thread.  tmp holds NW ints.  TRAIL = false leaves out the closing
// barrier: the caller then passes a barrier before tmp is written again.
template <int NW, bool TRAIL = true>
__device__ __forceinline__ int block_suffix_sum(int v, int* tmp) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int incl = wave_prefix_sum(v);
    const int total = __builtin_amdgcn_readlane(incl, 63);
    v = total - incl + v;  // this lane's suffix within the wave
    if (lane == 0) tmp[wave] = total;
    __syncthreads();
    int after = 0;
    for (int w = wave + 1; w < NW; ++w) after += tmp[w];
    if (TRAIL) __syncthreads();
    return v + after;
}

// Exclusive prefix sum over the block (thread order) of two ints per thread.
// TRAIL as for block_suffix_sum.
template <int NW, bool TRAIL = true>
__device__ __forceinline__ void block_exclusive_scan2(int& a, int& b, int* tmp) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int ia = wave_prefix_sum(a), ib = wave_prefix_sum(b);
    if (lane == 63) {
        tmp[wave] = ia;
        tmp[NW + wave] = ib;
    }
    __syncthreads();
    int ba = 0, bb = 0;
    for (int w = 0; w < wave; ++w) {
        ba += tmp[w];
        bb += tmp[NW + w];
    }
    if (TRAIL) __syncthreads();
    a = ba + ia - a;
    b = bb + ib - b;
}

}  // namespace qsa
