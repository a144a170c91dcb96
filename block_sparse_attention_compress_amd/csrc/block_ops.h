// Workgroup-wide prefix sums (wave shuffles, then one LDS exchange), shared by
// the top-k selection kernels.
#pragma once

#include "qsa_device.h"

namespace qsa {

// Suffix sum over the block (thread t gets the sum over threads >= t) of one
// int per thread.  tmp holds NW ints.
template <int NW>
__device__ __forceinline__ int block_suffix_sum(int v, int* tmp) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int other = __shfl_down(v, o);
        if (lane + o < 64) v += other;
    }
    if (lane == 0) tmp[wave] = v;
    __syncthreads();
    int after = 0;
    for (int w = wave + 1; w < NW; ++w) after += tmp[w];
    __syncthreads();
    return v + after;
}

// Exclusive prefix sum over the block (thread order) of two ints per thread.
template <int NW>
__device__ __forceinline__ void block_exclusive_scan2(int& a, int& b, int* tmp) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    int ia = a, ib = b;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int pa = __shfl_up(ia, o), pb = __shfl_up(ib, o);
        if (lane >= o) {
            ia += pa;
            ib += pb;
        }
    }
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
    __syncthreads();
    a = ba + ia - a;
    b = bb + ib - b;
}

}  // namespace qsa
