// a5 -- log-sum-exp merge of split-KV partial results.
//
// Decode context parallelism has every partition of the context produce a
// partial attention result and combines them at the end ("Qwen 4 QSA krijgt
// decode-contextparallellisme", the section on how it differs from tensor
// parallelism).  A partial is (o_s normalised, lse_s); the combination is
//   lse = M + ln sum_s exp(lse_s - M),  out = sum_s exp(lse_s - lse) o_s.
//
// One wave per output row: lane s < S holds lse_s, the wave max / sum give M and
// the normaliser, and each lane then accumulates 4 dims at a time with the split
// weights broadcast from their lanes.
#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ part_out,
                                                    const float* __restrict__ part_lse, int S, int N, int D,
                                                    uint16_t* __restrict__ out, float* __restrict__ out_lse) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + wave_id();
    if (row >= N) return;
    const float ls = lane < S ? part_lse[(int64_t)lane * N + row] : -INFINITY;
    const float M = wave_max(ls);
    if (M == -INFINITY) {
        for (int d = 4 * lane; d < D; d += 256)
            *reinterpret_cast<uint2*>(out + row * D + d) = make_uint2(0u, 0u);
        if (lane == 0 && out_lse) out_lse[row] = -INFINITY;
        return;
    }
    const float w = lane < S ? expf(ls - M) : 0.f;
    const float z = wave_sum(w);
    const float wn = w / z;
    for (int d = 4 * lane; d < D; d += 256) {
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int sp = 0; sp < S; ++sp) {
            const float ws = __shfl(wn, sp);
            const float4 o = *reinterpret_cast<const float4*>(part_out + ((int64_t)sp * N + row) * D + d);
            acc.x += ws * o.x;
            acc.y += ws * o.y;
            acc.z += ws * o.z;
            acc.w += ws * o.w;
        }
        *reinterpret_cast<uint2*>(out + row * D + d) = make_uint2(pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w));
    }
    if (lane == 0 && out_lse) out_lse[row] = M + logf(z);
}

hipError_t launch_merge(const float* part_out, const float* part_lse, int S, int N, int D, uint16_t* out,
                        float* out_lse, hipStream_t st) {
    if (N == 0) return hipSuccess;
    hipLaunchKernelGGL(merge_kernel, dim3((N + 3) / 4), dim3(256), 0, st, part_out, part_lse, S, N, D, out, out_lse);
    return hipGetLastError();
}

}  // namespace qsa
