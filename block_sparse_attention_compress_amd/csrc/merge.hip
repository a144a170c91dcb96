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
// weights broadcast from their lanes.  The lane's first 16 partials are loaded
// together with the lse, so a row costs one memory round trip when S <= 16 and
// D <= 256.
#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

constexpr int kMergeBatch = 16;  // partial loads in flight per lane

__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ part_out,
                                                    const float* __restrict__ part_lse, int S, int N, int D,
                                                    uint16_t* __restrict__ out, float* __restrict__ out_lse) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + wave_id();
    if (row >= N) return;  // uniform per wave
    // Every pass over the dims runs on all 64 lanes (a lane past D only skips its
    // loads and stores), so the split weights broadcast from lanes 0..S-1 are
    // always read from active lanes, whatever D is.
    const int d0 = 4 * lane;
    float4 o[kMergeBatch];
    auto load_batch = [&](int d, int sp0) {
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j)
            o[j] = (sp0 + j < S && d < D)
                       ? *reinterpret_cast<const float4*>(part_out + ((int64_t)(sp0 + j) * N + row) * D + d)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
    };
    // the partials do not depend on the lse: their first batch is requested with it
    load_batch(d0, 0);
    const float ls = lane < S ? part_lse[(int64_t)lane * N + row] : -INFINITY;
    const float M = wave_max(ls);
    if (M == -INFINITY) {
        for (int d = d0; d < D; d += 256)
            *reinterpret_cast<uint2*>(out + row * D + d) = make_uint2(0u, 0u);
        if (lane == 0 && out_lse) out_lse[row] = -INFINITY;
        return;
    }
    const float w = lane < S ? expf(ls - M) : 0.f;
    const float z = wave_sum(w);
    const float wn = w / z;
    for (int db = 0; db < D; db += 256) {
        const int d = db + d0;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int sp0 = 0; sp0 < S; sp0 += kMergeBatch) {
            if (sp0 > 0 || db > 0) load_batch(d, sp0);
#pragma unroll
            for (int j = 0; j < kMergeBatch; ++j) {
                if (sp0 + j >= S) break;  // uniform
                const float ws = __shfl(wn, sp0 + j);
                acc.x += ws * o[j].x;
                acc.y += ws * o[j].y;
                acc.z += ws * o[j].z;
                acc.w += ws * o[j].w;
            }
        }
        if (d < D)
            *reinterpret_cast<uint2*>(out + row * D + d) =
                make_uint2(pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w));
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
