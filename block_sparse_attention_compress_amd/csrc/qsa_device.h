// Device-side helpers shared by the QSA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

constexpr int kHeadDim = 256;
constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// The same packing by the hardware conversion (one v_cvt_pk_bf16_f32, round to
// nearest even): equal to pack_bf16x2 for finite inputs.  Used where the
// rounding sits in a hot loop (attention weights, outputs); block keys keep the
// integer form above.
typedef float qsa_f2v __attribute__((ext_vector_type(2)));
typedef __bf16 qsa_bf2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2_hw(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((qsa_f2v){lo, hi}, qsa_bf2v));
}

// Streaming loads: the nontemporal hint keeps data read once (the block-key
// scan) from being allocated in the caches on its way through.
typedef float qsa_f4v __attribute__((ext_vector_type(4)));
typedef unsigned int qsa_u2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float4 load_stream(const float4* p) {
    const qsa_f4v x = __builtin_nontemporal_load(reinterpret_cast<const qsa_f4v*>(p));
    return make_float4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ uint2 load_stream(const uint2* p) {
    const qsa_u2v x = __builtin_nontemporal_load(reinterpret_cast<const qsa_u2v*>(p));
    return make_uint2(x[0], x[1]);
}
__device__ __forceinline__ uint32_t load_stream(const uint32_t* p) { return __builtin_nontemporal_load(p); }

// Block-key storage types (qsa_kv_t.ckey_dtype).
constexpr int kKeyF32 = 0;
constexpr int kKeyBF16 = 1;
constexpr int kKeyFP8 = 2;  // OCP E4M3 ("fn": bias 7, largest finite 448)

// 4 floats -> 4 E4M3 codes (first value in the low byte), rounded to nearest
// even by the conversion unit; magnitudes past 448 are held at 448.
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
    auto sat = [](float x) { return fminf(fmaxf(x, -448.0f), 448.0f); };
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(a), sat(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(c), sat(d), w, true);
    return (uint32_t)w;
}

// 4 E4M3 codes (low byte first) -> 4 floats (exact).
__device__ __forceinline__ float4 unpack_fp8x4(uint32_t w) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    return make_float4(lo[0], lo[1], hi[0], hi[1]);
}

// Block key element: the fp32 mean of the first n (1..4) of a block's keys,
// ((k0 + k1) + (k2 + k3)) * 0.25 for a full block, the left-to-right sum divided
// by n (correctly rounded) for a partial last block.
__device__ __forceinline__ float block_mean(float k0, float k1, float k2, float k3, int n) {
    if (n == 4) {
        const float s01 = k0 + k1;
        const float s23 = k2 + k3;
        return (s01 + s23) * 0.25f;
    }
    if (n == 3) return __fdiv_rn((k0 + k1) + k2, 3.0f);
    if (n == 2) return (k0 + k1) * 0.5f;  // exact halving == division by 2
    return k0;
}

// Row index (in 256-element rows) of token `pos` of sequence `seq`, KV head h,
// in a paged [num_pages][Hkv][page_size][256] pool.
__device__ __forceinline__ int64_t token_row(const int32_t* __restrict__ block_table, int seq, int max_pages,
                                             int Hkv, int h, int lg_ps, int64_t pos) {
    const int64_t page = block_table[(int64_t)seq * max_pages + (pos >> lg_ps)];
    return ((page * Hkv + h) << lg_ps) + (pos & ((1 << lg_ps) - 1));
}

// Order-preserving map float -> uint32 (larger float, larger key); -0 maps as +0.
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ int wave_max_int(int v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

}  // namespace qsa
