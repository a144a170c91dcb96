// a1 -- block keys: the fp32 mean of each 4-token microblock's keys.
//
// The QSA indexer compresses keys into microblocks of 4 tokens ("Qwen 4 QSA
// krijgt decode-contextparallellisme", section "Wat de pull request
// daadwerkelijk verandert").  How a block key is pooled is not stated; the
// library uses the fp32 mean with a fixed add order, ((k0+k1)+(k2+k3))*0.25 for
// a full block and (left-to-right sum) / n for a partial last block, so that the
// result is reproducible bit for bit.
//
// One workgroup per (64-token chunk, KV head, sequence); chunks start at the
// one holding first_token, so a decode refresh launches one chunk per
// (sequence, KV head).  Thread t handles
// microblock t/16 of the chunk and dims 16*(t%16) .. +15: four 32-byte key reads
// (16-byte reads of fp8 E4M3 keys, decoded exactly),
// one 64-byte block-key write (32 bytes for bf16 block keys, 16 for fp8 E4M3
// ones, which store the same mean rounded to nearest, ties to even, fp8 held at
// +-448).  A pure HBM stream (read 2 B, write 1 B -- 0.5 B for bf16, 0.25 B for
// fp8 -- per key element of a block).
#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

template <int KT, bool KV8>
__global__ __launch_bounds__(256) void compress_kernel(const void* __restrict__ k, void* __restrict__ ckey,
                                                       const int32_t* __restrict__ block_table,
                                                       const int32_t* __restrict__ seq_lens,
                                                       const int32_t* __restrict__ first_token, int Hkv, int lg_ps,
                                                       int max_pages) {
    const int seq = blockIdx.z;
    const int h = blockIdx.y;
    const int L = seq_lens[seq];
    const int first = first_token ? max(first_token[seq], 0) : 0;
    const int mb = threadIdx.x >> 4;
    const int e = threadIdx.x & 15;
    // chunks are counted from the one holding first_token
    const int64_t chunk = (int64_t)(first >> 6) + blockIdx.x;
    const int64_t pos0 = (chunk * 16 + mb) * 4;
    if (pos0 >= L || pos0 + 3 < first) return;
    const int n = (L - pos0) < 4 ? (int)(L - pos0) : 4;

    const int64_t row = token_row(block_table, seq, max_pages, Hkv, h, lg_ps, pos0);
    // the 4 tokens of a block are consecutive rows of one page (page_size is a
    // power of two >= 4); this thread reads dims 16 e .. 16 e + 15 of each
    float r[16];
    if (KV8) {
        // fp8 rows: 16 codes (one uint4) per token, token u 256 bytes = 16 uint4 on
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(k) + row * kHeadDim + 16 * e);
        uint4 a[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) a[u] = u < n ? src[u * 16] : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float4 k0 = unpack_fp8x4((&a[0].x)[w]), k1 = unpack_fp8x4((&a[1].x)[w]);
            const float4 k2 = unpack_fp8x4((&a[2].x)[w]), k3 = unpack_fp8x4((&a[3].x)[w]);
            r[4 * w + 0] = block_mean(k0.x, k1.x, k2.x, k3.x, n);
            r[4 * w + 1] = block_mean(k0.y, k1.y, k2.y, k3.y, n);
            r[4 * w + 2] = block_mean(k0.z, k1.z, k2.z, k3.z, n);
            r[4 * w + 3] = block_mean(k0.w, k1.w, k2.w, k3.w, n);
        }
    } else {
        // bf16 rows: token u is 256 elements = 32 uint4 further on
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(k) + row * kHeadDim + 16 * e);
        uint4 a[4][2];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (u < n) {
                a[u][0] = src[u * 32];
                a[u][1] = src[u * 32 + 1];
            } else {
                a[u][0] = make_uint4(0, 0, 0, 0);
                a[u][1] = make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            const uint32_t w0 = (&a[0][w >> 2].x)[w & 3];
            const uint32_t w1 = (&a[1][w >> 2].x)[w & 3];
            const uint32_t w2 = (&a[2][w >> 2].x)[w & 3];
            const uint32_t w3 = (&a[3][w >> 2].x)[w & 3];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const float k0 = half ? bf16_hi(w0) : bf16_lo(w0);
                const float k1 = half ? bf16_hi(w1) : bf16_lo(w1);
                const float k2 = half ? bf16_hi(w2) : bf16_lo(w2);
                const float k3 = half ? bf16_hi(w3) : bf16_lo(w3);
                r[2 * w + half] = block_mean(k0, k1, k2, k3, n);
            }
        }
    }
    // block-key row in [num_pages][Hkv][page_size / 4][256]
    const int64_t brow = ((row >> lg_ps) << (lg_ps - 2)) + ((row & ((1 << lg_ps) - 1)) >> 2);
    if (KT == kKeyFP8) {
        uint4* dst = reinterpret_cast<uint4*>(static_cast<uint8_t*>(ckey) + brow * kHeadDim + 16 * e);
        *dst = make_uint4(pack_fp8x4(r[0], r[1], r[2], r[3]), pack_fp8x4(r[4], r[5], r[6], r[7]),
                          pack_fp8x4(r[8], r[9], r[10], r[11]), pack_fp8x4(r[12], r[13], r[14], r[15]));
    } else if (KT == kKeyBF16) {
        uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(ckey) + brow * kHeadDim + 16 * e);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            dst[i] = make_uint4(pack_bf16x2(r[8 * i], r[8 * i + 1]), pack_bf16x2(r[8 * i + 2], r[8 * i + 3]),
                                pack_bf16x2(r[8 * i + 4], r[8 * i + 5]), pack_bf16x2(r[8 * i + 6], r[8 * i + 7]));
    } else {
        float4* dst = reinterpret_cast<float4*>(static_cast<float*>(ckey) + brow * kHeadDim + 16 * e);
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] = make_float4(r[4 * i], r[4 * i + 1], r[4 * i + 2], r[4 * i + 3]);
    }
}

hipError_t launch_compress(const PagedKV& kv, const int32_t* first_token, int span, hipStream_t st) {
    if (kv.batch == 0 || kv.max_seq_len == 0) return hipSuccess;
    // tokens [first, first + span) touch at most ceil(span / 64) + 1 chunks
    const int chunks = first_token ? (span + 63) / 64 + 1 : (kv.max_seq_len + 63) / 64;
    dim3 grid(chunks, kv.Hkv, kv.batch);
#define QSA_COMPRESS2(KT, KV8)                                                                                  \
    hipLaunchKernelGGL((compress_kernel<KT, KV8>), grid, dim3(256), 0, st, kv.k, kv.ckey, kv.block_table,       \
                       kv.seq_lens, first_token, kv.Hkv, kv.lg_ps, kv.max_pages)
#define QSA_COMPRESS(KT)               \
    do {                               \
        if (kv.kv_fp8)                 \
            QSA_COMPRESS2(KT, true);   \
        else                           \
            QSA_COMPRESS2(KT, false);  \
    } while (0)
    if (kv.ckey_type == kKeyFP8)
        QSA_COMPRESS(kKeyFP8);
    else if (kv.ckey_type == kKeyBF16)
        QSA_COMPRESS(kKeyBF16);
    else
        QSA_COMPRESS(kKeyF32);
#undef QSA_COMPRESS
#undef QSA_COMPRESS2
    return hipGetLastError();
}

}  // namespace qsa
