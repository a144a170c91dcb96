// a4 / a6 -- exact softmax attention over the tokens of the selected blocks.
//
// After selection, QSA's softmax and value sum run on the uncompressed K and V
// of only the selected tokens ("Qwen 4 QSA krijgt decode-contextparallellisme",
// section "Wat de pull request daadwerkelijk verandert").  Decode and extend
// share this kernel: a decode row sits at t = L - 1, an extend row at its own t
// with the tokens after t masked.  Split-KV: the selected token slots, in order,
// have ranks p; split s of S takes p mod S == s (the partitions whose partial
// results the same page combines at the end).
//
// Work unit = one workgroup of 4 waves per (row, KV head, split).  The g query
// heads of the KV head form the 16 rows of a matrix-core tile (g <= 16; extra rows
// are zero and discarded, as the Ascend page pads 12 -> 16 heads).  A wave takes
// 32 selected tokens at a time:
//   S^T[token][head] = K . Q^T   8 x v_mfma_f32_16x16x32_bf16 per 16 tokens
//                                (lane (r, q) reads 128 contiguous bytes of the
//                                K row of token r, A operand; Q is the B operand)
//   online softmax in fp32, base 2 (x * scale * log2 e)
//   O[head][dim] += P . V        16 x v_mfma_f32_16x16x32_bf16 per 32 tokens
//                                (P rounded to bf16; lane (c, q) reads 32
//                                contiguous bytes of 8 V rows -- the tokens it
//                                holds in P -- and dim 16c + n feeds output tile n)
// The 4 waves' (m, l, O) are merged in LDS and written as the final bf16 output
// or as an fp32 partial (o, lse) for the log-sum-exp merge.
#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

constexpr int kAttnWaves = 4;
constexpr int kMaxSel = 2048;

struct AttnParams {
    const uint16_t* k;
    const uint16_t* v;
    const int32_t* block_table;
    const int32_t* seq_lens;
    int Hkv, lg_ps, max_pages;
    const uint16_t* q;
    int64_t q_stride;
    const int32_t* q_seq;
    const int32_t* q_pos;
    int R, Hq, g;
    const int32_t* sel;
    const int32_t* cnt;
    int kstride;
    float scale_log2;
    int S;
    uint16_t* out;
    int64_t out_stride;
    float* lse;
    float* part_out;
    float* part_lse;
};

__device__ __forceinline__ uint32_t word_of(const uint4& a, const uint4& b, int e) {
    // dword e (0..7) of the 32-byte pair (a, b)
    const uint4& src = e < 4 ? a : b;
    const int w = e & 3;
    return w == 0 ? src.x : (w == 1 ? src.y : (w == 2 ? src.z : src.w));
}

__global__ __launch_bounds__(256) void attn_kernel(const AttnParams P) {
    __shared__ float smem[kAttnWaves * 16 * kHeadDim];  // 64 KiB; first 10 KiB double as token tables
    __shared__ float wm[kAttnWaves][16], wl[kAttnWaves][16];
    int32_t* tok_base = reinterpret_cast<int32_t*>(smem);               // [kMaxSel]
    uint8_t* tok_nv = reinterpret_cast<uint8_t*>(smem + kMaxSel);       // [kMaxSel]

    const int S = P.S;
    const int unit = blockIdx.x;
    const int s = unit % S;
    const int uh = unit / S;
    const int h = uh % P.Hkv;
    const int row = uh / P.Hkv;
    const int seq = P.q_seq ? P.q_seq[row] : row;
    const int L = P.seq_lens[seq];
    const int t = P.q_pos ? P.q_pos[row] : L - 1;
    const int64_t lim = min((int64_t)L, (int64_t)t + 1);  // tokens at positions < lim are visible
    const int g = P.g;
    const int tid = threadIdx.x;

    int nsel = P.cnt[(int64_t)row * P.Hkv + h];
    nsel = max(0, min(nsel, P.kstride));
    const int32_t* sel_row = P.sel + ((int64_t)row * P.Hkv + h) * P.kstride;
    for (int j = tid; j < nsel; j += 256) {
        const int b = sel_row[j];
        const int64_t pos0 = 4 * (int64_t)b;
        if (b < 0 || pos0 >= lim) {
            tok_base[j] = 0;
            tok_nv[j] = 0;
        } else {
            tok_base[j] = (int32_t)token_row(P.block_table, seq, P.max_pages, P.Hkv, h, P.lg_ps, pos0);
            tok_nv[j] = (uint8_t)min(lim - pos0, (int64_t)4);
        }
    }
    __syncthreads();

    const int ntok = 4 * nsel;                                   // token slots of the selection
    const int n_s = ntok > s ? (ntok - s + S - 1) / S : 0;      // slots of this split
    const int ntiles = (n_s + 31) / 32;

    const int lane = tid & 63;
    const int wave = wave_id();
    const int c = lane & 15;
    const int qq = lane >> 4;

    bf16x8 qb[8];
    if (c < g) {
        const uint16_t* qp = P.q + (int64_t)row * P.q_stride + (int64_t)(h * g + c) * kHeadDim + 64 * qq;
#pragma unroll
        for (int m = 0; m < 8; ++m) qb[m] = *reinterpret_cast<const bf16x8*>(qp + 8 * m);
    } else {
#pragma unroll
        for (int m = 0; m < 8; ++m) qb[m] = bf16x8{};
    }

    float m_run = -INFINITY;
    float l_run = 0.f;
    floatx4 O[16];
#pragma unroll
    for (int nt = 0; nt < 16; ++nt) O[nt] = floatx4{0.f, 0.f, 0.f, 0.f};

    for (int tile = wave; tile < ntiles; tile += kAttnWaves) {
        const int n0 = tile * 32;
        // ---- K rows of tokens 16 th + c (A operand)
        bf16x8 kb[2][8];
#pragma unroll
        for (int th = 0; th < 2; ++th) {
            const int n = n0 + 16 * th + c;
            const int p = s + S * n;
            const bool valid = n < n_s && (p & 3) < tok_nv[p >> 2];
            if (valid) {
                const uint16_t* kp = P.k + (int64_t)(tok_base[p >> 2] + (p & 3)) * kHeadDim + 64 * qq;
#pragma unroll
                for (int m = 0; m < 8; ++m) kb[th][m] = *reinterpret_cast<const bf16x8*>(kp + 8 * m);
            } else {
#pragma unroll
                for (int m = 0; m < 8; ++m) kb[th][m] = bf16x8{};
            }
        }
        // ---- V rows of tokens 16 th + 4 qq + i, dims 16c .. 16c+15 (B operand)
        uint4 vv[2][4][2];
        bool vok[2][4];
#pragma unroll
        for (int th = 0; th < 2; ++th) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int n = n0 + 16 * th + 4 * qq + i;
                const int p = s + S * n;
                const bool valid = n < n_s && (p & 3) < tok_nv[p >> 2];
                vok[th][i] = valid;
                if (valid) {
                    const uint4* vp = reinterpret_cast<const uint4*>(
                        P.v + (int64_t)(tok_base[p >> 2] + (p & 3)) * kHeadDim + 16 * c);
                    vv[th][i][0] = vp[0];
                    vv[th][i][1] = vp[1];
                } else {
                    vv[th][i][0] = make_uint4(0, 0, 0, 0);
                    vv[th][i][1] = make_uint4(0, 0, 0, 0);
                }
            }
        }
        // ---- S^T = K . Q^T: st[th][i] = S[head c][token 16 th + 4 qq + i]
        floatx4 st[2];
#pragma unroll
        for (int th = 0; th < 2; ++th) {
            st[th] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < 8; ++m) st[th] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[th][m], qb[m], st[th], 0, 0, 0);
        }
        // ---- online softmax (base 2)
        float x[8];
        float mx = -INFINITY;
#pragma unroll
        for (int th = 0; th < 2; ++th)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[4 * th + i] = vok[th][i] ? st[th][i] * P.scale_log2 : -INFINITY;
                mx = fmaxf(mx, x[4 * th + i]);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        m_run = m_new;
        uint32_t pb[4];
        float psum = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t lo = f32_to_bf16_rne(__builtin_amdgcn_exp2f(x[2 * w] - m_use));
            const uint32_t hi = f32_to_bf16_rne(__builtin_amdgcn_exp2f(x[2 * w + 1] - m_use));
            psum += __uint_as_float(lo << 16) + __uint_as_float(hi << 16);
            pb[w] = lo | (hi << 16);
        }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float a_i = __shfl(alpha, 4 * qq + i);
#pragma unroll
            for (int nt = 0; nt < 16; ++nt) O[nt][i] *= a_i;
        }
        // ---- O += P . V; k-slot 4 th + i of lane (., qq) is token 16 th + 4 qq + i
        bf16x8 pa;
        {
            uint32_t* pw = reinterpret_cast<uint32_t*>(&pa);
            pw[0] = pb[0];
            pw[1] = pb[1];
            pw[2] = pb[2];
            pw[3] = pb[3];
        }
#pragma unroll
        for (int nt = 0; nt < 16; ++nt) {
            const int e = nt >> 1;
            uint32_t bw[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const int th = w >> 1;
                const int i0 = 2 * (w & 1);
                const uint32_t d0 = word_of(vv[th][i0][0], vv[th][i0][1], e);
                const uint32_t d1 = word_of(vv[th][i0 + 1][0], vv[th][i0 + 1][1], e);
                bw[w] = (nt & 1) ? ((d0 >> 16) | (d1 & 0xffff0000u)) : ((d0 & 0xffffu) | (d1 << 16));
            }
            bf16x8 vb;
            uint32_t* vw = reinterpret_cast<uint32_t*>(&vb);
            vw[0] = bw[0];
            vw[1] = bw[1];
            vw[2] = bw[2];
            vw[3] = bw[3];
            O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, O[nt], 0, 0, 0);
        }
    }

    // ---- merge the 4 waves in LDS
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    __syncthreads();  // token tables are dead; smem becomes the O exchange
    if (qq == 0) {
        wm[wave][c] = m_run;
        wl[wave][c] = l_tot;
    }
    float* ow = smem + wave * 16 * kHeadDim;
#pragma unroll
    for (int nt = 0; nt < 16; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) ow[(4 * qq + i) * kHeadDim + 16 * c + nt] = O[nt][i];
    __syncthreads();

    const float kLn2 = 0.6931471805599453f;
    for (int e = tid; e < g * kHeadDim; e += 256) {
        const int hh = e >> 8;
        const int d = e & (kHeadDim - 1);
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, wm[w][hh]);
        float o = 0.f, lse_v = -INFINITY;
        if (M != -INFINITY) {
            float num = 0.f, den = 0.f;
#pragma unroll
            for (int w = 0; w < kAttnWaves; ++w) {
                const float f = __builtin_amdgcn_exp2f(wm[w][hh] - M);
                num += f * smem[(w * 16 + hh) * kHeadDim + d];
                den += f * wl[w][hh];
            }
            o = num / den;
            lse_v = (M + __log2f(den)) * kLn2;
        }
        const int head = h * g + hh;
        if (P.part_out) {
            const int64_t prow = ((int64_t)s * P.R + row) * P.Hq + head;
            P.part_out[prow * kHeadDim + d] = o;
            if (d == 0) P.part_lse[prow] = lse_v;
        } else {
            P.out[(int64_t)row * P.out_stride + (int64_t)head * kHeadDim + d] = (uint16_t)f32_to_bf16_rne(o);
            if (d == 0 && P.lse) P.lse[(int64_t)row * P.Hq + head] = lse_v;
        }
    }
}

hipError_t launch_attn(const PagedKV& kv, const Rows& rows, const int32_t* sel_idx, const int32_t* sel_cnt, int k,
                       float scale, int num_splits, const AttnOut& o, hipStream_t st) {
    if (rows.R == 0) return hipSuccess;
    AttnParams P;
    P.k = kv.k;
    P.v = kv.v;
    P.block_table = kv.block_table;
    P.seq_lens = kv.seq_lens;
    P.Hkv = kv.Hkv;
    P.lg_ps = kv.lg_ps;
    P.max_pages = kv.max_pages;
    P.q = rows.q;
    P.q_stride = rows.q_stride;
    P.q_seq = rows.q_seq;
    P.q_pos = rows.q_pos;
    P.R = rows.R;
    P.Hq = rows.Hq;
    P.g = rows.Hq / kv.Hkv;
    P.sel = sel_idx;
    P.cnt = sel_cnt;
    P.kstride = k;
    P.scale_log2 = scale * 1.4426950408889634f;
    P.S = num_splits;
    P.out = o.out;
    P.out_stride = o.out_stride;
    P.lse = o.lse;
    P.part_out = o.part_out;
    P.part_lse = o.part_lse;
    const int64_t nblocks = (int64_t)rows.R * kv.Hkv * num_splits;
    hipLaunchKernelGGL(attn_kernel, dim3((unsigned)nblocks), dim3(256), 0, st, P);
    return hipGetLastError();
}

}  // namespace qsa
