// a6 variant -- extend attention over the union of a query tile's selections.
//
// Extend rows attend each over their own selected tokens ("Qwen4-Exp QSA komt
// naar Huawei's Ascend", section "Wat de pull request daadwerkelijk toevoegt";
// the selection itself: "Qwen 4 QSA krijgt decode-contextparallellisme",
// section "Wat de pull request daadwerkelijk verandert").  The per-row kernel
// (attn.hip) gathers every row's K/V rows on its own, so a block chosen by
// several rows of a chunk is read once per row.  This kernel takes a tile of
// kUT consecutive query rows (one KV head) and reads each block of the union
// of their selections once, into LDS, where every row of the tile that chose
// it uses it.  The result is the same set-defined attention per row:
//   T_r = { 4b + u : b in sel_r, 4b + u < L, 4b + u <= t_r },
// only the order in which each row's tokens are summed differs.
//
// Work unit = one workgroup of kUT waves per (tile, KV head); wave w owns row
// tile * kUT + w for the whole launch, with its (m, l, O) in registers, so no
// exchange or merge between waves is needed.  Per sequence present in the tile
// and per window of kUWin blocks:
//   1. membership bitmaps, one per row, from the rows' selections (LDS atomics);
//   2. their union, compacted in ascending block order;
//   3. each union block's first K/V row from the block table, and per row and
//      group of kUG union blocks a mask of the blocks the row chose;
//   4. groups of kUG union blocks (4 kUG token rows) staged in LDS -- the next
//      group's loads in flight in registers, two staging buffers, one barrier
//      per group -- and each wave runs its own members of the group, 4 blocks
//      (16 tokens) at a time, through the same matrix-core tile as the per-row
//      kernel (S^T = K Q^T on v_mfma_f32_16x16x32_bf16, lazy-rescaled online
//      softmax in base 2, P rounded to bf16, O += P V on
//      v_mfma_f32_16x16x16bf16_1k), reading the operands from the staged rows by
//      per-lane address.  Only a row's last tile of a group and its partly
//      visible block carry masked tokens.
#include "qsa_device.h"
#include "qsa_launch.h"
#include "attn_body.h"

namespace qsa {

constexpr int kUT = 8;         // query rows per tile (one wave each)
constexpr int kUThreads = 64 * kUT;
constexpr int kUWin = 4096;    // blocks per union window
constexpr int kUWords = kUWin / 32;
constexpr int kUG = 16;        // union blocks per staged group (64 token rows)

struct UnionParams {
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
    uint16_t* out;
    int64_t out_stride;
    float* lse;
};

template <bool KV8>
__global__ __launch_bounds__(kUThreads) void attn_union_kernel(const UnionParams P) {
    typedef typename KVRaw<KV8>::type Raw;  // 8 elements of a row
    constexpr int RB = kTileRowBytes<KV8>;  // bytes of a staged row
    constexpr int EB = KV8 ? 1 : 2;         // bytes per element
    // K/V staging: [buffer][K, V][token row].  While a window is set up, its first
    // bytes hold the rows' membership bitmaps and the union list instead.
    __shared__ __attribute__((aligned(16))) uint8_t stage[2][2][4 * kUG * RB];
    static_assert(sizeof(stage) >= (size_t)(kUT * kUWords + kUWin) * 4, "setup arrays fit the staging space");
    uint32_t (*bm)[kUWords] = reinterpret_cast<uint32_t (*)[kUWords]>(&stage[0][0][0]);  // row w chose block j
    int32_t* ublk = reinterpret_cast<int32_t*>(&stage[0][0][0]) + kUT * kUWords;       // union, ascending
    __shared__ int32_t ubase[kUWin];        // union block i: K/V row of its first token
    __shared__ uint16_t gmask[kUT][kUWin / kUG];  // row w: which blocks of union group gi it chose
    __shared__ int rdiag[kUT];              // row w: union index of its partly visible block, or -1
    __shared__ int rseq[kUT], rvis[kUT];    // per row: sequence (-1: none), last visible position
    __shared__ int wsum[kUThreads / 64];
    __shared__ int sh_nu;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = wave_id();
    const int c = lane & 15;
    const int qq = lane >> 4;
    const int h = blockIdx.y;
    const int g = P.g;
    const int row = blockIdx.x * kUT + wave;
    const bool has_row = row < P.R;

    // ---- this wave's row: query operand, sequence, visible range
    bf16x8 qb[8];
    {
        const int rr = has_row ? row : 0;
        const uint16_t* qp = P.q + (int64_t)rr * P.q_stride + (int64_t)(h * g + min(c, g - 1)) * kHeadDim + 8 * qq;
#pragma unroll
        for (int m = 0; m < 8; ++m) qb[m] = *reinterpret_cast<const bf16x8*>(qp + 32 * m);
        if (c >= g) {
#pragma unroll
            for (int m = 0; m < 8; ++m) qb[m] = bf16x8{};
        }
    }
    if (lane == 0) {
        int sq = -1, vis = -1;
        if (has_row) {
            sq = P.q_seq[row];
            const int L = P.seq_lens[sq];
            vis = min(P.q_pos[row], L - 1);  // tokens at positions <= vis are visible
        }
        rseq[wave] = sq;
        rvis[wave] = vis;
    }
    __syncthreads();
    const int my_seq = rseq[wave];
    const int my_vis = rvis[wave];
    const int my_cnt = has_row ? max(0, min(P.cnt[(int64_t)row * P.Hkv + h], P.kstride)) : 0;

    float m_run = -INFINITY;  // reference max of head c (log2 units), same in every qq group
    float l_run = 0.f;        // this lane's share of the head's normaliser
    floatx4 O[16];
#pragma unroll
    for (int nt = 0; nt < 16; ++nt) O[nt] = floatx4{0.f, 0.f, 0.f, 0.f};

    // staging: thread -> token rows ts + 16 p of a group (union block (ts + 16 p) / 4), piece pc of the row
    const int ts = tid >> 5;
    const int pc = tid & 31;
    const uint8_t* kbytes = reinterpret_cast<const uint8_t*>(P.k);
    const uint8_t* vbytes = reinterpret_cast<const uint8_t*>(P.v);

    for (int pass = 0; pass < kUT; ++pass) {
        // one pass per distinct sequence of the tile, in row order (uniform)
        const int sq = rseq[pass];
        if (sq < 0) continue;
        bool seen = false;
        for (int j = 0; j < pass; ++j) seen |= rseq[j] == sq;
        if (seen) continue;
        int nb = 0;  // blocks holding a token visible to some row of this sequence
        for (int j = 0; j < kUT; ++j)
            if (rseq[j] == sq && rvis[j] >= 0) nb = max(nb, rvis[j] / 4 + 1);
        const bool mine = my_seq == sq && my_vis >= 0;

        for (int w0 = 0; w0 < nb; w0 += kUWin) {
            // ---- 1. membership bitmaps of the window
            for (int i = tid; i < kUT * kUWords; i += kUThreads) (&bm[0][0])[i] = 0u;
            __syncthreads();
            for (int j = lane; j < my_cnt; j += 64) {
                if (!mine) break;
                const int b = P.sel[((int64_t)row * P.Hkv + h) * P.kstride + j];
                if (b >= w0 && b < w0 + kUWin && 4 * (int64_t)b <= my_vis)
                    atomicOr(&bm[wave][(b - w0) >> 5], 1u << ((b - w0) & 31));
            }
            __syncthreads();
            // ---- 2. the union, compacted in ascending order
            {
                int pcnt = 0;
                uint32_t u = 0;
                if (tid < kUWords) {
#pragma unroll
                    for (int w = 0; w < kUT; ++w) u |= bm[w][tid];
                    pcnt = __popc(u);
                }
                int incl = pcnt;  // inclusive scan within the wave
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const int y = __shfl_up(incl, o);
                    if (lane >= o) incl += y;
                }
                if (lane == 63) wsum[wave] = incl;
                __syncthreads();
                int before = 0;
                for (int w = 0; w < wave; ++w) before += wsum[w];
                if (tid == kUThreads - 1) sh_nu = before + incl;
                int pos = before + incl - pcnt;
                while (u) {
                    const int bit = __ffs(u) - 1;
                    u &= u - 1;
                    ublk[pos++] = w0 + 32 * tid + bit;
                }
                __syncthreads();
            }
            const int nu = sh_nu;
            const int ngrp = (nu + kUG - 1) / kUG;
            // ---- 3. the union blocks' K/V rows, and per row and group the chosen blocks
            if (tid < kUT) rdiag[tid] = -1;
            __syncthreads();
            for (int e = tid; e < nu; e += kUThreads)
                ubase[e] = (int32_t)token_row(P.block_table, sq, P.max_pages, P.Hkv, h, P.lg_ps, 4 * (int64_t)ublk[e]);
            for (int e = tid; e < kUT * ngrp; e += kUThreads) {
                const int w = e / ngrp, gi = e % ngrp;
                const int dblk = rseq[w] == sq && rvis[w] >= 0 ? rvis[w] >> 2 : -1;  // block holding t
                uint32_t msk = 0;
                for (int j = 0; j < kUG; ++j) {
                    const int ui = kUG * gi + j;
                    if (ui >= nu) break;
                    const int b = ublk[ui];
                    if ((bm[w][(b - w0) >> 5] >> ((b - w0) & 31)) & 1u) {
                        msk |= 1u << j;
                        if (b == dblk) rdiag[w] = ui;
                    }
                }
                gmask[w][gi] = (uint16_t)msk;
            }
            __syncthreads();
            const int my_diag = rdiag[wave];
            const int diag_live = (2 << (my_vis & 3)) - 1;  // its tokens up to t

            // ---- 4. groups of kUG union blocks (4 kUG token rows) staged in LDS
            // this thread's K/V row piece p of group gi (token row ts + 16 p; past the
            // end of the union: row 0)
            auto issue1 = [&](int gi, int p, Raw& kr, Raw& vr) {
                const int tr = ts + 16 * p;
                const int ui = kUG * gi + (tr >> 2);
                // a block's 4 rows lie in one page, so the rows of its tokens at or past L
                // exist too (they are masked)
                const int64_t rr = ui < nu ? (int64_t)ubase[ui] + (tr & 3) : 0;
                const int64_t off = rr * kHeadDim * EB + (int64_t)sizeof(Raw) * pc;
                kr = *reinterpret_cast<const Raw*>(kbytes + off);
                vr = *reinterpret_cast<const Raw*>(vbytes + off);
            };
            auto stage1 = [&](int buf, int p, const Raw& kr, const Raw& vr) {
                const int tr = ts + 16 * p;
                *reinterpret_cast<Raw*>(&stage[buf][0][tr * RB + sizeof(Raw) * pc]) = kr;
                *reinterpret_cast<Raw*>(&stage[buf][1][tr * RB + sizeof(Raw) * pc]) = vr;
            };
            // (named registers, not an array: an array here was kept in scratch memory)
            Raw k0, k1, k2, k3, v0, v1, v2, v3;
            auto issue = [&](int gi) {
                issue1(gi, 0, k0, v0);
                issue1(gi, 1, k1, v1);
                issue1(gi, 2, k2, v2);
                issue1(gi, 3, k3, v3);
            };
            auto stage_write = [&](int buf) {
                stage1(buf, 0, k0, v0);
                stage1(buf, 1, k1, v1);
                stage1(buf, 2, k2, v2);
                stage1(buf, 3, k3, v3);
            };
            // group gi from staging buffer buf, for this wave's row: its member blocks
            // of the group, 4 at a time (16 tokens), gathered from the staged rows
            auto compute = [&](int gi, int buf) {
                // the group's blocks this row chose (bit j: union block kUG gi + j)
                const uint32_t mask = mine ? gmask[wave][gi] : 0u;
                const int nm = __popc(mask);
                if (nm == 0) return;  // wave-uniform
                // lane l < nm: the group slot of member l (the l-th set bit of mask)
                int slot = 0;
                {
                    uint32_t mm = mask;
                    for (int j = 0; j < lane && mm; ++j) mm &= mm - 1;
                    slot = mm ? __ffs(mm) - 1 : 0;
                }
                const uint8_t* ktile = stage[buf][0];
                const uint8_t* vtile = stage[buf][1];
                for (int j0 = 0; j0 < nm; j0 += 4) {
                    // K operand: token c of the tile = token c & 3 of member j0 + c / 4
                    const int sk = __shfl(slot, min(j0 + (c >> 2), nm - 1));
                    const uint8_t* krow = ktile + (4 * sk + (c & 3)) * RB;
                    // this lane's tokens 4 qq + i: member j0 + qq, all visible unless it is
                    // the block holding t
                    const int jm = j0 + qq;
                    const int sv = __shfl(slot, min(jm, nm - 1));
                    const int live = jm < nm ? (kUG * gi + sv == my_diag ? diag_live : 15) : 0;
                    floatx4 st = {0.f, 0.f, 0.f, 0.f};
                    {
                        bf16x8 kb[8];
#pragma unroll
                        for (int m = 0; m < 8; ++m) {
                            const uint4 x = kv_bf16x8(*reinterpret_cast<const Raw*>(krow + EB * (32 * m + 8 * qq)));
                            kb[m] = __builtin_bit_cast(bf16x8, x);
                        }
#pragma unroll
                        for (int m = 0; m < 8; ++m) st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[m], qb[m], st, 0, 0, 0);
                    }
                    uint4 vv[4][2];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint8_t* vr = vtile + (4 * sv + i) * RB + EB * 8 * c;
                        vv[i][0] = kv_bf16x8(*reinterpret_cast<const Raw*>(vr));
                        vv[i][1] = kv_bf16x8(*reinterpret_cast<const Raw*>(vr + EB * 128));
                    }
                    float x[4];
                    float mx = -INFINITY;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        x[i] = (live >> i) & 1 ? st[i] * P.scale_log2 : -INFINITY;
                        mx = fmaxf(mx, x[i]);
                    }
                    mx = fmaxf(mx, __shfl_xor(mx, 16));
                    mx = fmaxf(mx, __shfl_xor(mx, 32));
                    if (__ballot(mx > m_run + kLazy)) {
                        const float m_new = mx > m_run + kLazy ? fmaxf(m_run, mx) : m_run;
                        const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
                        m_run = m_new;
                        l_run *= alpha;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float a_i = __shfl(alpha, 4 * qq + i);
#pragma unroll
                            for (int nt = 0; nt < 16; ++nt) O[nt][i] *= a_i;
                        }
                    }
                    const float m_use = m_run == -INFINITY ? 0.f : m_run;
                    uint32_t pw[2];
                    float psum = 0.f;
#pragma unroll
                    for (int w = 0; w < 2; ++w) {
                        pw[w] = pack_bf16x2_hw(__builtin_amdgcn_exp2f(x[2 * w] - m_use),
                                               __builtin_amdgcn_exp2f(x[2 * w + 1] - m_use));
                        psum += bf16_lo(pw[w]) + bf16_hi(pw[w]);
                    }
                    l_run += psum;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (!((live >> i) & 1)) {
                            vv[i][0] = make_uint4(0, 0, 0, 0);
                            vv[i][1] = make_uint4(0, 0, 0, 0);
                        }
                    bf16x4s pa;
                    {
                        uint32_t* p32 = reinterpret_cast<uint32_t*>(&pa);
                        p32[0] = pw[0];
                        p32[1] = pw[1];
                    }
#pragma unroll
                    for (int nt = 0; nt < 16; ++nt) {
                        const int hf = nt >> 3, e = (nt & 7) >> 1;
                        const uint32_t d0 = u4_word(vv[0][hf], e), d1 = u4_word(vv[1][hf], e);
                        const uint32_t d2 = u4_word(vv[2][hf], e), d3 = u4_word(vv[3][hf], e);
                        bf16x4s vb;
                        uint32_t* v32 = reinterpret_cast<uint32_t*>(&vb);
                        constexpr uint32_t kLo = 0x05040100u, kHi = 0x07060302u;
                        v32[0] = __builtin_amdgcn_perm(d1, d0, (nt & 1) ? kHi : kLo);
                        v32[1] = __builtin_amdgcn_perm(d3, d2, (nt & 1) ? kHi : kLo);
                        O[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, O[nt], 0, 0, 0);
                    }
                }
            };

            // group 0 staged, group 1 in flight in registers; then per group: compute
            // it, stage the next, issue the one after, barrier (every step stages and
            // issues, past the end too, so the waits stay exact)
            issue(0);
            stage_write(0);
            issue(1);
            __syncthreads();
            for (int gi = 0; gi < ngrp; ++gi) {
                compute(gi, gi & 1);
                stage_write((gi + 1) & 1);
                issue(gi + 2);
                __syncthreads();
            }
        }
    }

    // ---- this wave's row: O / l and the lse per head
    if (!has_row) return;
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    // lane (c, qq) holds O for heads 4 qq + i; their m and l sit in lanes (4 qq + i, .)
    const float kLn2 = 0.6931471805599453f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int hh = 4 * qq + i;
        const float lh = __shfl(l_tot, hh);
        const float mh = __shfl(m_run, hh);
        if (hh >= g) continue;
        const float inv = lh > 0.f ? 1.0f / lh : 0.f;
        const int head = h * g + hh;
        uint16_t* dst = P.out + (int64_t)row * P.out_stride + (int64_t)head * kHeadDim;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int d = 128 * hf + 8 * c;
            uint32_t w[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) w[j] = pack_bf16x2_hw(O[8 * hf + 2 * j][i] * inv, O[8 * hf + 2 * j + 1][i] * inv);
            uint16_t* p = dst + d;
            if (((reinterpret_cast<uintptr_t>(p)) & 15) == 0) {
                *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    p[2 * j] = (uint16_t)(w[j] & 0xffffu);
                    p[2 * j + 1] = (uint16_t)(w[j] >> 16);
                }
            }
        }
        if (c == 0 && P.lse) P.lse[(int64_t)row * P.Hq + head] = lh > 0.f ? (mh + __log2f(lh)) * kLn2 : -INFINITY;
    }
}

hipError_t launch_attn_union(const PagedKV& kv, const Rows& rows, const int32_t* sel_idx, const int32_t* sel_cnt, int k,
                             float scale, uint16_t* out, int64_t out_stride, float* lse, hipStream_t st) {
    if (rows.R == 0) return hipSuccess;
    UnionParams P;
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
    P.out = out;
    P.out_stride = out_stride;
    P.lse = lse;
    dim3 grid((unsigned)((rows.R + kUT - 1) / kUT), (unsigned)kv.Hkv);
    if (kv.kv_fp8)
        hipLaunchKernelGGL(attn_union_kernel<true>, grid, dim3(kUThreads), 0, st, P);
    else
        hipLaunchKernelGGL(attn_union_kernel<false>, grid, dim3(kUThreads), 0, st, P);
    return hipGetLastError();
}

}  // namespace qsa
