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
// are zero and discarded, as the Ascend page pads 12 -> 16 heads).  The prologue
// turns the selection into a per-slot table of K/V row indices in LDS (-1 for a
// masked slot).  A wave then takes 16 selected tokens at a time:
//   S^T[token][head] = K . Q^T   8 x v_mfma_f32_16x16x32_bf16; MFMA m covers dims
//                                32m..32m+31, lane (r, q) giving dims 32m + 8q..+7
//                                of token r, so each operand read covers 64
//                                contiguous bytes of each of the 16 K rows
//   online softmax in fp32, base 2 (x * scale * log2 e), with a lazy reference
//                                max: O and l are rescaled only when a head's
//                                max grows by more than 2^8, so P <= 256
//   O[head][dim] += P . V        16 x v_mfma_f32_16x16x16bf16_1k (P rounded to
//                                bf16; lane (c, q) reads dims 8c..8c+7 and
//                                128+8c..128+8c+7 of the V rows of tokens
//                                4q..4q+3 -- 256 contiguous bytes per 16 lanes --
//                                and output tile n takes dim 128 (n / 8) + 8c +
//                                n % 8)
// The raw K and V rows of a tile are loaded coalesced, all before the first wait
// (their row indices come from the slot table in back-to-back LDS reads), and
// staged in a per-wave LDS tile from which the operands above are read.  An fp8
// cache's rows are loaded and staged as codes (8 per lane instead of 8 bf16) and
// widened exactly to bf16, two codes per conversion, as the operands are read.
// The 4 waves' (m, l, O) are merged in LDS and written as the final bf16 output or
// as an fp32 partial (o, lse) for the log-sum-exp merge.
#include "qsa_device.h"
#include "qsa_launch.h"
#include "attn_body.h"

namespace qsa {

template <bool KV8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(KV8 ? 3 : 2, 8))) void attn_kernel(const AttnParams P) {
    extern __shared__ float smem[];
    const int unit = blockIdx.x;
    const int uh = unit / P.S;
    attend_split<KV8>(P, uh / P.Hkv, uh % P.Hkv, unit % P.S, smem);
}

hipError_t launch_attn(const PagedKV& kv, const Rows& rows, const int32_t* sel_idx, const int32_t* sel_cnt, int k,
                       float scale, int num_splits, bool blocked, const AttnOut& o, hipStream_t st) {
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
    P.blocked = blocked ? 1 : 0;
    P.out = o.out;
    P.out_stride = o.out_stride;
    P.lse = o.lse;
    P.part_out = o.part_out;
    P.part_lse = o.part_lse;
    const int64_t nblocks = (int64_t)rows.R * kv.Hkv * num_splits;
    const int blocks_per_wg = num_splits > 1 && blocked ? (k + num_splits - 1) / num_splits : k;
    P.table_words = 4 * ((blocks_per_wg + 3) & ~3) + kSlotPad;  // keeps the K tiles 16-byte aligned
    const size_t loop = attn_loop_bytes(P.table_words, kv.kv_fp8 != 0);
    const size_t xchg = (size_t)kAttnWaves * P.g * kHeadDim * sizeof(float);
    const size_t lds = loop > xchg ? loop : xchg;
    if (kv.kv_fp8)
        hipLaunchKernelGGL(attn_kernel<true>, dim3((unsigned)nblocks), dim3(256), lds, st, P);
    else
        hipLaunchKernelGGL(attn_kernel<false>, dim3((unsigned)nblocks), dim3(256), lds, st, P);
    return hipGetLastError();
}

}  // namespace qsa
