/*
 * qsa.h -- C ABI of libqsa.so, the MI355X (gfx950) hot path of QSA
 * micro-block sparse attention.
 *
 * The method: a light indexer compresses the keys of a sequence into
 * microblocks of 4 tokens, scores every block against the query, keeps the
 * best 512 blocks (about 2048 token positions), and exact softmax attention
 * then runs over the uncompressed K and V of only those tokens ("Qwen 4 QSA
 * krijgt decode-contextparallellisme", section "Wat de pull request
 * daadwerkelijk verandert").  The same page splits the main KV read into
 * partitions whose partial attention results are combined at the end; here
 * the partitions are split-KV work units on one GPU merged by log-sum-exp.
 * Head dimension 256 in bf16 and the (query, KV) head pairs (16,2), (24,2),
 * (12,1), (6,1), (3,1) come from "Qwen4-Exp QSA komt naar Huawei's Ascend",
 * section "Wat de pull request daadwerkelijk toevoegt".
 *
 * Conventions shared by every entry point
 *  - Every pointer argument is a DEVICE pointer owned by the caller, except
 *    the qsa_kv_t descriptor itself, which lives in host memory.  The library
 *    never allocates device memory and keeps no pointer after a call returns.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  No call synchronises or copies device -> host, so every call
 *    may be captured in a HIP graph.
 *  - Arguments are validated on the host before anything is launched; a
 *    rejected call launches nothing and returns QSA_ERR_INVALID_ARG or
 *    QSA_ERR_UNSUPPORTED.  There is no silent fallback.  Contents of device
 *    buffers (block tables, lengths, selections) are trusted: they must obey
 *    the rules stated below.
 *  - qsa_last_error() describes the most recent failure on the calling thread.
 *
 * Notation: B sequences, Hq query heads, Hkv KV heads, g = Hq / Hkv (query
 * head j belongs to KV head j / g), D = 256, L_i the length of sequence i,
 * nb_i = ceil(L_i / 4) blocks.  A query row r has a sequence q_seq[r] and a
 * position t = q_pos[r] (decode: one row per sequence with t = L_i - 1).
 * Block b is eligible for the row iff 4b <= t.
 */
#ifndef QSA_H
#define QSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QSA_API __attribute__((visibility("default")))

#define QSA_OK 0
#define QSA_ERR_INVALID_ARG (-1) /* bad pointer, size, stride or range */
#define QSA_ERR_UNSUPPORTED (-2) /* valid but outside what the kernels handle */
#define QSA_ERR_HIP (-3)         /* a HIP launch reported an error */

#define QSA_HEAD_DIM 256
#define QSA_MICROBLOCK 4
#define QSA_DEFAULT_TOPK 512
#define QSA_MAX_TOPK 2048
#define QSA_MAX_GROUP 16            /* query heads per KV head */
#define QSA_MAX_SPLITS 64
#define QSA_MAX_SEQ_LEN (1 << 20)   /* tokens per sequence */
#define QSA_CKEY_FP32 0             /* block keys stored as fp32 */
#define QSA_CKEY_BF16 1             /* block keys stored as bf16 (rounded fp32 means) */
#define QSA_CKEY_FP8 2              /* block keys stored as fp8 E4M3 (rounded, saturated fp32 means) */
#define QSA_KV_BF16 0               /* K and V rows stored as bf16 */
#define QSA_KV_FP8 1                /* K and V rows stored as fp8 E4M3 codes, unit scale */
#define QSA_NOALLOC_SCRATCH_BYTES (8u << 20) /* static device scratch of qsa_sparse_attn_decode_noalloc, per GPU */

/*
 * Paged KV cache.  Page p of the pool holds, for every KV head, page_size
 * consecutive tokens of one sequence:
 *   k, v   bf16  [num_pages][Hkv][page_size][256]; with kv_dtype QSA_KV_FP8
 *                fp8 E4M3 codes in the same layout (256 B per row), each code
 *                being the value itself (unit scale: an fp8 cache without
 *                calibration scales; the batch-sharded sampling page, section on
 *                the surrounding patch cluster, records an FP8 main KV cache
 *                for this attention path).  Every kernel reads them as their
 *                exact bf16 values: results are those of a bf16 cache holding
 *                the decoded values.
 *   ckey   fp32  [num_pages][Hkv][page_size / 4][256]   block keys, paged by
 *                the same block table, so a page's keys and block keys never
 *                diverge (the DCP page keeps selector and main cache in one
 *                cache group for that reason).  With ckey_dtype
 *                QSA_CKEY_BF16 the same layout holds bf16 block keys: each is
 *                the fp32 mean below rounded to the nearest bf16, ties to even
 *                (half the bytes of the dominant decode stream; the page on
 *                batch-sharded sampling, section on the surrounding patch
 *                cluster, records smaller cache formats for this path).  With
 *                QSA_CKEY_FP8 it holds one byte per element: OCP E4M3 ("fn":
 *                bias 7, 3 mantissa bits, largest finite 448, no infinities),
 *                the fp32 mean rounded to nearest, ties to the even code, and
 *                held at +-448 past that range (a quarter of the fp32 bytes).
 *   block_table int32 [batch][max_pages_per_seq]: token i of sequence s lives
 *                in page block_table[s][i / page_size], slot i % page_size.
 *   seq_lens    int32 [batch]: L_s, 0 <= L_s <= max_seq_len.
 * page_size is a power of two >= 4 (a contiguous cache is one page of
 * page_size >= max_seq_len with an identity table).  max_seq_len is a host
 * bound on every L_s, used to size grids.
 */
typedef struct qsa_kv {
    const void* k;
    const void* v;
    void* ckey;              /* fp32, bf16 or fp8 block keys, by ckey_dtype */
    const int32_t* block_table;
    const int32_t* seq_lens;
    int32_t batch;
    int32_t num_kv_heads;
    int32_t head_dim;        /* must be 256 */
    int32_t page_size;
    int32_t num_pages;
    int32_t max_pages_per_seq;
    int32_t max_seq_len;
    int32_t ckey_dtype;      /* QSA_CKEY_FP32 (0), QSA_CKEY_BF16 (1) or QSA_CKEY_FP8 (2) */
    int32_t kv_dtype;        /* QSA_KV_BF16 (0) or QSA_KV_FP8 (1) */
} qsa_kv_t;

/* Library version (major * 10000 + minor * 100 + patch). */
QSA_API int qsa_version(void);

/* Message of the last failed call on this thread ("" if none). */
QSA_API const char* qsa_last_error(void);

/*
 * a1 -- block keys.  Source: "Qwen 4 QSA krijgt decode-contextparallellisme", section "Wat de pull
 * request daadwerkelijk verandert" (the indexer compresses the keys into microblocks at
 * compression ratio 4). For every sequence s and KV head h, and every block b with 4b < L_s and
 * 4b + 3 >= first_token[s] (first_token NULL = 0), writes
 *   ckey[b] = fp32 mean of the block's n = min(4, L_s - 4b) keys,
 * computed exactly as ((k0 + k1) + (k2 + k3)) * 0.25 for n = 4 and as the left-to-right sum
 * divided by n (correctly rounded) for n < 4 (bf16 and fp8 block keys: that mean rounded to
 * nearest, ties to even; fp8 held at +-448).  The pages say only that keys are compressed into
 * 4-token microblocks; this pooling is the stated reading.  Idempotent: a page shared by two
 * sequences gets the same values from both.  Decode calls it with first_token = L_s - 1 to refresh
 * the block holding the newest token; extend with the first new position.  max_new_tokens is a
 * host bound on L_s - first_token[s] used to size the grid (<= 0: max_seq_len); it is ignored when
 * first_token is NULL.
 */
QSA_API int qsa_compress_keys(const qsa_kv_t* kv, const int32_t* first_token, int32_t max_new_tokens,
                              void* stream);

/*
 * a2 -- block scores.  Source: "Qwen 4 QSA krijgt decode-contextparallellisme", section "Wat de
 * pull request daadwerkelijk verandert" (the indexer scores the microblocks against the query). q:
 * bf16 rows, row r at q + r * q_row_stride (elements), heads contiguous inside a row ([Hq][256]).
 * q_seq / q_pos (int32 [R]) give each row's sequence and position (0 <= t < L of that sequence; a
 * negative t gives the row no eligible block); both may be NULL for decode
 * (row r = sequence r at t = L_r - 1, R must equal batch).  Writes
 *   scores[(r * Hkv + h) * score_stride + b] = (sum_{j in group h} q[r][j]) . ckey[b]
 * in fp32 for b < n_elig(r) = min(t / 4 + 1, score_stride); entries at or after n_elig(r) are not
 * written.  The scale is not applied (it does not change the order).  Rows sharing a sequence are
 * scored with matrix cores when there are more rows than sequences (extend).  R <= 65535 per call.
 */
QSA_API int qsa_block_scores(const qsa_kv_t* kv, const void* q, int64_t q_row_stride, const int32_t* q_seq,
                     const int32_t* q_pos, int32_t R, int32_t Hq, float* scores, int32_t score_stride,
                     void* stream);

/*
 * a1 + a2 for one decode step in one launch (source as for a1 and a2: "Qwen 4 QSA krijgt
 * decode-contextparallellisme", section "Wat de pull request daadwerkelijk verandert"). The same
 * results, bit for bit, as
 *   qsa_compress_keys(kv, first_token = {L_s - 1}, 1, stream);
 *   qsa_block_scores(kv, q, q_row_stride, NULL, NULL, batch, Hq, scores, score_stride, stream);
 * i.e. the block key holding each sequence's newest token is rebuilt from K (and stored), and
 * every eligible block of every row is scored, the newest one with its rebuilt key.  Sequences
 * with L_s = 0 are skipped.  The block keys rebuilt here must not be read by another sequence of
 * the same call (the page holding a sequence's newest token belongs to that sequence alone, as in
 * a paged cache that copies a shared page before appending to it).  Arguments and errors as for
 * the two calls.
 */
QSA_API int qsa_decode_scores_refresh(const qsa_kv_t* kv, const void* q, int64_t q_row_stride, int32_t Hq,
                                      float* scores, int32_t score_stride, void* stream);

/*
 * a3 -- top-k selection.  Source: "Qwen 4 QSA krijgt decode-contextparallellisme", section "Wat de
 * pull request daadwerkelijk verandert" (the best 512 blocks, about 2,048 token positions, are
 * kept); the -1 padding of a selection list is the one on "Qwen4-Exp QSA komt naar Huawei's
 * Ascend", section "Wat de pull request daadwerkelijk toevoegt". For each (row, KV head): among
 * the n_elig(r) scores (q_pos as above; NULL means n_elig = score_stride for every row), keeps the
 * k largest under the order (score descending, block index ascending; -0 equals +0), and writes
 * them in ascending block order to
 *   sel_idx[(r * Hkv + h) * k + j], j < cnt, then -1 up to k,
 *   sel_cnt[r * Hkv + h] = cnt = min(k, n_elig(r)).
 * 0 <= k <= QSA_MAX_TOPK.  Scores must be finite.  Rows are read with 16-byte loads when
 * score_stride is a multiple of 4 and scores is 16-byte aligned (any stride works).
 */
QSA_API int qsa_topk_blocks(const float* scores, int32_t score_stride, const int32_t* q_pos, int32_t R, int32_t Hkv,
                    int32_t k, int32_t* sel_idx, int32_t* sel_cnt, void* stream);

/*
 * a3, long rows (source as for a3: "Qwen 4 QSA krijgt decode-contextparallellisme", section "Wat
 * de pull request daadwerkelijk verandert"). The same selection as qsa_topk_blocks, bit for bit,
 * for rows longer than 16,384 blocks computed in two launches: every 8,192-block slice of a row
 * keeps its own top k (so one row spreads over many compute units), then the top k of those
 * candidates is taken.  The candidates live in `workspace` (device memory, 16-byte aligned,
 * caller-owned, contents on entry ignored and on return unspecified), which must hold
 * qsa_topk_workspace_bytes(R, Hkv, k, score_stride) bytes; when that is 0 the call is
 * qsa_topk_blocks and workspace may be NULL.  Arguments and errors as qsa_topk_blocks, plus
 * QSA_ERR_INVALID_ARG for a missing, short or misaligned workspace.  Calls sharing one workspace
 * must be ordered on one stream.
 */
QSA_API int qsa_topk_blocks_ws(const float* scores, int32_t score_stride, const int32_t* q_pos, int32_t R,
                               int32_t Hkv, int32_t k, int32_t* sel_idx, int32_t* sel_cnt, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Workspace bytes qsa_topk_blocks_ws needs (0 for rows that are selected in
 * one stage, for k == 0, and for arguments qsa_topk_blocks would reject). */
QSA_API size_t qsa_topk_workspace_bytes(int32_t R, int32_t Hkv, int32_t k, int32_t score_stride);

/*
 * a4 -- sparse attention, decode (one row per sequence at t = L_s - 1). Source: "Qwen 4 QSA krijgt
 * decode-contextparallellisme", section "Wat de pull request daadwerkelijk verandert" (softmax and
 * value sum run over the uncompressed K and V of the selected tokens; the split read whose partial
 * results are combined at the end), and "Qwen4-Exp QSA komt naar Huawei's Ascend", section "Wat de
 * pull request daadwerkelijk toevoegt" (head dimension 256 in bf16, the original 1/sqrt(256)
 * scale, zero output for fully masked rows). sel_idx / sel_cnt as written by qsa_topk_blocks
 * ([batch][Hkv][k], ascending, every block eligible).  For query head j of KV head h the token set
 * is
 *   T = { 4b + u : b selected, 0 <= u < 4, 4b + u < L_s }
 * and the result is softmax(scale * q_j . K_T^T) . V_T; scale <= 0 selects 1/sqrt(256) = 1/16.
 * Arithmetic: the g query heads of a KV head form one 16-row bf16 matrix-core tile; q . K^T
 * accumulates in fp32, the online softmax (running max and normaliser) is fp32, the weights P are
 * rounded to bf16 for the P . V product (fp32 accumulation), and the normaliser sums the rounded
 * weights.  An empty T gives output 0 and lse = -inf (fully masked rows keep a zero output, as on
 * the Ascend page).
 *
 * Split-KV: the selected tokens, in order, have ranks p = 0..|T|-1.
 *  - part_out != NULL: num_splits = S >= 1 partials are written, split s
 *    holding the tokens with p mod S == s (interleaved),
 *      part_out fp32 [S][batch][Hq][256] (normalised), part_lse fp32 [S][batch][Hq]
 *    (natural log); out / lse are not touched.  qsa_merge_lse combines them.
 *  - part_out == NULL: the final result is written, out bf16 at
 *    out + row * out_row_stride ([Hq][256] per row), lse fp32 [batch][Hq]
 *    (lse may be NULL).  num_splits = 0 lets the library choose the split
 *    count; any S > 1 splits the selected blocks into S contiguous ranges
 *    (the merged result does not depend on the partition) and merges them
 *    internally through `workspace`, which must hold
 *    qsa_decode_workspace_bytes(batch, Hq, num_splits) bytes.
 */
QSA_API int qsa_sparse_attn_decode(const qsa_kv_t* kv, const void* q, int64_t q_row_stride, int32_t Hq,
                           const int32_t* sel_idx, const int32_t* sel_cnt, int32_t k, float scale,
                           int32_t num_splits, void* out, int64_t out_row_stride, float* lse, float* part_out,
                           float* part_lse, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes qsa_sparse_attn_decode needs for num_splits (0 = the
 * library's own choice) when it writes the final result. */
QSA_API size_t qsa_decode_workspace_bytes(int32_t batch, int32_t Hq, int32_t num_splits);

/*
 * qsa_sparse_attn_decode without a workspace argument, for callers that cannot allocate device memory:
 * code under HIP graph capture that must not call hipMalloc, tight serving loops that keep a fixed
 * memory budget, and harnesses that forbid allocation.  The same computation and result, bit for bit,
 * as qsa_sparse_attn_decode writing the final result (part_out == NULL) with the same num_splits
 * (0 = the library's choice); the arguments mean the same.
 *
 * The split partials (qsa_decode_workspace_bytes(batch, Hq, S) bytes for the split count S used) live
 * in a static device array of QSA_NOALLOC_SCRATCH_BYTES (8 MiB), one per GPU, held from the library's
 * load until the process ends.  The library looks its address up once per device, on the first call
 * with that device current.  The call allocates nothing and calls no allocating routine.  Nothing in the
 * scratch needs clearing: every partial the merge reads is written earlier in the same call.
 *
 * Errors: as qsa_sparse_attn_decode; QSA_ERR_UNSUPPORTED, with a message and nothing launched, when the
 * partials would exceed QSA_NOALLOC_SCRATCH_BYTES (use qsa_sparse_attn_decode with a workspace, or fewer
 * splits); QSA_ERR_HIP if the scratch's address cannot be looked up.  All calls on one GPU share its
 * scratch: calls that may overlap on one GPU (several streams, several host threads) race and must be
 * ordered by the caller, e.g. issued on one stream.
 */
QSA_API int qsa_sparse_attn_decode_noalloc(const qsa_kv_t* kv, const void* q, int64_t q_row_stride, int32_t Hq,
                                           const int32_t* sel_idx, const int32_t* sel_cnt, int32_t k, float scale,
                                           int32_t num_splits, void* out, int64_t out_row_stride, float* lse,
                                           void* stream);

/*
 * Fused decode (source as for a2-a5: "Qwen 4 QSA krijgt decode-contextparallellisme", section "Wat
 * de pull request daadwerkelijk verandert"). a2 + a3 + a4 + a5 of one decode step in a single
 * launch -- the same block scores, the same top-k order and selection, and the same split
 * attention and log-sum-exp merge as the separate calls above, with the steps of different
 * (sequence, KV head) units overlapping.  As qsa_decode_scores_refresh does, the block key holding
 * each sequence's newest token is rebuilt from K, stored and scored with (a rebuilt key must not
 * be read by another sequence of the same call); every other block key must be current
 * (qsa_compress_keys).
 *   sel_idx int32 [batch][Hkv][k] and sel_cnt int32 [batch][Hkv] receive the
 *     selection, exactly as qsa_topk_blocks writes it;
 *   out bf16 at out + row * out_row_stride ([Hq][256] per row, 8-byte aligned,
 *     stride a multiple of 4) and lse fp32 [batch][Hq] (may be NULL) receive
 *     the result, as qsa_sparse_attn_decode writes it;
 *   num_splits: attention splits per (sequence, KV head), 0 = the library's
 *     choice; the result does not depend on it beyond rounding.
 * workspace: qsa_decode_fused_workspace_bytes(kv, Hq, k, num_splits) bytes, 256-byte aligned. It
 * holds the scores, the partials and a control area of counters and flags.  Zero-fill the
 * workspace once before its first use; the library keeps the control area consistent from then
 * on, so later calls need no clearing (a workspace may also serve a later call with fewer
 * sequences).  After every call its ticket and arrival counters are zero again, the int32 word at
 * workspace + 12 counts the calls made on the workspace, and each unit's ready word holds the
 * number of the call that last raised it.  Calls that share a workspace must not overlap (issue
 * them on one stream).  An attention item waits for its unit's selection for at most about a
 * second (only a stalled device takes that long): when a wait is abandoned, the int32 word at
 * workspace + 8 is incremented (it is never reset by the library) and that unit's out and lse
 * rows are written as NaN, never as a result computed from a selection that may be stale.
 */
QSA_API int qsa_decode_fused(const qsa_kv_t* kv, const void* q, int64_t q_row_stride, int32_t Hq, int32_t k,
                             float scale, int32_t num_splits, int32_t* sel_idx, int32_t* sel_cnt, void* out,
                             int64_t out_row_stride, float* lse, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Workspace bytes of qsa_decode_fused (0 if the arguments are invalid). */
QSA_API size_t qsa_decode_fused_workspace_bytes(const qsa_kv_t* kv, int32_t Hq, int32_t k, int32_t num_splits);

/*
 * a6 -- sparse attention, extend.  Source: "Qwen4-Exp QSA komt naar Huawei's Ascend", section "Wat
 * de pull request daadwerkelijk toevoegt" (extend / prefill rows, bf16 head dimension 256, heads
 * padded to a power of two with the padded outputs discarded, zero output for fully masked rows)
 * and "Qwen 4 QSA krijgt decode-contextparallellisme", section "Wat de pull request daadwerkelijk
 * verandert" (attention over the selected tokens' uncompressed K and V).  Like decode, but every
 * query row r has its own sequence q_seq[r], position t = q_pos[r] and selection, and tokens after
 * t are masked: T = { 4b + u : b selected, 4b + u < L, 4b + u <= t }. Writes out (bf16, row stride
 * out_row_stride) and lse ([R][Hq], may be NULL). The g heads of a KV head are padded to 16
 * matrix-core rows in the kernel; the padded rows are discarded (the Ascend page pads 12 -> 16 for
 * its tiler).
 */
QSA_API int qsa_sparse_attn_extend(const qsa_kv_t* kv, const void* q, int64_t q_row_stride, const int32_t* q_seq,
                           const int32_t* q_pos, int32_t R, int32_t Hq, const int32_t* sel_idx,
                           const int32_t* sel_cnt, int32_t k, float scale, void* out, int64_t out_row_stride,
                           float* lse, void* stream);

/*
 * a6 with a split read -- qsa_sparse_attn_extend for chunks of few rows.  Source: the extend rows
 * of "Qwen4-Exp QSA komt naar Huawei's Ascend", section "Wat de pull request daadwerkelijk
 * toevoegt", with the split read of "Qwen 4 QSA krijgt decode-contextparallellisme", section "Wat
 * de pull request daadwerkelijk verandert" (partial attention results over parts of the selected
 * tokens, combined at the end by log-sum-exp).  Arguments, token sets T and outputs as
 * qsa_sparse_attn_extend; the selected blocks of each (row, KV head) are cut into S contiguous
 * ranges, each attended by its own workgroup, and the S partials are merged as qsa_merge_lse does.
 * The merged result does not depend on the partition, so it equals the unsplit one up to rounding
 * (fp32 partials, then one bf16 rounding).  num_splits = 0 lets the library choose S from R * Hkv
 * and k (about 256 workgroups, at least 16 blocks per split, at most 16 splits; 1 once R * Hkv
 * reaches 256); S = 1 is the unsplit call.  With S > 1, out must be dense (out_row_stride ==
 * Hq * 256, 8-byte aligned) and `workspace` (device memory owned by the caller, 256-byte aligned)
 * must hold qsa_extend_workspace_bytes(R, Hq, num_splits) bytes; it holds the partials between
 * the two launches, so calls sharing it must be ordered on one stream.  Errors: those of
 * qsa_sparse_attn_extend, QSA_ERR_INVALID_ARG for num_splits outside [0, QSA_MAX_SPLITS] or a
 * missing, short or misaligned workspace, QSA_ERR_UNSUPPORTED for a strided out with S > 1.
 */
QSA_API int qsa_sparse_attn_extend_split(const qsa_kv_t* kv, const void* q, int64_t q_row_stride,
                                         const int32_t* q_seq, const int32_t* q_pos, int32_t R, int32_t Hq,
                                         const int32_t* sel_idx, const int32_t* sel_cnt, int32_t k, float scale,
                                         int32_t num_splits, void* out, int64_t out_row_stride, float* lse,
                                         void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of qsa_sparse_attn_extend_split: partials for R rows of Hq heads at num_splits
 * splits (num_splits = 0: enough for any split count the library chooses).  0 when no workspace
 * is needed (S <= 1) or the arguments are invalid. */
QSA_API size_t qsa_extend_workspace_bytes(int32_t R, int32_t Hq, int32_t num_splits);

/*
 * a6, query-tile union -- the same attention as qsa_sparse_attn_extend (same arguments, same
 * result set T per row, outputs within rounding of it: only the order in which a row's tokens are
 * summed differs), computed per tile of 8 consecutive query rows and KV head over the union of the
 * tile's selections: each selected block is read from the cache once per tile, into LDS, and used
 * there by every row of the tile that selected it; a row's unselected or invisible tokens are
 * masked.  Source: the per-row sets of "Qwen4-Exp QSA komt naar Huawei's Ascend", section "Wat de
 * pull request daadwerkelijk toevoegt", and the selection of "Qwen 4 QSA krijgt
 * decode-contextparallellisme", section "Wat de pull request daadwerkelijk verandert"; the tiling
 * is this library's.  Rows of a tile may belong to different sequences (each sequence of a tile is
 * a pass of its own).  It reads fewer cache bytes than the per-row kernel when adjacent rows
 * share selected blocks, and does more masked matrix-core work when they do not.
 */
QSA_API int qsa_sparse_attn_extend_union(const qsa_kv_t* kv, const void* q, int64_t q_row_stride,
                                         const int32_t* q_seq, const int32_t* q_pos, int32_t R, int32_t Hq,
                                         const int32_t* sel_idx, const int32_t* sel_cnt, int32_t k, float scale,
                                         void* out, int64_t out_row_stride, float* lse, void* stream);

/*
 * a5 -- log-sum-exp merge of S partial results.  Source: "Qwen 4 QSA krijgt
 * decode-contextparallellisme", section "Wat de pull request daadwerkelijk verandert" (the
 * attention results of the split read are combined at the end) and its question "Hoe verschilt
 * decode-contextparallellisme van tensorparallellisme?" (each rank reads its own slice, the
 * partial results are merged):  part_out fp32 [S][N][D], part_lse fp32 [S][N] ->
 *   lse = M + ln sum_s exp(lse_s - M),  M = max_s lse_s,
 *   out = sum_s exp(lse_s - lse) * o_s   (bf16 [N][D]),
 * all partials -inf -> out 0, lse -inf.  1 <= S <= QSA_MAX_SPLITS, D a multiple of 4 up to 1024.
 * out_lse may be NULL.
 */
QSA_API int qsa_merge_lse(const float* part_out, const float* part_lse, int32_t S, int32_t N, int32_t D, void* out_bf16,
                  float* out_lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */
