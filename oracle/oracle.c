/*
 * CPU oracle for the QSA (micro-block sparse attention) hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark call this code; the product path never does.
 * It shares no source with the HIP library.
 *
 * It is deliberately plain: one (sequence, KV head) or one (query row,
 * KV head) per call, fp64 arithmetic wherever the method does not fix a
 * precision, no blocking and no reordering beyond the definitions below.
 *
 * The method (pages "Qwen 4 QSA krijgt decode-contextparallellisme", section
 * "Wat de pull request daadwerkelijk verandert", and its Hebrew and Arabic
 * versions): a light indexer compresses keys into microblocks of 4 tokens,
 * scores the blocks against the query, keeps the best 512 blocks (about 2048
 * token positions), and the softmax and value sum then run over the
 * uncompressed K and V of only those tokens.  The same page (section on how
 * decode context parallelism differs from tensor parallelism) has each
 * partition of the context produce a partial attention result that is then
 * combined; here that is the log-sum-exp merge.
 *
 * Points the pages leave open are fixed as follows (one reading each):
 *  - a block key is the fp32 mean of the block's (up to) 4 keys, summed in the
 *    order ((k0+k1)+(k2+k3)) * 0.25 for a full block, left to right then
 *    divided by n for a partial last block of n < 4 keys;
 *  - one selection per (query row, KV head), scored with the sum of the
 *    group's query heads (query head j belongs to KV head j / (Hq/Hkv));
 *  - a block b is eligible for a row at position t iff 4b <= t;
 *  - order is (score descending, block index ascending): ties go to the lower
 *    index; -0 and +0 compare equal;
 *  - an empty token set gives output 0 and lse = -inf (the Ascend page,
 *    section "Wat de pull request daadwerkelijk toevoegt", keeps fully
 *    masked rows at zero output);
 *  - a split S partitions the ordered selected token list by rank p mod S.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static inline float bf16f(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* ------------------------------------------------------------------ O1
 * Block keys of one (sequence, KV head): keys [L][D] bf16 -> ckey [nb][D]
 * fp32, nb = ceil(L / 4).  Built with -ffp-contract=off so every operation
 * is one correctly rounded fp32 operation. */
int oracle_compress(const uint16_t* keys, int64_t L, int32_t D, float* ckey) {
    if (L < 0 || D <= 0) return -1;
    int64_t nb = (L + 3) / 4;
    for (int64_t b = 0; b < nb; ++b) {
        int64_t n = L - 4 * b < 4 ? L - 4 * b : 4;
        const uint16_t* k = keys + (size_t)(4 * b) * D;
        for (int32_t d = 0; d < D; ++d) {
            float r;
            if (n == 4) {
                float s01 = bf16f(k[d]) + bf16f(k[D + d]);
                float s23 = bf16f(k[2 * D + d]) + bf16f(k[3 * D + d]);
                float s = s01 + s23;
                r = s * 0.25f;
            } else if (n == 3) {
                float s = bf16f(k[d]) + bf16f(k[D + d]);
                s = s + bf16f(k[2 * D + d]);
                r = s / 3.0f;
            } else if (n == 2) {
                float s = bf16f(k[d]) + bf16f(k[D + d]);
                r = s / 2.0f;
            } else {
                r = bf16f(k[d]);
            }
            ckey[(size_t)b * D + d] = r;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ O1b
 * Reduced-precision block keys.  The pages record smaller cache formats for
 * this attention path (an FP8 main KV cache for the sparse-attention path, in
 * "Pengambilan sampel batch-sharded Qwen4Exp: di dalam vLLM PR #61018, dan apa
 * yang dikatakannya tentang Qwen 4", section "Apa yang dikatakan oleh klaster
 * patch di sekitarnya tentang Qwen4Exp"); the library's variant stores block
 * keys in bf16.  A bf16 block key is the O1 fp32 mean rounded to the nearest
 * bf16 value, ties to the even one.  It is returned widened to fp32 (exact), so
 * O2 applies unchanged. */
static float round_to_bf16(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    /* finite inputs: add half an ulp of bf16, plus one if the kept part is odd */
    const uint32_t keep_odd = (u >> 16) & 1u;
    u = (u + 0x7fffu + keep_odd) & 0xffff0000u;
    float r;
    memcpy(&r, &u, 4);
    return r;
}

int oracle_compress_bf16(const uint16_t* keys, int64_t L, int32_t D, float* ckey) {
    int rc = oracle_compress(keys, L, D, ckey);
    if (rc) return rc;
    const int64_t nb = (L + 3) / 4;
    for (int64_t i = 0; i < nb * D; ++i) ckey[i] = round_to_bf16(ckey[i]);
    return 0;
}

/* ------------------------------------------------------------------ O1c
 * fp8 block keys, the same source as O1b: OCP E4M3 ("fn": sign, 4 exponent bits
 * with bias 7, 3 mantissa bits, largest finite value 448, no infinities).  An
 * fp8 block key is the O1 fp32 mean rounded to the nearest E4M3 value, ties to
 * the even code; a mean whose magnitude rounds past 448 is held at 448 (the
 * saturating conversion fp8 caches use, so no key becomes NaN).  The decoded
 * value (exact in fp32) feeds O2 unchanged; the codes are what the cache holds. */
static uint8_t e4m3_encode(float x) {
    const uint8_t sign = signbit(x) ? 0x80 : 0x00;
    const double a = fabs((double)x);
    if (a >= 448.0) return sign | 0x7E;                  /* saturate */
    if (a < 0.015625) {                                  /* below 2^-6: steps of 2^-9 */
        const double q = nearbyint(a * 512.0);           /* 0..8; 8 is 2^-6, code 0x08 */
        return sign | (uint8_t)q;
    }
    int e;
    const double m = frexp(a, &e);                       /* a = m 2^e, m in [0.5, 1) */
    int E = e - 1;                                       /* a = (2m) 2^E, 2m in [1, 2) */
    double q = nearbyint((2.0 * m - 1.0) * 8.0);         /* 3-bit fraction, ties to even */
    if (q == 8.0) {
        q = 0.0;
        E += 1;
    }
    return sign | (uint8_t)(((E + 7) << 3) | (int)q);
}

static float e4m3_decode(uint8_t c) {
    const int E = (c >> 3) & 15, M = c & 7;
    const double v = E ? ldexp(8.0 + M, E - 10) : ldexp((double)M, -9);
    return (float)((c & 0x80) ? -v : v);
}

int oracle_compress_fp8(const uint16_t* keys, int64_t L, int32_t D, float* ckey, uint8_t* codes) {
    int rc = oracle_compress(keys, L, D, ckey);
    if (rc) return rc;
    const int64_t nb = (L + 3) / 4;
    for (int64_t i = 0; i < nb * D; ++i) {
        const uint8_t c = e4m3_encode(ckey[i]);
        if (codes) codes[i] = c;
        ckey[i] = e4m3_decode(c);
    }
    return 0;
}

/* ------------------------------------------------------------------ O2
 * Block scores of one (row, KV head): q [g][D] bf16 holds the g query heads
 * of the group; s[b] = sum_d (sum_j q[j][d]) * ckey[b][d] for b < n_elig,
 * everything in fp64. */
int oracle_scores(const uint16_t* q, int32_t g, int32_t D, const float* ckey, int64_t n_elig, double* s) {
    if (g <= 0 || D <= 0 || n_elig < 0) return -1;
    double* qs = (double*)calloc((size_t)D, sizeof(double));
    if (!qs) return -2;
    for (int32_t j = 0; j < g; ++j)
        for (int32_t d = 0; d < D; ++d) qs[d] += (double)bf16f(q[(size_t)j * D + d]);
    for (int64_t b = 0; b < n_elig; ++b) {
        double acc = 0.0;
        for (int32_t d = 0; d < D; ++d) acc += qs[d] * (double)ckey[(size_t)b * D + d];
        s[b] = acc;
    }
    free(qs);
    return 0;
}

/* ------------------------------------------------------------------ O3
 * Top-k of n scores under (score desc, index asc); the first min(k, n) in
 * that order, returned in ascending index order, -1 padded to k. */
static int by_index(const void* a, const void* b) {
    int32_t ia = *(const int32_t*)a, ib = *(const int32_t*)b;
    return ia < ib ? -1 : (ia > ib ? 1 : 0);
}

typedef struct { double s; int32_t i; } scored;

static int scored_cmp(const void* a, const void* b) {
    const scored* x = (const scored*)a;
    const scored* y = (const scored*)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return x->i < y->i ? -1 : (x->i > y->i ? 1 : 0);
}

int oracle_topk(const double* s, int64_t n, int32_t k, int32_t* sel, int32_t* cnt) {
    if (n < 0 || k < 0) return -1;
    scored* v = (scored*)malloc((size_t)(n > 0 ? n : 1) * sizeof(scored));
    if (!v) return -2;
    for (int64_t b = 0; b < n; ++b) {
        v[b].s = s[b] == 0.0 ? 0.0 : s[b]; /* -0 -> +0 */
        v[b].i = (int32_t)b;
    }
    qsort(v, (size_t)n, sizeof(scored), scored_cmp);
    int64_t m = n < k ? n : k;
    for (int64_t j = 0; j < m; ++j) sel[j] = v[j].i;
    qsort(sel, (size_t)m, sizeof(int32_t), by_index);
    for (int64_t j = m; j < k; ++j) sel[j] = -1;
    *cnt = (int32_t)m;
    free(v);
    return 0;
}

/* ------------------------------------------------------------------ O4
 * Attention of one (row, KV head) over the tokens of the selected blocks.
 *   q    [g][D] bf16     the group's query heads
 *   K, V [L][D] bf16     the sequence's logical keys / values for this KV head
 *   t                    the row's position (decode: L - 1)
 *   sel  [cnt]           selected block indices (ascending)
 * T = { 4b + u : b in sel, 0 <= u < 4, 4b + u < L, 4b + u <= t } in the order
 * of sel; split s of S keeps the tokens whose rank p in T has p mod S == s.
 * For each head: x_p = scale * q.k_p, m = max x, w_p = exp(x_p - m),
 * l = sum w, out = sum w_p v_p / l, lse = m + ln l.  Empty: out 0, lse -inf.
 * out [g][D], lse [g], fp64. */
int oracle_attend(const uint16_t* q, int32_t g, int32_t D, const uint16_t* K, const uint16_t* V, int64_t L,
                  int64_t t, const int32_t* sel, int32_t cnt, double scale, int32_t S, int32_t s, double* out,
                  double* lse) {
    if (g <= 0 || D <= 0 || L < 0 || cnt < 0 || S < 1 || s < 0 || s >= S) return -1;
    int64_t cap = (int64_t)cnt * 4;
    int64_t* tok = (int64_t*)malloc((size_t)(cap > 0 ? cap : 1) * sizeof(int64_t));
    double* x = (double*)malloc((size_t)(cap > 0 ? cap : 1) * sizeof(double));
    if (!tok || !x) { free(tok); free(x); return -2; }
    int64_t nT = 0, p = 0;
    for (int32_t j = 0; j < cnt; ++j) {
        for (int u = 0; u < 4; ++u) {
            int64_t pos = 4 * (int64_t)sel[j] + u;
            if (pos < L && pos <= t) {
                if (p % S == s) tok[nT++] = pos;
                ++p;
            }
        }
    }
    for (int32_t h = 0; h < g; ++h) {
        const uint16_t* qh = q + (size_t)h * D;
        double* oh = out + (size_t)h * D;
        for (int32_t d = 0; d < D; ++d) oh[d] = 0.0;
        if (nT == 0) {
            lse[h] = -INFINITY;
            continue;
        }
        double m = -INFINITY;
        for (int64_t i = 0; i < nT; ++i) {
            const uint16_t* kp = K + (size_t)tok[i] * D;
            double acc = 0.0;
            for (int32_t d = 0; d < D; ++d) acc += (double)bf16f(qh[d]) * (double)bf16f(kp[d]);
            x[i] = scale * acc;
            if (x[i] > m) m = x[i];
        }
        double l = 0.0;
        for (int64_t i = 0; i < nT; ++i) {
            double w = exp(x[i] - m);
            l += w;
            const uint16_t* vp = V + (size_t)tok[i] * D;
            for (int32_t d = 0; d < D; ++d) oh[d] += w * (double)bf16f(vp[d]);
        }
        for (int32_t d = 0; d < D; ++d) oh[d] /= l;
        lse[h] = m + log(l);
    }
    free(tok);
    free(x);
    return 0;
}

/* ------------------------------------------------------------------ O5
 * Merge S partial results: part_out [S][N][D], part_lse [S][N] ->
 * lse = M + ln sum_s exp(lse_s - M) with M = max_s lse_s,
 * out = sum_s exp(lse_s - lse) * o_s; all partials empty -> 0 and -inf. */
int oracle_merge(const double* part_out, const double* part_lse, int32_t S, int64_t N, int32_t D, double* out,
                 double* lse) {
    if (S < 1 || N < 0 || D <= 0) return -1;
    for (int64_t r = 0; r < N; ++r) {
        double M = -INFINITY;
        for (int32_t s = 0; s < S; ++s)
            if (part_lse[(size_t)s * N + r] > M) M = part_lse[(size_t)s * N + r];
        double* o = out + (size_t)r * D;
        for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
        if (M == -INFINITY) {
            lse[r] = -INFINITY;
            continue;
        }
        double z = 0.0;
        for (int32_t s = 0; s < S; ++s) z += exp(part_lse[(size_t)s * N + r] - M);
        double lr = M + log(z);
        for (int32_t s = 0; s < S; ++s) {
            double w = exp(part_lse[(size_t)s * N + r] - lr);
            const double* os = part_out + ((size_t)s * N + r) * D;
            for (int32_t d = 0; d < D; ++d) o[d] += w * os[d];
        }
        lse[r] = lr;
    }
    return 0;
}
