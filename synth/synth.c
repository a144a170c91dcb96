/*
 * Seeded synthetic inputs for the QSA decode / extend workloads.
 *
 * This file holds no attention arithmetic: it only turns (seed, stream,
 * counter) triples into numbers and scatters them into the logical and the
 * paged layouts.  Both the CPU oracle and the HIP library are fed from it.
 *
 * Generator definition (counter based, so any element can be produced on its
 * own and the logical and paged copies agree exactly):
 *   mix(z)          = SplitMix64 finaliser (Steele, Lea, Flood 2014):
 *                     z ^= z>>30; z *= 0xBF58476D1CE4E5B9;
 *                     z ^= z>>27; z *= 0x94D049BB133111EB; z ^= z>>31
 *   key(seed, s)    = mix(mix(seed) ^ mix(s + 0x632BE59BD9B4E019))
 *   u64(key, i)     = mix(key + (i + 1) * 0x9E3779B97F4A7C15)
 *                     (the i-th SplitMix64 output of a generator seeded with key)
 *   unit_open(x)    = ((x >> 11) + 1) * 2^-53         in (0, 1]
 *   unit(x)         = (x >> 11) * 2^-53               in [0, 1)
 *   normal(key, i)  = Box-Muller on the pair j = i/2:
 *                     r = sqrt(-2 ln unit_open(u64(key, 2j))),
 *                     th = 2 pi unit(u64(key, 2j+1)),
 *                     even i -> r cos th, odd i -> r sin th   (double)
 *   bf16(x)         = round-to-nearest-even of the float32 value (float)x.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t synth_key(uint64_t seed, uint64_t stream) {
    return mix64(mix64(seed) ^ mix64(stream + 0x632BE59BD9B4E019ULL));
}

uint64_t synth_u64(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GOLDEN); }

static inline double unit_open(uint64_t x) { return (double)((x >> 11) + 1) * 0x1.0p-53; }
static inline double unit_closed_open(uint64_t x) { return (double)(x >> 11) * 0x1.0p-53; }

double synth_uniform(uint64_t key, uint64_t i) { return unit_closed_open(synth_u64(key, i)); }

double synth_normal(uint64_t key, uint64_t i) {
    uint64_t j = i >> 1;
    double r = sqrt(-2.0 * log(unit_open(synth_u64(key, 2 * j))));
    double th = 6.283185307179586476925286766559 * unit_closed_open(synth_u64(key, 2 * j + 1));
    return (i & 1) ? r * sin(th) : r * cos(th);
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)(u >> 16); /* inf / nan: truncate */
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

uint16_t synth_bf16_from_float(float f) { return f32_to_bf16_rne(f); }

/* ---------------------------------------------------------------- threading */

typedef void (*range_fn)(void* ctx, int64_t lo, int64_t hi);
typedef struct { range_fn fn; void* ctx; int64_t lo, hi; } range_job;

static void* range_thread(void* p) {
    range_job* j = (range_job*)p;
    j->fn(j->ctx, j->lo, j->hi);
    return NULL;
}

static void parallel_for(range_fn fn, void* ctx, int64_t n, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (n < 4096 || nthreads == 1) { fn(ctx, 0, n); return; }
    pthread_t th[256];
    range_job jobs[256];
    int joined[256];
    int64_t per = (n + nthreads - 1) / nthreads;
    int nt = 0;
    for (int t = 0; t < nthreads; ++t) {
        int64_t lo = t * per, hi = lo + per < n ? lo + per : n;
        if (lo >= hi) break;
        jobs[t] = (range_job){fn, ctx, lo, hi};
        joined[t] = pthread_create(&th[t], NULL, range_thread, &jobs[t]) == 0;
        if (!joined[t]) fn(ctx, lo, hi); /* no thread: do the range here */
        nt = t + 1;
    }
    for (int t = 0; t < nt; ++t)
        if (joined[t]) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------- flat normal arrays */

typedef struct { uint64_t key; uint64_t start; double scale; uint16_t* out16; float* out32; } flat_ctx;

static void flat_bf16_range(void* p, int64_t lo, int64_t hi) {
    flat_ctx* c = (flat_ctx*)p;
    for (int64_t i = lo; i < hi; ++i)
        c->out16[i] = f32_to_bf16_rne((float)(c->scale * synth_normal(c->key, c->start + (uint64_t)i)));
}

static void flat_f32_range(void* p, int64_t lo, int64_t hi) {
    flat_ctx* c = (flat_ctx*)p;
    for (int64_t i = lo; i < hi; ++i)
        c->out32[i] = (float)(c->scale * synth_normal(c->key, c->start + (uint64_t)i));
}

/* out[i] = bf16(scale * normal(key, start + i)), i < n */
void synth_normal_bf16(uint64_t key, uint64_t start, int64_t n, double scale, uint16_t* out, int nthreads) {
    flat_ctx c = {key, start, scale, out, NULL};
    parallel_for(flat_bf16_range, &c, n, nthreads);
}

/* out[i] = (float)(scale * normal(key, start + i)), i < n */
void synth_normal_f32(uint64_t key, uint64_t start, int64_t n, double scale, float* out, int nthreads) {
    flat_ctx c = {key, start, scale, NULL, out};
    parallel_for(flat_f32_range, &c, n, nthreads);
}

/* ------------------------------------------------------------ K / V tensors */

/*
 * One (sequence, tensor) of the cache.  The element (h, pos, d) takes the
 * counter (h * 2^21 + pos) * D + d of stream `key`:
 *     z = normal(key, counter)
 *     if key_jitter != 0:  z *= 0.5 + 1.5 * unit(u64(key_jitter, h * 2^21 + pos))
 *     if bias_mask && bias_mask[h * nb + pos / 4]:  z += bias_mag * bias_dir[h * D + d]
 *     value = bf16(z)
 * and is written to logical[(h * L + pos) * D + d] (if logical != NULL) and to
 * paged[((block_table[pos / page_size] * Hkv + h) * page_size + pos % page_size) * D + d]
 * (if paged != NULL).
 */
typedef struct {
    uint64_t key, key_jitter;
    const float* bias_dir;
    const uint8_t* bias_mask;
    double bias_mag;
    int32_t Hkv, D, page_size;
    int64_t L, nb;
    const int32_t* block_table;
    uint16_t* logical;
    uint16_t* paged;
} kv_ctx;

static void kv_range(void* p, int64_t lo, int64_t hi) {
    kv_ctx* c = (kv_ctx*)p;
    const int D = c->D;
    for (int64_t row = lo; row < hi; ++row) { /* row = h * L + pos */
        int64_t h = row / c->L, pos = row % c->L;
        uint64_t tok = ((uint64_t)h << 21) + (uint64_t)pos;
        double jit = 1.0;
        if (c->key_jitter) jit = 0.5 + 1.5 * synth_uniform(c->key_jitter, tok);
        int biased = c->bias_mask && c->bias_mask[h * c->nb + pos / 4];
        uint16_t* dl = c->logical ? c->logical + (size_t)row * D : NULL;
        uint16_t* dp = NULL;
        if (c->paged) {
            int64_t page = c->block_table[pos / c->page_size];
            dp = c->paged + ((size_t)(page * c->Hkv + h) * c->page_size + (size_t)(pos % c->page_size)) * D;
        }
        for (int d = 0; d < D; ++d) {
            double z = synth_normal(c->key, tok * (uint64_t)D + (uint64_t)d) * jit;
            if (biased) z += c->bias_mag * (double)c->bias_dir[h * D + d];
            uint16_t v = f32_to_bf16_rne((float)z);
            if (dl) dl[d] = v;
            if (dp) dp[d] = v;
        }
    }
}

int synth_kv(uint64_t key, uint64_t key_jitter, const float* bias_dir, const uint8_t* bias_mask, double bias_mag,
             int32_t Hkv, int64_t L, int32_t D, int32_t page_size, const int32_t* block_table, uint16_t* logical,
             uint16_t* paged, int nthreads) {
    if (L < 0 || L >= (1LL << 21) || Hkv <= 0 || D <= 0) return -1;
    if (paged && (page_size <= 0 || !block_table)) return -1;
    kv_ctx c = {key, key_jitter, bias_dir, bias_mask, bias_mag, Hkv, D, page_size, L, (L + 3) / 4,
                block_table, logical, paged};
    parallel_for(kv_range, &c, (int64_t)Hkv * L, nthreads);
    return 0;
}

/* ----------------------------------------------------- integer recipe steps */

/* Fisher-Yates: out becomes a permutation of 0..n-1; step i (from n-1 down to 1)
 * swaps out[i] with out[u64(key, n-1-i) mod (i+1)]. */
void synth_permutation(uint64_t key, int64_t n, int32_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = (int32_t)i;
    for (int64_t i = n - 1; i >= 1; --i) {
        int64_t j = (int64_t)(synth_u64(key, (uint64_t)(n - 1 - i)) % (uint64_t)(i + 1));
        int32_t t = out[i];
        out[i] = out[j];
        out[j] = t;
    }
}

/* k distinct values of 0..n-1 (the last k slots of a partial Fisher-Yates),
 * returned in increasing order.  scratch must hold n int32. */
void synth_choose(uint64_t key, int64_t n, int64_t k, int32_t* scratch, int32_t* out) {
    for (int64_t i = 0; i < n; ++i) scratch[i] = (int32_t)i;
    for (int64_t s = 0; s < k; ++s) {
        int64_t i = n - 1 - s;
        int64_t j = (int64_t)(synth_u64(key, (uint64_t)s) % (uint64_t)(i + 1));
        int32_t t = scratch[i];
        scratch[i] = scratch[j];
        scratch[j] = t;
    }
    /* mark-and-scan keeps the result sorted */
    uint8_t* mark = (uint8_t*)calloc((size_t)n, 1);
    for (int64_t s = 0; s < k; ++s) mark[scratch[n - 1 - s]] = 1;
    int64_t w = 0;
    for (int64_t i = 0; i < n; ++i)
        if (mark[i]) out[w++] = (int32_t)i;
    free(mark);
}

/* lo + u64(key, i) mod (hi - lo + 1) */
int64_t synth_uniform_int(uint64_t key, uint64_t i, int64_t lo, int64_t hi) {
    return lo + (int64_t)(synth_u64(key, i) % (uint64_t)(hi - lo + 1));
}
