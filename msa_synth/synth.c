/*
 * Seeded synthetic inputs for MiniMax Sparse Attention workloads.
 *
 * This module produces input bytes only. It holds no part of the attention
 * method: no dot products, no pooling, no selection, no softmax. Both the
 * kernel library's tests/benchmark and the CPU oracle read the buffers it
 * fills, so the two sides always see identical inputs.
 *
 * Generator: every element i of a tensor is a pure function of (seed, i).
 * The counter is mixed with SplitMix64 (G. Steele, D. Lea, C. Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014; the
 * finaliser constants are S. Vigna's public-domain splitmix64.c), so any
 * element can be regenerated alone and the fill can run on many threads.
 *
 * Distributions:
 *   - normal: Box-Muller (G. Box, M. Muller, 1958), cosine branch only,
 *     computed in double, rounded double -> float -> bfloat16 (round to
 *     nearest, ties to even);
 *   - uniform integers in [lo, hi]: lo + floor((hi-lo+1) * u), u in [0,1)
 *     with 53 random bits; stored exactly as bfloat16 or as OCP FP8 E4M3FN.
 */
#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>

static inline uint64_t splitmix64_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* The k-th output of a SplitMix64 stream whose state starts at `seed`. */
static inline uint64_t stream_word(uint64_t seed, uint64_t k) {
    return splitmix64_mix(seed + (k + 1) * 0x9E3779B97F4A7C15ULL);
}

/* u in [0, 1) with 53 random bits. */
static inline double unit_double(uint64_t w) { return (double)(w >> 11) * 0x1.0p-53; }

static inline uint16_t float_to_bf16_rne(float f) {
    union { float f; uint32_t u; } v = { f };
    uint32_t u = v.u;
    if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/* Exact E4M3FN code of an integer with |v| <= 16 (every such integer is representable). */
static uint8_t int_to_e4m3(int v) {
    uint8_t sign = v < 0 ? 0x80 : 0x00;
    int a = v < 0 ? -v : v;
    if (a == 0) return sign;
    int e = 0;
    while ((a >> (e + 1)) != 0) e++;          /* a in [2^e, 2^(e+1)) */
    int mant = ((a << 3) >> e) & 7;            /* 3 fraction bits, exact for a <= 16 */
    return (uint8_t)(sign | ((e + 7) << 3) | mant);
}

static inline int uniform_int(uint64_t w, int lo, int hi) {
    double u = unit_double(w);
    return lo + (int)floor((double)(hi - lo + 1) * u);
}

enum { K_NORMAL_BF16 = 0, K_INT_BF16 = 1, K_INT_E4M3 = 2 };

typedef struct {
    int kind;
    void *out;
    size_t begin, end;
    uint64_t seed, offset;
    int lo, hi;
} fill_job;

static void fill_range(const fill_job *j) {
    for (size_t i = j->begin; i < j->end; ++i) {
        uint64_t k = j->offset + i;
        if (j->kind == K_NORMAL_BF16) {
            double u1 = 1.0 - unit_double(stream_word(j->seed, 2 * k));   /* (0, 1] */
            double u2 = unit_double(stream_word(j->seed, 2 * k + 1));
            double z = sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
            ((uint16_t *)j->out)[i] = float_to_bf16_rne((float)z);
        } else {
            int v = uniform_int(stream_word(j->seed, k), j->lo, j->hi);
            if (j->kind == K_INT_BF16)
                ((uint16_t *)j->out)[i] = float_to_bf16_rne((float)v);
            else
                ((uint8_t *)j->out)[i] = int_to_e4m3(v);
        }
    }
}

static void *fill_thread(void *arg) {
    fill_range((const fill_job *)arg);
    return NULL;
}

static int fill(int kind, void *out, size_t n, uint64_t seed, uint64_t offset, int lo, int hi,
                int nthreads) {
    if (kind != K_NORMAL_BF16 && (lo > hi || lo < -16 || hi > 16)) return -1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (n < (size_t)1 << 16) nthreads = 1;
    pthread_t tid[256];
    fill_job job[256];
    size_t chunk = (n + (size_t)nthreads - 1) / (size_t)nthreads;
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        size_t b = (size_t)t * chunk, e = b + chunk;
        if (b >= n) break;
        if (e > n) e = n;
        job[t] = (fill_job){ kind, out, b, e, seed, offset, lo, hi };
        if (nthreads == 1) {
            fill_range(&job[t]);
        } else if (pthread_create(&tid[t], NULL, fill_thread, &job[t]) != 0) {
            fill_range(&job[t]);
            tid[t] = 0;
            started++;
            continue;
        }
        started++;
    }
    if (nthreads > 1)
        for (int t = 0; t < started; ++t)
            if (tid[t]) pthread_join(tid[t], NULL);
    return 0;
}

/* N(0,1) samples rounded to bfloat16; element i uses counter offset + i. */
int synth_normal_bf16(uint16_t *out, size_t n, uint64_t seed, uint64_t offset, int nthreads) {
    return fill(K_NORMAL_BF16, out, n, seed, offset, 0, 0, nthreads);
}

/* Uniform integers in [lo, hi] (|lo|, |hi| <= 16) stored exactly as bfloat16. */
int synth_int_bf16(uint16_t *out, size_t n, uint64_t seed, uint64_t offset, int lo, int hi,
                   int nthreads) {
    return fill(K_INT_BF16, out, n, seed, offset, lo, hi, nthreads);
}

/* Uniform integers in [lo, hi] (|lo|, |hi| <= 16) stored exactly as OCP FP8 E4M3FN. */
int synth_int_e4m3(uint8_t *out, size_t n, uint64_t seed, uint64_t offset, int lo, int hi,
                   int nthreads) {
    return fill(K_INT_E4M3, out, n, seed, offset, lo, hi, nthreads);
}

/* Derives a per-tensor seed from a workload seed and a small tensor id. */
uint64_t synth_stream_seed(uint64_t base, uint64_t tensor_id) {
    return splitmix64_mix(base ^ splitmix64_mix(tensor_id + 0x632BE59BD9B4E019ULL));
}
