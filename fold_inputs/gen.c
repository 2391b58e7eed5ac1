/*
 * Seeded synthetic inputs for the fixed-order fold.
 *
 * This module produces input values only; it contains no part of the fold's
 * arithmetic.  Both the CPU oracle's tests and the GPU path's tests and bench
 * draw their addends from here, so both sides see the same bits.
 *
 * Every family starts from the same 64-bit xorshift stream
 * (memra-engine tests/tp_ar_gpu.rs, helper `vecf`; memra-engine
 * tests/gdn_packed_gpu.rs, helper `varied`): the state is seeded as
 * seed * 0x9E3779B97F4A7C15 with the low bit forced on, and every element takes
 * one step of x ^= x<<13; x ^= x>>7; x ^= x<<17 before it is drawn.
 *
 *   vecf   top 24 bits of the state, centred and scaled: (k - 2^23) / 2^23 for
 *          k = state >> 40.  Every value is an exact multiple of 2^-23 in
 *          [-1, 1), so the conversion involves no rounding at all.
 *   varied top 53 bits of the state mapped to [-1, 1) in binary64, rounded to
 *          binary32, then multiplied by `spread` in binary32 (full mantissa).
 *   mixed  sign random, binary exponent uniform over [-20, 20], mantissa
 *          uniform: integer bit assembly only, no float arithmetic.
 *
 * Multi-slot fills give slot r the seed `seed0 + r` and run one thread per
 * slot; each slot is still one sequential stream, so threading does not change
 * any value.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared -pthread (no fast-math).
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static inline uint64_t stream_seed(uint64_t seed)
{
    return (seed * 0x9E3779B97F4A7C15ULL) | 1ULL;
}

static inline uint64_t stream_step(uint64_t x)
{
    x ^= x << 13;
    x ^= x >> 7;
    x ^= x << 17;
    return x;
}

void gen_vecf(float *out, int64_t n, uint64_t seed)
{
    uint64_t x = stream_seed(seed);
    for (int64_t i = 0; i < n; ++i) {
        x = stream_step(x);
        int32_t k = (int32_t)(x >> 40) - 0x800000; /* in [-2^23, 2^23) */
        out[i] = (float)k * 0x1p-23f;              /* exact: |k| <= 2^23 */
    }
}

void gen_varied(float *out, int64_t n, uint64_t seed, float spread)
{
    uint64_t x = stream_seed(seed);
    for (int64_t i = 0; i < n; ++i) {
        x = stream_step(x);
        double u = (double)(x >> 11) * 0x1p-53; /* exact, in [0, 1) */
        float v = (float)(u * 2.0 - 1.0);       /* the only rounding: to binary32 */
        out[i] = v * spread;
    }
}

void gen_mixed(float *out, int64_t n, uint64_t seed)
{
    uint64_t x = stream_seed(seed);
    for (int64_t i = 0; i < n; ++i) {
        x = stream_step(x);
        uint32_t sign = (uint32_t)(x >> 63);
        uint32_t mant = (uint32_t)(x >> 40) & 0x7FFFFFu;
        /* Lemire's multiply-shift maps the low 32 bits onto 0..40 */
        int32_t e = (int32_t)(((x & 0xFFFFFFFFULL) * 41ULL) >> 32) - 20;
        uint32_t bits = (sign << 31) | ((uint32_t)(e + 127) << 23) | mant;
        memcpy(&out[i], &bits, sizeof bits);
    }
}

enum { FAM_VECF = 0, FAM_VARIED = 1, FAM_MIXED = 2 };

struct slot_job {
    int family;
    float *dst;
    int64_t len;
    uint64_t seed;
    float spread;
};

static void *slot_worker(void *arg)
{
    struct slot_job *j = (struct slot_job *)arg;
    switch (j->family) {
    case FAM_VECF: gen_vecf(j->dst, j->len, j->seed); break;
    case FAM_VARIED: gen_varied(j->dst, j->len, j->seed, j->spread); break;
    default: gen_mixed(j->dst, j->len, j->seed); break;
    }
    return NULL;
}

/*
 * Fill W slots of `len` values; slot r starts at out + r * slot_stride and is
 * drawn with seed seed0 + r.  Returns 0, or -1 on bad arguments.
 */
int gen_slots(int family, float *out, int32_t W, int64_t len, int64_t slot_stride,
              uint64_t seed0, float spread, int32_t max_threads)
{
    if (W < 0 || len < 0 || slot_stride < len || (W > 0 && len > 0 && !out))
        return -1;
    if (W == 0 || len == 0)
        return 0;
    struct slot_job *jobs = (struct slot_job *)calloc((size_t)W, sizeof *jobs);
    pthread_t *tid = (pthread_t *)calloc((size_t)W, sizeof *tid);
    if (!jobs || !tid) {
        free(jobs);
        free(tid);
        return -1;
    }
    for (int32_t r = 0; r < W; ++r) {
        jobs[r].family = family;
        jobs[r].dst = out + (int64_t)r * slot_stride;
        jobs[r].len = len;
        jobs[r].seed = seed0 + (uint64_t)r;
        jobs[r].spread = spread;
    }
    if (max_threads < 1)
        max_threads = 1;
    /* run in waves of at most max_threads threads */
    for (int32_t base = 0; base < W; base += max_threads) {
        int32_t end = base + max_threads < W ? base + max_threads : W;
        int32_t started = base;
        for (int32_t r = base; r < end; ++r) {
            if (pthread_create(&tid[r], NULL, slot_worker, &jobs[r]) != 0)
                break;
            started = r + 1;
        }
        for (int32_t r = started; r < end; ++r)
            slot_worker(&jobs[r]); /* thread creation failed: do it inline */
        for (int32_t r = base; r < started; ++r)
            pthread_join(tid[r], NULL);
    }
    free(jobs);
    free(tid);
    return 0;
}
