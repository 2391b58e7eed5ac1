/* A C caller of libdetfold with no Python and no torch: device buffers from
 * hipMalloc, streams and events from the HIP runtime, every fold entry point
 * called through include/detfold.h, and each result compared bit for bit with
 * the CPU oracle (oracle/liboracle.so, linked here as test infrastructure).
 *
 * Built by the repository's build step (tests/c/build_driver.py) and run by
 * tests/test_c_gpu.py on a GPU.  Prints "case <name>" before each device step
 * and "ok <name>" after its check; exits 1 at the first mismatch or error.
 * Every buffer is allocated at exactly the size the call reads or writes. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "detfold.h"

#define MAX_SLOTS 16 /* fold_slots and detfold_loopback_round take W <= 16 */

/* the oracle's entry points (oracle/oracle.c) */
int oracle_fold_slots(float *out, const float *const *slots, int32_t W, int64_t len);
int oracle_fold_stacked(float *out, const float *stacked, int32_t W, int64_t len);
int oracle_fold_stacked_scaled(float *out, const float *stacked, int32_t W, int64_t len, float inv_w);
int oracle_fold_into(float *dst, const float *stage, int64_t n);

static hipStream_t g_stream;

#define HIP_OK(call)                                                                       \
    do {                                                                                   \
        hipError_t e_ = (call);                                                            \
        if (e_ != hipSuccess) {                                                            \
            printf("hip error %d (%s) at %s:%d\n", (int)e_, hipGetErrorString(e_), __FILE__, \
                   __LINE__);                                                              \
            exit(1);                                                                       \
        }                                                                                  \
    } while (0)

static void begin(const char *name)
{
    printf("case %s\n", name);
    fflush(stdout);
}

static void expect_rc(const char *what, int got, int want)
{
    if (got != want) {
        printf("FAIL %s: rc %d (%s), want %d\n", what, got, detfold_strerror(got), want);
        exit(1);
    }
}

static void expect_bits(const char *name, const float *got, const float *want, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        uint32_t a, b;
        memcpy(&a, got + i, 4);
        memcpy(&b, want + i, 4);
        if (a != b) {
            printf("FAIL %s: element %lld is %08x, oracle %08x\n", name, (long long)i, a, b);
            exit(1);
        }
    }
    printf("ok %s\n", name);
    fflush(stdout);
}

/* Test inputs only: an xorshift64 stream turned into binary32 values with a
 * random sign, a 24-bit significand and an exponent spread over 2^-12 .. 2^8,
 * so that the order of the additions changes the rounded sums. */
static uint64_t g_state;

static void seed(uint64_t s) { g_state = s * 0x9E3779B97F4A7C15ull + 1; }

static float next_value(void)
{
    g_state ^= g_state << 13;
    g_state ^= g_state >> 7;
    g_state ^= g_state << 17;
    const uint64_t x = g_state;
    const float mag = (float)((x >> 8) & 0xFFFFFF) * 0x1p-24f;  /* [0, 1), exact */
    const float v = ldexpf(mag, (int)(x % 21) - 12);
    return (x >> 63) ? -v : v;
}

static float *host_values(int64_t n, uint64_t s)
{
    float *h = malloc((size_t)(n > 0 ? n : 1) * 4);
    if (!h) {
        printf("host allocation failed\n");
        exit(1);
    }
    seed(s);
    for (int64_t i = 0; i < n; ++i)
        h[i] = next_value();
    return h;
}

static float *dev_alloc(int64_t n)
{
    void *p = NULL;
    HIP_OK(hipMalloc(&p, (size_t)(n > 0 ? n : 1) * 4));
    return (float *)p;
}

static void to_dev(float *d, const float *h, int64_t n) { HIP_OK(hipMemcpy(d, h, (size_t)n * 4, hipMemcpyHostToDevice)); }
static void to_host(float *h, const float *d, int64_t n) { HIP_OK(hipMemcpy(h, d, (size_t)n * 4, hipMemcpyDeviceToHost)); }

/* fold_ranks / fold_ranks_scaled over a stacked arena that starts `off`
 * elements into its allocation (so its 16-byte phase differs from out's). */
static void stacked_case(const char *name, int32_t W, int64_t n, int off, int scaled, float inv_w,
                         uint64_t s)
{
    begin(name);
    const int64_t total = (int64_t)W * n + off;
    float *h = host_values(total, s);
    float *want = malloc((size_t)n * 4 + 4), *got = malloc((size_t)n * 4 + 4);
    float *d = dev_alloc(total), *out = dev_alloc(n);
    to_dev(d, h, total);
    int rc = scaled ? fold_ranks_scaled(out, d + off, W, n, inv_w, g_stream)
                    : fold_ranks(out, d + off, W, n, g_stream);
    expect_rc(name, rc, DETFOLD_OK);
    HIP_OK(hipStreamSynchronize(g_stream));
    to_host(got, out, n);
    if (scaled)
        oracle_fold_stacked_scaled(want, h + off, W, n, inv_w);
    else
        oracle_fold_stacked(want, h + off, W, n);
    expect_bits(name, got, want, n);
    HIP_OK(hipFree(d));
    HIP_OK(hipFree(out));
    free(h);
    free(want);
    free(got);
}

/* fold_into twice: dst = a + b, then dst = dst + dst' where dst' is a copy of
 * the first result, which must be exactly twice it. */
static void into_case(const char *name, int64_t n, uint64_t s)
{
    begin(name);
    float *a = host_values(n, s), *b = host_values(n, s + 1);
    float *got = malloc((size_t)n * 4 + 4);
    float *da = dev_alloc(n), *db = dev_alloc(n);
    to_dev(da, a, n);
    to_dev(db, b, n);
    expect_rc(name, fold_into(da, db, n, g_stream), DETFOLD_OK);
    HIP_OK(hipStreamSynchronize(g_stream));
    to_host(got, da, n);
    oracle_fold_into(a, b, n);
    expect_bits(name, got, a, n);
    HIP_OK(hipMemcpy(db, da, (size_t)n * 4, hipMemcpyDeviceToDevice));
    expect_rc(name, fold_into(da, db, n, g_stream), DETFOLD_OK);
    HIP_OK(hipStreamSynchronize(g_stream));
    to_host(got, da, n);
    for (int64_t i = 0; i < n; ++i)
        a[i] = a[i] * 2.0f; /* exact: no overflow at these magnitudes */
    expect_bits("second fold doubles", got, a, n);
    HIP_OK(hipFree(da));
    HIP_OK(hipFree(db));
    free(a);
    free(b);
    free(got);
}

/* fold_slots over W separate buffers at mixed 16-byte phases. */
static void slots_case(const char *name, int32_t W, int64_t n, uint64_t s)
{
    begin(name);
    float *h[MAX_SLOTS], *d[MAX_SLOTS];
    const float *hs[MAX_SLOTS], *ds[MAX_SLOTS];
    for (int32_t r = 0; r < W; ++r) {
        const int off = r % 4;
        h[r] = host_values(n, s + (uint64_t)r);
        d[r] = dev_alloc(n + off);
        to_dev(d[r] + off, h[r], n);
        hs[r] = h[r];
        ds[r] = d[r] + off;
    }
    float *want = malloc((size_t)n * 4 + 4), *got = malloc((size_t)n * 4 + 4);
    float *out = dev_alloc(n);
    expect_rc(name, fold_slots(out, ds, W, n, g_stream), DETFOLD_OK);
    HIP_OK(hipStreamSynchronize(g_stream));
    to_host(got, out, n);
    oracle_fold_slots(want, hs, W, n);
    expect_bits(name, got, want, n);
    for (int32_t r = 0; r < W; ++r) {
        HIP_OK(hipFree(d[r]));
        free(h[r]);
    }
    HIP_OK(hipFree(out));
    free(want);
    free(got);
}

/* detfold_loopback_round: every arena must end equal to the fold of all. */
static void round_case(const char *name, int32_t W, int64_t n, int32_t flags, uint64_t s)
{
    begin(name);
    float *h[MAX_SLOTS], *d[MAX_SLOTS];
    const float *hs[MAX_SLOTS];
    for (int32_t r = 0; r < W; ++r) {
        h[r] = host_values(n, s + (uint64_t)r);
        d[r] = dev_alloc(n);
        to_dev(d[r], h[r], n);
        hs[r] = h[r];
    }
    const int64_t stage_elems = (int64_t)W * ((n + W - 1) / W);
    float *stage = (flags & (DETFOLD_ROUND_DIRECT | DETFOLD_ROUND_FUSED)) ? NULL : dev_alloc(stage_elems);
    expect_rc(name, detfold_loopback_round(d, W, n, stage, stage ? stage_elems : 0, flags, g_stream),
              DETFOLD_OK);
    HIP_OK(hipStreamSynchronize(g_stream));
    float *want = malloc((size_t)n * 4 + 4), *got = malloc((size_t)n * 4 + 4);
    oracle_fold_slots(want, hs, W, n);
    for (int32_t r = 0; r < W; ++r) {
        to_host(got, d[r], n);
        expect_bits(name, got, want, n);
    }
    for (int32_t r = 0; r < W; ++r) {
        HIP_OK(hipFree(d[r]));
        free(h[r]);
    }
    if (stage)
        HIP_OK(hipFree(stage));
    free(want);
    free(got);
}

/* The two-rank links: x0 and x1 must both end as x0 + x1. */
static void links_case(int64_t n, uint64_t s)
{
    float *a = host_values(n, s), *b = host_values(n, s + 1);
    float *want = malloc((size_t)n * 4 + 4), *got = malloc((size_t)n * 4 + 4);
    memcpy(want, a, (size_t)n * 4);
    oracle_fold_into(want, b, n);
    float *x0 = dev_alloc(n), *x1 = dev_alloc(n);

    begin("pair link all-reduce");
    detfold_pair_link pair;
    memset(&pair, 0, sizeof pair);
    for (int r = 0; r < 2; ++r) {
        hipStream_t st;
        hipEvent_t e0, e1;
        HIP_OK(hipStreamCreate(&st));
        HIP_OK(hipEventCreateWithFlags(&e0, hipEventDisableTiming));
        HIP_OK(hipEventCreateWithFlags(&e1, hipEventDisableTiming));
        pair.stream[r] = st;
        pair.pushed[r] = e0;
        pair.folded[r] = e1;
        pair.stage[r] = dev_alloc(n);
    }
    pair.capacity = n;
    to_dev(x0, a, n);
    to_dev(x1, b, n);
    expect_rc("pair_link_init", detfold_pair_link_init(&pair), DETFOLD_OK);
    expect_rc("pair_all_reduce", detfold_pair_all_reduce(&pair, x0, x1, n), DETFOLD_OK);
    for (int r = 0; r < 2; ++r)
        HIP_OK(hipStreamSynchronize((hipStream_t)pair.stream[r]));
    to_host(got, x0, n);
    expect_bits("pair rank 0", got, want, n);
    to_host(got, x1, n);
    expect_bits("pair rank 1", got, want, n);

    begin("one-shot all-reduce");
    detfold_one_shot_link shot;
    memset(&shot, 0, sizeof shot);
    shot.stream = g_stream;
    shot.stage[0] = dev_alloc(n);
    shot.stage[1] = dev_alloc(n);
    shot.capacity = n;
    void *flags = NULL, *words = NULL;
    HIP_OK(hipMalloc(&flags, DETFOLD_ONE_SHOT_FLAG_WORDS * 4));
    HIP_OK(hipMalloc(&words, 2 * 4));
    shot.flags = (uint32_t *)flags;
    shot.words = (int32_t *)words;
    to_dev(x0, a, n);
    to_dev(x1, b, n);
    expect_rc("one_shot_init", detfold_one_shot_init(&shot), DETFOLD_OK);
    expect_rc("one_shot_all_reduce", detfold_one_shot_all_reduce(&shot, x0, x1, n), DETFOLD_OK);
    HIP_OK(hipStreamSynchronize(g_stream));
    int32_t w[2];
    HIP_OK(hipMemcpy(w, words, 8, hipMemcpyDeviceToHost));
    if (w[0] || w[1]) {
        printf("FAIL one-shot barrier words %d %d\n", w[0], w[1]);
        exit(1);
    }
    to_host(got, x0, n);
    expect_bits("one-shot rank 0", got, want, n);
    to_host(got, x1, n);
    expect_bits("one-shot rank 1", got, want, n);

    for (int r = 0; r < 2; ++r) {
        HIP_OK(hipFree(pair.stage[r]));
        HIP_OK(hipEventDestroy((hipEvent_t)pair.pushed[r]));
        HIP_OK(hipEventDestroy((hipEvent_t)pair.folded[r]));
        HIP_OK(hipStreamDestroy((hipStream_t)pair.stream[r]));
        HIP_OK(hipFree(shot.stage[r]));
    }
    HIP_OK(hipFree(flags));
    HIP_OK(hipFree(words));
    HIP_OK(hipFree(x0));
    HIP_OK(hipFree(x1));
    free(a);
    free(b);
    free(want);
    free(got);
}

int main(void)
{
    int ndev = 0;
    HIP_OK(hipGetDeviceCount(&ndev));
    if (ndev < 1) {
        printf("no HIP device\n");
        return 1;
    }
    HIP_OK(hipSetDevice(0));
    HIP_OK(hipStreamCreate(&g_stream));

    begin("argument errors");
    float *probe = dev_alloc(64);
    expect_rc("W = 0", fold_ranks(probe, probe + 32, 0, 16, g_stream), DETFOLD_EINVAL);
    expect_rc("overlap", fold_ranks(probe, probe + 8, 2, 16, g_stream), DETFOLD_EOVERLAP);
    expect_rc("empty", fold_into(NULL, NULL, 0, g_stream), DETFOLD_OK);
    HIP_OK(hipFree(probe));
    printf("ok argument errors\n");

    stacked_case("fold_ranks W=8 n=100003", 8, 100003, 0, 0, 1.0f, 1);
    stacked_case("fold_ranks W=16 n=10007 at base+1", 16, 10007, 1, 0, 1.0f, 2);
    stacked_case("fold_ranks_scaled W=4 n=65537 inv_w=0.25", 4, 65537, 0, 1, 0.25f, 3);
    stacked_case("fold_ranks W=37 n=4099 at base+2", 37, 4099, 2, 0, 1.0f, 4);
    stacked_case("fold_ranks W=3 n=5 at base+3", 3, 5, 3, 0, 1.0f, 5);
    stacked_case("fold_ranks W=1 n=1000 (a copy)", 1, 1000, 0, 0, 1.0f, 6);
    into_case("fold_into n=4096", 4096, 7);
    into_case("fold_into n=1", 1, 8);
    slots_case("fold_slots W=5 n=1027 mixed phases", 5, 1027, 9);
    round_case("loopback_round W=4 n=1001 direct", 4, 1001, DETFOLD_ROUND_DIRECT, 10);
    round_case("loopback_round W=4 n=1001 staged reversed", 4, 1001, DETFOLD_ROUND_REVERSE_DELIVERY, 11);
    round_case("loopback_round W=8 n=70001 fused", 8, 70001, DETFOLD_ROUND_FUSED, 13);
    links_case(4096, 12);

    HIP_OK(hipStreamDestroy(g_stream));
    printf("all ok\n");
    return 0;
}
