/* Host-side stress of the detfold C ABI under AddressSanitizer and
 * UndefinedBehaviorSanitizer: every planning and argument-checking path with
 * extreme widths, lengths, addresses, compute-unit counts and launch
 * overrides.  No call here reaches the device: the planning functions are
 * host only, and the fold entry points are given arguments that their checks
 * reject.  Every accepted plan is checked for the invariants the kernels rely
 * on; the program prints a summary line and exits nonzero on a violation. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "detfold.h"

static long violations = 0;

static void fail(const char *what, int64_t w, int64_t len)
{
    if (violations < 20)
        printf("violation: %s (W=%lld len=%lld)\n", what, (long long)w, (long long)len);
    ++violations;
}

/* What a kernel launch needs from a plan. */
static void check_plan(const detfold_plan *p, int32_t W, int64_t len, int coaligned, int32_t forced_block,
                       int32_t forced_group)
{
    if (p->group < 1 || p->group > 64)
        fail("XCD group out of range", W, len);
    if (len == 0) {
        if (p->grid != 0)
            fail("empty fold with a grid", W, len);
        return;
    }
    if (p->grid < 1 || p->grid > 0x7FFFFFFF)
        fail("grid out of range", W, len);
    if (p->block < 64 || p->block > 1024 || p->block % 64)
        fail("block out of range", W, len);
    if (p->tile < 1)
        fail("empty tile", W, len);
    if (p->path == DETFOLD_PATH_SCALAR) {
        if (p->body != len || p->head || p->tail)
            fail("scalar body does not cover len", W, len);
    } else {
        if (p->head < 0 || p->head > 3 || p->tail < 0 || p->tail > 3)
            fail("head or tail out of range", W, len);
        if ((int64_t)p->head + 4 * p->body + p->tail != len)
            fail("head + body + tail != len", W, len);
    }
    if (p->path == DETFOLD_PATH_ROWS && forced_block) {
        /* an override names the shape: the plan keeps it, with that shape's tile */
        const int64_t tile = W > 16 ? (forced_block == 1024 ? 256 : 64)
                                    : forced_block == 64 * W ? 64 * (W <= 2 ? 8 : (W + 3) / 4) : 64;
        if (p->block != forced_block || p->tile != tile)
            fail("row body override not kept", W, len);
        return;
    }
    /* slots per wave: eight slots one where len is a multiple of 2^24 or the
     * slots do not repeat the low 16 MiB of address, else two; seven and nine
     * to sixteen two; five and six two only co-aligned and repeating.  XCD
     * group: shifted slots runs of 32 (8 at three and four slots that do not
     * repeat; beyond sixteen slots 16 where they do not repeat); co-aligned
     * plain round-robin when repeating, else 32 from five to ten slots and 8 */
    const int repeat = len % ((int64_t)1 << 22) == 0;
    const int spw = (W < 5 || W > 16) ? 1
                    : W == 8 ? ((len % ((int64_t)1 << 24) == 0 || !repeat) ? 1 : 2)
                    : (W == 7 || W >= 9) ? 2
                    : (coaligned && repeat) ? 2 : 1;
    const int group = (W < 3 || W > 16) ? 1
                      : !coaligned ? (W <= 4 && !repeat ? 8 : 32)
                      : repeat ? 1 : (W >= 5 && W <= 10 ? 32 : 8);
    if (p->path == DETFOLD_PATH_ROWS && W <= 16 && p->group != (forced_group ? forced_group : group))
        fail("row body with the wrong XCD group", W, len);
    /* two slots per wave: ceil(W/2) waves, eight at thirteen and fourteen slots */
    const int waves = W > 16 ? 0 : (spw == 2 && (W == 13 || W == 14)) ? 8 : (W + spw - 1) / spw;
    if (p->path == DETFOLD_PATH_ROWS && W > 16 && p->group != (forced_group ? forced_group
                                                              : coaligned ? 1 : repeat ? 32 : 16))
        fail("wide row body with the wrong XCD group", W, len);
    const int wide8 = coaligned || (repeat && (W % 16 == 0 || W % 16 >= 8));
    if (p->path == DETFOLD_PATH_ROWS && p->block != (W <= 16 ? 64 * waves : wide8 ? 512 : 1024))
        fail("row body with the wrong workgroup size", W, len);
    if (p->path == DETFOLD_PATH_ROWS && W <= 16 && spw == 2 && p->tile != 64)
        fail("two-slot row body with the wrong tile", W, len);
    if (p->path == DETFOLD_PATH_ROWS && W == 8 && p->tile != (spw == 2 ? 64 : 128))
        fail("eight-slot row body with the wrong tile", W, len);
    if (p->path == DETFOLD_PATH_ROWS && W == 16 && p->tile != (spw == 2 ? 64 : 256))
        fail("sixteen-slot row body with the wrong tile", W, len);
    if (p->path == DETFOLD_PATH_ROWS && W < 2)
        fail("row body for one slot", W, len);
}

int main(void)
{
    static const int32_t widths[] = {-5, -1, 0, 1, 2, 3, 4, 7, 8, 9, 15, 16, 17, 31, 32, 33, 64, 100, 1000,
                                     INT32_MAX};
    static const int64_t lens[] = {-1, 0, 1, 2, 3, 4, 5, 7, 1023, 4096, 65537, 10000019, (int64_t)1 << 31,
                                   ((int64_t)1 << 31) + 13, (int64_t)1 << 40, INT64_MAX / 4096,
                                   INT64_MAX / 64, INT64_MAX / 8, INT64_MAX / 4, INT64_MAX - 1, INT64_MAX,
                                   INT64_MIN};
    static const uintptr_t bases[] = {0, 4, 16, 0x7F0000000000ull, 0x7F0000000004ull, 0x7F0000000008ull,
                                      0x7F000000000Cull, 0x7F0000000001ull, 0x7F0000000002ull,
                                      UINTPTR_MAX - 15, UINTPTR_MAX - 3};
    static const int32_t cus[] = {-1, 0, 1, 7, 256, INT32_MAX};
    const detfold_launch overrides[] = {
        {DETFOLD_PATH_AUTO, 0, 0, 0, DETFOLD_POLICY_DEFAULT, 0},
        {DETFOLD_PATH_VECTOR, 256, 7, 2, DETFOLD_POLICY_DEFAULT, 0},
        {DETFOLD_PATH_SCALAR, 1024, 1, 4, DETFOLD_POLICY_STREAM, 0},
        {DETFOLD_PATH_ROWS, 0, 3, 0, DETFOLD_POLICY_DEFAULT, 0},
        {DETFOLD_PATH_ROWS, 1024, 0, 1, DETFOLD_POLICY_DEFAULT, 0},
        {DETFOLD_PATH_ROWS, 512, 0, 0, DETFOLD_POLICY_DEFAULT, 4},
        {DETFOLD_PATH_ROWS, 256, 0, 0, DETFOLD_POLICY_DEFAULT, 8},
        {DETFOLD_PATH_ROWS, 0, 0, 0, DETFOLD_POLICY_DEFAULT, 64},
        {DETFOLD_PATH_ROWS, 0, 0, 0, DETFOLD_POLICY_DEFAULT, 65},
        {DETFOLD_PATH_ROWS, 0, 0, 0, DETFOLD_POLICY_DEFAULT, 12},
        {DETFOLD_PATH_AUTO, 0, 0, 0, DETFOLD_POLICY_DEFAULT, -1},
        {DETFOLD_PATH_AUTO, 0, 0, 0, DETFOLD_POLICY_CACHED, 0},
        {DETFOLD_PATH_AUTO, 64, 0x7FFFFFFF, 1, DETFOLD_POLICY_CACHED, 0},
        {7, 0, 0, 0, 0, 0},
        {DETFOLD_PATH_AUTO, 100, 0, 0, 0, 0},
        {DETFOLD_PATH_AUTO, 0, -1, 0, 0, 0},
        {DETFOLD_PATH_AUTO, 0, 0, 3, 0, 0},
        {DETFOLD_PATH_AUTO, 0, 0, 2, DETFOLD_POLICY_CACHED, 0},
        {DETFOLD_PATH_AUTO, 0, 0, 0, 9, 0},
    };
    const int nb = (int)(sizeof bases / sizeof bases[0]);
    long calls = 0, accepted = 0;
    uint64_t sum = 0;
    detfold_plan plan;

    for (size_t wi = 0; wi < sizeof widths / sizeof widths[0]; ++wi)
        for (size_t li = 0; li < sizeof lens / sizeof lens[0]; ++li)
            for (int oi = 0; oi < nb; ++oi)
                for (int si = 0; si < nb; ++si)
                    for (size_t ci = 0; ci < sizeof cus / sizeof cus[0]; ++ci)
                        for (int ki = -1; ki < (int)(sizeof overrides / sizeof overrides[0]); ++ki) {
                            const int32_t W = widths[wi];
                            const int64_t len = lens[li];
                            /* keep the arena clear of out unless both bases coincide */
                            const uintptr_t out = bases[oi];
                            const uintptr_t st = bases[si] + (bases[si] < (uintptr_t)1 << 62 ? (uintptr_t)1 << 50 : 0);
                            memset(&plan, 0xA5, sizeof plan);
                            const int rc = detfold_plan_fold_ranks(out, st, W, len, cus[ci],
                                                                   ki < 0 ? NULL : &overrides[ki], &plan);
                            ++calls;
                            sum = sum * 31 + (uint64_t)rc;
                            if (rc == DETFOLD_OK) {
                                ++accepted;
                                const int co = ((out >> 2) & 3) == ((st >> 2) & 3) && (out & 3) == 0 &&
                                               (st & 3) == 0 && len % 4 == 0;
                                const int rows_ovr = ki >= 0 && overrides[ki].path == DETFOLD_PATH_ROWS;
                                check_plan(&plan, W, len, co, rows_ovr ? overrides[ki].block : 0,
                                           ki >= 0 ? overrides[ki].group : 0);
                                sum = sum * 31 + (uint64_t)plan.grid + (uint64_t)plan.path;
                            } else if (rc != DETFOLD_EINVAL && rc != DETFOLD_EOVERLAP) {
                                fail("unexpected return code", W, len);
                            }
                        }

    for (size_t li = 0; li < sizeof lens / sizeof lens[0]; ++li)
        for (int oi = 0; oi < nb; ++oi)
            for (int si = 0; si < nb; ++si)
                for (size_t ci = 0; ci < sizeof cus / sizeof cus[0]; ++ci) {
                    memset(&plan, 0xA5, sizeof plan);
                    const int rc = detfold_plan_fold_into(bases[oi], bases[si] + ((uintptr_t)1 << 40),
                                                          lens[li], cus[ci], &plan);
                    ++calls;
                    if (rc == DETFOLD_OK) {
                        ++accepted;
                        check_plan(&plan, 2, lens[li], 0, 0, 0);
                    }
                }

    /* batched folds: every job's workgroups, each job at least one, within int32 */
    static const int64_t jlens[] = {0, 1, 3, 4, 5, 1023, 65537, 10000019, (int64_t)1 << 31,
                                    (int64_t)1 << 40, INT64_MAX / 64, -1};
    const int nj = (int)(sizeof jlens / sizeof jlens[0]);
    detfold_fold_job jobs[DETFOLD_MAX_JOBS + 1];
    for (int32_t W = -1; W <= 18; ++W)
        for (int count = 0; count <= DETFOLD_MAX_JOBS + 1; count += (count < 4 ? 1 : 7))
            for (int rot = 0; rot < nj; ++rot)
                for (int ph = 0; ph < 4; ++ph) {
                    uintptr_t out = 0x7F0000000000ull + 4 * (uintptr_t)ph;
                    uintptr_t arena = (uintptr_t)1 << 56;
                    int64_t total = 0;
                    for (int j = 0; j < count; ++j) {
                        const int64_t n = jlens[(rot + j) % nj];
                        jobs[j].out = (float *)out;
                        jobs[j].stacked = (const float *)arena;
                        jobs[j].len = n;
                        /* packed, padded, below len (rejected) and past any range (rejected) */
                        const int pk = (rot + j + ph) % 4;
                        jobs[j].pitch = pk == 0 ? 0 : pk == 1 ? (n > 0 ? n + 7 : 0)
                                        : pk == 2 ? (n > 1 ? n - 1 : 0) : INT64_MAX / 2;
                        if (n > 0 && n < ((int64_t)1 << 41)) {
                            out += (uintptr_t)n * 4 + 4 * (uintptr_t)ph;
                            arena += ((uintptr_t)n + 8) * 4 * 20 + 64;
                        }
                        total += n > 0 ? n : 0;
                    }
                    memset(&plan, 0xA5, sizeof plan);
                    const int rc = detfold_plan_fold_ranks_batch(jobs, count, W, 256, &plan);
                    ++calls;
                    sum = sum * 31 + (uint64_t)rc;
                    if (rc != DETFOLD_OK)
                        continue;
                    ++accepted;
                    if (plan.group < 1 || plan.group > 64)
                        fail("batch XCD group out of range", W, count);
                    if (total == 0 && plan.grid != 0)
                        fail("empty batch with a grid", W, count);
                    if (total > 0 && (plan.grid < 1 || plan.grid > 0x7FFFFFFF || plan.tile < 1 ||
                                      plan.block < 64 || plan.block > 1024))
                        fail("batch plan out of range", W, count);
                    if (total > 0 && plan.grid * plan.tile < plan.body)
                        fail("batch grid does not cover its groups", W, count);
                }

    /* owner shards: coverage, order and balance for every world and length */
    int64_t start[64], length[64];
    for (int32_t world = -1; world <= 64; ++world)
        for (size_t li = 0; li < sizeof lens / sizeof lens[0]; ++li) {
            const int64_t n = lens[li];
            const int rc = detfold_shard_plan(n, world, start, length);
            ++calls;
            if (rc != DETFOLD_OK)
                continue;
            int64_t s = 0, lo = INT64_MAX, hi = 0;
            for (int32_t p = 0; p < world; ++p) {
                if (start[p] != s || length[p] < 0)
                    fail("shards not contiguous", world, n);
                s += length[p];
                lo = length[p] < lo ? length[p] : lo;
                hi = length[p] > hi ? length[p] : hi;
            }
            if (s != n || hi - lo > 1)
                fail("shards do not cover n evenly", world, n);
        }

    /* the device entry points, each with an argument its checks reject */
    float *const fp = (float *)(uintptr_t)0x7F0000000000ull;
    for (size_t li = 0; li < sizeof lens / sizeof lens[0]; ++li) {
        const int64_t len = lens[li];
        if (fold_ranks(fp, fp + 64, 0, len, NULL) != DETFOLD_EINVAL)
            fail("fold_ranks accepted W = 0", 0, len);
        if (len > 0 && fold_ranks(NULL, fp, 2, len, NULL) != DETFOLD_EINVAL)
            fail("fold_ranks accepted a NULL out", 2, len);
        if (len > 0 && fold_into(fp, (const float *)((uintptr_t)fp + 2), len, NULL) != DETFOLD_EINVAL)
            fail("fold_into accepted a misaligned stage", 2, len);
        if (fold_ranks_scaled(fp, fp, 3, len < 0 ? len : -len - 1, 0.5f, NULL) != DETFOLD_EINVAL)
            fail("fold_ranks_scaled accepted a negative length", 3, len);
        const float *slots[17];
        for (int r = 0; r < 17; ++r)
            slots[r] = fp + 1024 * (r + 1);
        if (fold_slots(fp, slots, 17, len, NULL) != DETFOLD_EINVAL)
            fail("fold_slots accepted 17 slots", 17, len);
        calls += 5;
    }
    detfold_one_shot_link shot;
    memset(&shot, 0, sizeof shot);
    shot.capacity = INT64_MAX;
    shot.flags = (uint32_t *)(uintptr_t)0x7F0000100000ull;
    shot.words = (int32_t *)(uintptr_t)0x7F0000200000ull;
    shot.stage[0] = fp + (1 << 24);
    shot.stage[1] = fp + (2 << 24);
    for (size_t li = 0; li < sizeof lens / sizeof lens[0]; ++li) {
        const int64_t len = lens[li];
        if (len > 0 && detfold_one_shot_all_reduce(&shot, fp, fp, len) != DETFOLD_EOVERLAP &&
            detfold_one_shot_all_reduce(&shot, fp, fp, len) != DETFOLD_EINVAL)
            fail("one-shot accepted x0 == x1", 2, len);
        if (detfold_one_shot_rank(&shot, 2, fp, len, NULL) != DETFOLD_EINVAL)
            fail("one-shot accepted rank 2", 2, len);
        calls += 2;
    }

    printf("calls %ld accepted %ld violations %ld checksum %016llx\n", calls, accepted, violations,
           (unsigned long long)sum);
    return violations ? 1 : 0;
}
