/* A plain C99 caller of the detfold C ABI: argument checks and host-only
 * planning, no device work (it runs without a GPU).  Prints one line per
 * check; the pytest wrapper compares them. */
#include <stdint.h>
#include <stdio.h>

#include "detfold.h"

int main(void)
{
    const uintptr_t base = (uintptr_t)0x7F0000000000ull;
    float *out = (float *)base;
    const float *stacked = (const float *)(base + (1u << 30));
    int64_t start[3], length[3];
    detfold_plan plan;
    detfold_launch launch = {DETFOLD_PATH_ROWS, 0, 0, 0, DETFOLD_POLICY_DEFAULT, 0};

    printf("abi %d\n", detfold_abi_version());
    printf("w0 %d\n", fold_ranks(out, stacked, 0, 16, NULL));
    printf("overlap %d\n", fold_ranks((float *)stacked, stacked, 2, 16, NULL));
    printf("timed_w0 %d\n", detfold_fold_ranks_timed(out, stacked, 0, 16, 0, 1.0f, NULL, NULL, NULL, NULL));
    printf("timed_overlap %d\n",
           detfold_fold_ranks_timed((float *)stacked, stacked, 2, 16, 1, 0.5f, NULL, NULL, NULL, NULL));
    printf("timed_empty %d\n", detfold_fold_ranks_timed(out, stacked, 4, 0, 0, 1.0f, NULL, NULL, NULL, NULL));
    printf("empty %d\n", fold_into(NULL, NULL, 0, NULL));
    printf("strerror %s\n", detfold_strerror(DETFOLD_EOVERLAP));
    int rc = detfold_shard_plan(10, 3, start, length);
    printf("shards %d %lld %lld %lld\n", rc, (long long)length[0], (long long)length[1],
           (long long)length[2]);
    rc = detfold_plan_fold_ranks(base, base + (1u << 30), 8, (int64_t)1 << 24, 256, &launch, &plan);
    printf("plan %d %d %d %lld %lld\n", rc, plan.path, plan.block, (long long)plan.grid,
           (long long)plan.tile);

    /* the two-rank links from C: struct layout and the checks made before any HIP call */
    detfold_one_shot_link shot = {0};
    shot.capacity = 1024;
    shot.stage[0] = (float *)(base + (2u << 20));
    shot.stage[1] = (float *)(base + (3u << 20));
    printf("shot_noflags %d\n", detfold_one_shot_all_reduce(&shot, out, out + 4096, 16));
    shot.flags = (uint32_t *)(base + (4u << 20));
    shot.words = (int32_t *)(base + (5u << 20));
    printf("shot_capacity %d\n", detfold_one_shot_all_reduce(&shot, out, out + 4096, 1025));
    printf("shot_rank %d\n", detfold_one_shot_rank(&shot, 2, out, 16, NULL));
    printf("shot_empty %d\n", detfold_one_shot_all_reduce(&shot, out, out + 4096, 0));
    printf("shot_words %d %d %d\n", DETFOLD_ONE_SHOT_FLAG_WORDS, DETFOLD_BARRIER_ENTRY_EXPIRED,
           DETFOLD_BARRIER_EXIT_EXPIRED);
    detfold_pair_link pair = {{NULL, NULL}, {NULL, NULL}, 0, {NULL, NULL}, {NULL, NULL}};
    printf("bcast_noevents %d\n", detfold_pair_broadcast(&pair, 0, stacked, out, 16));
    printf("gather_noevents %d\n", detfold_pair_all_gather(&pair, stacked, stacked, out, out + 64, 16));
    return 0;
}
