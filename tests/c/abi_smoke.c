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
    detfold_launch launch = {DETFOLD_PATH_ROWS, 0, 0, 0, DETFOLD_POLICY_DEFAULT};

    printf("abi %d\n", detfold_abi_version());
    printf("w0 %d\n", fold_ranks(out, stacked, 0, 16, NULL));
    printf("overlap %d\n", fold_ranks((float *)stacked, stacked, 2, 16, NULL));
    printf("empty %d\n", fold_into(NULL, NULL, 0, NULL));
    printf("strerror %s\n", detfold_strerror(DETFOLD_EOVERLAP));
    int rc = detfold_shard_plan(10, 3, start, length);
    printf("shards %d %lld %lld %lld\n", rc, (long long)length[0], (long long)length[1],
           (long long)length[2]);
    rc = detfold_plan_fold_ranks(base, base + (1u << 30), 8, (int64_t)1 << 24, 256, &launch, &plan);
    printf("plan %d %d %d %lld %lld\n", rc, plan.path, plan.block, (long long)plan.grid,
           (long long)plan.tile);
    return 0;
}
