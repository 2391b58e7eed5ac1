/*
 * CPU oracle for the fixed-order fold.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file; only the tests, the smoke check and the bench's CPU-baseline leg
 * do.  It shares no code, header or constant with the HIP library.
 *
 * What it computes is the plain definition of the method, written out as a
 * serial loop (mamba-rs src/dist/reducer.rs: the module note on the FixedOrder
 * contract, the `det_sum_ranks` kernel source and the host function
 * `reduce_sum_reference`):
 *
 *   for every element i, with W >= 1 addend slots s_0 .. s_{W-1}:
 *     acc = s_0[i]                       (the first addend itself, not 0 + s_0[i])
 *     acc = acc + s_r[i]  for r = 1, 2, .., W-1, strictly ascending
 *     out[i] = acc
 *
 * Every "+" is one IEEE 754 binary32 addition, round-to-nearest-even, with
 * subnormals kept.  The scaled variant multiplies the finished sum once by the
 * caller's inverse world size (the module note: the kernel produces the sum,
 * the mean scale is a separate multiply by 1/W that is exact for power-of-two
 * worlds).  The in-place variant is the two-addend case dst = dst + stage
 * (memra-engine tests/tp_ar_gpu.rs, the C-ABI fold `memra_tp_ar_fold`).
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math (x86-64, SSE arithmetic, so
 * every float operation is a single binary32 rounding).  At entry each call
 * makes sure the calling thread's SSE control word asks for round-to-nearest
 * with neither flush-to-zero nor denormals-are-zero, and restores the caller's
 * word on return, so a library that changed that word cannot change the
 * oracle's bits.
 */
#include <stdint.h>
#include <xmmintrin.h>

#define MXCSR_DAZ (1u << 6)
#define MXCSR_RC_MASK (3u << 13)
#define MXCSR_FTZ (1u << 15)

static unsigned int ieee_mode_enter(void)
{
    unsigned int saved = _mm_getcsr();
    _mm_setcsr(saved & ~(MXCSR_DAZ | MXCSR_FTZ | MXCSR_RC_MASK));
    return saved;
}

static void ieee_mode_leave(unsigned int saved)
{
    _mm_setcsr(saved);
}

/* Returns 0 on success, -1 when W < 1 or len < 0 (the host reference asserts
 * a non-empty world). */
int oracle_fold_slots(float *out, const float *const *slots, int32_t W, int64_t len)
{
    if (W < 1 || len < 0)
        return -1;
    unsigned int saved = ieee_mode_enter();
    for (int64_t i = 0; i < len; ++i) {
        float acc = slots[0][i];
        for (int32_t r = 1; r < W; ++r)
            acc = acc + slots[r][i];
        out[i] = acc;
    }
    ieee_mode_leave(saved);
    return 0;
}

/* Stacked arena: slot r is the row stacked[r * len .. r * len + len). */
int oracle_fold_stacked(float *out, const float *stacked, int32_t W, int64_t len)
{
    if (W < 1 || len < 0)
        return -1;
    unsigned int saved = ieee_mode_enter();
    for (int64_t i = 0; i < len; ++i) {
        float acc = stacked[i];
        for (int32_t r = 1; r < W; ++r)
            acc = acc + stacked[(int64_t)r * len + i];
        out[i] = acc;
    }
    ieee_mode_leave(saved);
    return 0;
}

/* The stacked fold followed by one binary32 multiply of the finished sum. */
int oracle_fold_stacked_scaled(float *out, const float *stacked, int32_t W, int64_t len,
                               float inv_w)
{
    if (W < 1 || len < 0)
        return -1;
    unsigned int saved = ieee_mode_enter();
    for (int64_t i = 0; i < len; ++i) {
        float acc = stacked[i];
        for (int32_t r = 1; r < W; ++r)
            acc = acc + stacked[(int64_t)r * len + i];
        out[i] = acc * inv_w;
    }
    ieee_mode_leave(saved);
    return 0;
}

/* In place: dst[i] = dst[i] + stage[i]. */
int oracle_fold_into(float *dst, const float *stage, int64_t n)
{
    if (n < 0)
        return -1;
    unsigned int saved = ieee_mode_enter();
    for (int64_t i = 0; i < n; ++i)
        dst[i] = dst[i] + stage[i];
    ieee_mode_leave(saved);
    return 0;
}
