// detfold.hip -- the fixed-order fold for AMD Instinct MI355X (gfx950, CDNA4).
//
// Operation (mamba-rs src/dist/reducer.rs: FixedOrder-contract module note,
// `det_sum_ranks`, `reduce_sum_reference`; memra-engine tests/tp_ar_gpu.rs:
// `memra_tp_ar_fold`): out[i] = (((s_0[i] + s_1[i]) + s_2[i]) + ...) + s_{W-1}[i],
// each "+" one binary32 add, round-to-nearest-even, subnormals kept.
//
// Design for CDNA4:
//  * The fold is pure HBM streaming: (W+1)*4 bytes moved per element against
//    W-1 adds, about 0.2 flop/byte, so memory bandwidth bounds it and matrix
//    cores have nothing to do.  Every choice below is about keeping enough
//    16-byte loads in flight on all 256 compute units.
//  * One thread owns a group of 4 consecutive elements: it issues one 16-byte
//    load per slot (a wave covers 1 KiB of each slot, fully coalesced), then
//    runs four independent add chains, each in ascending slot order, then one
//    16-byte store.  All loads of a thread's pass are issued before the first
//    add, so the adds wait on data, not the reverse.  `unroll` groups per thread
//    per pass multiply the bytes in flight.
//  * When `out` and the slots sit at different offsets modulo 16 bytes no
//    element index lines them all up, so the scalar body gives each lane one
//    4-byte element per slot (a wave still reads 256 contiguous bytes per
//    slot).  Loads are pure data movement: the chain, and so the bits, is the
//    same on either body.
//  * A grid-stride loop lets any grid cover any length; the default grid is
//    sized from the device's compute-unit count.
//  * No atomics, no flags, no waits on other work: a launch completes on its
//    own, whatever else is resident (the latency path of fold_into relies on
//    this).
//  * Compiled with -ffp-contract=off, no fast-math, packed-FP32 instructions
//    disabled, and f32 denormals enabled (the HIP default on gfx9), so every
//    add is a single v_add_f32 under IEEE round-to-nearest-even.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "detfold.h"

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kMaxBlock = 1024;
constexpr int kDefaultBlock = 256;
constexpr int kWorkgroupsPerCU = 8;  // default cap for the grid-stride grid
constexpr int kLatencyBlock = 256;
constexpr int kChunk = 8;            // slots loaded per batch when W is a runtime value

// ---------------------------------------------------------------------------
// Device side

// Fold one tile: U independent positions (U groups of 4 elements, or U single
// elements), each at offset off[u] of `out` and of every slot.  Slot 0 is s0,
// slot r >= 1 is s1 + (r-1)*stride.  WS > 0 is a compile-time slot count; WS
// == 0 reads it from w.
template <int WS, int U, typename T, bool SCALED>
__device__ __forceinline__ void fold_tile(T *out, const T *s0, const T *s1, int64_t stride, int w,
                                          const int64_t (&off)[U], float inv_w)
{
    if constexpr (WS > 0) {
        T v[U][WS];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u][0] = s0[off[u]];
#pragma unroll
        for (int r = 1; r < WS; ++r)
#pragma unroll
            for (int u = 0; u < U; ++u)
                v[u][r] = s1[(int64_t)(r - 1) * stride + off[u]];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            T acc = v[u][0];
#pragma unroll
            for (int r = 1; r < WS; ++r)
                acc = acc + v[u][r];  // ascending slot order, one rounding per add
            if constexpr (SCALED)
                acc = acc * inv_w;  // one rounding of the finished sum
            out[off[u]] = acc;
        }
    } else {
        T acc[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            acc[u] = s0[off[u]];
        for (int r0 = 1; r0 < w; r0 += kChunk) {
            T v[U][kChunk];
#pragma unroll
            for (int k = 0; k < kChunk; ++k)
                if (r0 + k < w)
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        v[u][k] = s1[(int64_t)(r0 + k - 1) * stride + off[u]];
#pragma unroll
            for (int k = 0; k < kChunk; ++k)
                if (r0 + k < w)
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        acc[u] = acc[u] + v[u][k];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            T a = acc[u];
            if constexpr (SCALED)
                a = a * inv_w;
            out[off[u]] = a;
        }
    }
}

// Grid-stride over `n` positions, U per thread per pass; a pass whose last
// position is in range needs no per-position guard.
template <int WS, int U, typename T, bool SCALED>
__device__ __forceinline__ void fold_span(T *out, const T *s0, const T *s1, int64_t stride, int w,
                                          int64_t n, float inv_w)
{
    const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (int64_t base = gid; base < n; base += nthreads * U) {
        if (base + (int64_t)(U - 1) * nthreads < n) {
            int64_t off[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                off[u] = base + (int64_t)u * nthreads;
            fold_tile<WS, U, T, SCALED>(out, s0, s1, stride, w, off, inv_w);
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t one[1] = {base + (int64_t)u * nthreads};
                if (one[0] < n)
                    fold_tile<WS, 1, T, SCALED>(out, s0, s1, stride, w, one, inv_w);
            }
        }
    }
}

// Vector body: elements [head, head + 4*groups) as 16-byte groups; the up to 3
// elements before (head) and after (tail) are folded one by one by the first
// threads of the grid.
template <int WS, int U, bool SCALED>
__global__ __launch_bounds__(kMaxBlock) void k_fold_vector(float *out, const float *s0,
                                                           const float *s1, int64_t stride, int w,
                                                           int64_t len, int64_t head, float inv_w)
{
    const int64_t groups = (len - head) >> 2;
    const int64_t tail0 = head + (groups << 2);
    const int64_t edges = head + (len - tail0);
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid < edges) {
        const int64_t one[1] = {gid < head ? gid : tail0 + (gid - head)};
        fold_tile<WS, 1, float, SCALED>(out, s0, s1, stride, w, one, inv_w);
    }
    fold_span<WS, U, f4, SCALED>(reinterpret_cast<f4 *>(out + head),
                                 reinterpret_cast<const f4 *>(s0 + head),
                                 reinterpret_cast<const f4 *>(s1 + head), stride >> 2, w, groups,
                                 inv_w);
}

// Scalar body: every element with 4-byte loads (slots at mixed 16-byte phases).
template <int WS, int U, bool SCALED>
__global__ __launch_bounds__(kMaxBlock) void k_fold_scalar(float *out, const float *s0,
                                                           const float *s1, int64_t stride, int w,
                                                           int64_t len, float inv_w)
{
    fold_span<WS, U, float, SCALED>(out, s0, s1, stride, w, len, inv_w);
}

// ---------------------------------------------------------------------------
// Host side: planning (pure integer logic, no HIP calls)

struct Geometry {
    uintptr_t out, s0, s1;  // byte addresses
    int64_t stride;         // elements between slots r and r+1 for r >= 1
    int32_t w;
    int64_t len;
};

inline int phase16(uintptr_t a) { return (int)((a >> 2) & 3); }

// Whether out and every slot share one offset modulo 16 bytes.
bool vector_legal(const Geometry &g)
{
    const int p = phase16(g.out);
    if (phase16(g.s0) != p)
        return false;
    if (g.w >= 2 && phase16(g.s1) != p)
        return false;
    if (g.w >= 3 && (g.stride & 3) != 0)
        return false;
    return true;
}

int default_unroll(int path, int32_t w)
{
    if (path == DETFOLD_PATH_VECTOR)
        return w >= 16 || w == 0 ? 1 : 2;
    return 4;
}

int check_override(const detfold_launch *o)
{
    if (!o)
        return DETFOLD_OK;
    if (o->path < DETFOLD_PATH_AUTO || o->path > DETFOLD_PATH_SCALAR)
        return DETFOLD_EINVAL;
    if (o->block != 0 && (o->block < 64 || o->block > kMaxBlock || (o->block % 64) != 0))
        return DETFOLD_EINVAL;
    if (o->grid < 0 || o->grid > 0x7FFFFFFF)
        return DETFOLD_EINVAL;
    if (o->unroll != 0 && o->unroll != 1 && o->unroll != 2 && o->unroll != 4)
        return DETFOLD_EINVAL;
    return DETFOLD_OK;
}

// Path and geometry for one call.  The default grid covers the body in one
// pass when that takes at most cu_count * kWorkgroupsPerCU workgroups, and is
// capped there otherwise (the grid-stride loop does the rest).
int make_plan(const Geometry &g, int32_t cu_count, const detfold_launch *ovr, detfold_plan *p)
{
    if (cu_count < 1)
        return DETFOLD_EINVAL;
    int rc = check_override(ovr);
    if (rc != DETFOLD_OK)
        return rc;
    const detfold_launch o = ovr ? *ovr : detfold_launch{DETFOLD_PATH_AUTO, 0, 0, 0};

    const bool vec_ok = vector_legal(g);
    int path = o.path;
    if (path == DETFOLD_PATH_AUTO)
        path = vec_ok ? DETFOLD_PATH_VECTOR : DETFOLD_PATH_SCALAR;
    if (path == DETFOLD_PATH_VECTOR && !vec_ok)
        return DETFOLD_EINVAL;

    p->path = path;
    p->block = o.block ? o.block : kDefaultBlock;
    p->unroll = o.unroll ? o.unroll : default_unroll(path, g.w <= 16 ? g.w : 0);
    if (path == DETFOLD_PATH_VECTOR) {
        int64_t head = (4 - phase16(g.out)) & 3;
        if (head > g.len)
            head = g.len;
        p->head = (int32_t)head;
        p->body = (g.len - head) >> 2;
        p->tail = (int32_t)((g.len - head) & 3);
    } else {
        p->head = 0;
        p->tail = 0;
        p->body = g.len;
    }
    if (g.len == 0) {
        p->grid = 0;
        return DETFOLD_OK;
    }
    const int64_t per_block = (int64_t)p->block * p->unroll;
    int64_t need = (p->body + per_block - 1) / per_block;
    if (need < 1)
        need = 1;  // a body of zero groups still needs threads for head and tail
    const int64_t cap = (int64_t)cu_count * kWorkgroupsPerCU;
    p->grid = o.grid ? o.grid : (need < cap ? need : cap);
    return DETFOLD_OK;
}

bool ranges_overlap(uintptr_t a, uint64_t a_bytes, uintptr_t b, uint64_t b_bytes)
{
    if (a_bytes == 0 || b_bytes == 0)
        return false;
    return a < b + b_bytes && b < a + a_bytes;
}

int check_ranks_args(const float *out, const float *stacked, int32_t W, int64_t len)
{
    if (W < 1 || len < 0)
        return DETFOLD_EINVAL;
    if (len == 0)
        return DETFOLD_OK;
    if (!out || !stacked)
        return DETFOLD_EINVAL;
    if ((((uintptr_t)out) & 3) || (((uintptr_t)stacked) & 3))
        return DETFOLD_EINVAL;
    if (len > INT64_MAX / 4 / W)
        return DETFOLD_EINVAL;
    if (ranges_overlap((uintptr_t)out, (uint64_t)len * 4, (uintptr_t)stacked,
                       (uint64_t)len * 4 * (uint64_t)W))
        return DETFOLD_EOVERLAP;
    return DETFOLD_OK;
}

int check_into_args(const float *dst, const float *stage, int64_t n)
{
    if (n < 0)
        return DETFOLD_EINVAL;
    if (n == 0)
        return DETFOLD_OK;
    if (!dst || !stage)
        return DETFOLD_EINVAL;
    if ((((uintptr_t)dst) & 3) || (((uintptr_t)stage) & 3))
        return DETFOLD_EINVAL;
    if (n > INT64_MAX / 4)
        return DETFOLD_EINVAL;
    if (ranges_overlap((uintptr_t)dst, (uint64_t)n * 4, (uintptr_t)stage, (uint64_t)n * 4))
        return DETFOLD_EOVERLAP;
    return DETFOLD_OK;
}

Geometry ranks_geometry(uintptr_t out, uintptr_t stacked, int32_t W, int64_t len)
{
    // slot 1 starts one row after slot 0; slot r >= 1 at slot 1 + (r-1)*len
    return Geometry{out, stacked, stacked + (uintptr_t)len * 4, len, W, len};
}

Geometry into_geometry(uintptr_t dst, uintptr_t stage, int64_t n)
{
    return Geometry{dst, dst, stage, 0, 2, n};
}

// ---------------------------------------------------------------------------
// Host side: device query and launch

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

int current_cu_count(int32_t *cu)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return DETFOLD_EDEVICE;
    if (dev < kMaxDevices) {
        int c = g_cu_count[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *cu = c;
            return DETFOLD_OK;
        }
    }
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c < 1)
        return DETFOLD_EDEVICE;
    if (dev < kMaxDevices)
        g_cu_count[dev].store(c, std::memory_order_relaxed);
    *cu = c;
    return DETFOLD_OK;
}

typedef void (*vector_kernel_t)(float *, const float *, const float *, int64_t, int, int64_t,
                                int64_t, float);
typedef void (*scalar_kernel_t)(float *, const float *, const float *, int64_t, int, int64_t,
                                float);

template <int WS, bool SCALED>
vector_kernel_t pick_vector_u(int unroll)
{
    switch (unroll) {
    case 1: return k_fold_vector<WS, 1, SCALED>;
    case 2: return k_fold_vector<WS, 2, SCALED>;
    default: return k_fold_vector<WS, 4, SCALED>;
    }
}

template <int WS, bool SCALED>
scalar_kernel_t pick_scalar_u(int unroll)
{
    switch (unroll) {
    case 1: return k_fold_scalar<WS, 1, SCALED>;
    case 2: return k_fold_scalar<WS, 2, SCALED>;
    default: return k_fold_scalar<WS, 4, SCALED>;
    }
}

// Compile-time slot counts for the common power-of-two worlds; others use the
// runtime-W body, which loads slots in batches of kChunk.
template <bool SCALED>
vector_kernel_t pick_vector(int32_t w, int unroll)
{
    switch (w) {
    case 1: return pick_vector_u<1, SCALED>(unroll);
    case 2: return pick_vector_u<2, SCALED>(unroll);
    case 4: return pick_vector_u<4, SCALED>(unroll);
    case 8: return pick_vector_u<8, SCALED>(unroll);
    case 16: return pick_vector_u<16, SCALED>(unroll);
    default: return pick_vector_u<0, SCALED>(unroll);
    }
}

template <bool SCALED>
scalar_kernel_t pick_scalar(int32_t w, int unroll)
{
    switch (w) {
    case 1: return pick_scalar_u<1, SCALED>(unroll);
    case 2: return pick_scalar_u<2, SCALED>(unroll);
    case 4: return pick_scalar_u<4, SCALED>(unroll);
    case 8: return pick_scalar_u<8, SCALED>(unroll);
    case 16: return pick_scalar_u<16, SCALED>(unroll);
    default: return pick_scalar_u<0, SCALED>(unroll);
    }
}

int launch_plan(const Geometry &g, const detfold_plan &p, bool scaled, float inv_w,
                hipStream_t stream)
{
    float *out = reinterpret_cast<float *>(g.out);
    const float *s0 = reinterpret_cast<const float *>(g.s0);
    const float *s1 = reinterpret_cast<const float *>(g.s1);
    int64_t stride = g.stride;
    int w = g.w;
    int64_t len = g.len;
    int64_t head = p.head;
    const dim3 grid((unsigned)p.grid), block((unsigned)p.block);
    hipError_t e;
    if (p.path == DETFOLD_PATH_VECTOR) {
        vector_kernel_t k = scaled ? pick_vector<true>(w, p.unroll) : pick_vector<false>(w, p.unroll);
        void *args[] = {&out, &s0, &s1, &stride, &w, &len, &head, &inv_w};
        e = hipLaunchKernel(reinterpret_cast<const void *>(k), grid, block, args, 0, stream);
    } else {
        scalar_kernel_t k = scaled ? pick_scalar<true>(w, p.unroll) : pick_scalar<false>(w, p.unroll);
        void *args[] = {&out, &s0, &s1, &stride, &w, &len, &inv_w};
        e = hipLaunchKernel(reinterpret_cast<const void *>(k), grid, block, args, 0, stream);
    }
    return e == hipSuccess ? DETFOLD_OK : DETFOLD_ELAUNCH;
}

int run_ranks(float *out, const float *stacked, int32_t W, int64_t len, bool scaled, float inv_w,
              const detfold_launch *ovr, void *stream)
{
    int rc = check_ranks_args(out, stacked, W, len);
    if (rc == DETFOLD_OK)
        rc = check_override(ovr);
    if (rc != DETFOLD_OK || len == 0)
        return rc;
    const Geometry g = ranks_geometry((uintptr_t)out, (uintptr_t)stacked, W, len);
    if (ovr && ovr->path == DETFOLD_PATH_VECTOR && !vector_legal(g))
        return DETFOLD_EINVAL;  // rejected before the device is touched
    int32_t cu = 0;
    if ((rc = current_cu_count(&cu)) != DETFOLD_OK)
        return rc;
    detfold_plan p;
    if ((rc = make_plan(g, cu, ovr, &p)) != DETFOLD_OK)
        return rc;
    return launch_plan(g, p, scaled, inv_w, static_cast<hipStream_t>(stream));
}

// The decode-join path.  Payloads of 16-256 KiB are launch-latency bound:
// one position per thread, one pass, a grid just large enough for that.  A
// payload too large for one pass of cu_count * kWorkgroupsPerCU workgroups is
// bandwidth bound and takes the default streaming plan instead.
int plan_into(const Geometry &g, int32_t cu_count, detfold_plan *p)
{
    const detfold_launch one_pass = {DETFOLD_PATH_AUTO, kLatencyBlock, 0, 1};
    int rc = make_plan(g, cu_count, &one_pass, p);
    if (rc != DETFOLD_OK || g.len == 0)
        return rc;
    const int64_t blocks = (p->body + kLatencyBlock - 1) / kLatencyBlock;
    if (blocks <= (int64_t)cu_count * kWorkgroupsPerCU)
        return DETFOLD_OK;  // make_plan's grid is already the one-pass grid
    return make_plan(g, cu_count, nullptr, p);
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI

extern "C" {

int fold_ranks(float *out, const float *stacked, int32_t W, int64_t len, void *stream)
{
    return run_ranks(out, stacked, W, len, false, 1.0f, nullptr, stream);
}

int fold_ranks_scaled(float *out, const float *stacked, int32_t W, int64_t len, float inv_w,
                      void *stream)
{
    return run_ranks(out, stacked, W, len, true, inv_w, nullptr, stream);
}

int detfold_fold_ranks_ex(float *out, const float *stacked, int32_t W, int64_t len, int32_t scaled,
                          float inv_w, const detfold_launch *launch, void *stream)
{
    return run_ranks(out, stacked, W, len, scaled != 0, inv_w, launch, stream);
}

int fold_into(float *dst, const float *stage, int64_t n, void *stream)
{
    int rc = check_into_args(dst, stage, n);
    if (rc != DETFOLD_OK || n == 0)
        return rc;
    const Geometry g = into_geometry((uintptr_t)dst, (uintptr_t)stage, n);
    int32_t cu = 0;
    if ((rc = current_cu_count(&cu)) != DETFOLD_OK)
        return rc;
    detfold_plan p;
    if ((rc = plan_into(g, cu, &p)) != DETFOLD_OK)
        return rc;
    return launch_plan(g, p, false, 1.0f, static_cast<hipStream_t>(stream));
}

const char *detfold_strerror(int rc)
{
    switch (rc) {
    case DETFOLD_OK: return "ok";
    case DETFOLD_EINVAL: return "invalid argument (W < 1, negative length, NULL or misaligned "
                                "pointer, size overflow, or bad launch override)";
    case DETFOLD_EOVERLAP: return "output overlaps an input range";
    case DETFOLD_ELAUNCH: return "HIP kernel launch failed";
    case DETFOLD_EDEVICE: return "no usable current HIP device";
    default: return "unknown detfold return code";
    }
}

int detfold_abi_version(void) { return DETFOLD_ABI_VERSION; }

int detfold_shard_plan(int64_t n, int32_t world, int64_t *start, int64_t *length)
{
    if (world < 1 || n < 0 || !start || !length)
        return DETFOLD_EINVAL;
    const int64_t q = n / world, r = n % world;
    int64_t s = 0;
    for (int32_t p = 0; p < world; ++p) {
        const int64_t l = q + (p < r ? 1 : 0);
        start[p] = s;
        length[p] = l;
        s += l;
    }
    return DETFOLD_OK;
}

int detfold_plan_fold_ranks(uintptr_t out, uintptr_t stacked, int32_t W, int64_t len,
                            int32_t cu_count, const detfold_launch *launch, detfold_plan *plan)
{
    if (!plan)
        return DETFOLD_EINVAL;
    int rc = check_ranks_args(reinterpret_cast<const float *>(out),
                              reinterpret_cast<const float *>(stacked), W, len);
    if (rc != DETFOLD_OK)
        return rc;
    return make_plan(ranks_geometry(out, stacked, W, len), cu_count, launch, plan);
}

int detfold_plan_fold_into(uintptr_t dst, uintptr_t stage, int64_t n, int32_t cu_count,
                           detfold_plan *plan)
{
    if (!plan)
        return DETFOLD_EINVAL;
    int rc = check_into_args(reinterpret_cast<const float *>(dst),
                             reinterpret_cast<const float *>(stage), n);
    if (rc != DETFOLD_OK)
        return rc;
    return plan_into(into_geometry(dst, stage, n), cu_count, plan);
}

}  // extern "C"
