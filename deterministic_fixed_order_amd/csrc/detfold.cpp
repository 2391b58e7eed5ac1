// detfold.cpp -- the host side of libdetfold: the device query, the call
// sequences of every entry point (argument checks, plan, launches, stream
// ordering) and the C ABI declared in include/detfold.h.  The kernels and
// their launches live in fold_kernels.hip; the host-only planning and
// argument checks in plan.cpp.
//
// Every entry point checks its arguments before any HIP call, so an argument
// error never touches the device; nothing here allocates or synchronizes,
// except detfold_one_shot_init, which waits for its counters to be zeroed.

#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cstdint>

#include "internal.h"

namespace detfold_impl {
namespace {

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

int run_ranks(float *out, const float *stacked, int32_t W, int64_t len, bool scaled, float inv_w,
              const detfold_launch *ovr, void *stream, void *begin = nullptr, void *done = nullptr)
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
    if ((rc = make_plan(g, cu, ovr, DETFOLD_POLICY_STREAM, &p)) != DETFOLD_OK)
        return rc;
    return launch_plan(g, p, scaled, inv_w, static_cast<hipStream_t>(stream), done, begin);
}

// Launch the fold of separate slots (arguments already checked, len > 0).
int launch_slots(const float *out, const float *const *slots, int32_t W, int64_t len, bool scaled,
                 float inv_w, int32_t cu, hipStream_t stream)
{
    const Geometry g = slots_geometry(out, slots, W, len);
    detfold_plan p;
    int rc = make_plan(g, cu, nullptr, DETFOLD_POLICY_STREAM, &p);
    if (rc != DETFOLD_OK)
        return rc;
    return launch_plan(g, p, scaled, inv_w, stream);
}

int run_slots(float *out, const float *const *slots, int32_t W, int64_t len, bool scaled,
              float inv_w, void *stream)
{
    int rc = check_slots_args(out, slots, W, len);
    if (rc != DETFOLD_OK || len == 0)
        return rc;
    int32_t cu = 0;
    if ((rc = current_cu_count(&cu)) != DETFOLD_OK)
        return rc;
    return launch_slots(out, slots, W, len, scaled, inv_w, cu, static_cast<hipStream_t>(stream));
}

// One fixed-order reduction round over W arenas on one device (mamba-rs
// src/dist/reducer.rs, LoopbackWorld::run_round, with the transport's
// owner-shard dataflow of reduce_sum_fixed_order_nccl):
//   A. every owner p gathers the W copies of its shard, slot = source rank,
//      and folds them in ascending slot order into its own arena's shard;
//   B. every owner's reduced shard is copied to the other W-1 arenas.
// Staged (the transport's shape): the gather copies each source's shard into
// `stage` ([W][l_p], slot = source rank) in ascending or, with
// DETFOLD_ROUND_REVERSE_DELIVERY, descending source order, then fold_ranks
// folds `stage`.  Direct: the owner folds straight from the W arenas
// (fold_slots, in place on its own shard), since on one device every arena is
// already in the same HBM.  Fused: no owner shards at all -- one kernel folds
// every tile from the W arenas and writes the sum back into that tile of each
// (k_fold_rows_all), the shape an owner takes when its peers' buffers are
// mapped.  Bytes move by device-to-device copies only, so the bits are the
// fold's whatever the mode or the delivery order.
int run_round(float *const *arenas, int32_t W, int64_t n, float *stage, int32_t flags,
              hipStream_t stream)
{
    int32_t cu = 0;
    int rc = current_cu_count(&cu);
    if (rc != DETFOLD_OK)
        return rc;
    if (flags & DETFOLD_ROUND_FUSED) {
        const Geometry g = slots_geometry(arenas[0], arenas, W, n);
        detfold_plan p;
        if ((rc = make_plan(g, cu, nullptr, DETFOLD_POLICY_STREAM, &p)) != DETFOLD_OK)
            return rc;
        return launch_rows_all(g, p, stream);
    }
    int64_t start[kMaxRowsW], length[kMaxRowsW];
    balanced_shards(n, W, start, length);
    const bool direct = flags & DETFOLD_ROUND_DIRECT;
    const bool reverse = flags & DETFOLD_ROUND_REVERSE_DELIVERY;
    for (int32_t me = 0; me < W; ++me) {
        const int64_t s = start[me], l = length[me];
        if (l == 0)
            continue;
        if (direct) {
            const float *slots[kMaxRowsW];
            for (int32_t r = 0; r < W; ++r)
                slots[r] = arenas[r] + s;
            rc = launch_slots(arenas[me] + s, slots, W, l, false, 1.0f, cu, stream);
        } else {
            for (int32_t k = 0; k < W && rc == DETFOLD_OK; ++k) {
                const int32_t src = reverse ? W - 1 - k : k;
                float *slot = stage + (int64_t)src * l;
                rc = launch_copy(&slot, 1, arenas[src] + s, l, cu, stream);
            }
            if (rc == DETFOLD_OK) {
                const Geometry g = ranks_geometry((uintptr_t)(arenas[me] + s), (uintptr_t)stage, W, l);
                detfold_plan p;
                rc = make_plan(g, cu, nullptr, DETFOLD_POLICY_STREAM, &p);
                if (rc == DETFOLD_OK)
                    rc = launch_plan(g, p, false, 1.0f, stream);
            }
        }
        if (rc != DETFOLD_OK)
            return rc;
    }
    for (int32_t o = 0; o < W; ++o) {  // owner o's shard, read once, written to the other arenas
        float *dsts[kMaxRowsW];
        int nd = 0;
        for (int32_t r = 0; r < W; ++r)
            if (r != o)
                dsts[nd++] = arenas[r] + start[o];
        if ((rc = launch_copy(dsts, nd, arenas[o] + start[o], length[o], cu, stream)) != DETFOLD_OK)
            return rc;
    }
    return DETFOLD_OK;
}

// ---------------------------------------------------------------------------
// Two ranks on one device (memra-engine tests/tp_ar_gpu.rs, ArLink's pipeline
// arm, on the same-device emulation its module note describes): each rank is
// a stream; a rank pushes its partial into the peer's staging buffer (a device
// copy), and once the peer's push has landed in its own staging buffer it
// folds in place.  Ordering is by events on the streams only -- no device
// flag, no spin -- so neither rank's kernel ever waits on the other's.

// The pair link's launches have their dispatch record the link's events
// (hipExtLaunchKernel), which is not a form stream capture takes: refuse a
// link whose streams are being captured, before any work is enqueued.
int link_not_capturing(const detfold_pair_link *k)
{
    for (int r = 0; r < 2; ++r) {
        hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(static_cast<hipStream_t>(k->stream[r]), &st) != hipSuccess)
            return DETFOLD_ELAUNCH;
        if (st != hipStreamCaptureStatusNone)
            return DETFOLD_ECAPTURE;
    }
    return DETFOLD_OK;
}

int run_pair(const detfold_pair_link *k, float *x0, float *x1, int64_t n)
{
    int32_t cu = 0;
    int rc = current_cu_count(&cu);
    if (rc != DETFOLD_OK || (rc = link_not_capturing(k)) != DETFOLD_OK)
        return rc;
    float *x[2] = {x0, x1};
    hipStream_t st[2] = {static_cast<hipStream_t>(k->stream[0]), static_cast<hipStream_t>(k->stream[1])};
    for (int r = 0; r < 2; ++r) {
        const int peer = 1 - r;
        // the peer's previous fold has finished reading the staging buffer we refill
        if (hipStreamWaitEvent(st[r], static_cast<hipEvent_t>(k->folded[peer]), 0) != hipSuccess)
            return DETFOLD_ELAUNCH;
        float *dst = k->stage[peer];
        if ((rc = launch_copy(&dst, 1, x[r], n, cu, st[r], static_cast<hipEvent_t>(k->pushed[r]))) != DETFOLD_OK)
            return rc;
    }
    for (int r = 0; r < 2; ++r) {
        const int peer = 1 - r;
        if (hipStreamWaitEvent(st[r], static_cast<hipEvent_t>(k->pushed[peer]), 0) != hipSuccess)
            return DETFOLD_ELAUNCH;
        const Geometry g = into_geometry((uintptr_t)x[r], (uintptr_t)k->stage[r], n);
        detfold_plan p;
        if ((rc = plan_into(g, cu, &p)) != DETFOLD_OK ||
            (rc = launch_plan(g, p, false, 1.0f, st[r], static_cast<hipEvent_t>(k->folded[r]))) != DETFOLD_OK)
            return rc;
    }
    return DETFOLD_OK;
}

// Broadcast: stream[o] marks where it stands (folded[o]), stream[root] waits
// for that mark, copies, and the copy's end (pushed[root]) gates stream[o].
int run_broadcast(const detfold_pair_link *k, int32_t root, const float *src, float *dst, int64_t n)
{
    int32_t cu = 0;
    int rc = current_cu_count(&cu);
    if (rc != DETFOLD_OK || (rc = link_not_capturing(k)) != DETFOLD_OK)
        return rc;
    const int32_t o = 1 - root;
    hipStream_t sr = static_cast<hipStream_t>(k->stream[root]);
    hipStream_t so = static_cast<hipStream_t>(k->stream[o]);
    if (hipEventRecord(static_cast<hipEvent_t>(k->folded[o]), so) != hipSuccess ||
        hipStreamWaitEvent(sr, static_cast<hipEvent_t>(k->folded[o]), 0) != hipSuccess)
        return DETFOLD_ELAUNCH;
    if ((rc = launch_copy(&dst, 1, src, n, cu, sr, static_cast<hipEvent_t>(k->pushed[root]))) != DETFOLD_OK)
        return rc;
    return hipStreamWaitEvent(so, static_cast<hipEvent_t>(k->pushed[root]), 0) == hipSuccess
               ? DETFOLD_OK
               : DETFOLD_ELAUNCH;
}

// All-gather: both streams mark where they stand; rank r, once the peer has
// reached its mark, writes x_r into slot r of f_r and of f_peer in one copy
// kernel; then each stream waits for the peer's copy.
int run_all_gather(const detfold_pair_link *k, const float *x0, const float *x1, float *f0,
                   float *f1, int64_t span)
{
    int32_t cu = 0;
    int rc = current_cu_count(&cu);
    if (rc != DETFOLD_OK || (rc = link_not_capturing(k)) != DETFOLD_OK)
        return rc;
    const float *x[2] = {x0, x1};
    float *f[2] = {f0, f1};
    hipStream_t st[2] = {static_cast<hipStream_t>(k->stream[0]), static_cast<hipStream_t>(k->stream[1])};
    for (int r = 0; r < 2; ++r)
        if (hipEventRecord(static_cast<hipEvent_t>(k->folded[r]), st[r]) != hipSuccess)
            return DETFOLD_ELAUNCH;
    for (int r = 0; r < 2; ++r) {
        if (hipStreamWaitEvent(st[r], static_cast<hipEvent_t>(k->folded[1 - r]), 0) != hipSuccess)
            return DETFOLD_ELAUNCH;
        float *dsts[2] = {f[r] + (int64_t)r * span, f[1 - r] + (int64_t)r * span};
        if ((rc = launch_copy(dsts, 2, x[r], span, cu, st[r], static_cast<hipEvent_t>(k->pushed[r]))) != DETFOLD_OK)
            return rc;
    }
    for (int r = 0; r < 2; ++r)
        if (hipStreamWaitEvent(st[r], static_cast<hipEvent_t>(k->pushed[1 - r]), 0) != hipSuccess)
            return DETFOLD_ELAUNCH;
    return DETFOLD_OK;
}

int run_one_shot(const detfold_one_shot_link *k, int32_t rank0, int nranks, float *xa, float *xb,
                 int64_t n, void *stream)
{
    return launch_one_shot(one_shot_args(k, rank0, nranks, xa, xb, n), nranks, stream);
}

// Many stacked folds of one width: one launch of the batched row body for
// 2 <= W <= 16, else one launch per job.
int run_batch(const detfold_fold_job *jobs, int32_t count, int32_t W, bool scaled, float inv_w,
              void *stream)
{
    int rc = check_batch_args(jobs, count, W);
    if (rc != DETFOLD_OK)
        return rc;
    bool any = false;
    for (int32_t j = 0; j < count; ++j)
        any = any || jobs[j].len > 0;
    if (!any)
        return DETFOLD_OK;
    int32_t cu = 0;
    if ((rc = current_cu_count(&cu)) != DETFOLD_OK)
        return rc;
    if (W == 1 || W > kMaxRowsW) {  // no batched body: one launch per job, at its pitch
        for (int32_t j = 0; j < count && rc == DETFOLD_OK; ++j) {
            if (jobs[j].len == 0)
                continue;
            const Geometry g = job_geometry(jobs[j], W);
            detfold_plan p;
            if ((rc = make_plan(g, cu, nullptr, DETFOLD_POLICY_STREAM, &p)) == DETFOLD_OK)
                rc = launch_plan(g, p, scaled, inv_w, stream);
        }
        return rc;
    }
    BatchArgs a;
    detfold_plan p;
    if ((rc = plan_batch(jobs, count, W, cu, &a, &p)) != DETFOLD_OK)
        return rc;
    a.inv_w = inv_w;
    return launch_batch(a, W, p, scaled, stream);
}

}  // namespace
}  // namespace detfold_impl

using namespace detfold_impl;


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

int detfold_fold_ranks_timed(float *out, const float *stacked, int32_t W, int64_t len, int32_t scaled,
                             float inv_w, const detfold_launch *launch, void *stream, void *start,
                             void *stop)
{
    return run_ranks(out, stacked, W, len, scaled != 0, inv_w, launch, stream, start, stop);
}

int fold_ranks_batch(const detfold_fold_job *jobs, int32_t count, int32_t W, void *stream)
{
    return run_batch(jobs, count, W, false, 1.0f, stream);
}

int fold_ranks_batch_scaled(const detfold_fold_job *jobs, int32_t count, int32_t W, float inv_w,
                            void *stream)
{
    return run_batch(jobs, count, W, true, inv_w, stream);
}

int detfold_plan_fold_ranks_batch(const detfold_fold_job *jobs, int32_t count, int32_t W,
                                  int32_t cu_count, detfold_plan *plan)
{
    if (!plan || W < 2 || W > kMaxRowsW)
        return DETFOLD_EINVAL;
    int rc = check_batch_args(jobs, count, W);
    if (rc != DETFOLD_OK)
        return rc;
    BatchArgs a;
    return plan_batch(jobs, count, W, cu_count, &a, plan);
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
    case DETFOLD_ESIZE: return "request exceeds the library's static stage "
                               "(DETFOLD_STATIC_STAGE_FLOATS floats)";
    case DETFOLD_ECAPTURE: return "the pair link's streams are being captured into a graph, "
                                  "which the pair link does not support";
    default: return "unknown detfold return code";
    }
}

int detfold_abi_version(void) { return DETFOLD_ABI_VERSION; }

int detfold_shard_plan(int64_t n, int32_t world, int64_t *start, int64_t *length)
{
    return balanced_shards(n, world, start, length);
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
    return make_plan(ranks_geometry(out, stacked, W, len), cu_count, launch, DETFOLD_POLICY_STREAM,
                     plan);
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

int fold_slots(float *out, const float *const *slots, int32_t W, int64_t len, void *stream)
{
    return run_slots(out, slots, W, len, false, 1.0f, stream);
}

int fold_slots_scaled(float *out, const float *const *slots, int32_t W, int64_t len, float inv_w,
                      void *stream)
{
    return run_slots(out, slots, W, len, true, inv_w, stream);
}

int detfold_loopback_round(float *const *arenas, int32_t W, int64_t n, float *stage,
                           int64_t stage_elems, int32_t flags, void *stream)
{
    int rc = check_round_args(arenas, W, n, stage, stage_elems, flags);
    if (rc != DETFOLD_OK || W == 1 || n == 0)
        return rc;
    return run_round(arenas, W, n, stage, flags, static_cast<hipStream_t>(stream));
}

int detfold_loopback_round_static(float *const *arenas, int32_t W, int64_t n, int32_t flags,
                                  void *stream)
{
    if (flags & ~DETFOLD_ROUND_REVERSE_DELIVERY)
        return DETFOLD_EINVAL;  // the staged round only
    // the arenas alone first (no stage yet: DIRECT skips the stage checks)
    int rc = check_round_args(arenas, W, n, nullptr, 0, flags | DETFOLD_ROUND_DIRECT);
    if (rc != DETFOLD_OK || W == 1 || n == 0)
        return rc;
    const int64_t need = (int64_t)W * ((n + W - 1) / W);
    if (need > DETFOLD_STATIC_STAGE_FLOATS)
        return DETFOLD_ESIZE;
    float *stage = nullptr;
    if ((rc = static_stage(&stage)) != DETFOLD_OK)
        return rc;
    if ((rc = check_round_args(arenas, W, n, stage, DETFOLD_STATIC_STAGE_FLOATS, flags)) != DETFOLD_OK)
        return rc;
    return run_round(arenas, W, n, stage, flags, static_cast<hipStream_t>(stream));
}

int detfold_pair_link_init(const detfold_pair_link *link)
{
    if (!link || !link->folded[0] || !link->folded[1] || !link->pushed[0] || !link->pushed[1])
        return DETFOLD_EINVAL;
    for (int r = 0; r < 2; ++r)
        if (hipEventRecord(static_cast<hipEvent_t>(link->folded[r]), static_cast<hipStream_t>(link->stream[r])) != hipSuccess)
            return DETFOLD_ELAUNCH;
    return DETFOLD_OK;
}

int detfold_pair_all_reduce(const detfold_pair_link *link, float *x0, float *x1, int64_t n)
{
    int rc = check_pair_args(link, x0, x1, n);
    if (rc != DETFOLD_OK || n == 0)
        return rc;
    return run_pair(link, x0, x1, n);
}

int detfold_pair_broadcast(const detfold_pair_link *link, int32_t root, const float *src,
                           float *dst, int64_t n)
{
    if (check_link_events(link) != DETFOLD_OK || (root != 0 && root != 1) || n < 0)
        return DETFOLD_EINVAL;
    if (n == 0)
        return DETFOLD_OK;
    if (bad_buffer(src, n) || bad_buffer(dst, n))
        return DETFOLD_EINVAL;
    if (ranges_overlap((uintptr_t)src, (uint64_t)n * 4, (uintptr_t)dst, (uint64_t)n * 4))
        return DETFOLD_EOVERLAP;
    return run_broadcast(link, root, src, dst, n);
}

int detfold_pair_all_gather(const detfold_pair_link *link, const float *x0, const float *x1,
                            float *f0, float *f1, int64_t span)
{
    if (check_link_events(link) != DETFOLD_OK || span < 0)
        return DETFOLD_EINVAL;
    if (span == 0)
        return DETFOLD_OK;
    if (bad_buffer(x0, span) || bad_buffer(x1, span) || bad_buffer(f0, 2 * span) || bad_buffer(f1, 2 * span))
        return DETFOLD_EINVAL;
    const uint64_t xb = (uint64_t)span * 4, fb = xb * 2;
    if (ranges_overlap((uintptr_t)f0, fb, (uintptr_t)f1, fb) ||
        ranges_overlap((uintptr_t)f0, fb, (uintptr_t)x0, xb) || ranges_overlap((uintptr_t)f0, fb, (uintptr_t)x1, xb) ||
        ranges_overlap((uintptr_t)f1, fb, (uintptr_t)x0, xb) || ranges_overlap((uintptr_t)f1, fb, (uintptr_t)x1, xb))
        return DETFOLD_EOVERLAP;
    return run_all_gather(link, x0, x1, f0, f1, span);
}

int detfold_one_shot_init(const detfold_one_shot_link *link)
{
    int rc = check_one_shot_link(link);
    if (rc != DETFOLD_OK)
        return rc;
    if ((rc = launch_zero_words(link->flags, DETFOLD_ONE_SHOT_FLAG_WORDS, link->stream)) != DETFOLD_OK ||
        (rc = launch_zero_words(reinterpret_cast<uint32_t *>(link->words), 2, link->stream)) != DETFOLD_OK)
        return rc;
    return hipStreamSynchronize(static_cast<hipStream_t>(link->stream)) == hipSuccess ? DETFOLD_OK
                                                                                      : DETFOLD_ELAUNCH;
}

int detfold_one_shot_all_reduce(const detfold_one_shot_link *link, float *x0, float *x1, int64_t n)
{
    int rc = check_one_shot_link(link);
    if (rc != DETFOLD_OK)
        return rc;
    float *x[2] = {x0, x1};
    if ((rc = check_one_shot_buffers(link, x, 2, n)) != DETFOLD_OK || n == 0)
        return rc;
    return run_one_shot(link, 0, 2, x0, x1, n, link->stream);
}

int detfold_one_shot_rank(const detfold_one_shot_link *link, int32_t rank, float *x, int64_t n,
                          void *stream)
{
    int rc = check_one_shot_link(link);
    if (rc != DETFOLD_OK)
        return rc;
    if (rank != 0 && rank != 1)
        return DETFOLD_EINVAL;
    float *xs[1] = {x};
    if ((rc = check_one_shot_buffers(link, xs, 1, n)) != DETFOLD_OK || n == 0)
        return rc;
    return run_one_shot(link, rank, 1, x, nullptr, n, stream);
}

}  // extern "C"
