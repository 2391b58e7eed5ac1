/*
 * detfold.h -- deterministic fixed-order fold of float32 partial buffers on
 * AMD Instinct MI355X (gfx950), C ABI.
 *
 * The operation (mamba-rs src/dist/reducer.rs: module note on the
 * ReduceContract::FixedOrder contract, the `det_sum_ranks` kernel source and
 * the host function `reduce_sum_reference`): W partial buffers s_0 .. s_{W-1}
 * of `len` float32 values are combined elementwise as
 *
 *     acc = s_0[i];  acc = acc + s_r[i]  for r = 1 .. W-1, strictly ascending;
 *
 * every "+" a single IEEE 754 binary32 addition, round-to-nearest-even, with
 * subnormals kept and no fused multiply-add.  The association order is fixed by
 * program text, never by launch geometry, scheduling or memory layout, so the
 * result is bit-identical to a host serial add chain of the same addends.
 *
 * Conventions shared by every entry point:
 *   - Pointers named as device pointers address memory of the calling thread's
 *     current HIP device; `stream` is a hipStream_t of that device passed as
 *     void* (NULL = the null stream).
 *   - The caller owns every buffer.  The library allocates nothing, keeps no
 *     pointer after it returns, and does not synchronize (detfold_one_shot_init
 *     excepted): work is enqueued on `stream` and the call returns.  Faults
 *     inside the kernels surface at the caller's next synchronization of that
 *     stream.
 *   - Float pointers must be 4-byte aligned; any 4-byte alignment is accepted
 *     (buffers at different offsets modulo 16 bytes and ragged lengths are
 *     handled by dword-addressed or 4-byte loads, never an error).
 *   - A call with zero elements returns DETFOLD_OK and launches nothing
 *     (mamba-rs src/dist/reducer.rs, `DetReduceKernel::launch`).
 *   - Every entry point validates its arguments before any HIP call, so an
 *     argument error never touches the device.
 *   - The library keeps one piece of state: a per-device cache of the compute
 *     unit count, filled on first use.  All entry points are thread-safe;
 *     calls that write overlapping memory race as any two kernels would.
 */
#ifndef DETFOLD_H
#define DETFOLD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes.  Only "0 = ok" is fixed by the pages (memra-engine
 * tests/tp_ar_gpu.rs, `memra_tp_ar_fold` returns 0 on success); the others
 * name the failure classes the pages describe as errors. */
#define DETFOLD_OK 0       /* work enqueued (or nothing to do)                           */
#define DETFOLD_EINVAL 1   /* W < 1, negative length, NULL or misaligned pointer with     */
                           /* len > 0, size overflow, or an invalid launch override      */
#define DETFOLD_EOVERLAP 2 /* output range overlaps an input range it must not alias     */
#define DETFOLD_ELAUNCH 3  /* the HIP launch was refused                                 */
#define DETFOLD_EDEVICE 4  /* no current HIP device, or its properties could not be read */
#define DETFOLD_ESIZE 5    /* the request needs more than the library's static stage     */
#define DETFOLD_ECAPTURE 6 /* a pair-link stream is being captured into a graph         */

/*
 * fold_ranks -- out[i] = ((s_0[i] + s_1[i]) + ...) + s_{W-1}[i]
 *
 * Stacked arena layout (mamba-rs src/dist/reducer.rs, `det_sum_ranks` and
 * `reduce_sum_fixed_order_nccl`): `stacked` is row-major [W][len], slot r
 * (the addend from source rank r) at stacked + r*len.  `out` holds len floats.
 *   out      device pointer, written (len floats)
 *   stacked  device pointer, read (W*len floats)
 *   W        number of addend slots, >= 1 (W = 1 copies slot 0 bit for bit)
 *   len      elements per slot, >= 0 (64-bit; W*len*4 bytes must fit int64)
 *   stream   hipStream_t of the current device
 * Errors: DETFOLD_EINVAL, DETFOLD_EOVERLAP when [out, out+len) intersects
 * [stacked, stacked+W*len) (the launch contract requires the regions not to
 * overlap), DETFOLD_EDEVICE, DETFOLD_ELAUNCH.
 */
int fold_ranks(float *out, const float *stacked, int32_t W, int64_t len, void *stream);

/*
 * fold_into -- dst[i] = dst[i] + stage[i]   (in place; the two-addend fold)
 *
 * The decode-join fold of memra-engine tests/tp_ar_gpu.rs (C-ABI
 * `memra_tp_ar_fold(dst, stage, n, stream)`): dst holds this rank's partial
 * (slot 0), stage the peer's partial (slot 1).  Small payloads (16-256 KiB)
 * take a latency path: a small grid, no device-side flags and no waits of any
 * kind, so the fold completes whatever else is resident on the device (the
 * page's note on the flag-spinning first cut that deadlocked on one card).
 *   dst    device pointer, read and written (n floats)
 *   stage  device pointer, read (n floats)
 *   n      elements, >= 0
 * Errors: DETFOLD_EINVAL, DETFOLD_EOVERLAP when the two ranges intersect,
 * DETFOLD_EDEVICE, DETFOLD_ELAUNCH.
 */
int fold_into(float *dst, const float *stage, int64_t n, void *stream);

/*
 * fold_ranks_scaled -- out[i] = fold_ranks(...)[i] * inv_w
 *
 * The mean scale applied after the sum, as one binary32 multiply of the
 * finished sum (mamba-rs src/dist/reducer.rs module note: the kernel forms the
 * sum and the caller's 1/W scale follows it, exact for power-of-two W).  The
 * scale is the caller's: inv_w is not checked against W, and any value
 * (including non-powers of two) is applied as given, with one rounding of
 * sum * inv_w.  For W that is not a power of two this can differ from
 * sum / W (5 * RN(1/3) rounds to 0x3fd55556, 5 / 3 to 0x3fd55555).
 * Arguments and errors as fold_ranks.
 */
int fold_ranks_scaled(float *out, const float *stacked, int32_t W, int64_t len, float inv_w,
                      void *stream);

/*
 * fold_slots -- out[i] = ((s_0[i] + s_1[i]) + ...) + s_{W-1}[i] over W separate buffers
 *
 * The same fold as fold_ranks when the addends do not sit in one stacked arena
 * (for example W per-rank arenas on one device, as in mamba-rs
 * src/dist/reducer.rs LoopbackWorld, or buffers of another device mapped into
 * this one's address space).
 *   out      device pointer, written (len floats).  It may be identical to one
 *            or more of the slots (the fold then runs in place); any other
 *            overlap with a slot is DETFOLD_EOVERLAP.
 *   slots    HOST array of W device pointers, each to len floats (read); the
 *            pointers are passed to the kernel by value, the array may be
 *            reused as soon as the call returns.  Slots may overlap each other.
 *   W        1 <= W <= 16
 *   len      elements, >= 0
 * Errors: DETFOLD_EINVAL (also for W > 16), DETFOLD_EOVERLAP, DETFOLD_EDEVICE,
 * DETFOLD_ELAUNCH.
 */
int fold_slots(float *out, const float *const *slots, int32_t W, int64_t len, void *stream);

/* fold_slots followed by one binary32 multiply of each sum by inv_w. */
int fold_slots_scaled(float *out, const float *const *slots, int32_t W, int64_t len, float inv_w,
                      void *stream);

/*
 * fold_ranks_batch -- many stacked folds of one width in one launch: for each
 * job j, jobs[j].out = fold_ranks of jobs[j].stacked ([W][jobs[j].len]), bit
 * for bit what `count` separate fold_ranks calls would write.
 *
 * On one device the W owners of the transport dataflow each fold their own
 * shard (mamba-rs src/dist/reducer.rs, reduce_sum_fixed_order_nccl and
 * LoopbackWorld::run_round); one launch over all the owners' shards keeps the
 * whole device busy where one owner's shard alone is too small to (a shard of
 * a 40 MB arena is a wave or two of workgroups).  The same holds for any set
 * of buffers of equal width, such as the buckets of one reduction.
 *   jobs     HOST array of `count` jobs (copied into the launch; reusable as
 *            soon as the call returns); a job with len == 0 is skipped.  A
 *            job's slots may sit `pitch` floats apart (a receive buffer whose
 *            slots are padded), which gives the same bits as a packed arena
 *   count    0 <= count <= DETFOLD_MAX_JOBS
 *   W        >= 1, shared by every job.  2 <= W <= 16 is one launch; W = 1
 *            and W > 16 run one launch per job.
 * Every job is checked as fold_ranks checks its arguments (its arena being
 * [stacked, stacked + (W-1)*pitch + len)); besides, no job's output may
 * overlap another job's output or arena (DETFOLD_EOVERLAP), and a pitch below
 * len is DETFOLD_EINVAL.  Arenas may overlap each other (they are only read).
 * Errors: DETFOLD_EINVAL (also for count out of range or NULL jobs with
 * count > 0), DETFOLD_EOVERLAP, DETFOLD_EDEVICE, DETFOLD_ELAUNCH.
 */
#define DETFOLD_MAX_JOBS 32
typedef struct detfold_fold_job {
    float *out;           /* device, len floats, written */
    const float *stacked; /* device, slot r at stacked + r*pitch (read) */
    int64_t len;          /* elements per slot, >= 0 */
    int64_t pitch;        /* floats from one slot's start to the next: 0 = len (a packed
                             [W][len] arena), else >= len (slots padded apart) */
} detfold_fold_job;
int fold_ranks_batch(const detfold_fold_job *jobs, int32_t count, int32_t W, void *stream);

/* fold_ranks_batch followed by one binary32 multiply of every sum by inv_w. */
int fold_ranks_batch_scaled(const detfold_fold_job *jobs, int32_t count, int32_t W, float inv_w,
                            void *stream);

/*
 * detfold_loopback_round -- one fixed-order reduction round across W arenas on
 * one device: afterwards every arena holds, bit for bit, the ascending-rank
 * fold of the W arenas' original contents.
 *
 * The dataflow of mamba-rs src/dist/reducer.rs (LoopbackWorld::run_round and
 * the owner-shard exchange of reduce_sum_fixed_order_nccl): [0, n) is split
 * into W contiguous owner shards (detfold_shard_plan); owner p folds the W
 * copies of shard p into its own arena; then every owner's reduced shard is
 * copied into the other W-1 arenas.  Movement is device-to-device copies only.
 *   arenas       HOST array of W device pointers, each to n floats (read and
 *                written); arenas must not overlap each other
 *   W            1 <= W <= 16 (W = 1: nothing to do)
 *   n            elements per arena, >= 0
 *   stage        device scratch of at least W * ceil(n / W) floats, owned by
 *                the caller, overwritten; unused (may be NULL) with
 *                DETFOLD_ROUND_DIRECT or DETFOLD_ROUND_FUSED
 *   stage_elems  capacity of `stage` in floats
 *   flags        DETFOLD_ROUND_REVERSE_DELIVERY: gather the sources' shards
 *                into the stage in descending source order (slot placement is
 *                still by source rank, so the bits do not change);
 *                DETFOLD_ROUND_DIRECT: fold each owner's shard straight from
 *                the W arenas, with no stage and no gather copies;
 *                DETFOLD_ROUND_FUSED: one kernel and no owner shards -- each
 *                workgroup reads one tile of all W arenas, folds it and writes
 *                the sum back into that tile of every arena, so each arena
 *                byte is read once and written once (W*n*4 bytes each way).
 *                Not combinable with the other flags; no stage.
 * Arenas may sit at any 4-byte-aligned addresses (any 16-byte phases).
 * Errors: DETFOLD_EINVAL (also for an unknown flag or FUSED with another
 * flag), DETFOLD_EOVERLAP (arenas overlap each other or the stage),
 * DETFOLD_EDEVICE, DETFOLD_ELAUNCH.  Stream-ordered; no synchronize.
 */
#define DETFOLD_ROUND_REVERSE_DELIVERY 1
#define DETFOLD_ROUND_DIRECT 2
#define DETFOLD_ROUND_FUSED 4
int detfold_loopback_round(float *const *arenas, int32_t W, int64_t n, float *stage,
                           int64_t stage_elems, int32_t flags, void *stream);

/*
 * detfold_loopback_round_static -- the staged detfold_loopback_round with its
 * stage in device memory the library owns, for callers that cannot allocate
 * device memory (code under stream or graph capture, tight serving loops,
 * harnesses that forbid allocation): the call allocates nothing and frees
 * nothing.  The stage is a file-scope device array of
 * DETFOLD_STATIC_STAGE_FLOATS floats (16 MiB), one per device the library
 * runs on, held until the process ends.
 *   arenas, W, n  as detfold_loopback_round; W * ceil(n / W) must not exceed
 *                 DETFOLD_STATIC_STAGE_FLOATS, else DETFOLD_ESIZE before any
 *                 device work
 *   flags         0 or DETFOLD_ROUND_REVERSE_DELIVERY (the staged round;
 *                 anything else is DETFOLD_EINVAL)
 * The bits equal detfold_loopback_round's with a caller stage.  The stage is
 * shared by every call on a device and keeps the last call's contents; every
 * call overwrites the part it reads before reading it, so nothing needs
 * clearing.  Calls that overlap in time on one device (other streams, other
 * threads, other processes do not share it) race on the stage: order them.
 * Errors: as detfold_loopback_round, plus DETFOLD_ESIZE, and DETFOLD_EDEVICE
 * when the stage's device address cannot be obtained.
 */
#define DETFOLD_STATIC_STAGE_FLOATS (1 << 22)
int detfold_loopback_round_static(float *const *arenas, int32_t W, int64_t n, int32_t flags,
                                  void *stream);

/*
 * A two-rank all-reduce on one device: the pipeline arm of memra-engine
 * tests/tp_ar_gpu.rs (ArLink: push the peer partial into staging, order with
 * events, fold) with each rank a stream.  Rank r pushes its partial into
 * stage[1-r] by a device copy, and folds x_r += stage[r] once the peer's push
 * has landed.  All ordering is by events between the two streams; no kernel
 * spins on a flag, so neither rank can starve the other however much other
 * work is resident.  The caller owns every buffer, stream and event; the
 * library keeps no state between calls.
 * The link's launches have their dispatch record the link's events, a form
 * stream capture does not take: every pair-link call on a stream that is
 * being captured into a graph returns DETFOLD_ECAPTURE before enqueueing
 * anything.
 */
typedef struct detfold_pair_link {
    void *stream[2];  /* hipStream_t of rank 0 and rank 1 (one device; may be equal) */
    float *stage[2];  /* stage[r]: rank r's staging buffer, capacity floats, device */
    int64_t capacity; /* floats each staging buffer holds */
    void *pushed[2];  /* hipEvent_t: recorded on stream[r] after rank r's push */
    void *folded[2];  /* hipEvent_t: recorded on stream[r] after rank r's fold */
} detfold_pair_link;

/* Record folded[0] and folded[1] once on their streams before the first
 * detfold_pair_all_reduce, so the first call's waits have an event to wait for. */
int detfold_pair_link_init(const detfold_pair_link *link);

/*
 * detfold_pair_all_reduce -- x0 = x0 + x1 on stream[0] and x1 = x1 + x0 on
 * stream[1], bit-identical (binary32 addition is commutative), each the
 * two-addend fold of fold_into.  A call may be repeated on the same link: a
 * rank refills the peer's staging buffer only after the peer's previous fold
 * has read it (folded[peer]).
 *   x0, x1  device pointers to n floats each (read and written)
 *   n       0 <= n <= capacity
 * Errors: DETFOLD_EINVAL (NULL link, event, buffer, or n > capacity),
 * DETFOLD_EOVERLAP (x0, x1, stage[0], stage[1] must be disjoint over n
 * floats), DETFOLD_EDEVICE, DETFOLD_ELAUNCH.
 */
int detfold_pair_all_reduce(const detfold_pair_link *link, float *x0, float *x1, int64_t n);

/*
 * detfold_pair_broadcast -- pure movement: the other rank's dst becomes a byte
 * copy of rank `root`'s src (memra-engine tests/tp_ar_gpu.rs, the broadcast
 * half of broadcast_and_all_gather_move_bytes_exactly).  The copy runs on
 * stream[root] once stream[1-root] has reached this call (so earlier work
 * there that reads dst is done); stream[1-root] then waits for the copy.
 *   root    0 or 1
 *   src     device pointer, n floats of rank root (read)
 *   dst     device pointer, n floats of rank 1-root (overwritten)
 * Errors: DETFOLD_EINVAL (NULL link or event, root not 0 or 1, n < 0, NULL or
 * misaligned buffer), DETFOLD_EOVERLAP (src and dst intersect), DETFOLD_ELAUNCH.
 * Uses the link's events (folded[], pushed[]) but not its staging buffers.
 */
int detfold_pair_broadcast(const detfold_pair_link *link, int32_t root, const float *src,
                           float *dst, int64_t n);

/*
 * detfold_pair_all_gather -- pure movement: on both ranks f_r becomes the
 * rank-order concatenation [x0 | x1] (2*span floats).  Rank r writes x_r into
 * its own slot of f_r and into the same slot of the peer's f_{1-r} with one
 * copy kernel on stream[r]; each stream then waits for the peer's copy.
 *   x0, x1  device pointers, span floats each (read; they may alias each other)
 *   f0, f1  device pointers, 2*span floats each (overwritten)
 * Errors: DETFOLD_EINVAL, DETFOLD_EOVERLAP (f0, f1 and the x must not intersect),
 * DETFOLD_ELAUNCH.
 */
int detfold_pair_all_gather(const detfold_pair_link *link, const float *x0, const float *x1,
                            float *f0, float *f1, int64_t span);

/*
 * The one-shot arm of the two-rank all-reduce (memra-engine
 * tests/tp_ar_gpu.rs, one_shot_all_reduce_matches_the_host_sum_bitwise; the
 * module note there describes why a spinning fold can starve its peer on one
 * device).  One kernel and no events: each workgroup b of rank r
 *   1. copies its chunk of x_r into stage[1-r],
 *   2. arrives at the entry barrier (counter flags[entry][r][b]) and waits
 *      until the peer's workgroup b has arrived as often,
 *   3. folds x_r[i] = x_r[i] + stage[r][i] over its chunk,
 *   4. arrives at the exit barrier and waits for the peer's workgroup b (so
 *      the next call's push cannot overwrite a stage the peer still reads).
 * Every wait polls at most spin_limit times.  A wait that expires stores a
 * barrier word and the workgroup returns: DETFOLD_BARRIER_ENTRY_EXPIRED
 * (the fold was skipped, that chunk of x_r is untouched) or
 * DETFOLD_BARRIER_EXIT_EXPIRED (the fold is done; the peer may still read
 * the stage).  The first word stored for a rank stays until init.  After a
 * nonzero word the counters disagree and the link must be re-initialised.
 * The counters live on the device and are advanced by the kernel itself, so
 * a call captured in a HIP graph replays correctly.
 */
#define DETFOLD_ONE_SHOT_BLOCKS 64 /* workgroups per rank, at most */
#define DETFOLD_ONE_SHOT_FLAG_WORDS (2 * 2 * DETFOLD_ONE_SHOT_BLOCKS)
#define DETFOLD_BARRIER_ENTRY_EXPIRED 40043
#define DETFOLD_BARRIER_EXIT_EXPIRED 40044
typedef struct detfold_one_shot_link {
    void *stream;       /* hipStream_t for init and for detfold_one_shot_all_reduce */
    float *stage[2];    /* stage[r]: rank r's staging buffer, capacity floats, device */
    int64_t capacity;   /* floats each staging buffer holds */
    uint32_t *flags;    /* device, DETFOLD_ONE_SHOT_FLAG_WORDS barrier counters */
    int32_t *words;     /* device, 2 barrier words (rank 0, rank 1); 0 = no expiry */
    int32_t spin_limit; /* polls per barrier wait before it expires; 0 = 1 << 20 */
} detfold_one_shot_link;

/* Zero flags and words with a kernel on link->stream and synchronize that
 * stream.  Call once before the first all-reduce and after any nonzero word. */
int detfold_one_shot_init(const detfold_one_shot_link *link);

/*
 * detfold_one_shot_all_reduce -- x0 = x0 + x1 and x1 = x1 + x0 (bit-identical),
 * both ranks' workgroups in one launch on link->stream.  On one device that
 * launch holds at most 2 * DETFOLD_ONE_SHOT_BLOCKS workgroups of 256 threads,
 * all resident at once, so the barriers complete.
 *   x0, x1  device pointers to n floats each (read and written)
 *   n       0 <= n <= capacity
 * Errors: DETFOLD_EINVAL (NULL link, flags, words or buffer, misaligned
 * pointer, spin_limit < 0, n > capacity), DETFOLD_EOVERLAP (x0, x1, stage[0],
 * stage[1] must be disjoint over n floats), DETFOLD_ELAUNCH.  An expired
 * barrier is reported in link->words, not by the return code.
 */
int detfold_one_shot_all_reduce(const detfold_one_shot_link *link, float *x0, float *x1,
                                int64_t n);

/*
 * detfold_one_shot_rank -- rank `rank`'s kernel alone, on `stream`: the shape
 * each rank launches on its own device.  Both ranks must make the call with
 * the same n.  On one device the two kernels must run concurrently for the
 * barriers to meet; when they do not (both streams on one hardware queue, or
 * the peer never launched), the waits expire and the words say so.
 *   rank    0 or 1;  x  device pointer to n floats of that rank
 * Errors: as detfold_one_shot_all_reduce, plus DETFOLD_EINVAL for a bad rank.
 */
int detfold_one_shot_rank(const detfold_one_shot_link *link, int32_t rank, float *x, int64_t n,
                          void *stream);

/* Static, NUL-terminated description of a return code (never NULL). */
const char *detfold_strerror(int rc);

/* ABI revision of this header; bumped on any incompatible change. */
#define DETFOLD_ABI_VERSION 12
int detfold_abi_version(void);

/* ------------------------------------------------------------------------
 * Owner shards (host only; no device access).
 *
 * detfold_shard_plan -- split [0, n) into `world` contiguous owner shards, as
 * the transport dataflow does before each owner folds its own shard
 * (mamba-rs src/dist/reducer.rs, `shard_plan` as used by
 * `reduce_sum_fixed_order_nccl` and `LoopbackWorld::run_round`; the split
 * itself is not printed there).  Balanced split: shard p has
 * n/world + (p < n%world) elements, shards in ascending order, so a shard may
 * be empty when n < world.  The fold's bits do not depend on the split.
 *   start, length  host arrays of `world` int64, written
 * Errors: DETFOLD_EINVAL for world < 1, n < 0 or NULL arrays.
 */
int detfold_shard_plan(int64_t n, int32_t world, int64_t *start, int64_t *length);

/* ------------------------------------------------------------------------
 * Launch planning and the test-only launch override.
 *
 * Three bodies compute the same per-element chain, so the path, the geometry
 * and the cache policy never change a bit:
 *   ROWS    (default for W >= 2 on the streaming policy) one workgroup of
 *           W waves per tile (beyond 16 slots: 16 waves making passes of 16
 *           slots, the running sums kept in registers between passes); wave r
 *           streams a contiguous run of slot r into
 *           LDS with 16-byte loads addressed from the slot's own first element
 *           of the tile, so a slot at another 16-byte phase than out's lands
 *           aligned all the same; every thread then folds whole 16-byte groups
 *           and stores them.  Up to 3 elements before the first 16-byte
 *           boundary of `out` (head) and up to 3 after the last (tail) are
 *           folded one by one.
 *   VECTOR  (default for W = 1 when `out` and slot 0 share one 16-byte phase,
 *           and for the small in-place fold) each thread loads 16 bytes of
 *           every slot directly; head and tail as above.
 *   SCALAR  (otherwise) each thread loads 4 bytes of every slot directly.
 *
 * Cache policy: the bandwidth path (fold_ranks, fold_ranks_scaled, and
 * fold_into above 8 MiB per buffer) streams: loads and stores carry the
 * non-temporal hint.  fold_into at or below 8 MiB per buffer uses no hints,
 * since the folded result is read again soon.
 */
#define DETFOLD_PATH_AUTO 0
#define DETFOLD_PATH_VECTOR 1 /* direct body, 16-byte loads (out and every slot co-aligned) */
#define DETFOLD_PATH_SCALAR 2 /* direct body, 4-byte loads (any alignment)                 */
#define DETFOLD_PATH_ROWS 3   /* LDS row body, W >= 2, any alignment, streaming only        */

#define DETFOLD_POLICY_DEFAULT 0
#define DETFOLD_POLICY_STREAM 1 /* non-temporal loads and stores */
#define DETFOLD_POLICY_CACHED 2 /* no cache hints (available with unroll 1 only) */

typedef struct detfold_launch {
    int32_t path;   /* DETFOLD_PATH_*; VECTOR where the alignment forbids it is EINVAL */
    int32_t block;  /* threads per workgroup: 0 = default, else a multiple of 64 in [64, 1024].
                       ROWS names the shape: W <= 16: 64*W (one slot per wave) or, W >= 5,
                       64*ceil(W/2) (two slots per wave); W > 16: 1024 or 512 (the pass shapes) */
    int64_t grid;   /* workgroups: 0 = one pass, else >= 1 (workgroups loop over the tiles) */
    int32_t unroll; /* groups (vector) or elements (scalar) per thread per tile: 0 = default, 1, 2 or 4
                       (ROWS: 0 or 1) */
    int32_t policy; /* DETFOLD_POLICY_*: 0 = the entry point's own policy */
    int32_t group;  /* ROWS, one pass: each XCD takes runs of this many neighbouring tiles
                       (0 = the plan's choice, else a power of two up to 64; 1 = plain
                       round-robin) */
} detfold_launch;

typedef struct detfold_plan {
    int32_t path;   /* DETFOLD_PATH_ROWS, _VECTOR or _SCALAR */
    int32_t block;
    int64_t grid;
    int32_t unroll;
    int32_t head;   /* elements folded one by one before the 16-byte-aligned body (rows, vector) */
    int32_t tail;   /* elements folded one by one after it (rows, vector) */
    int32_t policy; /* DETFOLD_POLICY_STREAM or DETFOLD_POLICY_CACHED */
    int64_t body;   /* 4-element groups (rows, vector) or elements (scalar) */
    int64_t tile;   /* body positions one workgroup folds per pass */
    int32_t group;  /* XCD tile group of the row body (1 = plain round-robin) */
} detfold_plan;

/*
 * detfold_plan_fold_ranks -- the path and geometry fold_ranks (and, with a
 * launch override, detfold_fold_ranks_ex) would use for these addresses and
 * sizes on a device with `cu_count` compute units.  Host only: addresses are
 * plain integers and nothing is dereferenced.  `launch` may be NULL.
 * Errors: as fold_ranks's argument checks, plus DETFOLD_EINVAL for a bad
 * override or cu_count < 1.  With len == 0 the plan has grid = 0.
 */
int detfold_plan_fold_ranks(uintptr_t out, uintptr_t stacked, int32_t W, int64_t len,
                            int32_t cu_count, const detfold_launch *launch, detfold_plan *plan);

/* The plan of fold_ranks_batch's one launch for 2 <= W <= 16 (host only, as
 * above): block and tile of the shape, grid = the workgroups of all jobs,
 * body = their 16-byte groups.  With no element to fold the grid is 0. */
int detfold_plan_fold_ranks_batch(const detfold_fold_job *jobs, int32_t count, int32_t W,
                                  int32_t cu_count, detfold_plan *plan);

/* The plan fold_into would use (host only, as above). */
int detfold_plan_fold_into(uintptr_t dst, uintptr_t stage, int64_t n, int32_t cu_count,
                           detfold_plan *plan);

/*
 * detfold_fold_ranks_ex -- fold_ranks / fold_ranks_scaled with an explicit
 * launch override.  For tests and tuning sweeps: it exists to show that the
 * bits do not depend on path or geometry.  scaled = 0 ignores inv_w.
 */
int detfold_fold_ranks_ex(float *out, const float *stacked, int32_t W, int64_t len, int32_t scaled,
                          float inv_w, const detfold_launch *launch, void *stream);

/*
 * detfold_fold_ranks_timed -- detfold_fold_ranks_ex whose kernel dispatch
 * itself records two caller-owned events: `start` when the fold kernel begins
 * and `stop` when it has finished (hipExtLaunchKernel's start and stop
 * events).  hipEventElapsedTime(start, stop) is then the kernel's own
 * duration, free of the launch and event-record latency that an event pair
 * recorded around the call includes (memra-engine src/bin/moe_tp2_repro.rs
 * times with timing-enabled events and warns that a harness can end up timing
 * itself rather than the device).  The fold is one kernel on every path, so
 * the pair brackets all of its work.  For measurement; the bits are those of
 * fold_ranks / fold_ranks_scaled.
 *   start, stop  hipEvent_t of the current device created with timing
 *                enabled, or NULL (that event is not recorded)
 *   launch       may be NULL (the default plan)
 * Errors: as detfold_fold_ranks_ex.  With len == 0 nothing is launched and
 * neither event is recorded.
 */
int detfold_fold_ranks_timed(float *out, const float *stacked, int32_t W, int64_t len, int32_t scaled,
                             float inv_w, const detfold_launch *launch, void *stream, void *start,
                             void *stop);

#ifdef __cplusplus
}
#endif

#endif /* DETFOLD_H */
