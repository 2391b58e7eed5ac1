// plan.cpp -- host-only planning and argument checks of libdetfold: plain
// integer logic on addresses and sizes, no device access and no HIP calls, so
// every path here can be exercised without a GPU (the library's host tests
// and its sanitizer build do).

#include <cstdint>

#include "internal.h"

namespace detfold_impl {

// Whether out and every slot share one offset modulo 16 bytes.
bool vector_legal(const Geometry &g)
{
    const int p = phase16(g.out);
    if (g.has_table) {
        for (int32_t r = 0; r < g.w; ++r)
            if (phase16(g.table[r]) != p)
                return false;
        return true;
    }
    if (phase16(g.s0) != p)
        return false;
    if (g.w >= 2 && phase16(g.s1) != p)
        return false;
    if (g.w >= 3 && (g.stride & 3) != 0)
        return false;
    return true;
}

// Whether the slots of a stacked arena repeat every address bit below
// kRepeatBytes (the slot length in bytes is a multiple of it).  Separate
// slot buffers (a table) count as repeating: the rules below were measured
// on stacked arenas, and tables keep the shapes they had before.
bool slots_repeat(const Geometry &g)
{
    return g.has_table || (g.stride * 4) % kRepeatBytes == 0;
}

// Slots each wave of the row body streams.
//  * Separate slot buffers (a table): two from five slots up when every slot
//    shares out's 16-byte phase, and from seven up when some slot does not;
//    else one.
//  * Stacked arenas of eight slots: one where the slot length is a multiple
//    of kOneSlotAlign or the slots do not repeat the low address bits, else
//    two.
//  * Stacked arenas of seven and of nine to sixteen slots: two.
//  * Stacked arenas of five or six slots: two when every slot shares out's
//    phase and the slots repeat the low address bits, else one.
int rows_slots_per_wave(const Geometry &g)
{
    if (g.w > kMaxRowsW || g.w < 5)
        return 1;
    if (g.has_table)
        return vector_legal(g) || g.w >= 7 ? 2 : 1;
    if (g.w == 8)
        return g.stride % kOneSlotAlign == 0 || !slots_repeat(g) ? 1 : 2;
    if (g.w == 7 || g.w >= 9)
        return 2;
    return vector_legal(g) && slots_repeat(g) ? 2 : 1;
}

// Whether a wide fold (beyond 16 slots) takes the eight-wave pass shape: when
// every slot shares out's phase, or when the slots repeat the low address bits
// and the last pass holds at least half of 16 slots (a pass of a few slots
// leaves most of the eight-wave shape's waves idle: W = 17 loses 7.7%).
static bool wide_eight_waves(const Geometry &g)
{
    const int last = g.w % kWideSlots;
    return vector_legal(g) || (slots_repeat(g) && (last == 0 || last >= kWideSlots / 2));
}

// Workgroup size and tile (16-byte groups) of the row bodies: one wave per
// one or two slots up to 16 slots; beyond that, passes of 16 slots by
// 16 waves, or 8 waves (wide_eight_waves).
int rows_block(const Geometry &g)
{
    if (g.w <= kMaxRowsW)
        return 64 * rows_waves(g.w, rows_slots_per_wave(g));
    return 64 * (wide_eight_waves(g) ? kWideAlignedWaves : kWideWaves);
}

int64_t rows_tile(const Geometry &g)
{
    if (g.w <= kMaxRowsW)
        return (int64_t)rows_kib_per_wave(g.w, rows_slots_per_wave(g)) * 64;
    return (int64_t)(wide_eight_waves(g) ? kWideAlignedKiB : kWideKiB) * 64;
}

// The tile of the row-body shape a workgroup size names, or 0 if it names
// none: up to 16 slots, 64*W threads (one slot per wave) or, from five slots
// up, 64*ceil(W/2) (two slots per wave); beyond 16, 64*kWideWaves or
// 64*kWideAlignedWaves threads (the two pass shapes).  Any shape folds any
// alignment, with the same bits; the plan picks the faster one.
int64_t rows_tile_for_block(const Geometry &g, int block)
{
    if (g.w > kMaxRowsW) {
        if (block == 64 * kWideWaves)
            return (int64_t)kWideKiB * 64;
        if (block == 64 * kWideAlignedWaves)
            return (int64_t)kWideAlignedKiB * 64;
        return 0;
    }
    if (block == 64 * g.w)
        return (int64_t)rows_kib_per_wave(g.w, 1) * 64;
    if (g.w >= 5 && block == 64 * rows_waves(g.w, 2))
        return (int64_t)rows_kib_per_wave(g.w, 2) * 64;
    return 0;
}

// XCD tile group of the row body (xcd_tile in fold_kernels.hip), for stacked
// arenas of three to sixteen slots: with slots shifted from out's 16-byte
// phase, runs of kSlotGroupMid tiles per XCD (kSlotGroup at three and four
// slots that do not repeat the low address bits); co-aligned, plain
// round-robin where the slots repeat the low address bits, else runs of
// kSlotGroupMid tiles from five to ten slots and of kSlotGroup otherwise.
// Beyond sixteen slots, shifted slots take runs of kSlotGroupMid where they
// repeat the low address bits and of kWideShiftedGroup where they do not;
// co-aligned ones plain round-robin.  Separate slot buffers: shifted ones as
// shifted stacked slots that do not repeat, co-aligned ones plain
// round-robin.
int rows_group(const Geometry &g, int block)
{
    (void)block;
    if (g.w > kMaxRowsW && !g.has_table)
        return vector_legal(g) ? 1 : (slots_repeat(g) ? kSlotGroupMid : kWideShiftedGroup);
    if (g.has_table)
        return vector_legal(g) || g.w < 3 || g.w > kMaxRowsW ? 1 : (g.w <= 4 ? kSlotGroup : kSlotGroupMid);
    if (g.w < 3 || g.w > kMaxRowsW)
        return 1;
    if (!vector_legal(g))
        return g.w <= 4 && !slots_repeat(g) ? kSlotGroup : kSlotGroupMid;
    if (slots_repeat(g))
        return 1;
    return g.w >= 5 && g.w <= 10 ? kSlotGroupMid : kSlotGroup;
}

// Positions per thread per pass.  The vector body moves 16 bytes per slot per
// position, and one position per thread keeps the most waves in flight (the
// measured best on MI355X); the scalar body moves 4 bytes per slot per
// position, so each thread takes four.
static int default_unroll(int path) { return path == DETFOLD_PATH_VECTOR ? 1 : 4; }

int check_override(const detfold_launch *o)
{
    if (!o)
        return DETFOLD_OK;
    if (o->path < DETFOLD_PATH_AUTO || o->path > DETFOLD_PATH_ROWS)
        return DETFOLD_EINVAL;
    if (o->block != 0 && (o->block < 64 || o->block > kMaxBlock || (o->block % 64) != 0))
        return DETFOLD_EINVAL;
    if (o->grid < 0 || o->grid > 0x7FFFFFFF)
        return DETFOLD_EINVAL;
    if (o->unroll != 0 && o->unroll != 1 && o->unroll != 2 && o->unroll != 4)
        return DETFOLD_EINVAL;
    if (o->policy < 0 || o->policy > DETFOLD_POLICY_CACHED)
        return DETFOLD_EINVAL;
    if (o->policy == DETFOLD_POLICY_CACHED && o->unroll > 1)
        return DETFOLD_EINVAL;  // the unhinted kernels exist with unroll 1 only
    if (o->group < 0 || o->group > kMaxGroup || (o->group & (o->group - 1)))
        return DETFOLD_EINVAL;  // 0 (the plan's choice) or a power of two up to kMaxGroup
    return DETFOLD_OK;
}

// Path and geometry for one call.
//  * Streaming policy, W >= 2: the LDS row body, one wave per slot
//    (block = 64*W), a tile of 64 * rows_kib_per_wave(W) groups per
//    workgroup, one pass; beyond 16 slots (stacked arenas) the wide row body,
//    16 waves making passes of 16 slots over tiles of 256 groups.
//  * Otherwise the direct bodies: vector when `out` and every slot share a
//    16-byte phase, else scalar; kStreamBlock threads, halved (down to 64)
//    while that would leave compute units without a workgroup; one pass.
// An override replaces any of path, block, grid, unroll and policy; a grid
// smaller than one pass makes the workgroups loop over the tiles.
int make_plan(const Geometry &g, int32_t cu_count, const detfold_launch *ovr, int policy,
              detfold_plan *p)
{
    if (cu_count < 1)
        return DETFOLD_EINVAL;
    int rc = check_override(ovr);
    if (rc != DETFOLD_OK)
        return rc;
    const detfold_launch o = ovr ? *ovr : detfold_launch{DETFOLD_PATH_AUTO, 0, 0, 0, 0, 0};
    if (o.policy)
        policy = o.policy;

    const bool vec_ok = vector_legal(g);
    const bool rows_ok = g.w >= 2 && (g.w <= kMaxRowsW || !g.has_table);
    if (g.has_table && g.w >= 2 && (o.path == DETFOLD_PATH_VECTOR || o.path == DETFOLD_PATH_SCALAR ||
                                    policy == DETFOLD_POLICY_CACHED))
        return DETFOLD_EINVAL;  // separate slot buffers have only the LDS row body
    int path = o.path;
    if (path == DETFOLD_PATH_AUTO) {
        if (rows_ok && policy == DETFOLD_POLICY_STREAM)
            path = DETFOLD_PATH_ROWS;
        else
            path = vec_ok ? DETFOLD_PATH_VECTOR : DETFOLD_PATH_SCALAR;
    }
    if (path == DETFOLD_PATH_VECTOR && !vec_ok)
        return DETFOLD_EINVAL;
    if (path == DETFOLD_PATH_ROWS &&
        (!rows_ok || policy == DETFOLD_POLICY_CACHED || (o.block && !rows_tile_for_block(g, o.block)) ||
         o.unroll > 1))
        return DETFOLD_EINVAL;

    p->path = path;
    p->policy = policy;
    if (path == DETFOLD_PATH_SCALAR) {
        p->head = 0;
        p->tail = 0;
        p->body = g.len;
    } else {
        int64_t head = (4 - phase16(g.out)) & 3;
        if (head > g.len)
            head = g.len;
        p->head = (int32_t)head;
        p->body = (g.len - head) >> 2;
        p->tail = (int32_t)((g.len - head) & 3);
    }
    p->group = 1;
    if (path == DETFOLD_PATH_ROWS) {
        p->unroll = 1;
        p->block = o.block ? o.block : rows_block(g);
        p->tile = rows_tile_for_block(g, p->block);
        p->group = o.group ? o.group : rows_group(g, p->block);
    } else {
        p->unroll = policy == DETFOLD_POLICY_CACHED ? 1 : (o.unroll ? o.unroll : default_unroll(path));
        int block = o.block;
        if (!block) {
            block = kStreamBlock;
            while (block > 64 &&
                   (p->body + (int64_t)block * p->unroll - 1) / ((int64_t)block * p->unroll) < cu_count)
                block >>= 1;
        }
        p->block = block;
        p->tile = (int64_t)p->block * p->unroll;
    }
    if (g.len == 0) {
        p->grid = 0;
        return DETFOLD_OK;
    }
    int64_t need = (p->body + p->tile - 1) / p->tile;
    if (need < 1)
        need = 1;  // a body of zero groups still needs threads for head and tail
    if (need > 0x7FFFFFFF)
        need = 0x7FFFFFFF;  // the workgroups loop over the rest
    p->grid = o.grid ? o.grid : need;
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


// The decode-join path (fold_into): up to kLatencyBytes per buffer, the
// unhinted direct body with one position per thread; above, streaming.
int plan_into(const Geometry &g, int32_t cu_count, detfold_plan *p)
{
    if (g.len * 4 <= kLatencyBytes) {
        const detfold_launch o = {DETFOLD_PATH_AUTO, 0, 0, 1, 0, 0};
        return make_plan(g, cu_count, &o, DETFOLD_POLICY_CACHED, p);
    }
    return make_plan(g, cu_count, nullptr, DETFOLD_POLICY_STREAM, p);
}

// ---------------------------------------------------------------------------
// Separate slot buffers (fold_slots) and the one-GPU rounds built on them

// out may be exactly one (or more) of the slots -- the fold then runs in place,
// every element read before it is written by the same workgroup -- but may not
// partly overlap any slot.
int check_slots_args(const float *out, const float *const *slots, int32_t W, int64_t len)
{
    if (W < 1 || W > kMaxRowsW || len < 0)
        return DETFOLD_EINVAL;
    if (len == 0)
        return DETFOLD_OK;
    if (!out || !slots || (((uintptr_t)out) & 3) || len > INT64_MAX / 4)
        return DETFOLD_EINVAL;
    for (int32_t r = 0; r < W; ++r) {
        if (!slots[r] || (((uintptr_t)slots[r]) & 3))
            return DETFOLD_EINVAL;
        if (slots[r] != out &&
            ranges_overlap((uintptr_t)out, (uint64_t)len * 4, (uintptr_t)slots[r], (uint64_t)len * 4))
            return DETFOLD_EOVERLAP;
    }
    return DETFOLD_OK;
}

Geometry slots_geometry(const float *out, const float *const *slots, int32_t W, int64_t len)
{
    Geometry g{(uintptr_t)out, (uintptr_t)slots[0], W >= 2 ? (uintptr_t)slots[1] : (uintptr_t)slots[0],
               0, W, len};
    g.has_table = true;
    for (int32_t r = 0; r < W; ++r)
        g.table[r] = (uintptr_t)slots[r];
    return g;
}

int balanced_shards(int64_t n, int32_t world, int64_t *start, int64_t *length)
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

int64_t job_pitch(const detfold_fold_job &j) { return j.pitch ? j.pitch : j.len; }

Geometry job_geometry(const detfold_fold_job &j, int32_t W)
{
    const int64_t pitch = job_pitch(j);
    return Geometry{(uintptr_t)j.out, (uintptr_t)j.stacked, (uintptr_t)j.stacked + (uintptr_t)pitch * 4, pitch, W,
                    j.len};
}

// The floats a job's arena spans: (W-1)*pitch + len, or -1 when that
// overflows the byte range an int64 can hold.
static int64_t job_span(const detfold_fold_job &j, int32_t W)
{
    const int64_t pitch = job_pitch(j);
    if (pitch > (INT64_MAX / 4 - j.len) / (W > 1 ? W - 1 : 1))
        return -1;
    return (int64_t)(W - 1) * pitch + j.len;
}

// Each job as fold_ranks checks it (its arena spanning (W-1)*pitch + len
// floats), and no job's output may touch another job's output or arena (the
// workgroups of one launch run in any order).
int check_batch_args(const detfold_fold_job *jobs, int32_t count, int32_t W)
{
    if (count < 0 || count > kMaxJobs || W < 1 || (count > 0 && !jobs))
        return DETFOLD_EINVAL;
    for (int32_t j = 0; j < count; ++j) {
        const detfold_fold_job &b = jobs[j];
        if (b.len < 0 || b.pitch < 0 || (b.pitch && b.pitch < b.len))
            return DETFOLD_EINVAL;
        if (b.len == 0)
            continue;
        if (!b.out || !b.stacked || (((uintptr_t)b.out) & 3) || (((uintptr_t)b.stacked) & 3))
            return DETFOLD_EINVAL;
        const int64_t span = job_span(b, W);
        if (span < 0)
            return DETFOLD_EINVAL;
        if (ranges_overlap((uintptr_t)b.out, (uint64_t)b.len * 4, (uintptr_t)b.stacked, (uint64_t)span * 4))
            return DETFOLD_EOVERLAP;
    }
    for (int32_t j = 0; j < count; ++j) {
        if (jobs[j].len == 0)
            continue;
        const uint64_t ob = (uint64_t)jobs[j].len * 4;
        for (int32_t k = 0; k < count; ++k) {
            if (k == j || jobs[k].len == 0)
                continue;
            if (ranges_overlap((uintptr_t)jobs[j].out, ob, (uintptr_t)jobs[k].out, (uint64_t)jobs[k].len * 4) ||
                ranges_overlap((uintptr_t)jobs[j].out, ob, (uintptr_t)jobs[k].stacked,
                               (uint64_t)job_span(jobs[k], W) * 4))
                return DETFOLD_EOVERLAP;
        }
    }
    return DETFOLD_OK;
}

// The shape is the one the longest job would get alone (every shape gives
// the same bits); each job takes ceil(groups / tile) workgroups, at least one
// (for its head and tail elements).
int plan_batch(const detfold_fold_job *jobs, int32_t count, int32_t W, int32_t cu_count,
               BatchArgs *a, detfold_plan *p)
{
    if (W < 2 || W > kMaxRowsW || cu_count < 1)
        return DETFOLD_EINVAL;
    *a = BatchArgs{};
    int32_t longest = -1;
    for (int32_t j = 0; j < count; ++j)
        if (jobs[j].len > 0 && (longest < 0 || jobs[j].len > jobs[longest].len))
            longest = j;
    *p = detfold_plan{};
    p->path = DETFOLD_PATH_ROWS;
    p->policy = DETFOLD_POLICY_STREAM;
    p->unroll = 1;
    p->group = 1;
    a->group = 1;
    if (longest < 0)
        return DETFOLD_OK;  // nothing to fold
    const Geometry lg = job_geometry(jobs[longest], W);
    p->block = rows_block(lg);
    p->tile = rows_tile(lg);
    p->group = rows_group(lg, p->block);
    a->group = p->group;
    int64_t tiles = 0;
    for (int32_t j = 0; j < count; ++j) {
        if (jobs[j].len == 0)
            continue;
        BatchJob &b = a->job[a->count++];
        b.out = jobs[j].out;
        b.s0 = jobs[j].stacked;
        b.len = jobs[j].len;
        b.pitch = job_pitch(jobs[j]);
        b.head = (4 - phase16((uintptr_t)jobs[j].out)) & 3;
        if (b.head > b.len)
            b.head = b.len;
        a->tile0[a->count - 1] = (int32_t)(tiles < 0x7FFFFFFF ? tiles : 0x7FFFFFFF);
        const int64_t groups = (b.len - b.head) >> 2;
        const int64_t t = (groups + p->tile - 1) / p->tile;
        tiles += t > 0 ? t : 1;
        p->body += groups;
    }
    if (tiles > 0x7FFFFFFF)
        return DETFOLD_EINVAL;
    p->grid = tiles;
    // every job the same number of tiles: the kernel divides instead of looking up
    const int64_t t0 = tiles / a->count;
    bool uniform = t0 * a->count == tiles;
    for (int32_t j = 0; uniform && j < a->count; ++j)
        uniform = a->tile0[j] == (int64_t)j * t0;
    a->uniform_tiles = uniform ? (int32_t)t0 : 0;
    a->uniform_magic = uniform ? (uint32_t)(0xFFFFFFFFull / (uint64_t)t0) : 0u;
    return DETFOLD_OK;
}

int check_round_args(float *const *arenas, int32_t W, int64_t n, const float *stage,
                     int64_t stage_elems, int32_t flags)
{
    constexpr int32_t known = DETFOLD_ROUND_REVERSE_DELIVERY | DETFOLD_ROUND_DIRECT | DETFOLD_ROUND_FUSED;
    if (W < 1 || W > kMaxRowsW || n < 0 || (flags & ~known) ||
        ((flags & DETFOLD_ROUND_FUSED) && flags != DETFOLD_ROUND_FUSED))
        return DETFOLD_EINVAL;
    if (W == 1 || n == 0)
        return DETFOLD_OK;
    if (!arenas || n > INT64_MAX / 4 / W)
        return DETFOLD_EINVAL;
    for (int32_t r = 0; r < W; ++r) {
        if (!arenas[r] || (((uintptr_t)arenas[r]) & 3))
            return DETFOLD_EINVAL;
        for (int32_t q = 0; q < r; ++q)
            if (ranges_overlap((uintptr_t)arenas[r], (uint64_t)n * 4, (uintptr_t)arenas[q], (uint64_t)n * 4))
                return DETFOLD_EOVERLAP;
    }
    if (!(flags & (DETFOLD_ROUND_DIRECT | DETFOLD_ROUND_FUSED))) {
        const int64_t need = (int64_t)W * ((n + W - 1) / W);
        if (!stage || (((uintptr_t)stage) & 3) || stage_elems < need)
            return DETFOLD_EINVAL;
        for (int32_t r = 0; r < W; ++r)
            if (ranges_overlap((uintptr_t)stage, (uint64_t)need * 4, (uintptr_t)arenas[r], (uint64_t)n * 4))
                return DETFOLD_EOVERLAP;
    }
    return DETFOLD_OK;
}

// ---------------------------------------------------------------------------
// Two ranks on one device: the pair link and the one-shot link

int check_pair_args(const detfold_pair_link *k, const float *x0, const float *x1, int64_t n)
{
    if (!k || n < 0 || n > k->capacity || !k->pushed[0] || !k->pushed[1] || !k->folded[0] ||
        !k->folded[1])
        return DETFOLD_EINVAL;
    if (n == 0)
        return DETFOLD_OK;
    const float *p[4] = {x0, x1, k->stage[0], k->stage[1]};
    for (int i = 0; i < 4; ++i) {
        if (!p[i] || (((uintptr_t)p[i]) & 3) || n > INT64_MAX / 4)
            return DETFOLD_EINVAL;
        for (int j = 0; j < i; ++j)
            if (ranges_overlap((uintptr_t)p[i], (uint64_t)n * 4, (uintptr_t)p[j], (uint64_t)n * 4))
                return DETFOLD_EOVERLAP;
    }
    return DETFOLD_OK;
}

int check_link_events(const detfold_pair_link *k)
{
    return k && k->pushed[0] && k->pushed[1] && k->folded[0] && k->folded[1] ? DETFOLD_OK
                                                                               : DETFOLD_EINVAL;
}

bool bad_buffer(const void *p, int64_t n)
{
    return !p || (((uintptr_t)p) & 3) || n > INT64_MAX / 8;
}

int check_one_shot_link(const detfold_one_shot_link *k)
{
    if (!k || !k->flags || !k->words || (((uintptr_t)k->flags) & 3) || (((uintptr_t)k->words) & 3) ||
        k->spin_limit < 0 || k->capacity < 0)
        return DETFOLD_EINVAL;
    if (ranges_overlap((uintptr_t)k->flags, DETFOLD_ONE_SHOT_FLAG_WORDS * 4, (uintptr_t)k->words, 8))
        return DETFOLD_EOVERLAP;
    return DETFOLD_OK;
}

// The buffers one launch touches: the ranks' x (one or both) and both stages.
int check_one_shot_buffers(const detfold_one_shot_link *k, const float *const *x, int nx, int64_t n)
{
    if (n < 0 || n > k->capacity)
        return DETFOLD_EINVAL;
    if (n == 0)
        return DETFOLD_OK;
    const float *p[4] = {k->stage[0], k->stage[1], x[0], nx > 1 ? x[1] : nullptr};
    const int np = 2 + nx;
    for (int i = 0; i < np; ++i) {
        if (bad_buffer(p[i], n))
            return DETFOLD_EINVAL;
        for (int j = 0; j < i; ++j)
            if (ranges_overlap((uintptr_t)p[i], (uint64_t)n * 4, (uintptr_t)p[j], (uint64_t)n * 4))
                return DETFOLD_EOVERLAP;
    }
    return DETFOLD_OK;
}

// The one-shot launch: nranks = 2 puts both ranks in one launch (workgroups
// [0, G) rank 0, [G, 2G) rank 1); nranks = 1 launches rank `rank0` alone.
// G = ceil(n / kOneShotPerBlock) capped at DETFOLD_ONE_SHOT_BLOCKS; each
// workgroup takes a chunk rounded up to 4 floats.
OneShotArgs one_shot_args(const detfold_one_shot_link *k, int32_t rank0, int nranks, float *xa,
                          float *xb, int64_t n)
{
    OneShotArgs a = {};
    int64_t blocks = (n + kOneShotPerBlock - 1) / kOneShotPerBlock;
    if (blocks > DETFOLD_ONE_SHOT_BLOCKS)
        blocks = DETFOLD_ONE_SHOT_BLOCKS;
    int64_t chunk = (n + blocks - 1) / blocks;
    chunk = (chunk + 3) & ~(int64_t)3;
    a.x[rank0] = xa;
    if (nranks == 2)
        a.x[1 - rank0] = xb;
    a.stage[0] = k->stage[0];
    a.stage[1] = k->stage[1];
    a.flags = k->flags;
    a.words = k->words;
    a.n = n;
    a.chunk = chunk;
    a.blocks = (int32_t)blocks;
    a.rank0 = rank0;
    a.spin_limit = k->spin_limit ? k->spin_limit : kDefaultSpinLimit;
    bool vec = true;
    for (int r = 0; r < 2; ++r)
        vec = vec && phase16((uintptr_t)a.stage[r]) == 0 && (!a.x[r] || phase16((uintptr_t)a.x[r]) == 0);
    a.vec = vec;
    return a;
}

}  // namespace detfold_impl
