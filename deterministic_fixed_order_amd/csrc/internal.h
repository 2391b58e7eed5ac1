// internal.h -- declarations shared by the translation units of libdetfold:
// fold_kernels.hip (device code and its launches), plan.cpp (host-only
// planning and argument checks) and detfold.cpp (device queries, call
// sequencing and the C ABI).  Not installed; the public interface is
// include/detfold.h.  Only the C ABI is exported from the library.
#ifndef DETFOLD_INTERNAL_H
#define DETFOLD_INTERNAL_H

#include <cstdint>

#include "detfold.h"

namespace detfold_impl {

constexpr int kMaxBlock = 1024;
constexpr int kXcds = 8;           // accelerator complex dies of an MI355X; workgroups go round-robin
constexpr int kMaxGroup = 64;      // largest XCD tile group a launch override may ask for
constexpr int kStreamBlock = 512;  // largest default workgroup of the bandwidth path
constexpr int kChunk = 8;          // slots loaded per batch when W is a runtime value
constexpr int kMaxRowsW = 16;      // widest fold the LDS row body takes (one wave per slot)
constexpr int kWideSlots = 16;     // slots per pass of the wide row body (W > kMaxRowsW)

// The measured notes below compare shapes within one interleaved sweep.  Unless
// a note says otherwise, those sweeps folded one arena into one output over
// and over; the memory-side cache then serves part of the traffic, so their
// absolute rates run 2-5% above what the same fold reaches with its operands
// out of that cache, while the comparisons they support were rechecked with
// the operands rotating.

// Shapes of a pass of the wide row body: 16 waves x 1 slot x 4 KiB, or, when
// every slot shares out's 16-byte phase, 8 waves x 2 slots x 1 KiB (measured
// on MI355X at W = 24..64: 2.6-21.5% faster co-aligned, 2.7-5.5% slower with
// shifted slots).  Shifted slots whose length in bytes is a multiple of
// kRepeatBytes take runs of 32 tiles per XCD, and the eight-wave shape too
// where the last pass holds at least eight slots: +12% to +20% at W = 32
// and 64 (W=32 x 2^22 at base+1: 5,370 -> 6,441 GB/s), +3% at W = 24; W = 17
// in the eight-wave shape lost 7.7% (its second pass is one slot).  6
// interleaved rounds each, bit-checked.  Shifted slots that do not repeat
// keep the sixteen-wave shape and take runs of kWideShiftedGroup tiles per
// XCD: +0.4% to +2.1% over plain round-robin at six arenas of W = 17..48,
// lengths 5e6 to 1.2e7, one to three elements off (6 interleaved rounds,
// outputs rotating past the memory-side cache, one arena, bit-checked);
// runs of 8 gained +0.3% to +2.1%, of 32 -0.4% to +2.0%.  With copies of
// the arena rotating as well the same six read -1.6% to +2.2% (+0.4% on
// average), so the rule rests as much on the traffic: the shared boundary
// lines of the 4 KiB runs are fetched once per XCD run instead of twice
// (W=32 x 8,000,001 at base+1: 1.030x -> 1.012x the algorithmic bytes).
constexpr int kWideWaves = 16, kWideKiB = 4;
constexpr int kWideAlignedWaves = 8, kWideAlignedKiB = 1;
constexpr int kWideShiftedGroup = 16;

// KiB of one slot each wave of the LDS row body streams per tile: ceil(W/4)
// for W >= 3, 8 for W = 2.  Measured on MI355X over W = 2..16 and 1/2/4/8 KiB
// per wave: with every CU holding 32 waves (32/W workgroups), ceil(W/4) KiB
// per wave keeps about 8 KiB of output tiles in flight per CU and was the
// fastest or within 2% of it at W = 3, 4, 5, 6, 8 and 16 (W = 8: 7.1 TB/s at
// 64 MiB per slot, against 6.4 TB/s at 8 KiB per wave).  Two-slot folds have
// only two waves per workgroup and want long runs instead.
constexpr int rows_kib_per_wave(int w)
{
    return w <= 2 ? 8 : (w + 3) / 4;
}

// Widths from five to sixteen have a second shape, in which each wave streams
// 1 KiB of up to two slots per tile (SPW = 2; rows_waves and rows_wave_lo
// below say which; the plan picks the shape, see rows_slots_per_wave).  The
// first measurements on MI355X, before XCD tile groups (the notes on
// kRepeatBytes say what changed with them):
//  * W = 8, two slots per wave (four waves): 1.5-12% faster wherever the slot
//    length is not a multiple of 2^24 floats, 0.8-1.4% slower where it is
//    (2^24, 2^25, 2^26), whose 64 MiB-aligned runs the one-slot shape suits;
//  * W = 16, two slots per wave (eight waves): when every slot shares out's
//    16-byte phase, 0.4-4.3% faster than four slots per wave (four waves) on
//    the stacked fold at six lengths, 1.4-6% on separate slots, 2-16% on the
//    fused round, and up to 30% faster than one slot per wave (16 waves x
//    4 KiB); with shifted slots and plain round-robin tiles one slot per
//    wave was best (several slots per wave lost 3-12%);
//  * W = 6, 10, 12, 14, every slot at out's phase: 3.7-15% faster than one
//    slot per wave at slot lengths of 6e6 to 1.26e7 (arenas beyond the
//    memory-side cache); with shifted slots and plain round-robin tiles it
//    lost up to 5% at W = 10 and 12.  W = 4 keeps one slot per wave: two
//    lose 6-8% at 2^24 and 1e8;
//  * odd W = 5, 7, 9, 11 at out's phase: 4-21% faster; 13 and 15: 0.2-5.6%;
//    W = 3 loses up to 3% and keeps one slot per wave.
// The shapes differ only in which wave loads which slot; every element's
// chain is the same.
constexpr int64_t kOneSlotAlign = (int64_t)1 << 24;  // floats; stacked slot lengths at this multiple

// Stacked arenas whose slot length in bytes is not a multiple of kRepeatBytes
// (16 MiB) -- their W slots sit at unrelated low address bits -- take, from
// three slots up, runs of kSlotGroup neighbouring tiles per XCD, and from
// nine slots up two slots per wave.  Measured on MI355X over 23 widths,
// lengths and alignments (8 interleaved rounds each, every variant
// bit-checked): +5% to +13% at every shifted arena of three to sixteen slots
// (W=16 x 10,000,019 at base+1 element: 6,126 -> 6,514 GB/s; W=8 x 10^7 at
// base+1: 5,845 -> 6,610), +2% to +10% on co-aligned arenas of such lengths
// (W=8 x 6,291,456: 6,615 -> 7,279), a tie at W=4 x 10^8.  Where the slot
// length is such a multiple (W=8 x 2^24, W=4 x 2^24, W=2 x 2^26) plain
// round-robin stays best: groups lose up to 8% (W=8), and groups of 2 or 4
// up to 35% at W=4.  At W=2 groups of 8 lose up to 2.5%, so two-slot folds
// keep plain round-robin.  Later sweeps (6 interleaved rounds each, every
// variant bit-checked) refined this:
//  * Co-aligned arenas of five to ten slots whose slots do not repeat take
//    runs of kSlotGroupMid tiles: +0.3% to +3.2% against runs of 8 over 11
//    arenas (W=8 x 3*10^7: 6,536 -> 6,745 GB/s), never a loss; from eleven
//    slots up runs of 32 tie or lose up to 1.9%.
//  * Shifted arenas (some slot off out's 16-byte phase) whose slot length is
//    a multiple of kRepeatBytes were a cliff under one slot per wave and
//    plain round-robin: 4.9-5.6 TB/s at slot lengths 2^22 to 3*2^22 for
//    W = 5..16.  Runs of 32 tiles per XCD, with two slots per wave from
//    seven slots up (eight slots excepted), measured +10% to +36% there
//    (W=16 x 2^22 at base+1: 4,950 -> 6,747 GB/s; W=9 x 3*2^22: +28%), +5%
//    at W=8 x 2^24 at base+1 and a tie at W=16 x 2^24.  Shifted arenas whose
//    slots do not repeat tie or gain up to 2.2% with runs of 32 against 8
//    (the W=16 x 10,000,019 arena at base+1: +0.1% to +0.4%), except at
//    three and four slots, which keep runs of 8 there (W=4 x 1e8 at base+1:
//    runs of 8 +2.6% over 32); shifted repeating arenas of three and four
//    slots take runs of 32 too (W=3 x 2^23 at base+2: +10% over 8; W=4 x
//    2^24 at base+1: +4.5% over plain round-robin).  Two-slot folds keep
//    plain round-robin everywhere (groups tie or lose up to 4.6%).
//  * Seven slots take two slots per wave on every stacked arena: one slot
//    per wave means seven-wave workgroups, 28 of a CU's 32 wave slots
//    (+3% to +6% at slot lengths 10^7 and 1.5*10^7).
//  * Separate slot buffers (fold_slots) shifted from out's phase take the
//    same shapes and groups as shifted stacked slots that do not repeat:
//    +3% to +21% at W = 4..16 on buffers of 2^22 and 10^7 floats (W=12 x
//    2^22 two elements off: 5,326 -> 6,422 GB/s; W=7: +18.8%), a tie at W=3,
//    -2.3% at W=16 x 2^24.  Co-aligned tables keep their shapes.
constexpr int64_t kRepeatBytes = (int64_t)1 << 24;
constexpr int kSlotGroup = 8;
constexpr int kSlotGroupMid = 32;
constexpr int rows_kib_per_wave(int w, int spw)
{
    return spw == 1 ? rows_kib_per_wave(w) : 1;
}

// Waves of the row body: w with one slot per wave; with two, ceil(w/2),
// except eight at thirteen and fourteen slots.  A CU holds 32 waves, so
// workgroups of seven waves fill only 28 of them (four workgroups); eight-wave
// workgroups fill all 32.  Measured on MI355X (6 interleaved rounds,
// bit-checked), eight waves against seven: +11% to +15% at W = 13 and 14,
// co-aligned and shifted (W=14 x 8e6: 5,961 -> 6,741 GB/s).
constexpr int rows_waves(int w, int spw)
{
    return spw == 2 && (w == 13 || w == 14) ? 8 : (w + spw - 1) / spw;
}

// Slots [rows_wave_lo(w, spw, q), rows_wave_lo(w, spw, q + 1)) are wave q's:
// the w slots in ascending runs over the waves, at most spw per wave (one or
// two each where there are more waves than ceil(w/spw)).
constexpr int rows_wave_lo(int w, int spw, int q) { return q * w / rows_waves(w, spw); }

// The slots per wave of a row-body workgroup of `waves` waves over w slots
// (the inverse of rows_waves for the shapes the plan makes).
constexpr int rows_spw(int w, int waves) { return (w + waves - 1) / waves; }

// Memory policy of a launch.
//  kStream  the bandwidth path: every input byte is read once and every
//           output byte written once, so loads and stores carry the
//           non-temporal hint.  With the output rotating through buffers
//           twice the size of the memory-side cache (every store reaches
//           HBM), non-temporal stores beat stores written through to system
//           scope (sc0 sc1) by 2.8-3.9% at W=8 x 2^24, 9% at W=16 x
//           10,000,019 at base+1, 14% on its owner shards in one launch,
//           4.5% at W=32, 4.9% at W=2, 2% on fold_into; write-back stores
//           lose 5-6% to both.
//  kCached  the decode-join path: no hints; its output is read again soon.
enum Policy : int { kCached = 0, kStream = 1 };

// The decode-join path: payloads up to kLatencyBytes per buffer are
// launch-latency bound and their result is read again soon, so they take one
// position per thread, one pass and no cache hints; larger payloads are
// bandwidth bound and stream.  Copies up to kCopyCachedBytes take no cache
// hints either (a decode-join push is read by the peer's fold right away).
constexpr int64_t kLatencyBytes = 8 << 20;
constexpr int64_t kCopyCachedBytes = 1 << 20;

// One-shot two-rank all-reduce: workgroup size, payload floats per workgroup
// before the DETFOLD_ONE_SHOT_BLOCKS cap, and the default poll limit of a
// barrier wait (about a second).
constexpr int kOneShotBlock = 256;
constexpr int64_t kOneShotPerBlock = 1024;
constexpr int32_t kDefaultSpinLimit = 1 << 20;

// Slot base pointers of the LDS row body, passed by value in the kernel
// arguments (slot r of a stacked arena is stacked + r*len; fold_slots takes
// them from the caller).  Also the destination list of the copy kernel.
struct SlotTable {
    const float *p[kMaxRowsW];
};

// Kernel arguments of the batched fold: the jobs with at least one element,
// in the caller's order; job j owns workgroups [tile0[j], tile0[j+1]).  The
// first workgroups of all jobs sit together at the front, so that a
// workgroup finds its job from a few wide scalar loads at fixed offsets
// rather than a chain of dependent ones.
constexpr int kMaxJobs = DETFOLD_MAX_JOBS;
struct BatchJob {
    float *out;
    const float *s0;  // slot 0; slot r at s0 + r*pitch
    int64_t len;
    int64_t pitch;    // floats between slot starts (>= len)
    int64_t head;     // elements before out's first 16-byte boundary
};
struct BatchArgs {
    int32_t tile0[kMaxJobs];  // each job's first workgroup (the grid is below 2^31)
    int32_t count;
    int32_t group;            // XCD tile group (xcd_tile) over the launch's workgroups
    float inv_w;
    // When every job has the same number of tiles T (balanced owner shards),
    // uniform_tiles = T and the job of workgroup b is b / T, computed as
    // q = (b * uniform_magic) >> 32 plus one correction step, with
    // uniform_magic = floor((2^32 - 1) / T); 0 = look the job up in tile0.
    int32_t uniform_tiles;
    uint32_t uniform_magic;
    BatchJob job[kMaxJobs];
};

// Kernel arguments of the one-shot all-reduce.
struct OneShotArgs {
    float *x[2];      // the ranks' partials, folded in place
    float *stage[2];  // stage[r]: where the peer's partial lands for rank r
    uint32_t *flags;  // [entry|exit][rank][DETFOLD_ONE_SHOT_BLOCKS] counters
    int32_t *words;   // per-rank barrier word
    int64_t n;
    int64_t chunk;    // floats per workgroup, a multiple of 4
    int32_t blocks;   // workgroups per rank
    int32_t rank0;    // rank of workgroups [0, blocks); a two-rank launch adds rank 1 after them
    int32_t spin_limit;
    int32_t vec;      // every buffer 16-byte aligned: 16-byte accesses
};

// The addresses and sizes one fold works on (host side, plain integers).
struct Geometry {
    uintptr_t out, s0, s1;  // byte addresses
    int64_t stride;         // elements between slots r and r+1 for r >= 1
    int32_t w;
    int64_t len;
    // Every slot's base address when the slots are not one stacked arena
    // (fold_slots); otherwise empty and derived from s0, s1 and stride.
    bool has_table = false;
    uintptr_t table[kMaxRowsW] = {};

    uintptr_t slot(int32_t r) const
    {
        if (has_table)
            return table[r];
        return r == 0 ? s0 : s1 + (uintptr_t)((r - 1) * stride) * 4;
    }
};

// Offset of an address modulo 16 bytes, in floats.
inline int phase16(uintptr_t a) { return (int)((a >> 2) & 3); }

// --- plan.cpp: host only, no device access ---------------------------------
bool vector_legal(const Geometry &g);
bool slots_repeat(const Geometry &g);
int rows_slots_per_wave(const Geometry &g);
int rows_block(const Geometry &g);
int64_t rows_tile(const Geometry &g);
int64_t rows_tile_for_block(const Geometry &g, int block);
int rows_group(const Geometry &g, int block);
int check_override(const detfold_launch *o);
int make_plan(const Geometry &g, int32_t cu_count, const detfold_launch *ovr, int policy,
              detfold_plan *p);
int plan_into(const Geometry &g, int32_t cu_count, detfold_plan *p);
bool ranges_overlap(uintptr_t a, uint64_t a_bytes, uintptr_t b, uint64_t b_bytes);
int check_ranks_args(const float *out, const float *stacked, int32_t W, int64_t len);
int check_into_args(const float *dst, const float *stage, int64_t n);
int check_slots_args(const float *out, const float *const *slots, int32_t W, int64_t len);
Geometry ranks_geometry(uintptr_t out, uintptr_t stacked, int32_t W, int64_t len);
Geometry into_geometry(uintptr_t dst, uintptr_t stage, int64_t n);
Geometry slots_geometry(const float *out, const float *const *slots, int32_t W, int64_t len);
int balanced_shards(int64_t n, int32_t world, int64_t *start, int64_t *length);
int check_batch_args(const detfold_fold_job *jobs, int32_t count, int32_t W);
// A batch job's slot pitch (its pitch, or len when 0) and its geometry.
int64_t job_pitch(const detfold_fold_job &j);
Geometry job_geometry(const detfold_fold_job &j, int32_t W);
// The batched fold's kernel arguments and plan (2 <= W <= 16, arguments
// checked): jobs without elements are dropped; a.count == 0 when none is left.
int plan_batch(const detfold_fold_job *jobs, int32_t count, int32_t W, int32_t cu_count,
               BatchArgs *a, detfold_plan *p);
int check_round_args(float *const *arenas, int32_t W, int64_t n, const float *stage,
                     int64_t stage_elems, int32_t flags);
int check_pair_args(const detfold_pair_link *k, const float *x0, const float *x1, int64_t n);
int check_link_events(const detfold_pair_link *k);
bool bad_buffer(const void *p, int64_t n);
int check_one_shot_link(const detfold_one_shot_link *k);
int check_one_shot_buffers(const detfold_one_shot_link *k, const float *const *x, int nx, int64_t n);
OneShotArgs one_shot_args(const detfold_one_shot_link *k, int32_t rank0, int nranks, float *xa,
                          float *xb, int64_t n);

// --- fold_kernels.hip: launches (hipStream_t and hipEvent_t passed as void*) -
// With `done`, the event is recorded by the dispatch itself when the kernel
// completes, with `begin` when it starts.  Each returns DETFOLD_OK or
// DETFOLD_ELAUNCH.
int launch_plan(const Geometry &g, const detfold_plan &p, bool scaled, float inv_w, void *stream,
                void *done = nullptr, void *begin = nullptr);
int launch_copy(float *const *dsts, int ndst, const float *src, int64_t len, int32_t cu,
                void *stream, void *done = nullptr);
// Every slot of a table geometry becomes the fold of all (the fused round);
// `p` is the plan make_plan gives that geometry.
int launch_rows_all(const Geometry &g, const detfold_plan &p, void *stream);
// The batched fold (k_fold_rows_batch); `p` from plan_batch.
int launch_batch(const BatchArgs &a, int32_t w, const detfold_plan &p, bool scaled, void *stream);
int launch_one_shot(const OneShotArgs &a, int nranks, void *stream);
// The current device's address of the library's static stage
// (DETFOLD_STATIC_STAGE_FLOATS floats), or DETFOLD_EDEVICE.
int static_stage(float **stage);
int launch_zero_words(uint32_t *p, int64_t n, void *stream);

}  // namespace detfold_impl

#endif  // DETFOLD_INTERNAL_H
