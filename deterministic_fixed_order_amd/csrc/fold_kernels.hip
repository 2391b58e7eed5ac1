// fold_kernels.hip -- the device code of the fixed-order fold for AMD Instinct
// MI355X (gfx950, CDNA4), and the launches that pick its instances.
//
// Operation (mamba-rs src/dist/reducer.rs: FixedOrder-contract module note,
// `det_sum_ranks`, `reduce_sum_reference`; memra-engine tests/tp_ar_gpu.rs:
// `memra_tp_ar_fold`): out[i] = (((s_0[i] + s_1[i]) + s_2[i]) + ...) + s_{W-1}[i],
// each "+" one binary32 add, round-to-nearest-even, subnormals kept.
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
//    element index lines them all up.  The LDS row bodies (W >= 2) still
//    moves 16-byte blocks: each wave's buffer descriptor starts at its own
//    slot's first element of the tile.  The direct bodies give each lane one
//    4-byte element per slot instead (a wave still reads 256 contiguous bytes
//    per slot).  Loads are pure data movement: the chain, and so the bits, is
//    the same on every body.
//  * A grid-stride loop lets any grid cover any length; the default grid is
//    sized from the device's compute-unit count.
//  * The fold kernels have no atomics, no flags and no waits on other work: a
//    launch completes on its own, whatever else is resident (the latency path
//    of fold_into relies on this).  The one-shot all-reduce kernel is the only
//    code that waits on another workgroup, and every one of its waits is
//    bounded by a poll count.
//  * Compiled with -ffp-contract=off, no fast-math, packed-FP32 instructions
//    disabled, and f32 denormals enabled (the HIP default on gfx9), so every
//    add is a single v_add_f32 under IEEE round-to-nearest-even.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "internal.h"

// The stage of detfold_loopback_round_static: device memory the library owns,
// one copy per device, held until the process ends.  Host code never uses
// this name as an address (on the host it is only a stand-in); it takes each
// device's address from hipGetSymbolAddress (static_stage below).
static __device__ __align__(256) float scratch[DETFOLD_STATIC_STAGE_FLOATS];

namespace detfold_impl {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned u4 __attribute__((ext_vector_type(4)));

// Cache-policy operand of the gfx950 buffer instructions: bit 0 = sc0,
// bit 1 = nt, bit 4 = sc1.
template <int POL> struct Aux {
    static constexpr int load = POL == kStream ? 2 : 0;   // nt
    static constexpr int store = POL == kStream ? 2 : 0;  // nt
};
// Written through to system scope (sc0 sc1): the fused round's stores of
// whole lines back into its arenas.
constexpr int kStoreThrough = 17;

// Raw buffer descriptor word 3 for gfx9-family parts (32-bit data format,
// no swizzle); the range check is num_records in bytes.
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kRsrcWord3);
}

template <int AUX> __device__ __forceinline__ void bload(f4 &v, __amdgpu_buffer_rsrc_t rs, uint32_t off)
{
    v = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, AUX));
}
template <int AUX> __device__ __forceinline__ void bload(float &v, __amdgpu_buffer_rsrc_t rs, uint32_t off)
{
    v = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, AUX));
}
template <int AUX> __device__ __forceinline__ void bstore(f4 v, __amdgpu_buffer_rsrc_t rs, uint32_t off)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), rs, off, 0, AUX);
}
template <int AUX> __device__ __forceinline__ void bstore(float v, __amdgpu_buffer_rsrc_t rs, uint32_t off)
{
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), rs, off, 0, AUX);
}


// ---------------------------------------------------------------------------
// Device side

// One tile of `cnt` positions (16-byte groups or single elements, T) starting
// at position `start` of `out` and of every slot; slot 0 is s0, slot r >= 1 is
// s1 + (r-1)*stride.  Thread tid owns positions tid + u*B for u < U.  Every
// slot is read through a buffer descriptor based at the tile's start, so the
// per-lane offsets are 32-bit however large the arena is.  GUARD: a partial
// (last) tile, whose positions are checked against cnt.
template <int WS, int U, typename T, bool SCALED, int POL, bool GUARD>
__device__ __forceinline__ void fold_tile(T *out, const T *s0, const T *s1, int64_t stride, int w,
                                          int64_t start, int64_t cnt, float inv_w)
{
    const uint32_t B = blockDim.x;
    const uint32_t bytes = (uint32_t)(cnt * (int64_t)sizeof(T));
    uint32_t off[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t p = threadIdx.x + (uint32_t)u * B;
        off[u] = p * (uint32_t)sizeof(T);
        ok[u] = !GUARD || (int64_t)p < cnt;
    }
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(out + start, bytes);
    if constexpr (WS > 0) {
        T v[U][WS];
        const __amdgpu_buffer_rsrc_t r0 = make_rsrc(s0 + start, bytes);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (ok[u])
                bload<Aux<POL>::load>(v[u][0], r0, off[u]);
#pragma unroll
        for (int r = 1; r < WS; ++r) {
            const __amdgpu_buffer_rsrc_t rr = make_rsrc(s1 + (int64_t)(r - 1) * stride + start, bytes);
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (ok[u])
                    bload<Aux<POL>::load>(v[u][r], rr, off[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (!ok[u])
                continue;
            T acc = v[u][0];
#pragma unroll
            for (int r = 1; r < WS; ++r)
                acc = acc + v[u][r];  // ascending slot order, one rounding per add
            if constexpr (SCALED)
                acc = acc * inv_w;  // one rounding of the finished sum
            bstore<Aux<POL>::store>(acc, ro, off[u]);
        }
    } else {
        T acc[U];
        const __amdgpu_buffer_rsrc_t r0 = make_rsrc(s0 + start, bytes);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (ok[u])
                bload<Aux<POL>::load>(acc[u], r0, off[u]);
        for (int r0i = 1; r0i < w; r0i += kChunk) {
            T v[U][kChunk];
#pragma unroll
            for (int k = 0; k < kChunk; ++k) {
                if (r0i + k < w) {
                    const __amdgpu_buffer_rsrc_t rr =
                        make_rsrc(s1 + (int64_t)(r0i + k - 1) * stride + start, bytes);
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        if (ok[u])
                            bload<Aux<POL>::load>(v[u][k], rr, off[u]);
                }
            }
#pragma unroll
            for (int k = 0; k < kChunk; ++k)
                if (r0i + k < w)
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        if (ok[u])
                            acc[u] = acc[u] + v[u][k];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (!ok[u])
                continue;
            T a = acc[u];
            if constexpr (SCALED)
                a = a * inv_w;
            bstore<Aux<POL>::store>(a, ro, off[u]);
        }
    }
}

// Tiles of B*U positions over [0, n); block b takes tiles b, b + grid, ...
// With the default one-pass grid every block takes exactly one tile.
template <int WS, int U, typename T, bool SCALED, int POL>
__device__ __forceinline__ void fold_tiles(T *out, const T *s0, const T *s1, int64_t stride, int w,
                                           int64_t n, float inv_w)
{
    const int64_t tile = (int64_t)blockDim.x * U;
    for (int64_t start = (int64_t)blockIdx.x * tile; start < n; start += (int64_t)gridDim.x * tile) {
        if (n - start >= tile)
            fold_tile<WS, U, T, SCALED, POL, false>(out, s0, s1, stride, w, start, tile, inv_w);
        else
            fold_tile<WS, U, T, SCALED, POL, true>(out, s0, s1, stride, w, start, n - start, inv_w);
    }
}

// A single element with plain loads: the head and tail of the vector body.
template <int WS, bool SCALED>
__device__ __forceinline__ void fold_one(float *out, const float *s0, const float *s1,
                                         int64_t stride, int w, int64_t i, float inv_w)
{
    const int nw = WS > 0 ? WS : w;
    float acc = s0[i];
    for (int r = 1; r < nw; ++r)
        acc = acc + s1[(int64_t)(r - 1) * stride + i];
    if constexpr (SCALED)
        acc = acc * inv_w;
    out[i] = acc;
}

// Vector body: elements [head, head + 4*groups) as 16-byte groups; the up to 3
// elements before (head) and after (tail) are folded one by one by the first
// threads of the grid.
template <int WS, int U, bool SCALED, int POL>
__global__ __launch_bounds__(kMaxBlock) void k_fold_vector(float *out, const float *s0,
                                                           const float *s1, int64_t stride, int w,
                                                           int64_t len, int64_t head, float inv_w)
{
    const int64_t groups = (len - head) >> 2;
    const int64_t tail0 = head + (groups << 2);
    const int64_t edges = head + (len - tail0);
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid < edges)
        fold_one<WS, SCALED>(out, s0, s1, stride, w, gid < head ? gid : tail0 + (gid - head), inv_w);
    fold_tiles<WS, U, f4, SCALED, POL>(reinterpret_cast<f4 *>(out + head),
                                       reinterpret_cast<const f4 *>(s0 + head),
                                       reinterpret_cast<const f4 *>(s1 + head), stride >> 2, w,
                                       groups, inv_w);
}

// Scalar body: every element with 4-byte loads (slots at mixed 16-byte phases).
template <int WS, int U, bool SCALED, int POL>
__global__ __launch_bounds__(kMaxBlock) void k_fold_scalar(float *out, const float *s0,
                                                           const float *s1, int64_t stride, int w,
                                                           int64_t len, float inv_w)
{
    fold_tiles<WS, U, float, SCALED, POL>(out, s0, s1, stride, w, len, inv_w);
}

// LDS row-transpose body (2 <= W <= 16).  One workgroup of rows_waves(W, SPW)
// waves folds a tile of T 16-byte groups of `out`: wave q streams the tile's
// bytes of its slots (a run of at most SPW consecutive slots, rows_wave_lo)
// -- LPW consecutive KiB of each, one contiguous run per slot -- straight into
// LDS rows (buffer loads with the lds bit, no register staging); after a
// barrier every thread folds whole groups from the W rows, in ascending row
// order, and stores them.  SPW is 1 or 2 (up to two slots of 1 KiB per wave;
// the plan's rows_slots_per_wave picks).
// Streaming whole runs of a slot keeps each wave on few runs of HBM rows; the
// direct body instead has every wave touch W runs 1 KiB at a time, which
// measured 3-8% slower on MI355X.
//
// Slot phases: the tile of `out` starts 16-byte aligned, but slot r's bytes
// for the tile may start at any dword.  The buffer descriptor of slot r is
// based at exactly that dword (gfx9 buffer loads need only dword alignment), so every
// row lands in LDS aligned to the tile whatever the slot's phase, and the
// fold reads 16-byte groups from every row alike.  The descriptor's range is
// the tile's bytes of the slot, so no lane reads past them.  Measured on
// MI355X against realigning shifted rows in LDS (one extra KiB loaded per
// wave, 4-byte LDS reads): +3% at W=16 x 10,000,019 at base+1, +10% at W=7,
// no change when every slot is aligned.
template <int W, int SPW> struct RowsShape {
    static constexpr int LPW = rows_kib_per_wave(W, SPW);  // KiB of each slot a wave streams per tile
    static constexpr int T = LPW * 64;                     // 16-byte groups per tile
    static constexpr int WAVES = rows_waves(W, SPW);       // wave q streams its run of slots (rows_wave_lo)
};

typedef __attribute__((address_space(3))) void lds_void;

// Where slot r starts: a table of base pointers passed in the kernel
// arguments, or, for the batched fold, base + r*pitch computed in scalar
// registers (a table built in the kernel would live in private memory).
struct TableSlots {
    const SlotTable &t;
    __device__ const float *operator()(int r) const { return t.p[r]; }
};
struct StrideSlots {
    const float *s0;
    int64_t pitch;
    __device__ const float *operator()(int r) const { return s0 + (int64_t)r * pitch; }
};

template <int W, bool SCALED, typename Slots>
__device__ __forceinline__ void fold_one_table(float *out, const Slots &slot, int64_t i, float inv_w)
{
    float acc = slot(0)[i];
#pragma unroll
    for (int r = 1; r < W; ++r)
        acc = acc + slot(r)[i];
    if constexpr (SCALED)
        acc = acc * inv_w;
    out[i] = acc;
}

// Wave `wave` streams the tile's bytes of its slots (its run of at most SPW,
// rows_wave_lo) into their LDS rows: LPW KiB of each, through a descriptor
// based at the slot's element e0 and limited to the tile's cnt groups.
template <int W, int SPW, int LPW, int T, typename Slots>
__device__ __forceinline__ void stream_rows(f4 (&rows)[W][T], const Slots &slot, int64_t e0,
                                            int64_t cnt, uint32_t wave, uint32_t lane)
{
    const uint32_t lo = (uint32_t)rows_wave_lo(W, SPW, (int)wave);
    const uint32_t hi = (uint32_t)rows_wave_lo(W, SPW, (int)wave + 1);
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
        const uint32_t r = lo + (uint32_t)j;
        if (r >= hi)
            break;  // this wave has fewer slots
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(slot(r) + e0, (uint32_t)(cnt * 16));
#pragma unroll
        for (int u = 0; u < LPW; ++u)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)&rows[r][u * 64], 16,
                                                     (uint32_t)(u * 64 + lane) * 16u, 0, 0,
                                                     Aux<kStream>::load);
    }
}

// The tile workgroup b folds when each XCD is to take runs of `group`
// neighbouring tiles.  Workgroups go to the 8 XCDs round-robin (b mod 8), so
// within each block of 8*group workgroups XCD x gets tiles x*group ..
// x*group+group-1; a last, partial block keeps b.  A 16-byte run of a slot
// that does not start on a 128-byte line shares its first and last line with
// the neighbouring tiles' runs; on one XCD that line is fetched once into its
// L2, across XCDs once per XCD.  Any group gives a permutation of the tiles,
// so the bits never depend on it.  group is a power of two (the plan and the
// override check see to it), so the index arithmetic is shifts and masks.
__device__ __forceinline__ int64_t xcd_tile(int64_t b, int64_t ntiles, int group)
{
    static_assert(kXcds == 8, "three bits of XCD index");
    if (group <= 1)
        return b;
    const int lg = __builtin_ctz((unsigned)group);
    const int64_t span = (int64_t)kXcds << lg;
    if (b >= (ntiles & ~(span - 1)))
        return b;
    const int64_t r = b & (span - 1);
    return b - r + ((r & (kXcds - 1)) << lg) + (r >> 3);
}

// One tile of the row body: the W slots' bytes for groups [tile*T, tile*T+cnt)
// of `out` streamed into the rows, then every thread folds whole groups in
// ascending row order and stores them.  Every thread of the workgroup calls
// it (it holds two barriers); a tile at or past `groups` does nothing.
template <int W, int SPW, bool SCALED, int T, typename Slots>
__device__ __forceinline__ void rows_tile(f4 (&rows)[W][T], float *out, const Slots &slots,
                                          int64_t groups, int64_t head, int64_t tile, float inv_w,
                                          uint32_t wave, uint32_t lane)
{
    constexpr int LPW = RowsShape<W, SPW>::LPW;
    static_assert(T == RowsShape<W, SPW>::T, "the rows hold one tile");
    constexpr int NT = RowsShape<W, SPW>::WAVES * 64;  // threads per workgroup
    const int64_t g0 = tile * T;
    if (g0 >= groups)
        return;
    const int64_t cnt = groups - g0 < T ? groups - g0 : T;
    const int64_t e0 = head + 4 * g0;  // first element of the tile; out + e0 is 16-byte aligned
    stream_rows<W, SPW, LPW, T>(rows, slots, e0, cnt, wave, lane);
    __syncthreads();  // every row has landed

    const __amdgpu_buffer_rsrc_t ro = make_rsrc(out + e0, (uint32_t)(cnt * 16));
    for (uint32_t t = threadIdx.x; t < (uint32_t)cnt; t += NT) {
        f4 acc = rows[0][t];
#pragma unroll
        for (int q = 1; q < W; ++q)
            acc = acc + rows[q][t];  // ascending slot order, one rounding per add
        if constexpr (SCALED)
            acc = acc * inv_w;  // one rounding of the finished sum
        bstore<Aux<kStream>::store>(acc, ro, t * 16u);
    }
    __syncthreads();  // the rows are refilled only after every thread has read them
}

// The up to 3 elements before out's first 16-byte boundary (head) and after
// its last (tail), one per thread: thread `k` < head + tail folds one.
template <int W, bool SCALED, typename Slots>
__device__ __forceinline__ void rows_edges(float *out, const Slots &slots, int64_t len, int64_t head,
                                           int64_t k, float inv_w)
{
    const int64_t groups = (len - head) >> 2;
    const int64_t tail0 = head + (groups << 2);
    if (k < head + (len - tail0))
        fold_one_table<W, SCALED>(out, slots, k < head ? k : tail0 + (k - head), inv_w);
}

template <int W, int SPW, bool SCALED>
__global__ __launch_bounds__(rows_waves(W, SPW) * 64) void k_fold_rows(float *out, SlotTable slots, int64_t len,
                                                            int64_t head, float inv_w, int group)
{
    constexpr int T = RowsShape<W, SPW>::T;
    __shared__ f4 rows[W][T];
    const TableSlots slot{slots};
    rows_edges<W, SCALED>(out, slot, len, head, (int64_t)blockIdx.x * blockDim.x + threadIdx.x, inv_w);
    const int64_t groups = (len - head) >> 2;
    const int64_t ntiles = (groups + T - 1) / T;
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if ((int64_t)gridDim.x == ntiles) {  // one pass: one tile per workgroup
        rows_tile<W, SPW, SCALED, T>(rows, out, slot, groups, head, xcd_tile(blockIdx.x, ntiles, group), inv_w,
                                     wave, lane);
        return;
    }
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x)
        rows_tile<W, SPW, SCALED, T>(rows, out, slot, groups, head, tile, inv_w, wave, lane);
}

// Many stacked folds of one width in one launch (fold_ranks_batch): job j
// owns workgroups [tile0_j, tile0_{j+1}), one tile each, and its first
// workgroup also folds the job's head and tail elements.  Within a job
// everything is k_fold_rows's, so every element's chain is the same.
template <int W, int SPW, bool SCALED>
__global__ __launch_bounds__(rows_waves(W, SPW) * 64) void k_fold_rows_batch(BatchArgs a)
{
    constexpr int T = RowsShape<W, SPW>::T;
    __shared__ f4 rows[W][T];
    // the grid is below 2^31 workgroups (the plan sees to it): 32-bit scalar compares
    const int32_t b = (int32_t)xcd_tile(blockIdx.x, gridDim.x, a.group);
    int j = 0;  // the last job that starts at or before workgroup b
    if (a.uniform_tiles > 0) {  // b / T by multiply-high and one correction step
        uint32_t q = __umulhi((uint32_t)b, a.uniform_magic);
        if ((uint32_t)b - q * (uint32_t)a.uniform_tiles >= (uint32_t)a.uniform_tiles)
            ++q;
        j = (int)q;
    } else {
#pragma unroll
        for (int k = 1; k < kMaxJobs; ++k)
            if (k < a.count && b >= a.tile0[k])
                j = k;
    }
    float *const out = a.job[j].out;
    const int64_t len = a.job[j].len, head = a.job[j].head;
    const StrideSlots slots{a.job[j].s0, a.job[j].pitch};
    const int64_t tile = (int64_t)(b - a.tile0[j]);
    if (tile == 0)
        rows_edges<W, SCALED>(out, slots, len, head, threadIdx.x, a.inv_w);
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    rows_tile<W, SPW, SCALED, T>(rows, out, slots, (len - head) >> 2, head, tile, a.inv_w, wave, lane);
}

// Fold and write back (the fused one-device round, W <= 16 separate
// buffers): every slot ends holding the fold of all.  The loads are the row
// body's; then each thread that owns a group folds it in ascending row order
// and leaves the sum in row 0, and after a second barrier wave q writes the
// tile of row 0 into the slots it loaded (rows_wave_lo), through a descriptor
// based at each slot's first element of the tile as its loads were, so any
// 16-byte phase works.  A workgroup has read its tile of every slot (first
// barrier) before it writes any of them, and workgroups own disjoint tiles;
// the head and tail elements are read, folded and written back by one thread
// each.  Every byte of every slot is read once and written once.
//
// With a one-pass grid the tiles go to the XCDs in runs of `group`
// (xcd_tile).  A slot's run that does not start on a 128-byte line shares
// its first and last line with the neighbouring tiles' runs of that slot, and
// those partial lines are written back through the L2 (no write-through) so
// that the neighbours' halves can meet there; runs on whole lines are
// written through (sc0 sc1).  Measured on MI355X (5 interleaved rounds,
// bit-checked) against write-through everywhere: +18% at W=8 x 10^7 with
// every arena one element off a line, +29% with the arenas at four different
// 16-byte phases, +4.5-5% at W=16; line-aligned arenas unchanged (write-back
// stores there lose 6-8%).  The non-temporal stores of the other stream
// kernels lose 1.1% here against write-through (W=8 x 2^24, line-aligned):
// the round writes back into the arenas it has just read.
template <int W, int SPW>
__global__ __launch_bounds__(rows_waves(W, SPW) * 64) void k_fold_rows_all(SlotTable slots, int64_t len,
                                                                int64_t head, int group)
{
    constexpr int LPW = RowsShape<W, SPW>::LPW, T = RowsShape<W, SPW>::T;
    constexpr int NT = RowsShape<W, SPW>::WAVES * 64;  // threads per workgroup
    __shared__ f4 rows[W][T];

    const int64_t groups = (len - head) >> 2;
    const int64_t tail0 = head + (groups << 2);
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid < head + (len - tail0)) {
        const int64_t i = gid < head ? gid : tail0 + (gid - head);
        float acc = slots.p[0][i];
#pragma unroll
        for (int r = 1; r < W; ++r)
            acc = acc + slots.p[r][i];
#pragma unroll
        for (int r = 0; r < W; ++r)
            const_cast<float *>(slots.p[r])[i] = acc;
    }

    const uint32_t lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t ntiles = (groups + T - 1) / T;
    const bool one_pass = (int64_t)gridDim.x == ntiles;
    for (int64_t b = blockIdx.x; b < ntiles; b += gridDim.x) {
        const int64_t tile = one_pass ? xcd_tile(b, ntiles, group) : b;
        const int64_t g0 = tile * T;
        const int64_t cnt = groups - g0 < T ? groups - g0 : T;
        const int64_t e0 = head + 4 * g0;
        stream_rows<W, SPW, LPW, T>(rows, TableSlots{slots}, e0, cnt, wave, lane);
        __syncthreads();  // every row has landed

        for (uint32_t t = threadIdx.x; t < (uint32_t)cnt; t += NT) {
            f4 acc = rows[0][t];
#pragma unroll
            for (int q = 1; q < W; ++q)
                acc = acc + rows[q][t];  // ascending slot order, one rounding per add
            rows[0][t] = acc;
        }
        __syncthreads();  // the sums are in row 0

        const uint32_t lo = (uint32_t)rows_wave_lo(W, SPW, (int)wave);
        const uint32_t hi = (uint32_t)rows_wave_lo(W, SPW, (int)wave + 1);
#pragma unroll
        for (int j = 0; j < SPW; ++j) {
            const uint32_t r = lo + (uint32_t)j;
            if (r >= hi)
                break;  // this wave has fewer slots
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(slots.p[r] + e0, (uint32_t)(cnt * 16));
            const bool on_line = ((uintptr_t)(slots.p[r] + e0) & 127) == 0;  // uniform per wave
#pragma unroll
            for (int u = 0; u < LPW; ++u) {
                const uint32_t g = (uint32_t)(u * 64) + lane;
                if (g < (uint32_t)cnt) {
                    if (on_line)
                        bstore<kStoreThrough>(rows[0][g], rs, g * 16u);
                    else
                        bstore<Aux<kCached>::store>(rows[0][g], rs, g * 16u);
                }
            }
        }
        __syncthreads();  // row 0 is read before the next tile refills the rows
    }
}

// Wide LDS row body (W > 16, stacked arena): a workgroup of WAVES waves folds
// a tile of KIB*64 groups in passes of 16 slots.  In pass p wave q streams KIB
// KiB of each of its SPW slots 16p + q*SPW + j into LDS row q*SPW + j, as the
// row body above does; after the barrier the thread that owns group t
// continues its chain with rows 0, 1, ... of the pass -- pass 0 starts it
// from slot 0 -- and a second barrier frees the rows for the next pass.  The
// running sum stays in the thread's registers between passes, so each element
// still sees the adds in strictly ascending slot order, one rounding each,
// and is stored once at the end.
// With a one-pass grid the tiles go to the XCDs in runs of `group` (xcd_tile).
template <int WAVES, int SPW, int KIB, bool SCALED>
__global__ __launch_bounds__(WAVES * 64) void k_fold_rows_wide(float *out, const float *s0,
                                                               const float *s1, int64_t stride, int w,
                                                               int64_t len, int64_t head, float inv_w,
                                                               int group)
{
    constexpr int T = KIB * 64;  // groups per tile, at most one per thread
    static_assert(T <= WAVES * 64, "one group per thread");
    static_assert(WAVES * SPW == kWideSlots, "a pass is 16 slots");
    __shared__ f4 rows[kWideSlots][T];

    const int64_t groups = (len - head) >> 2;
    const int64_t tail0 = head + (groups << 2);
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid < head + (len - tail0))
        fold_one<0, SCALED>(out, s0, s1, stride, w, gid < head ? gid : tail0 + (gid - head), inv_w);

    const uint32_t lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const uint32_t t = threadIdx.x;
    const int64_t ntiles = (groups + T - 1) / T;
    const bool one_pass = (int64_t)gridDim.x == ntiles;
    for (int64_t b = blockIdx.x; b < ntiles; b += gridDim.x) {
        const int64_t tile = one_pass ? xcd_tile(b, ntiles, group) : b;
        const int64_t g0 = tile * T;
        const int64_t cnt = groups - g0 < T ? groups - g0 : T;
        const int64_t e0 = head + 4 * g0;
        f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int base = 0; base < w; base += kWideSlots) {
            const int nr = w - base < kWideSlots ? w - base : kWideSlots;
#pragma unroll
            for (int j = 0; j < SPW; ++j) {  // this wave's slots of the pass
                const int q = wave * SPW + j;
                if (q < nr) {
                    const int r = base + q;
                    const float *slot = r == 0 ? s0 : s1 + (int64_t)(r - 1) * stride;
                    const __amdgpu_buffer_rsrc_t rs = make_rsrc(slot + e0, (uint32_t)(cnt * 16));
#pragma unroll
                    for (int u = 0; u < KIB; ++u)
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)&rows[q][u * 64], 16,
                                                                 (uint32_t)(u * 64 + lane) * 16u, 0, 0,
                                                                 Aux<kStream>::load);
                }
            }
            __syncthreads();  // this pass's rows have landed
            if (t < (uint32_t)cnt) {
                int q = 0;
                if (base == 0) {
                    acc = rows[0][t];  // the chain starts from slot 0 itself
                    q = 1;
                }
                // rows are read four at a time so the LDS reads overlap; the
                // adds still take slot base + q in ascending order
                for (; q + 4 <= nr; q += 4) {
                    const f4 a0 = rows[q][t], a1 = rows[q + 1][t], a2 = rows[q + 2][t], a3 = rows[q + 3][t];
                    acc = acc + a0;
                    acc = acc + a1;
                    acc = acc + a2;
                    acc = acc + a3;
                }
                for (; q < nr; ++q)
                    acc = acc + rows[q][t];
            }
            __syncthreads();  // every thread has read the rows before they are refilled
        }
        if (t < (uint32_t)cnt) {
            if constexpr (SCALED)
                acc = acc * inv_w;  // one rounding of the finished sum
            bstore<Aux<kStream>::store>(acc, make_rsrc(out + e0, (uint32_t)(cnt * 16)), t * 16u);
        }
    }
}

// Byte movement for the one-device rounds: copy `n` floats from `src` into
// every one of `ndst` destinations (src read once).  VEC: src and every
// destination share one 16-byte phase -- 16-byte groups after `head` scalar
// elements, `tail` after them; otherwise one 4-byte element per thread.  No
// arithmetic touches the data.
template <bool VEC, int POL>
__global__ __launch_bounds__(kMaxBlock) void k_copy_out(SlotTable dsts, int ndst, const float *src,
                                                        int64_t n, int64_t head)
{
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
    if constexpr (VEC) {
        const int64_t groups = (n - head) >> 2;
        const int64_t tail0 = head + (groups << 2);
        if (gid < head + (n - tail0)) {
            const int64_t i = gid < head ? gid : tail0 + (gid - head);
            const float v = src[i];
            for (int d = 0; d < ndst; ++d)
                const_cast<float *>(dsts.p[d])[i] = v;
        }
        const f4 *s4 = reinterpret_cast<const f4 *>(src + head);
        for (int64_t g = gid; g < groups; g += nthreads) {
            f4 v;
            if constexpr (POL == kStream)
                v = __builtin_nontemporal_load(s4 + g);
            else
                v = s4[g];
            for (int d = 0; d < ndst; ++d) {
                f4 *d4 = reinterpret_cast<f4 *>(const_cast<float *>(dsts.p[d]) + head) + g;
                if constexpr (POL == kStream)
                    __builtin_nontemporal_store(v, d4);
                else
                    *d4 = v;
            }
        }
    } else {
        for (int64_t i = gid; i < n; i += nthreads) {
            const float v = src[i];
            for (int d = 0; d < ndst; ++d)
                const_cast<float *>(dsts.p[d])[i] = v;
        }
    }
}

// ---------------------------------------------------------------------------
// One-shot two-rank all-reduce (memra-engine tests/tp_ar_gpu.rs, the one-shot
// arm: one kernel per rank, an in-kernel barrier with entry and exit refusal
// words, repeat calls on the same link).
//
// Workgroup b of rank r owns chunk b of the payload and pairs with workgroup b
// of the peer; the two meet through four counters per pair (entry and exit,
// one per rank).  A workgroup arrives by incrementing its own counter and
// waits until the peer's counter has caught up with the value it produced.
// Neither side can run a whole call ahead: the peer's next arrival at entry
// follows its exit wait, which needs this side's exit arrival.  Counters only
// ever grow, so a call needs no epoch from the host and a graph replay of a
// captured call is a fresh call.

// Poll *f (agent scope, acquire) until it reaches `target`, at most `limit`
// times.  Signed distance, so the comparison survives counter wrap.
__device__ bool await_count(const uint32_t *f, uint32_t target, int32_t limit)
{
    for (int32_t i = 0; i < limit; ++i) {
        const uint32_t v = __hip_atomic_load(f, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
        if ((int32_t)(v - target) >= 0)
            return true;
        __builtin_amdgcn_s_sleep(4);
    }
    return false;
}

// Arrive at a barrier: bump this workgroup's counter with an agent-scope
// release, which writes the L2 back before the increment lands, so the
// workgroup's stores (ordered before it by the caller's __syncthreads) are
// visible to the peer's acquire on any XCD.  Returns the count produced.
__device__ uint32_t arrive(uint32_t *f)
{
    return __hip_atomic_fetch_add(f, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT) + 1u;
}

// Keep the first refusal word stored for a rank.
__device__ void refuse(int32_t *word, int32_t code)
{
    int32_t expected = 0;
    __hip_atomic_compare_exchange_strong(word, &expected, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(kOneShotBlock) void k_one_shot(OneShotArgs a)
{
    __shared__ int passed;
    const int32_t rank = a.rank0 + (int32_t)blockIdx.x / a.blocks;
    const int32_t b = (int32_t)blockIdx.x % a.blocks;
    const int32_t peer = 1 - rank;
    uint32_t *const entry = a.flags;
    uint32_t *const exit = a.flags + 2 * DETFOLD_ONE_SHOT_BLOCKS;
    const int64_t lo = (int64_t)b * a.chunk;
    const int64_t hi = lo + a.chunk < a.n ? lo + a.chunk : a.n;
    const int64_t len = hi > lo ? hi - lo : 0;
    float *const x = a.x[rank] + lo;
    float *const push = a.stage[peer] + lo;
    const float *const mine = a.stage[rank] + lo;
    const int64_t groups = a.vec ? len >> 2 : 0;

    // 1. this rank's chunk goes to the peer's staging buffer
    for (int64_t g = threadIdx.x; g < groups; g += kOneShotBlock)
        reinterpret_cast<f4 *>(push)[g] = reinterpret_cast<const f4 *>(x)[g];
    for (int64_t i = (groups << 2) + threadIdx.x; i < len; i += kOneShotBlock)
        push[i] = x[i];
    __syncthreads();
    // 2. entry barrier: the peer's chunk has landed in stage[rank]
    if (threadIdx.x == 0) {
        const uint32_t mine_count = arrive(entry + rank * DETFOLD_ONE_SHOT_BLOCKS + b);
        const bool ok = await_count(entry + peer * DETFOLD_ONE_SHOT_BLOCKS + b, mine_count, a.spin_limit);
        if (!ok)
            refuse(a.words + rank, DETFOLD_BARRIER_ENTRY_EXPIRED);
        passed = ok;
    }
    __syncthreads();
    if (!passed)
        return;
    // 3. the fold, x_r + x_peer
    for (int64_t g = threadIdx.x; g < groups; g += kOneShotBlock) {
        const f4 v = reinterpret_cast<const f4 *>(x)[g] + reinterpret_cast<const f4 *>(mine)[g];
        reinterpret_cast<f4 *>(x)[g] = v;
    }
    for (int64_t i = (groups << 2) + threadIdx.x; i < len; i += kOneShotBlock)
        x[i] = x[i] + mine[i];
    __syncthreads();
    // 4. exit barrier: the peer has finished reading the stage this rank refills next call
    if (threadIdx.x == 0) {
        const uint32_t mine_count = arrive(exit + rank * DETFOLD_ONE_SHOT_BLOCKS + b);
        if (!await_count(exit + peer * DETFOLD_ONE_SHOT_BLOCKS + b, mine_count, a.spin_limit))
            refuse(a.words + rank, DETFOLD_BARRIER_EXIT_EXPIRED);
    }
}

__global__ __launch_bounds__(kOneShotBlock) void k_zero_words(uint32_t *p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

typedef void (*vector_kernel_t)(float *, const float *, const float *, int64_t, int, int64_t,
                                int64_t, float);
typedef void (*scalar_kernel_t)(float *, const float *, const float *, int64_t, int, int64_t,
                                float);

// Kernel instances: compile-time slot counts for the common power-of-two
// worlds (others use the runtime-W body, which loads slots in batches of
// kChunk), unroll 1, 2 or 4 with streaming hints, unroll 1 without hints.
template <int WS, bool SCALED>
vector_kernel_t pick_vector_w(int unroll, int policy)
{
    if (policy == kCached)
        return k_fold_vector<WS, 1, SCALED, kCached>;
    switch (unroll) {
    case 1: return k_fold_vector<WS, 1, SCALED, kStream>;
    case 2: return k_fold_vector<WS, 2, SCALED, kStream>;
    default: return k_fold_vector<WS, 4, SCALED, kStream>;
    }
}

template <int WS, bool SCALED>
scalar_kernel_t pick_scalar_w(int unroll, int policy)
{
    if (policy == kCached)
        return k_fold_scalar<WS, 1, SCALED, kCached>;
    switch (unroll) {
    case 1: return k_fold_scalar<WS, 1, SCALED, kStream>;
    case 2: return k_fold_scalar<WS, 2, SCALED, kStream>;
    default: return k_fold_scalar<WS, 4, SCALED, kStream>;
    }
}

typedef void (*rows_kernel_t)(float *, SlotTable, int64_t, int64_t, float, int);

template <bool SCALED>
rows_kernel_t pick_rows(int32_t w, int spw)
{
    switch (w) {
    case 2: return k_fold_rows<2, 1, SCALED>;
    case 3: return k_fold_rows<3, 1, SCALED>;
    case 4: return k_fold_rows<4, 1, SCALED>;
    case 5: return spw == 2 ? k_fold_rows<5, 2, SCALED> : k_fold_rows<5, 1, SCALED>;
    case 6: return spw == 2 ? k_fold_rows<6, 2, SCALED> : k_fold_rows<6, 1, SCALED>;
    case 7: return spw == 2 ? k_fold_rows<7, 2, SCALED> : k_fold_rows<7, 1, SCALED>;
    case 8: return spw == 2 ? k_fold_rows<8, 2, SCALED> : k_fold_rows<8, 1, SCALED>;
    case 9: return spw == 2 ? k_fold_rows<9, 2, SCALED> : k_fold_rows<9, 1, SCALED>;
    case 10: return spw == 2 ? k_fold_rows<10, 2, SCALED> : k_fold_rows<10, 1, SCALED>;
    case 11: return spw == 2 ? k_fold_rows<11, 2, SCALED> : k_fold_rows<11, 1, SCALED>;
    case 12: return spw == 2 ? k_fold_rows<12, 2, SCALED> : k_fold_rows<12, 1, SCALED>;
    case 13: return spw == 2 ? k_fold_rows<13, 2, SCALED> : k_fold_rows<13, 1, SCALED>;
    case 14: return spw == 2 ? k_fold_rows<14, 2, SCALED> : k_fold_rows<14, 1, SCALED>;
    case 15: return spw == 2 ? k_fold_rows<15, 2, SCALED> : k_fold_rows<15, 1, SCALED>;
    default: return spw == 2 ? k_fold_rows<16, 2, SCALED> : k_fold_rows<16, 1, SCALED>;
    }
}

typedef void (*rows_batch_kernel_t)(BatchArgs);

template <bool SCALED>
rows_batch_kernel_t pick_rows_batch(int32_t w, int spw)
{
    switch (w) {
    case 2: return k_fold_rows_batch<2, 1, SCALED>;
    case 3: return k_fold_rows_batch<3, 1, SCALED>;
    case 4: return k_fold_rows_batch<4, 1, SCALED>;
    case 5: return spw == 2 ? k_fold_rows_batch<5, 2, SCALED> : k_fold_rows_batch<5, 1, SCALED>;
    case 6: return spw == 2 ? k_fold_rows_batch<6, 2, SCALED> : k_fold_rows_batch<6, 1, SCALED>;
    case 7: return spw == 2 ? k_fold_rows_batch<7, 2, SCALED> : k_fold_rows_batch<7, 1, SCALED>;
    case 8: return spw == 2 ? k_fold_rows_batch<8, 2, SCALED> : k_fold_rows_batch<8, 1, SCALED>;
    case 9: return spw == 2 ? k_fold_rows_batch<9, 2, SCALED> : k_fold_rows_batch<9, 1, SCALED>;
    case 10: return spw == 2 ? k_fold_rows_batch<10, 2, SCALED> : k_fold_rows_batch<10, 1, SCALED>;
    case 11: return spw == 2 ? k_fold_rows_batch<11, 2, SCALED> : k_fold_rows_batch<11, 1, SCALED>;
    case 12: return spw == 2 ? k_fold_rows_batch<12, 2, SCALED> : k_fold_rows_batch<12, 1, SCALED>;
    case 13: return spw == 2 ? k_fold_rows_batch<13, 2, SCALED> : k_fold_rows_batch<13, 1, SCALED>;
    case 14: return spw == 2 ? k_fold_rows_batch<14, 2, SCALED> : k_fold_rows_batch<14, 1, SCALED>;
    case 15: return spw == 2 ? k_fold_rows_batch<15, 2, SCALED> : k_fold_rows_batch<15, 1, SCALED>;
    default: return spw == 2 ? k_fold_rows_batch<16, 2, SCALED> : k_fold_rows_batch<16, 1, SCALED>;
    }
}

typedef void (*rows_all_kernel_t)(SlotTable, int64_t, int64_t, int);

rows_all_kernel_t pick_rows_all(int32_t w, int spw)
{
    switch (w) {
    case 2: return k_fold_rows_all<2, 1>;
    case 3: return k_fold_rows_all<3, 1>;
    case 4: return k_fold_rows_all<4, 1>;
    case 5: return spw == 2 ? k_fold_rows_all<5, 2> : k_fold_rows_all<5, 1>;
    case 6: return spw == 2 ? k_fold_rows_all<6, 2> : k_fold_rows_all<6, 1>;
    case 7: return spw == 2 ? k_fold_rows_all<7, 2> : k_fold_rows_all<7, 1>;
    case 8: return spw == 2 ? k_fold_rows_all<8, 2> : k_fold_rows_all<8, 1>;
    case 9: return spw == 2 ? k_fold_rows_all<9, 2> : k_fold_rows_all<9, 1>;
    case 10: return spw == 2 ? k_fold_rows_all<10, 2> : k_fold_rows_all<10, 1>;
    case 11: return spw == 2 ? k_fold_rows_all<11, 2> : k_fold_rows_all<11, 1>;
    case 12: return spw == 2 ? k_fold_rows_all<12, 2> : k_fold_rows_all<12, 1>;
    case 13: return spw == 2 ? k_fold_rows_all<13, 2> : k_fold_rows_all<13, 1>;
    case 14: return spw == 2 ? k_fold_rows_all<14, 2> : k_fold_rows_all<14, 1>;
    case 15: return spw == 2 ? k_fold_rows_all<15, 2> : k_fold_rows_all<15, 1>;
    default: return spw == 2 ? k_fold_rows_all<16, 2> : k_fold_rows_all<16, 1>;
    }
}

template <bool SCALED>
vector_kernel_t pick_vector(int32_t w, int unroll, int policy)
{
    switch (w) {
    case 1: return pick_vector_w<1, SCALED>(unroll, policy);
    case 2: return pick_vector_w<2, SCALED>(unroll, policy);
    case 4: return pick_vector_w<4, SCALED>(unroll, policy);
    case 8: return pick_vector_w<8, SCALED>(unroll, policy);
    case 16: return pick_vector_w<16, SCALED>(unroll, policy);
    default: return pick_vector_w<0, SCALED>(unroll, policy);
    }
}

template <bool SCALED>
scalar_kernel_t pick_scalar(int32_t w, int unroll, int policy)
{
    switch (w) {
    case 1: return pick_scalar_w<1, SCALED>(unroll, policy);
    case 2: return pick_scalar_w<2, SCALED>(unroll, policy);
    case 4: return pick_scalar_w<4, SCALED>(unroll, policy);
    case 8: return pick_scalar_w<8, SCALED>(unroll, policy);
    case 16: return pick_scalar_w<16, SCALED>(unroll, policy);
    default: return pick_scalar_w<0, SCALED>(unroll, policy);
    }
}

// Launch a kernel; with `done`, the event is recorded by the dispatch itself
// when the kernel completes (cheaper than a separate event record), and with
// `begin` when it starts, so the pair times the kernel alone.
hipError_t launch(const void *k, dim3 grid, dim3 block, void **args, hipStream_t stream,
                  hipEvent_t done, hipEvent_t begin = nullptr)
{
    if (done || begin)
        return hipExtLaunchKernel(k, grid, block, args, 0, stream, begin, done, 0);
    return hipLaunchKernel(k, grid, block, args, 0, stream);
}

}  // namespace

// ---------------------------------------------------------------------------
// Launches (declared in internal.h): pick the kernel instance a plan names
// and enqueue it on the caller's stream.

int launch_plan(const Geometry &g, const detfold_plan &p, bool scaled, float inv_w, void *stream_,
                void *done_, void *begin_)
{
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    hipEvent_t done = static_cast<hipEvent_t>(done_);
    hipEvent_t begin = static_cast<hipEvent_t>(begin_);
    float *out = reinterpret_cast<float *>(g.out);
    const float *s0 = reinterpret_cast<const float *>(g.s0);
    const float *s1 = reinterpret_cast<const float *>(g.s1);
    int64_t stride = g.stride;
    int w = g.w;
    int64_t len = g.len;
    int64_t head = p.head;
    const int policy = p.policy == DETFOLD_POLICY_CACHED ? kCached : kStream;
    const dim3 grid((unsigned)p.grid), block((unsigned)p.block);
    hipError_t e;
    if (p.path == DETFOLD_PATH_ROWS && w > kMaxRowsW) {
        // the plan's workgroup size names the pass shape
        const bool aligned = p.block == 64 * kWideAlignedWaves;
        constexpr int AW = kWideAlignedWaves, AS = kWideSlots / kWideAlignedWaves, AK = kWideAlignedKiB;
        const void *k = aligned ? (scaled ? (const void *)k_fold_rows_wide<AW, AS, AK, true>
                                          : (const void *)k_fold_rows_wide<AW, AS, AK, false>)
                                : (scaled ? (const void *)k_fold_rows_wide<kWideWaves, 1, kWideKiB, true>
                                          : (const void *)k_fold_rows_wide<kWideWaves, 1, kWideKiB, false>);
        int group = p.group;
        void *args[] = {&out, &s0, &s1, &stride, &w, &len, &head, &inv_w, &group};
        e = launch(k, grid, block, args, stream, done, begin);
    } else if (p.path == DETFOLD_PATH_ROWS) {
        const int spw = rows_spw(w, p.block / 64);  // the plan's workgroup size names the shape
        rows_kernel_t k = scaled ? pick_rows<true>(w, spw) : pick_rows<false>(w, spw);
        SlotTable slots = {};
        for (int32_t r = 0; r < w; ++r)
            slots.p[r] = reinterpret_cast<const float *>(g.slot(r));
        int group = p.group;
        void *args[] = {&out, &slots, &len, &head, &inv_w, &group};
        e = launch(reinterpret_cast<const void *>(k), grid, block, args, stream, done, begin);
    } else if (p.path == DETFOLD_PATH_VECTOR) {
        vector_kernel_t k = scaled ? pick_vector<true>(w, p.unroll, policy)
                                   : pick_vector<false>(w, p.unroll, policy);
        void *args[] = {&out, &s0, &s1, &stride, &w, &len, &head, &inv_w};
        e = launch(reinterpret_cast<const void *>(k), grid, block, args, stream, done, begin);
    } else {
        scalar_kernel_t k = scaled ? pick_scalar<true>(w, p.unroll, policy)
                                   : pick_scalar<false>(w, p.unroll, policy);
        void *args[] = {&out, &s0, &s1, &stride, &w, &len, &inv_w};
        e = launch(reinterpret_cast<const void *>(k), grid, block, args, stream, done, begin);
    }
    return e == hipSuccess ? DETFOLD_OK : DETFOLD_ELAUNCH;
}

// The batched fold's launch (2 <= W <= 16): one workgroup per tile of every job.
int launch_batch(const BatchArgs &a, int32_t w, const detfold_plan &p, bool scaled, void *stream)
{
    if (p.path != DETFOLD_PATH_ROWS || w < 2 || w > kMaxRowsW || a.count < 1 || a.count > kMaxJobs)
        return DETFOLD_EINVAL;
    const int spw = rows_spw(w, p.block / 64);  // the plan's workgroup size names the shape
    rows_batch_kernel_t k = scaled ? pick_rows_batch<true>(w, spw) : pick_rows_batch<false>(w, spw);
    BatchArgs copy = a;
    void *args[] = {&copy};
    return launch(reinterpret_cast<const void *>(k), dim3((unsigned)p.grid), dim3((unsigned)p.block), args,
                  static_cast<hipStream_t>(stream), nullptr) == hipSuccess
               ? DETFOLD_OK
               : DETFOLD_ELAUNCH;
}

// The fused round's launch: the plan of a fold over the slot table (row
// body, 2 <= W <= 16), with k_fold_rows_all in place of k_fold_rows.
int launch_rows_all(const Geometry &g, const detfold_plan &p, void *stream)
{
    if (p.path != DETFOLD_PATH_ROWS || !g.has_table || g.w < 2 || g.w > kMaxRowsW)
        return DETFOLD_EINVAL;
    const int spw = rows_spw(g.w, p.block / 64);
    rows_all_kernel_t k = pick_rows_all(g.w, spw);
    SlotTable slots = {};
    for (int32_t r = 0; r < g.w; ++r)
        slots.p[r] = reinterpret_cast<const float *>(g.table[r]);
    int64_t len = g.len, head = p.head;
    int group = p.group;
    void *args[] = {&slots, &len, &head, &group};
    return launch(reinterpret_cast<const void *>(k), dim3((unsigned)p.grid), dim3((unsigned)p.block), args,
                  static_cast<hipStream_t>(stream), nullptr) == hipSuccess
               ? DETFOLD_OK
               : DETFOLD_ELAUNCH;
}

// Copy len floats from src to each of ndst destinations with k_copy_out.
// Payloads up to kCopyCachedBytes take no cache hints (a decode-join push is
// read by the peer's fold right away); larger ones stream.  One pass of
// 256-thread workgroups, capped at 8 per CU with the rest covered by the
// grid-stride loop.
int launch_copy(float *const *dsts, int ndst, const float *src, int64_t len, int32_t cu,
                void *stream, void *done)
{
    if (len == 0 || ndst == 0)
        return DETFOLD_OK;
    SlotTable t = {};
    bool vec = true;
    const int ph = phase16((uintptr_t)src);
    for (int d = 0; d < ndst; ++d) {
        t.p[d] = dsts[d];
        vec = vec && phase16((uintptr_t)dsts[d]) == ph;
    }
    int64_t head = (4 - ph) & 3;
    if (head > len)
        head = len;
    const int64_t units = vec ? ((len - head) >> 2) + 6 : len;
    const int block = 256;
    int64_t grid = (units + block - 1) / block;
    const int64_t cap = (int64_t)cu * 8;
    if (grid > cap)
        grid = cap;
    if (grid < 1)
        grid = 1;
    const bool stream_pol = len * 4 > kCopyCachedBytes;
    const void *k = vec ? (stream_pol ? (const void *)k_copy_out<true, kStream> : (const void *)k_copy_out<true, kCached>)
                        : (stream_pol ? (const void *)k_copy_out<false, kStream> : (const void *)k_copy_out<false, kCached>);
    void *args[] = {&t, &ndst, &src, &len, &head};
    return launch(k, dim3((unsigned)grid), dim3(block), args, static_cast<hipStream_t>(stream),
                  static_cast<hipEvent_t>(done)) == hipSuccess
               ? DETFOLD_OK
               : DETFOLD_ELAUNCH;
}

// Device address of `scratch` on the current device, looked up once per
// device with that device current.
int static_stage(float **stage)
{
    constexpr int kMaxDevices = 64;
    static std::atomic<float *> cached[kMaxDevices];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return DETFOLD_EDEVICE;
    if (dev < kMaxDevices) {
        float *p = cached[dev].load(std::memory_order_acquire);
        if (p) {
            *stage = p;
            return DETFOLD_OK;
        }
    }
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
        return DETFOLD_EDEVICE;
    if (dev < kMaxDevices)
        cached[dev].store(static_cast<float *>(p), std::memory_order_release);
    *stage = static_cast<float *>(p);
    return DETFOLD_OK;
}

int launch_one_shot(const OneShotArgs &a, int nranks, void *stream)
{
    OneShotArgs copy = a;
    void *args[] = {&copy};
    return hipLaunchKernel((const void *)k_one_shot, dim3((unsigned)(a.blocks * nranks)), dim3(kOneShotBlock),
                           args, 0, static_cast<hipStream_t>(stream)) == hipSuccess
               ? DETFOLD_OK
               : DETFOLD_ELAUNCH;
}

int launch_zero_words(uint32_t *p, int64_t n, void *stream)
{
    void *args[] = {&p, &n};
    return hipLaunchKernel((const void *)k_zero_words, dim3(1), dim3(kOneShotBlock), args, 0,
                           static_cast<hipStream_t>(stream)) == hipSuccess
               ? DETFOLD_OK
               : DETFOLD_ELAUNCH;
}

}  // namespace detfold_impl
