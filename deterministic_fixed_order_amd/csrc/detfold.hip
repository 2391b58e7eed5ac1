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

#include "detfold.h"

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned u4 __attribute__((ext_vector_type(4)));

constexpr int kMaxBlock = 1024;
constexpr int kStreamBlock = 512;  // largest default workgroup of the bandwidth path
constexpr int kChunk = 8;          // slots loaded per batch when W is a runtime value
constexpr int kMaxRowsW = 16;      // widest fold the LDS row body takes (one wave per slot)
constexpr int kWideWaves = 16;     // slots per pass of the wide row body (W > kMaxRowsW)
constexpr int kWideKiB = 4;        // KiB of one slot each wave of the wide body streams per pass

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

// Memory policy of a launch.
//  kStream  the bandwidth path: every input byte is read once, so loads carry
//           the non-temporal hint, and stores are written through the
//           per-XCD L2 (scope bits sc0 sc1) instead of sitting there dirty
//           until an eviction competes with the incoming loads.
//  kCached  the decode-join path: no hints; its output is read again soon.
enum Policy : int { kCached = 0, kStream = 1 };

// Cache-policy operand of the gfx950 buffer instructions: bit 0 = sc0,
// bit 1 = nt, bit 4 = sc1.
template <int POL> struct Aux {
    static constexpr int load = POL == kStream ? 2 : 0;    // nt
    static constexpr int store = POL == kStream ? 17 : 0;  // sc0 sc1
};

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

// LDS row-transpose body (2 <= W <= 16).  One workgroup of W waves folds a
// tile of T 16-byte groups of `out`: wave r streams the tile's bytes of slot r
// -- LPW consecutive KiB, one contiguous run per wave -- straight into LDS row
// r (buffer loads with the lds bit, no register staging); after a barrier
// every thread folds whole groups from the W rows, in ascending row order, and
// stores them.  Streaming one slot per wave keeps each wave on one run of HBM
// rows; the direct body instead has every wave touch W runs 1 KiB at a time,
// which measured 3-8% slower on MI355X.
//
// Slot phases: the tile of `out` starts 16-byte aligned, but slot r's bytes
// for the tile may start at any dword.  Wave r's buffer descriptor is based at
// exactly that dword (gfx9 buffer loads need only dword alignment), so every
// row lands in LDS aligned to the tile whatever the slot's phase, and the
// fold reads 16-byte groups from every row alike.  The descriptor's range is
// the tile's bytes of the slot, so no lane reads past them.  Measured on
// MI355X against realigning shifted rows in LDS (one extra KiB loaded per
// wave, 4-byte LDS reads): +3% at W=16 x 10,000,019 at base+1, +10% at W=7,
// no change when every slot is aligned.
template <int W> struct RowsShape {
    static constexpr int LPW = rows_kib_per_wave(W);  // KiB each wave streams per tile
    static constexpr int T = LPW * 64;                // 16-byte groups per tile
};

typedef __attribute__((address_space(3))) void lds_void;

// Slot base pointers of the LDS row body, passed by value in the kernel
// arguments (slot r of a stacked arena is stacked + r*len; fold_slots takes
// them from the caller).
struct SlotTable {
    const float *p[kMaxRowsW];
};

template <int W, bool SCALED>
__device__ __forceinline__ void fold_one_table(float *out, const SlotTable &slots, int64_t i,
                                               float inv_w)
{
    float acc = slots.p[0][i];
#pragma unroll
    for (int r = 1; r < W; ++r)
        acc = acc + slots.p[r][i];
    if constexpr (SCALED)
        acc = acc * inv_w;
    out[i] = acc;
}

template <int W, bool SCALED>
__global__ __launch_bounds__(W * 64) void k_fold_rows(float *out, SlotTable slots, int64_t len,
                                                      int64_t head, float inv_w)
{
    constexpr int LPW = RowsShape<W>::LPW, T = RowsShape<W>::T;
    __shared__ f4 rows[W][T];

    const int64_t groups = (len - head) >> 2;
    const int64_t tail0 = head + (groups << 2);
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid < head + (len - tail0))
        fold_one_table<W, SCALED>(out, slots, gid < head ? gid : tail0 + (gid - head), inv_w);

    const uint32_t lane = threadIdx.x & 63;
    const uint32_t r = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // this wave's slot
    const float *slot = slots.p[r];
    for (int64_t tile = blockIdx.x; tile * T < groups; tile += gridDim.x) {
        const int64_t g0 = tile * T;
        const int64_t cnt = groups - g0 < T ? groups - g0 : T;
        const int64_t e0 = head + 4 * g0;  // first element of the tile; out + e0 is 16-byte aligned
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(slot + e0, (uint32_t)(cnt * 16));
#pragma unroll
        for (int u = 0; u < LPW; ++u)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)&rows[r][u * 64], 16,
                                                     (uint32_t)(u * 64 + lane) * 16u, 0, 0,
                                                     Aux<kStream>::load);
        __syncthreads();  // every row has landed

        const __amdgpu_buffer_rsrc_t ro = make_rsrc(out + e0, (uint32_t)(cnt * 16));
        for (uint32_t t = threadIdx.x; t < (uint32_t)cnt; t += W * 64) {
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
}

// Wide LDS row body (W > 16, stacked arena): a workgroup of 16 waves folds a
// tile of 256 groups in passes of 16 slots.  In pass p wave q streams 4 KiB of
// slot 16p + q into LDS row q, exactly as the row body above does; after the
// barrier the thread that owns group t continues its chain with rows 0, 1, ...
// of the pass -- pass 0 starts it from slot 0 -- and a second barrier frees
// the rows for the next pass.  The running sum stays in the thread's
// registers between passes, so each element still sees the adds in strictly
// ascending slot order, one rounding each, and is stored once at the end.
template <bool SCALED>
__global__ __launch_bounds__(kWideWaves * 64) void k_fold_rows_wide(float *out, const float *s0,
                                                                    const float *s1, int64_t stride,
                                                                    int w, int64_t len, int64_t head,
                                                                    float inv_w)
{
    constexpr int T = kWideKiB * 64;  // groups per tile, at most one per thread
    static_assert(T <= kWideWaves * 64, "one group per thread");
    __shared__ f4 rows[kWideWaves][T];

    const int64_t groups = (len - head) >> 2;
    const int64_t tail0 = head + (groups << 2);
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid < head + (len - tail0))
        fold_one<0, SCALED>(out, s0, s1, stride, w, gid < head ? gid : tail0 + (gid - head), inv_w);

    const uint32_t lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const uint32_t t = threadIdx.x;
    for (int64_t tile = blockIdx.x; tile * T < groups; tile += gridDim.x) {
        const int64_t g0 = tile * T;
        const int64_t cnt = groups - g0 < T ? groups - g0 : T;
        const int64_t e0 = head + 4 * g0;
        f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int base = 0; base < w; base += kWideWaves) {
            const int nr = w - base < kWideWaves ? w - base : kWideWaves;
            if (wave < nr) {
                const int r = base + wave;
                const float *slot = r == 0 ? s0 : s1 + (int64_t)(r - 1) * stride;
                const __amdgpu_buffer_rsrc_t rs = make_rsrc(slot + e0, (uint32_t)(cnt * 16));
#pragma unroll
                for (int u = 0; u < kWideKiB; ++u)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)&rows[wave][u * 64], 16,
                                                             (uint32_t)(u * 64 + lane) * 16u, 0, 0,
                                                             Aux<kStream>::load);
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

constexpr int kOneShotBlock = 256;
constexpr int64_t kOneShotPerBlock = 1024;  // payload floats per workgroup before the cap
constexpr int32_t kDefaultSpinLimit = 1 << 20;

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

// ---------------------------------------------------------------------------
// Host side: planning (pure integer logic, no HIP calls)

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

inline int phase16(uintptr_t a) { return (int)((a >> 2) & 3); }

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

// Workgroup size and tile (16-byte groups) of the row bodies: one wave per
// slot up to 16 slots, 16 waves making passes over the slots beyond that.
int rows_block(int32_t w) { return w <= kMaxRowsW ? 64 * w : 64 * kWideWaves; }
int64_t rows_tile(int32_t w) { return (int64_t)(w <= kMaxRowsW ? rows_kib_per_wave(w) : kWideKiB) * 64; }

// Positions per thread per pass.  The vector body moves 16 bytes per slot per
// position, and one position per thread keeps the most waves in flight (the
// measured best on MI355X); the scalar body moves 4 bytes per slot per
// position, so each thread takes four.
int default_unroll(int path) { return path == DETFOLD_PATH_VECTOR ? 1 : 4; }

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
    const detfold_launch o = ovr ? *ovr : detfold_launch{DETFOLD_PATH_AUTO, 0, 0, 0, 0};
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
        (!rows_ok || policy == DETFOLD_POLICY_CACHED || (o.block && o.block != rows_block(g.w)) ||
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
    if (path == DETFOLD_PATH_ROWS) {
        p->unroll = 1;
        p->block = rows_block(g.w);
        p->tile = rows_tile(g.w);
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

typedef void (*rows_kernel_t)(float *, SlotTable, int64_t, int64_t, float);

template <bool SCALED>
rows_kernel_t pick_rows(int32_t w)
{
    switch (w) {
    case 2: return k_fold_rows<2, SCALED>;
    case 3: return k_fold_rows<3, SCALED>;
    case 4: return k_fold_rows<4, SCALED>;
    case 5: return k_fold_rows<5, SCALED>;
    case 6: return k_fold_rows<6, SCALED>;
    case 7: return k_fold_rows<7, SCALED>;
    case 8: return k_fold_rows<8, SCALED>;
    case 9: return k_fold_rows<9, SCALED>;
    case 10: return k_fold_rows<10, SCALED>;
    case 11: return k_fold_rows<11, SCALED>;
    case 12: return k_fold_rows<12, SCALED>;
    case 13: return k_fold_rows<13, SCALED>;
    case 14: return k_fold_rows<14, SCALED>;
    case 15: return k_fold_rows<15, SCALED>;
    default: return k_fold_rows<16, SCALED>;
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
// when the kernel completes (cheaper than a separate event record).
hipError_t launch(const void *k, dim3 grid, dim3 block, void **args, hipStream_t stream,
                  hipEvent_t done)
{
    if (done)
        return hipExtLaunchKernel(k, grid, block, args, 0, stream, nullptr, done, 0);
    return hipLaunchKernel(k, grid, block, args, 0, stream);
}

int launch_plan(const Geometry &g, const detfold_plan &p, bool scaled, float inv_w,
                hipStream_t stream, hipEvent_t done = nullptr)
{
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
        const void *k = scaled ? (const void *)k_fold_rows_wide<true> : (const void *)k_fold_rows_wide<false>;
        void *args[] = {&out, &s0, &s1, &stride, &w, &len, &head, &inv_w};
        e = launch(k, grid, block, args, stream, done);
    } else if (p.path == DETFOLD_PATH_ROWS) {
        rows_kernel_t k = scaled ? pick_rows<true>(w) : pick_rows<false>(w);
        SlotTable slots = {};
        for (int32_t r = 0; r < w; ++r)
            slots.p[r] = reinterpret_cast<const float *>(g.slot(r));
        void *args[] = {&out, &slots, &len, &head, &inv_w};
        e = launch(reinterpret_cast<const void *>(k), grid, block, args, stream, done);
    } else if (p.path == DETFOLD_PATH_VECTOR) {
        vector_kernel_t k = scaled ? pick_vector<true>(w, p.unroll, policy)
                                   : pick_vector<false>(w, p.unroll, policy);
        void *args[] = {&out, &s0, &s1, &stride, &w, &len, &head, &inv_w};
        e = launch(reinterpret_cast<const void *>(k), grid, block, args, stream, done);
    } else {
        scalar_kernel_t k = scaled ? pick_scalar<true>(w, p.unroll, policy)
                                   : pick_scalar<false>(w, p.unroll, policy);
        void *args[] = {&out, &s0, &s1, &stride, &w, &len, &inv_w};
        e = launch(reinterpret_cast<const void *>(k), grid, block, args, stream, done);
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
    if ((rc = make_plan(g, cu, ovr, DETFOLD_POLICY_STREAM, &p)) != DETFOLD_OK)
        return rc;
    return launch_plan(g, p, scaled, inv_w, static_cast<hipStream_t>(stream));
}

// The decode-join path.  Payloads up to kLatencyBytes per buffer are
// launch-latency bound and their result is read again soon: one position per
// thread, one pass, no cache hints.  Larger payloads are bandwidth bound and
// take the streaming policy.
constexpr int64_t kLatencyBytes = 8 << 20;
constexpr int64_t kCopyCachedBytes = 1 << 20;

int plan_into(const Geometry &g, int32_t cu_count, detfold_plan *p)
{
    if (g.len * 4 <= kLatencyBytes) {
        const detfold_launch o = {DETFOLD_PATH_AUTO, 0, 0, 1, 0};
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

// Copy len floats from src to each of ndst destinations with k_copy_out.
// Payloads up to kCopyCachedBytes take no cache hints (a decode-join push is
// read by the peer's fold right away); larger ones stream.  One pass of 256-thread workgroups, capped at 8
// per CU with the rest covered by the grid-stride loop.
int copy_out(float *const *dsts, int ndst, const float *src, int64_t len, int32_t cu,
             hipStream_t stream, hipEvent_t done = nullptr)
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
    return launch(k, dim3((unsigned)grid), dim3(block), args, stream, done) == hipSuccess ? DETFOLD_OK
                                                                                        : DETFOLD_ELAUNCH;
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

int check_round_args(float *const *arenas, int32_t W, int64_t n, const float *stage,
                     int64_t stage_elems, int32_t flags)
{
    if (W < 1 || W > kMaxRowsW || n < 0 || (flags & ~(DETFOLD_ROUND_REVERSE_DELIVERY | DETFOLD_ROUND_DIRECT)))
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
    if (!(flags & DETFOLD_ROUND_DIRECT)) {
        const int64_t need = (int64_t)W * ((n + W - 1) / W);
        if (!stage || (((uintptr_t)stage) & 3) || stage_elems < need)
            return DETFOLD_EINVAL;
        for (int32_t r = 0; r < W; ++r)
            if (ranges_overlap((uintptr_t)stage, (uint64_t)need * 4, (uintptr_t)arenas[r], (uint64_t)n * 4))
                return DETFOLD_EOVERLAP;
    }
    return DETFOLD_OK;
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
// already in the same HBM.  Bytes move by device-to-device copies only, so the
// bits are the fold's whatever the mode or the delivery order.
int run_round(float *const *arenas, int32_t W, int64_t n, float *stage, int32_t flags,
              hipStream_t stream)
{
    int32_t cu = 0;
    int rc = current_cu_count(&cu);
    if (rc != DETFOLD_OK)
        return rc;
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
                rc = copy_out(&slot, 1, arenas[src] + s, l, cu, stream);
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
        if ((rc = copy_out(dsts, nd, arenas[o] + start[o], length[o], cu, stream)) != DETFOLD_OK)
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

int run_pair(const detfold_pair_link *k, float *x0, float *x1, int64_t n)
{
    int32_t cu = 0;
    int rc = current_cu_count(&cu);
    if (rc != DETFOLD_OK)
        return rc;
    float *x[2] = {x0, x1};
    hipStream_t st[2] = {static_cast<hipStream_t>(k->stream[0]), static_cast<hipStream_t>(k->stream[1])};
    for (int r = 0; r < 2; ++r) {
        const int peer = 1 - r;
        // the peer's previous fold has finished reading the staging buffer we refill
        if (hipStreamWaitEvent(st[r], static_cast<hipEvent_t>(k->folded[peer]), 0) != hipSuccess)
            return DETFOLD_ELAUNCH;
        float *dst = k->stage[peer];
        if ((rc = copy_out(&dst, 1, x[r], n, cu, st[r], static_cast<hipEvent_t>(k->pushed[r]))) != DETFOLD_OK)
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

int check_link_events(const detfold_pair_link *k)
{
    return k && k->pushed[0] && k->pushed[1] && k->folded[0] && k->folded[1] ? DETFOLD_OK
                                                                               : DETFOLD_EINVAL;
}

bool bad_buffer(const void *p, int64_t n)
{
    return !p || (((uintptr_t)p) & 3) || n > INT64_MAX / 8;
}

// Broadcast: stream[o] marks where it stands (folded[o]), stream[root] waits
// for that mark, copies, and the copy's end (pushed[root]) gates stream[o].
int run_broadcast(const detfold_pair_link *k, int32_t root, const float *src, float *dst, int64_t n)
{
    int32_t cu = 0;
    int rc = current_cu_count(&cu);
    if (rc != DETFOLD_OK)
        return rc;
    const int32_t o = 1 - root;
    hipStream_t sr = static_cast<hipStream_t>(k->stream[root]);
    hipStream_t so = static_cast<hipStream_t>(k->stream[o]);
    if (hipEventRecord(static_cast<hipEvent_t>(k->folded[o]), so) != hipSuccess ||
        hipStreamWaitEvent(sr, static_cast<hipEvent_t>(k->folded[o]), 0) != hipSuccess)
        return DETFOLD_ELAUNCH;
    if ((rc = copy_out(&dst, 1, src, n, cu, sr, static_cast<hipEvent_t>(k->pushed[root]))) != DETFOLD_OK)
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
    if (rc != DETFOLD_OK)
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
        if ((rc = copy_out(dsts, 2, x[r], span, cu, st[r], static_cast<hipEvent_t>(k->pushed[r]))) != DETFOLD_OK)
            return rc;
    }
    for (int r = 0; r < 2; ++r)
        if (hipStreamWaitEvent(st[r], static_cast<hipEvent_t>(k->pushed[1 - r]), 0) != hipSuccess)
            return DETFOLD_ELAUNCH;
    return DETFOLD_OK;
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

// nranks = 2: both ranks in one launch (workgroups [0, G) rank 0, [G, 2G)
// rank 1); nranks = 1: rank `rank0` alone.  G = ceil(n / 1024) capped at
// DETFOLD_ONE_SHOT_BLOCKS; each workgroup takes a chunk rounded up to 4 floats.
int run_one_shot(const detfold_one_shot_link *k, int32_t rank0, int nranks, float *xa, float *xb,
                 int64_t n, hipStream_t stream)
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
    void *args[] = {&a};
    return hipLaunchKernel((const void *)k_one_shot, dim3((unsigned)(blocks * nranks)), dim3(kOneShotBlock),
                           args, 0, stream) == hipSuccess
               ? DETFOLD_OK
               : DETFOLD_ELAUNCH;
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
    hipStream_t st = static_cast<hipStream_t>(link->stream);
    uint32_t *flags = link->flags;
    int64_t nf = DETFOLD_ONE_SHOT_FLAG_WORDS;
    uint32_t *words = reinterpret_cast<uint32_t *>(link->words);
    int64_t nw = 2;
    void *a0[] = {&flags, &nf};
    void *a1[] = {&words, &nw};
    if (hipLaunchKernel((const void *)k_zero_words, dim3(1), dim3(kOneShotBlock), a0, 0, st) != hipSuccess ||
        hipLaunchKernel((const void *)k_zero_words, dim3(1), dim3(kOneShotBlock), a1, 0, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return DETFOLD_ELAUNCH;
    return DETFOLD_OK;
}

int detfold_one_shot_all_reduce(const detfold_one_shot_link *link, float *x0, float *x1, int64_t n)
{
    int rc = check_one_shot_link(link);
    if (rc != DETFOLD_OK)
        return rc;
    float *x[2] = {x0, x1};
    if ((rc = check_one_shot_buffers(link, x, 2, n)) != DETFOLD_OK || n == 0)
        return rc;
    return run_one_shot(link, 0, 2, x0, x1, n, static_cast<hipStream_t>(link->stream));
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
    return run_one_shot(link, rank, 1, x, nullptr, n, static_cast<hipStream_t>(stream));
}

}  // extern "C"
