// rk_scan.hpp -- scans (prefix folds) on gfx950.
//
// AcceleratedKernels.jl PR #202 (tile scans), opening paragraph: accumulate!
// over a whole array or along one dim; every output k of a line is the fold
// of the line's elements 0..k (inclusive) or 0..k-1 (exclusive), started
// from init.  The page's kernels give each thread a run of consecutive
// elements in shared memory and pad the runs to an odd stride against bank
// conflicts.  Here a scan keeps the data in registers instead: lane l of a
// wave holds the l-th 16-byte vector of a 64-vector chunk (one fully
// coalesced load), scans its own few elements, and a wave64 DPP scan of the
// lane totals gives every lane its offset, so no element goes through LDS.
//
// Kernels, chosen by plan_scan():
//   k_scan_tile     lines contiguous along the scan dim and at least one
//                   tile long (the whole array included; also lines contiguous
//                   on one side only, too few for the transposing tiles, the
//                   other side's elements moved one by one): one pass, tiles in
//                   the order of a counter, each tile's prefix from its
//                   predecessors by decoupled look-back (Merrill and Garland,
//                   "Single-pass Parallel Prefix Scan with Decoupled
//                   Look-back", 2016);
//   k_scan_rowwave  shorter contiguous lines: one wave per line;
//   k_scan_columns  a strided scan dim over runs of contiguous lines: tiles of
//                   lines x scan positions, look-back along the scan dim;
//   k_scan_transpose input and output contiguous along different axes (a
//                   transposed or permuted view): tiles staged through LDS,
//                   look-back along the scan dim;
//   k_scan_lines    any other layout: one thread per line, walking it.
#pragma once

#include "rk_kernels.hpp"
#include "rk_scan_plan.hpp"

namespace rk {

// ------------------------------------------------------------ lane moves

// DPP row shifts: lane i of a 16-lane row reads lane i - n of the same row;
// lanes without a source take `fill`.
template <int CTRL, class T>
__device__ __forceinline__ T dpp_shift(T v, T fill)
{
    if constexpr (sizeof(T) == 4) {
        return bitcast<T>((uint32_t)__builtin_amdgcn_update_dpp((int)bitcast<uint32_t>(fill), (int)bitcast<uint32_t>(v),
                                                                CTRL, 0xf, 0xf, false));
    } else {
        const uint64_t u = bitcast<uint64_t>(v), f = bitcast<uint64_t>(fill);
        const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)f, (int)(uint32_t)u, CTRL, 0xf,
                                                                  0xf, false);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)(f >> 32), (int)(uint32_t)(u >> 32),
                                                                  CTRL, 0xf, 0xf, false);
        return bitcast<T>(((uint64_t)hi << 32) | lo);
    }
}

constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;

// Inclusive scan over the 64 lanes of a wave: lane i gets v_0 (+) ... (+) v_i.
// Steps of 1, 2, 4 and 8 lanes inside each 16-lane row (Hillis and Steele),
// then every row adds the totals of the rows before it, read from lanes 15,
// 31 and 47.  All 64 lanes must be active.
template <class Op, class T>
__device__ __forceinline__ T wave_scan_incl(T v)
{
    const T id = Op::template identity<T>();
    v = Op::apply(dpp_shift<kDppRowShr1>(v, id), v);
    v = Op::apply(dpp_shift<kDppRowShr2>(v, id), v);
    v = Op::apply(dpp_shift<kDppRowShr4>(v, id), v);
    v = Op::apply(dpp_shift<kDppRowShr8>(v, id), v);
    const T r0 = read_lane(v, 15), r1 = read_lane(v, 31), r2 = read_lane(v, 47);
    const int row = lane_id() >> 4;
    T pre = r0;
    pre = row >= 2 ? Op::apply(pre, r1) : pre;
    pre = row >= 3 ? Op::apply(pre, r2) : pre;
    return row >= 1 ? Op::apply(pre, v) : v;
}

// Value of the previous lane; lane 0 gets `fill`.  All 64 lanes active.
template <class T>
__device__ __forceinline__ T lane_prev(T v, T fill)
{
    const int src = lane_id() > 0 ? lane_id() - 1 : 0;
    const T p = move_words(v, [src](uint32_t w) { return bpermute32(w, src); });
    return lane_id() > 0 ? p : fill;
}

// ---------------------------------------------------------------- outputs

// Storage type and conversion of an accumulator for each output dtype (the
// same rounding as store_out: nearest even, through round-to-odd from f64).
template <int OD> struct OutT;
template <> struct OutT<F32> {
    using S = float;
    template <class A> __device__ static S conv(A v) { return (float)v; }
};
template <> struct OutT<F64> {
    using S = double;
    template <class A> __device__ static S conv(A v) { return (double)v; }
};
template <> struct OutT<BF16> {
    using S = uint16_t;
    template <class A> __device__ static S conv(A v)
    {
        if constexpr (std::is_same_v<A, double>)
            return f32_to_bf16_rne(f64_to_f32_odd(v));
        else
            return f32_to_bf16_rne((float)v);
    }
};
template <> struct OutT<F16> {
    using S = uint16_t;
    template <class A> __device__ static S conv(A v)
    {
        float f;
        if constexpr (std::is_same_v<A, double>)
            f = f64_to_f32_odd(v);
        else
            f = (float)v;
        return bitcast<uint16_t>((_Float16)f);
    }
};
template <> struct OutT<I32> {
    using S = int32_t;
    template <class A> __device__ static S conv(A v) { return (int32_t)(uint32_t)(uint64_t)v; }
};
template <> struct OutT<I64> {
    using S = int64_t;
    template <class A> __device__ static S conv(A v) { return (int64_t)v; }
};

// Store V consecutive outputs at element idx of `out`, converted to OD, in
// the widest pieces their byte count allows (the caller guarantees that
// alignment when V > 1).
template <int OD, class Acc, int V, bool NTS = false>
__device__ __forceinline__ void store_run_as(void *out, int64_t idx, const Acc (&v)[V])
{
    using S = typename OutT<OD>::S;
    S t[V];
#pragma unroll
    for (int i = 0; i < V; ++i)
        t[i] = OutT<OD>::conv(v[i]);
    char *p = reinterpret_cast<char *>(static_cast<S *>(out) + idx);
    constexpr int NB = int(sizeof(t));
    // Non-temporal only when one store covers the lane's whole run: a wave's
    // store is then one contiguous piece.  Runs of 32 bytes and more take
    // several stores at a lane stride, each leaving holes in the lines that the
    // next one fills; streaming those past the cache measured 10-15% slower.
    constexpr bool NT = NTS && NB <= 16;
    if constexpr (NB % 16 == 0) {
#pragma unroll
        for (int b = 0; b < NB; b += 16) {
            u32x4 w;
            __builtin_memcpy(&w, reinterpret_cast<const char *>(t) + b, 16);
            if constexpr (NT)
                __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(p + b));
            else
                *reinterpret_cast<u32x4 *>(p + b) = w;
        }
    } else if constexpr (NB % 8 == 0) {
#pragma unroll
        for (int b = 0; b < NB; b += 8) {
            uint64_t w;
            __builtin_memcpy(&w, reinterpret_cast<const char *>(t) + b, 8);
            *reinterpret_cast<uint64_t *>(p + b) = w;
        }
    } else if constexpr (NB % 4 == 0) {
#pragma unroll
        for (int b = 0; b < NB; b += 4) {
            uint32_t w;
            __builtin_memcpy(&w, reinterpret_cast<const char *>(t) + b, 4);
            *reinterpret_cast<uint32_t *>(p + b) = w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < V; ++i)
            reinterpret_cast<S *>(p)[i] = t[i];
    }
}

template <class Acc, int V, bool NTS = false>
__device__ __forceinline__ void store_run(void *out, int64_t idx, int out_dtype, const Acc (&v)[V])
{
    if constexpr (std::is_floating_point_v<Acc>) {
        switch (out_dtype) {
        case F32: store_run_as<F32, Acc, V, NTS>(out, idx, v); break;
        case F64: store_run_as<F64, Acc, V, NTS>(out, idx, v); break;
        case BF16: store_run_as<BF16, Acc, V, NTS>(out, idx, v); break;
        case F16: store_run_as<F16, Acc, V, NTS>(out, idx, v); break;
        default: break;
        }
    } else {
        switch (out_dtype) {
        case I32: store_run_as<I32, Acc, V, NTS>(out, idx, v); break;
        case I64: store_run_as<I64, Acc, V, NTS>(out, idx, v); break;
        default: break;
        }
    }
}

// ------------------------------------------------------------ chunk scans

// A chunk is 64 * VL consecutive elements of a line: lane l holds elements
// l*VL .. l*VL+VL-1, loaded at once (16 bytes when VL is the input's 16-byte
// vector; 8 or 4 bytes when the outputs are wider than the inputs, so that a
// lane's outputs still make one 16-byte store).  Elements past the line's end
// hold the identity.
template <class In, int VL, int BYTES = VL * int(sizeof(typename InTraits<In>::S))>
struct ChunkRaw {
    using type = std::conditional_t<
        VL == 1, typename InTraits<In>::S,
        std::conditional_t<BYTES == 16, u32x4, std::conditional_t<BYTES == 8, uint64_t, uint32_t>>>;
};

template <class In, class Acc, class Op, int VL>
struct Chunk {
    using S = typename InTraits<In>::S;
    static constexpr int V = VL;
    using Raw = typename ChunkRaw<In, VL>::type;
    static_assert(VL == 1 || sizeof(Raw) == VL * sizeof(S), "a lane's elements are one load");

    __device__ static Raw load(const S *x, int64_t i, int64_t m)
    {
        Raw r{};
        if (i < m) {
            if constexpr (VL == 1)
                r = load1(x + i);
            else if constexpr (sizeof(Raw) == 16)
                r = load16(reinterpret_cast<const u32x4 *>(x + i));
            else
                r = load1(reinterpret_cast<const Raw *>(x + i));
        }
        return r;
    }

    __device__ static void decode(Raw r, bool valid, Acc (&e)[V])
    {
        if constexpr (VL == 1) {
            e[0] = InTraits<In>::template one<Acc>(r);
        } else if constexpr (VL == InTraits<In>::vec) {
            InTraits<In>::template decode<Acc>(r, e);
        } else {
            S t[VL];
            __builtin_memcpy(t, &r, sizeof r);
#pragma unroll
            for (int i = 0; i < V; ++i)
                e[i] = InTraits<In>::template one<Acc>(t[i]);
        }
#pragma unroll
        for (int i = 0; i < V; ++i)
            e[i] = valid ? e[i] : Op::template identity<Acc>();
    }
};

// Scan of one chunk: the lane's exclusive offset inside the chunk and the
// chunk's total (wave-uniform).
template <class Acc, class Op, int V>
__device__ __forceinline__ void chunk_scan(const Acc (&e)[V], Acc &lane_excl, Acc &total)
{
    Acc t = e[0];
#pragma unroll
    for (int i = 1; i < V; ++i)
        t = Op::apply(t, e[i]);
    const Acc incl = wave_scan_incl<Op>(t);
    total = read_lane(incl, 63);
    lane_excl = lane_prev(incl, Op::template identity<Acc>());
}

// Outputs of one chunk from `run` = everything before the lane's first element.
template <class Acc, class Op, int V>
__device__ __forceinline__ void chunk_outputs(const Acc (&e)[V], Acc run, bool inclusive, Acc (&o)[V])
{
#pragma unroll
    for (int i = 0; i < V; ++i) {
        if (inclusive) {
            run = Op::apply(run, e[i]);
            o[i] = run;
        } else {
            o[i] = run;
            run = Op::apply(run, e[i]);
        }
    }
}

// ------------------------------------------------------- look-back state

// Flags: 0 nothing yet, 1 aggregate, 2 inclusive prefix.  A value is stored,
// its store waited for, and only then its flag, all at device scope; a
// reader loads the flag first and the value after it.  The timeout word is
// nonzero if a look-back wait gave up (never in normal runs).
//
// With a library slot (ScanArgs::slot >= 0) the counter, timeout word and
// flags live in library memory instead of the workspace.  It starts zeroed
// and the last block of every scan puts it back to zero, so no launch has to
// clear it; the workspace header then receives the call's tile count and
// timeout word.  Calls on one stream share its slot in order; calls that may
// overlap have different slots.
constexpr uint32_t kFlagAggregate = 1;
constexpr uint32_t kFlagPrefix = 2;

// Columns-scan state: the header, flags and values laid out as the plan
// describes them (scan_columns_state_bytes); the flags of neighbouring tiles
// sit in different 128-byte lines, for the reason given for the tile scan's
// records below.
constexpr int kScanSlotWords = 64 + kScanFlagCapacity;
namespace RK_UNIT {
static __device__ __attribute__((aligned(128))) uint32_t g_scan_state[kArriveSlots * kScanSlotWords];
}
using RK_UNIT::g_scan_state;

struct ScanState {
    uint32_t *counter;
    uint32_t *timeout;
    uint32_t *done;       // slot state only: blocks finished, wraps to zero
    uint32_t *flagw;      // flag words
    uint32_t lines;       // flag lines
    uint64_t *aggs;
    uint64_t *pres;

    __device__ ScanState(void *ws, int64_t tiles, int slot, int64_t width = 1)
    {
        uint32_t *w = static_cast<uint32_t *>(ws);
        lines = (uint32_t)scan_flag_lines(tiles);
        aggs = reinterpret_cast<uint64_t *>(w + 64 + int64_t(lines) * 32);
        pres = aggs + tiles * width;
        uint32_t *h = slot >= 0 ? g_scan_state + int64_t(slot) * kScanSlotWords : w;
        counter = h;
        timeout = h + 1;
        done = slot >= 0 ? h + 32 : nullptr;   // a line of its own
        flagw = h + 64;
    }
    __device__ uint32_t *flag(int64_t g) const
    {
        const uint32_t u = (uint32_t)g;
        return flagw + (u % lines) * 32 + u / lines;
    }
};

// Tile-scan state: the header and per-tile records laid out as the plan
// describes them (kScanHeaderBytes, kScanRecBytes).  Device-scope accesses to
// one 128-byte line are serialised where they are performed, so the tiles
// that publish and poll at the same time -- neighbours -- are kept in
// different lines, and a reader finds a tile's flag and values in one line.
constexpr int kScanTileSlotWords = (kScanHeaderBytes + kScanRecCapacity * kScanRecBytes) / 4;
namespace RK_UNIT {
static __device__ __attribute__((aligned(128))) uint32_t g_scan_tile_state[kArriveSlots * kScanTileSlotWords];
}
using RK_UNIT::g_scan_tile_state;

struct TileState {
    uint32_t *counter;
    uint32_t *timeout;
    uint32_t *done;       // slot state only: blocks finished, wraps to zero
    char *recs;
    uint32_t lines;       // tile counts fit 32 bits (the counter is a 32-bit word)

    __device__ TileState(void *ws, int64_t tiles, int slot)
    {
        uint32_t *h = slot >= 0 ? g_scan_tile_state + int64_t(slot) * kScanTileSlotWords : static_cast<uint32_t *>(ws);
        counter = h;
        timeout = h + 1;
        done = slot >= 0 ? h + 32 : nullptr;  // a line of its own
        recs = reinterpret_cast<char *>(h) + kScanHeaderBytes;
        lines = (uint32_t)scan_rec_lines(tiles);
    }
    __device__ char *rec(int64_t g) const
    {
        const uint32_t u = (uint32_t)g;
        return recs + int64_t((u % lines) * 4 + u / lines) * kScanRecBytes;
    }
    __device__ uint32_t *flag(int64_t g) const { return reinterpret_cast<uint32_t *>(rec(g)); }
    template <class Acc>
    __device__ Acc *value(int64_t g, uint32_t flag) const
    {
        return reinterpret_cast<Acc *>(rec(g) + (flag == kFlagPrefix ? 16 : 8));
    }
};

// End of a block of a slot-state scan, run by wave 0 alone once the block's
// outputs are issued (the other waves end without waiting): lane 0 waits for
// its flag and output stores, then counts the block done; the last block of
// the call (every look-back has ended by then) copies the tile count and the
// timeout word into the workspace header and zeroes the counter, the timeout
// word and `nflags` flags (stride `fstride` words) for the next call.
__device__ __forceinline__ void release_slot(uint32_t *done, int64_t tiles, uint32_t *counter, uint32_t *timeout,
                                             uint32_t *flags, int64_t nflags, int64_t fstride, void *ws)
{
    if (!done || threadIdx.x >= 64)
        return;
    uint32_t prev = 0;
    if (threadIdx.x == 0) {
        wait_stores();
        prev = __builtin_amdgcn_atomic_inc32(done, (uint32_t)(tiles - 1), __ATOMIC_RELAXED, "agent");
    }
    prev = __builtin_amdgcn_readfirstlane(prev);
    if (prev != (uint32_t)(tiles - 1))
        return;
    for (int64_t i = threadIdx.x; i < nflags; i += 64)
        flags[i * fstride] = 0;
    if (threadIdx.x == 0) {
        uint32_t *hdr = static_cast<uint32_t *>(ws);
        hdr[0] = __hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        hdr[1] = __hip_atomic_load(timeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(timeout, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

__device__ __forceinline__ void scan_release(const ScanState &st, void *ws, int64_t tiles)
{
    release_slot(st.done, tiles, st.counter, st.timeout, st.flagw, int64_t(st.lines) * 32, 1, ws);
}

__device__ __forceinline__ void tile_release(const TileState &st, void *ws, int64_t tiles)
{
    release_slot(st.done, tiles, st.counter, st.timeout, reinterpret_cast<uint32_t *>(st.recs),
                 int64_t(st.lines) * 4, kScanRecBytes / 4, ws);
}

template <class Acc>
__device__ __forceinline__ void publish(const TileState &st, int64_t g, Acc v, uint32_t flag)
{
    store_partial(st.value<Acc>(g, flag), v);
    wait_stores();
    __hip_atomic_store(st.flag(g), flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Exclusive prefix of tile t (global index g) of a line, run by one whole
// wave: publish the tile's aggregate, then read the predecessors 64 at a time
// (lane 0 the nearest) until one with its inclusive prefix.  Every tile with
// a smaller counter value has already started, and it publishes its
// aggregate without waiting on anything, so every wait here ends.  As a
// safety net each wait is still bounded (a.spin_limit sleeps): past it the
// tile records the timeout in the header and in the library's count of waits
// that gave up, and goes on, so every wave exits.  Publishes the tile's own
// inclusive prefix before returning.
template <class Acc, class Op>
__device__ Acc scan_lookback(const TileState &st, const ScanArgs &a, int64_t g, int64_t t, Acc agg, Acc init)
{
    const int lane = lane_id();
    if (t == 0) {
        if (lane == 0)
            publish(st, g, Op::apply(init, agg), kFlagPrefix);
        return init;
    }
    if (lane == 0)
        publish(st, g, agg, kFlagAggregate);
    const int64_t g0 = g - t;                  // the line's first tile
    Acc acc = Op::template identity<Acc>();    // fold of the tiles after the window
    int64_t top = t - 1;
    for (;;) {
        const int64_t j = top - lane;
        const bool valid = j >= 0;
        uint32_t f;
        uint64_t pm, zm;
        for (uint32_t spin = 0;; ++spin) {
            f = valid ? __hip_atomic_load(st.flag(g0 + j), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : kFlagPrefix;
            pm = __ballot(f == kFlagPrefix);
            zm = __ballot(f == 0);
            // done when every lane before the first prefix has published
            const uint64_t need = pm ? (pm & (0 - pm)) - 1 : ~uint64_t(0);
            if ((zm & need) == 0 && !a.force_wait)
                break;
            if (spin >= a.spin_limit) {
                if (lane == 0) {
                    __hip_atomic_store(st.timeout, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    record_timeout(a.slot);
                }
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        const int first = pm ? __builtin_ctzll(pm) : 64;   // lane of the nearest prefix
        Acc v = Op::template identity<Acc>();
        if (valid && lane <= first)
            v = load_partial(st.value<Acc>(g0 + j, lane == first ? kFlagPrefix : kFlagAggregate));
        acc = Op::apply(wave_reduce<Op>(v), acc);
        if (pm)
            break;
        top -= 64;
    }
    if (lane == 0)
        publish(st, g, Op::apply(acc, agg), kFlagPrefix);
    return acc;
}

// ------------------------------------------------------------------ kernels

// Zero the tile counter and flags before a tile scan (a fill kernel, not a
// memset, so the call can be captured in a graph).
template <int BLOCK>
__global__ __launch_bounds__(BLOCK) void k_scan_clear(uint32_t *w, int64_t words)
{
    for (int64_t i = int64_t(blockIdx.x) * BLOCK + threadIdx.x; i < words; i += int64_t(gridDim.x) * BLOCK)
        w[i] = 0;
}

// Tile kernel: a tile is NW waves x UC chunks of consecutive elements of one
// line; tiles are numbered by a counter in the order blocks start.
// STR = 1: the outputs of a line are s_out apart (the scan dim contiguous in
// the input only: a few rows of a row-major matrix along their rows), each
// stored on its own.  STR = 2: the inputs are s_in apart (the scan dim
// contiguous in the output only), loaded one element a lane.
template <class In, class Acc, class Op, int BLOCK, int U, int VL, bool NTS = false, int STR = 0>
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(4))) void k_scan_tile(ScanArgs a)
{
    static_assert(STR != 2 || VL == 1, "strided inputs take element loads");
    using C = Chunk<In, Acc, Op, VL>;
    using S = typename C::S;
    constexpr int V = C::V;
    constexpr int UC = scan_lane_chunks(U, InTraits<In>::vec, VL);   // chunks per lane (the plan's tile size)
    constexpr int64_t CH = 64 * V;
    constexpr int NW = BLOCK / 64;
    constexpr int64_t T = int64_t(NW) * UC * CH;

    __shared__ uint32_t s_id;
    __shared__ Acc s_wave[NW];
    __shared__ Acc s_excl;
    const TileState st(a.ws, a.tiles, a.slot);
    if (threadIdx.x == 0)
        s_id = __hip_atomic_fetch_add(st.counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int64_t g = s_id;
    if (g >= a.tiles) {                        // never: the counter starts at zero every call
        if (threadIdx.x == 0) {
            __hip_atomic_store(st.timeout, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            record_timeout(a.slot);
        }
        return;
    }
    // tiles, and so lines, number below 2^31: 32-bit arithmetic
    const uint32_t line32 = uint32_t(g) / uint32_t(a.tiles_per_line);
    const int64_t line = line32;
    const int64_t t = g - line * a.tiles_per_line;
    const S *x = static_cast<const S *>(a.x) + layout_offset32(a.kept_nd, a.kept_ext, a.kept_in, line32);
    const int64_t ob = layout_offset32(a.kept_nd, a.kept_ext, a.kept_out, line32);
    // the wave's number, read as uniform so that its arithmetic is scalar
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int64_t first = t * T + int64_t(w) * UC * CH + int64_t(lane_id()) * V;
    // this lane's chunks inside the line, a count rather than a 64-bit index
    // per chunk held from the loads to the stores
    const int nk = first < a.m ? (int)((a.m - first + CH - 1) / CH < UC ? (a.m - first + CH - 1) / CH : UC) : 0;

    typename C::Raw raw[UC];
#pragma unroll
    for (int k = 0; k < UC; ++k) {
        raw[k] = typename C::Raw{};
        if (k < nk) {
            if constexpr (STR == 2)
                raw[k] = load1(x + (first + k * CH) * a.s_in);
            else
                raw[k] = C::load(x, first + k * CH, a.m);
        }
    }
    issue_barrier();

    // the wave's total first (the look-back needs only the tile's); the
    // chunks are scanned after it, so no per-chunk state is held across it
    Acc lt = Op::template identity<Acc>();
#pragma unroll
    for (int k = 0; k < UC; ++k) {
        Acc e[V];
        C::decode(raw[k], k < nk, e);
#pragma unroll
        for (int i = 0; i < V; ++i)
            lt = Op::apply(lt, e[i]);
    }
    const Acc wt = wave_reduce<Op>(lt);
    if (lane_id() == 0)
        s_wave[w] = wt;
    __syncthreads();
    Acc agg = s_wave[0], wpre = Op::template identity<Acc>();
#pragma unroll
    for (int v = 1; v < NW; ++v) {
        if (v == w)
            wpre = agg;
        agg = Op::apply(agg, s_wave[v]);
    }
    if (w == 0) {
        const Acc excl = scan_lookback<Acc, Op>(st, a, g, t, agg, from_bits<Acc>(a.init_bits));
        if (lane_id() == 0)
            s_excl = excl;
    }
    __syncthreads();

    // decode the raw loads again below rather than keeping the first decode
    // alive across the look-back (wider accumulators would double the registers)
#pragma unroll
    for (int k = 0; k < UC; ++k)
        asm volatile("" : "+v"(raw[k]));
    Acc carry = Op::apply(s_excl, wpre);
#pragma unroll
    for (int k = 0; k < UC; ++k) {
        Acc e[V], o[V], lane_excl, total;
        C::decode(raw[k], k < nk, e);
        chunk_scan<Acc, Op, V>(e, lane_excl, total);
        chunk_outputs<Acc, Op, V>(e, Op::apply(carry, lane_excl), a.inclusive != 0, o);
        if (k < nk) {
            if constexpr (STR == 1) {
#pragma unroll
                for (int i = 0; i < V; ++i) {
                    const Acc w[1] = {o[i]};
                    store_run<Acc, 1>(a.out, ob + (first + k * CH + i) * a.s_out, a.out_dtype, w);
                }
            } else {
                store_run<Acc, V, NTS>(a.out, ob + first + k * CH, a.out_dtype, o);
            }
        }
        carry = Op::apply(carry, total);
    }
    tile_release(st, a.ws, a.tiles);
}

// Row-wave kernel: one wave per line, UC chunks in flight, the carry passed
// from chunk to chunk.
template <class In, class Acc, class Op, int BLOCK, int U, int VL, bool NTS = true>
__global__ __launch_bounds__(BLOCK) void k_scan_rowwave(ScanArgs a)
{
    using C = Chunk<In, Acc, Op, VL>;
    using S = typename C::S;
    constexpr int V = C::V;
    constexpr int UC = scan_lane_chunks(U, InTraits<In>::vec, VL);
    constexpr int64_t CH = 64 * V;
    // the wave's number, read as uniform so that the index arithmetic runs on
    // the scalar unit
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int64_t line = int64_t(blockIdx.x) * (BLOCK / 64) + wave;
    if (line >= a.lines)
        return;                                // whole wave; no block barrier below
    // lines number below 2^33 here (grid below 2^31, 4 waves a block): the
    // 32-bit form whenever the count fits
    const bool small = uint64_t(a.lines) <= 0xffffffffu;
    const S *x = static_cast<const S *>(a.x) + (small ? layout_offset32(a.kept_nd, a.kept_ext, a.kept_in, uint32_t(line))
                                                      : layout_offset(a.kept_nd, a.kept_ext, a.kept_in, line));
    const int64_t ob = small ? layout_offset32(a.kept_nd, a.kept_ext, a.kept_out, uint32_t(line))
                             : layout_offset(a.kept_nd, a.kept_ext, a.kept_out, line);
    Acc carry = from_bits<Acc>(a.init_bits);
    for (int64_t c0 = int64_t(lane_id()) * V; c0 - int64_t(lane_id()) * V < a.m; c0 += UC * CH) {
        typename C::Raw raw[UC];
#pragma unroll
        for (int k = 0; k < UC; ++k)
            raw[k] = C::load(x, c0 + k * CH, a.m);
        issue_barrier();
#pragma unroll
        for (int k = 0; k < UC; ++k) {
            const int64_t i = c0 + k * CH;
            Acc e[V], o[V], lane_excl, total;
            C::decode(raw[k], i < a.m, e);
            chunk_scan<Acc, Op, V>(e, lane_excl, total);
            chunk_outputs<Acc, Op, V>(e, Op::apply(carry, lane_excl), a.inclusive != 0, o);
            if (i < a.m)
                store_run<Acc, V, NTS>(a.out, ob + i, a.out_dtype, o);
            carry = Op::apply(carry, total);
        }
    }
}

// Columns kernel: a strided scan dim over runs of contiguous lines (kept dim
// 0).  A tile is W = CL * V consecutive lines of one run by R = RG * RPG
// consecutive scan positions; row group rg of the block scans positions
// rg*RPG .. rg*RPG+RPG-1 for its V lines with 16-byte loads (a wave reads
// 64 / CL rows of W lines per instruction), the row groups' totals are
// combined through LDS, and the tile's prefix along the scan dim comes from
// the tiles before it by decoupled look-back (numbered chunk-major, so the
// tiles a tile waits on started before it).  Row group 0 does the look-back,
// each thread for its own lines, a window of K predecessors at a time.
template <class In, class Acc, class Op, int BLOCK, int CL, int RPG, bool VECTOR>
__global__ __launch_bounds__(BLOCK) void k_scan_columns(ScanArgs a)
{
    using S = typename InTraits<In>::S;
    constexpr int V = VECTOR ? InTraits<In>::vec : 1;
    constexpr int W = CL * V;
    constexpr int RG = BLOCK / CL;
    constexpr int64_t R = int64_t(RG) * RPG;
    constexpr int K = 8;
    using Raw = std::conditional_t<VECTOR, u32x4, S>;
    static_assert(BLOCK % CL == 0, "whole row groups");

    __shared__ uint32_t s_id;
    __shared__ Acc s_part[RG][W];
    __shared__ Acc s_excl[W];
    const ScanState st(a.ws, a.tiles, a.slot, W);
    if (threadIdx.x == 0)
        s_id = __hip_atomic_fetch_add(st.counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const uint32_t gu = s_id;
    if (gu >= a.tiles) {                       // never: the counter starts at zero every call
        if (threadIdx.x == 0) {
            __hip_atomic_store(st.timeout, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            record_timeout(a.slot);
        }
        return;
    }
    // tile numbers fit 32 bits (the plan refuses more), so they split in 32-bit
    // arithmetic: chunk t along the scan dim, tile ct across the lines
    const uint32_t t32 = gu / (uint32_t)a.col_tiles;
    const uint32_t ct32 = gu - t32 * (uint32_t)a.col_tiles;
    const uint32_t run32 = ct32 / (uint32_t)a.col_tiles_per_run;
    const int64_t g = gu, t = t32, ct = ct32;
    const int64_t col0 = int64_t(ct32 - run32 * (uint32_t)a.col_tiles_per_run) * W;
    const int c = (int)(threadIdx.x % CL), rg = (int)(threadIdx.x / CL);
    const int64_t run_len = a.kept_ext[0];
    const int64_t col = col0 + int64_t(c) * V;
    const bool active = col < run_len;                 // 16-byte loads: run_len % V == 0
    const int64_t r0 = t * R + int64_t(rg) * RPG;
    // this thread's positions r0 .. r0+nv-1 exist (none for lines past the run);
    // one count instead of a 64-bit row index per position keeps registers free
    const int nv = active ? (int)(a.m - r0 < RPG ? (a.m - r0 > 0 ? a.m - r0 : 0) : RPG) : 0;
    const S *x = static_cast<const S *>(a.x) +
                 layout_offset(a.kept_nd - 1, a.kept_ext + 1, a.kept_in + 1, int64_t(run32)) + col;
    const int64_t xo = r0 * a.s_in;
    const int64_t ob = layout_offset(a.kept_nd - 1, a.kept_ext + 1, a.kept_out + 1, int64_t(run32)) + col +
                       r0 * a.s_out;

    Raw raw[RPG];
#pragma unroll
    for (int q = 0; q < RPG; ++q) {
        raw[q] = Raw{};
        if (q < nv) {
            if constexpr (VECTOR)
                raw[q] = load16(reinterpret_cast<const u32x4 *>(x + (xo + q * a.s_in)));
            else
                raw[q] = load1(x + (xo + q * a.s_in));
        }
    }
    issue_barrier();

    // this thread's totals over its RPG positions, per line
    Acc tot[V];
    set_identity<Acc, Op>(tot);
#pragma unroll
    for (int q = 0; q < RPG; ++q) {
        Acc e[V];
        Chunk<In, Acc, Op, V>::decode(raw[q], q < nv, e);
#pragma unroll
        for (int i = 0; i < V; ++i)
            tot[i] = Op::apply(tot[i], e[i]);
    }
#pragma unroll
    for (int i = 0; i < V; ++i)
        s_part[rg][c * V + i] = tot[i];
    __syncthreads();
    // offset of this row group and the tile's aggregate, per line.  The loop
    // over row groups stays rolled: unrolled, every running value would stay
    // live until the pick by rg (RG * V registers on top of the raw loads).
    Acc gpre[V], agg[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        gpre[i] = Op::template identity<Acc>();
        agg[i] = Op::template identity<Acc>();
    }
#pragma unroll 1
    for (int k = 0; k < RG; ++k) {
#pragma unroll
        for (int i = 0; i < V; ++i) {
            if (k == rg)
                gpre[i] = agg[i];
            agg[i] = Op::apply(agg[i], s_part[k][c * V + i]);
        }
    }
    // tile g's W partials, packed as Acc, element i of thread c at i * CL + c:
    // the stores go through to memory, so one instruction must cover whole lines
    const int64_t slot = g * W + c;
    if (t > 0) {
        if (rg == 0 && active) {
#pragma unroll
            for (int i = 0; i < V; ++i)
                store_partial(reinterpret_cast<Acc *>(st.aggs) + slot + i * CL, agg[i]);
            wait_stores();
        }
        __syncthreads();
        if (threadIdx.x == 0)
            __hip_atomic_store(st.flag(g), kFlagAggregate, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (rg == 0) {
        Acc acc[V];
        const Acc init = from_bits<Acc>(a.init_bits);
#pragma unroll
        for (int i = 0; i < V; ++i)
            acc[i] = t == 0 ? init : Op::template identity<Acc>();
        if (t > 0 && active) {
            int64_t top = t - 1;
            for (;;) {
                uint32_t f[K];
#pragma unroll
                for (int q = 0; q < K; ++q)
                    f[q] = top - q >= 0 ? __hip_atomic_load(st.flag((top - q) * a.col_tiles + ct), __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT)
                                        : kFlagPrefix;
                int first = K;
                for (uint32_t spin = 0;; ++spin) {
                    first = K;
                    bool ready = !a.force_wait;
#pragma unroll
                    for (int q = K - 1; q >= 0; --q)
                        if (f[q] == kFlagPrefix)
                            first = q;
#pragma unroll
                    for (int q = 0; q < K; ++q)
                        if (q < first && f[q] == 0)
                            ready = false;
                    if (ready)
                        break;
                    if (spin >= a.spin_limit) {
                        __hip_atomic_store(st.timeout, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        record_timeout(a.slot);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
#pragma unroll
                    for (int q = 0; q < K; ++q)
                        if (f[q] == 0 && top - q >= 0)
                            f[q] = __hip_atomic_load(st.flag((top - q) * a.col_tiles + ct), __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
                }
#pragma unroll
                for (int q = 0; q < K; ++q) {
                    const int64_t j = top - q;
                    if (q <= first && j >= 0) {
                        const Acc *src = reinterpret_cast<const Acc *>(f[q] == kFlagPrefix ? st.pres : st.aggs);
                        const int64_t js = (j * a.col_tiles + ct) * W + c;
#pragma unroll
                        for (int i = 0; i < V; ++i)
                            acc[i] = Op::apply(load_partial(src + js + i * CL), acc[i]);
                    }
                }
                if (first < K)
                    break;
                top -= K;
            }
        }
#pragma unroll
        for (int i = 0; i < V; ++i) {
            s_excl[c * V + i] = acc[i];
            if (active)
                store_partial(reinterpret_cast<Acc *>(st.pres) + slot + i * CL, Op::apply(acc[i], agg[i]));
        }
        wait_stores();
    }
    __syncthreads();
    if (threadIdx.x == 0)
        __hip_atomic_store(st.flag(g), kFlagPrefix, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // decode the raw loads again below rather than keeping the first decode
    // alive across the look-back (wider accumulators would double the registers)
#pragma unroll
    for (int q = 0; q < RPG; ++q)
        asm volatile("" : "+v"(raw[q]));
    Acc runv[V];
#pragma unroll
    for (int i = 0; i < V; ++i)
        runv[i] = Op::apply(s_excl[c * V + i], gpre[i]);
#pragma unroll
    for (int q = 0; q < RPG; ++q) {
        Acc e[V], o[V];
        Chunk<In, Acc, Op, V>::decode(raw[q], q < nv, e);
#pragma unroll
        for (int i = 0; i < V; ++i) {
            if (a.inclusive) {
                runv[i] = Op::apply(runv[i], e[i]);
                o[i] = runv[i];
            } else {
                o[i] = runv[i];
                runv[i] = Op::apply(runv[i], e[i]);
            }
        }
        if (q < nv)
            store_run<Acc, V, true>(a.out, ob + q * a.s_out, a.out_dtype, o);
    }
    scan_release(st, a.ws, a.tiles);
}

// Lines kernel: one thread per line walking the scan dim, UNROLL elements in
// flight.  Consecutive threads take consecutive lines (the first kept dim).
template <class In, class Acc, class Op, int BLOCK, int UNROLL>
__global__ __launch_bounds__(BLOCK) void k_scan_lines(ScanArgs a)
{
    using S = typename InTraits<In>::S;
    for (int64_t line = int64_t(blockIdx.x) * BLOCK + threadIdx.x; line < a.lines;
         line += int64_t(gridDim.x) * BLOCK) {
        const S *x = static_cast<const S *>(a.x) + layout_offset(a.kept_nd, a.kept_ext, a.kept_in, line);
        const int64_t ob = layout_offset(a.kept_nd, a.kept_ext, a.kept_out, line);
        Acc run = from_bits<Acc>(a.init_bits);
        for (int64_t k0 = 0; k0 < a.m; k0 += UNROLL) {
            S v[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u)
                if (k0 + u < a.m)
                    v[u] = load1(x + (k0 + u) * a.s_in);
            issue_barrier();
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                if (k0 + u < a.m) {
                    const Acc e = InTraits<In>::template one<Acc>(v[u]);
                    Acc o[1];
                    if (a.inclusive) {
                        run = Op::apply(run, e);
                        o[0] = run;
                    } else {
                        o[0] = run;
                        run = Op::apply(run, e);
                    }
                    store_run<Acc, 1>(a.out, ob + (k0 + u) * a.s_out, a.out_dtype, o);
                }
            }
        }
    }
}

// Lines kernel, packed form, for lines contiguous along the scan dim in
// input and output and shorter than four waves (scan_lines_packed): a lane
// holds E consecutive elements, a line takes L = ceil(m / E) lanes and a wave
// 64 / L whole lines, lane j holding elements (j % L) * E, ... of its line
// j / L (the lanes past the last whole line idle).  A lane scans its own E
// elements, then the lines' lane totals go through a segmented wave scan: at
// distance d = 1, 2, 4, ... a lane folds in the lane d below it when that
// lane holds the same line.  An output is op(op(init, the lanes before), its
// lane's running value).  Waves stride over the groups of lines, U groups a
// round with their loads in flight together (one a round waited on memory
// latency every group).
//
// L32: the line count fits 32 bits, so a line's offsets take 32-bit
// divisions (the 64-bit ones sat on every group's path to its loads).
template <class In, class Acc, class Op, int BLOCK, int U, int E, bool L32>
__global__ __launch_bounds__(BLOCK) void k_scan_packed(ScanArgs a)
{
    using S = typename InTraits<In>::S;
    const int m = int(a.m);
    const int L = (m + E - 1) / E;
    const int per = 64 / L;
    const int lane = lane_id();
    const int g = lane / L;
    const int q = lane - g * L;
    const Acc init = from_bits<Acc>(a.init_bits);
    const int64_t groups = (a.lines + per - 1) / per;
    const int64_t nw = int64_t(gridDim.x) * (BLOCK / 64);
    for (int64_t w0 = int64_t(blockIdx.x) * (BLOCK / 64) + (threadIdx.x >> 6); w0 < groups; w0 += nw * U) {
        S raw[U][E];
        int64_t ob[U];
        bool act[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t line = (w0 + u * nw) * per + g;
            act[u] = g < per && w0 + u * nw < groups && line < a.lines;
            ob[u] = 0;
#pragma unroll
            for (int e = 0; e < E; ++e)
                raw[u][e] = S{};
            if (act[u]) {
                const S *x = static_cast<const S *>(a.x) +
                             (L32 ? layout_offset32(a.kept_nd, a.kept_ext, a.kept_in, uint32_t(line))
                                  : layout_offset(a.kept_nd, a.kept_ext, a.kept_in, line));
                ob[u] = L32 ? layout_offset32(a.kept_nd, a.kept_ext, a.kept_out, uint32_t(line))
                            : layout_offset(a.kept_nd, a.kept_ext, a.kept_out, line);
#pragma unroll
                for (int e = 0; e < E; ++e)
                    if (q * E + e < m)
                        raw[u][e] = load1(x + q * E + e);
            }
        }
        issue_barrier();
        Acc l[U][E], t[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            t[u] = Op::template identity<Acc>();
#pragma unroll
            for (int e = 0; e < E; ++e) {
                if (act[u] && q * E + e < m)
                    t[u] = Op::apply(t[u], InTraits<In>::template one<Acc>(raw[u][e]));
                l[u][e] = t[u];
            }
        }
        // each step's lane moves for all U groups at once, so their LDS
        // round trips overlap (group by group they went one at a time)
        for (int d = 1; d < L; d <<= 1) {
            Acc y[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                y[u] = __shfl_up(t[u], d, 64);
            if (q >= d) {
#pragma unroll
                for (int u = 0; u < U; ++u)
                    t[u] = Op::apply(y[u], t[u]);
            }
        }
        Acc before[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            before[u] = __shfl_up(t[u], 1, 64);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const Acc base = q == 0 ? init : Op::apply(init, before[u]);
            if (!act[u])
                continue;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                if (q * E + e < m) {
                    Acc o[1];
                    o[0] = a.inclusive ? Op::apply(base, l[u][e]) : e == 0 ? base : Op::apply(base, l[u][e - 1]);
                    store_run<Acc, 1>(a.out, ob[u] + q * E + e, a.out_dtype, o);
                }
            }
        }
    }
}

// A value kept in an LDS slot at least as wide as it.
template <class T, class Slot>
__device__ __forceinline__ void slot_put(Slot &s, T v)
{
    static_assert(sizeof(T) <= sizeof(Slot), "slot too narrow");
    __builtin_memcpy(&s, &v, sizeof(T));
}
template <class T, class Slot>
__device__ __forceinline__ T slot_get(const Slot &s)
{
    T v;
    __builtin_memcpy(&v, &s, sizeof(T));
    return v;
}

// Transposing kernel, for layouts whose input and output are contiguous
// along different axes (scan_tr_ta/tb/tp give a tile's extents for each
// mode).  A tile is TA x TB lines -- kept dims 0 and 1 after the plan's
// reordering, a and b -- by TP scan positions.  It is loaded with the
// input's contiguous axis across the lanes into LDS; each thread then scans
// its own lines along the positions there, its prefix per line from the
// tiles before it along the scan dim by decoupled look-back (tiles numbered
// chunk-major, as in the columns kernel; wave 0 polls a window of 64
// predecessors' flags and every thread folds its own lines' values), and
// writes the outputs back into the same slots; the tile is then stored with
// the output's contiguous axis across the lanes.  Column c of LDS row p sits
// at c ^ ((p + c / 32) % 32): a row, a column, and the b axis at a fixed a
// each cover 32 banks.
template <class In, class Acc, class Op, int MODE>
__global__ __launch_bounds__(tune::kScanTrBlock) void k_scan_transpose(ScanArgs a)
{
    using S = typename InTraits<In>::S;
    constexpr int BLOCK = tune::kScanTrBlock;
    constexpr int SB = (sizeof(S) > sizeof(Acc) ? sizeof(S) : sizeof(Acc)) > 4 ? 8 : 4;
    using Slot = std::conditional_t<SB == 8, uint64_t, uint32_t>;
    constexpr int TA = scan_tr_ta(MODE), TB = scan_tr_tb(MODE), TL = TA * TB, TP = scan_tr_tp(MODE, SB);
    constexpr int LPT = TL / BLOCK;            // lines per thread
    constexpr int EPT = TL * TP / BLOCK;       // tile elements per thread
    static_assert(TL % BLOCK == 0 && TL % 32 == 0 && BLOCK % TP == 0 && EPT % 16 == 0, "tile geometry");

    __shared__ Slot tile[TL * TP];
    __shared__ uint32_t s_id;
    __shared__ int s_first;
    const ScanState st(a.ws, a.tiles, a.slot, TL);
    if (threadIdx.x == 0)
        s_id = __hip_atomic_fetch_add(st.counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const uint32_t gu = s_id;
    if (gu >= a.tiles) {                       // never: the counter starts at zero every call
        if (threadIdx.x == 0) {
            __hip_atomic_store(st.timeout, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            record_timeout(a.slot);
        }
        return;
    }
    // chunk t along the scan dim, line tile ct = (run, tile along b, tile along a)
    const uint32_t t32 = gu / (uint32_t)a.col_tiles;
    const uint32_t ct32 = gu - t32 * (uint32_t)a.col_tiles;
    const uint32_t run32 = ct32 / (uint32_t)a.col_tiles_per_run;
    const uint32_t rem = ct32 - run32 * (uint32_t)a.col_tiles_per_run;
    const uint32_t nta = (uint32_t)((a.kept_ext[0] + TA - 1) / TA);
    const uint32_t tbi = rem / nta, tai = rem - tbi * nta;
    const int64_t g = gu, t = t32, ct = ct32;
    const int64_t a0 = int64_t(tai) * TA, b0 = int64_t(tbi) * TB, p0 = t * TP;
    const int na = (int)(a.kept_ext[0] - a0 < TA ? a.kept_ext[0] - a0 : TA);
    const int nb = (int)(a.kept_ext[1] - b0 < TB ? a.kept_ext[1] - b0 : TB);
    const int np = (int)(a.m - p0 < TP ? a.m - p0 : TP);
    const int64_t sb_in = a.kept_in[1], sa_out = a.kept_out[0];
    const S *x = static_cast<const S *>(a.x) + layout_offset32(a.kept_nd - 2, a.kept_ext + 2, a.kept_in + 2, run32) +
                 a0 * a.kept_in[0] + b0 * sb_in + p0 * a.s_in;
    const int64_t ob = layout_offset32(a.kept_nd - 2, a.kept_ext + 2, a.kept_out + 2, run32) + a0 * sa_out +
                       b0 * a.kept_out[1] + p0 * a.s_out;
    auto at = [](int ia, int ib, int ip) {
        const int c = ia + TA * ib;
        return ip * TL + (c ^ ((ip + (c >> 5)) & 31));
    };

    // loads: element e of the tile with the input's contiguous axis fastest
    // (p in mode 0, a otherwise; that axis has input stride 1).  Every lane
    // loads, those past the view's edge the tile's first element (never
    // used): loads under a branch each were issued one at a time.
    S raw[EPT];
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
        const int e = int(threadIdx.x) + k * BLOCK;
        const int ia = MODE == 0 ? 0 : e % TA;
        const int ib = MODE == 0 ? e / TP : (e / TA) % TB;
        const int ip = MODE == 0 ? e % TP : e / TL;
        const int64_t off = MODE == 0 ? ip + ib * sb_in : ia + ib * sb_in + ip * a.s_in;
        raw[k] = load1(x + (ia < na && ib < nb && ip < np ? off : 0));
    }
    issue_barrier();
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
        const int e = int(threadIdx.x) + k * BLOCK;
        const int ia = MODE == 0 ? 0 : e % TA;
        const int ib = MODE == 0 ? e / TP : (e / TA) % TB;
        const int ip = MODE == 0 ? e % TP : e / TL;
        if (ia < na && ib < nb && ip < np)
            slot_put<S>(tile[at(ia, ib, ip)], raw[k]);
    }
    __syncthreads();

    // this thread's lines c = threadIdx.x + j * BLOCK, every position of them
    // read from LDS at once (those past the view's edge hold no input and are
    // left out of the totals; their outputs are never stored)
    S vals[LPT][TP];
    Acc tot[LPT];
    bool act[LPT];
#pragma unroll
    for (int j = 0; j < LPT; ++j) {
        const int c = int(threadIdx.x) + j * BLOCK, ia = c % TA, ib = c / TA;
        act[j] = ia < na && ib < nb;
#pragma unroll
        for (int p = 0; p < TP; ++p)
            vals[j][p] = slot_get<S>(tile[at(ia, ib, p)]);
    }
#pragma unroll
    for (int j = 0; j < LPT; ++j) {
        tot[j] = Op::template identity<Acc>();
#pragma unroll
        for (int p = 0; p < TP; ++p)
            if (p < np)
                tot[j] = Op::apply(tot[j], InTraits<In>::template one<Acc>(vals[j][p]));
    }
    // the tile's per-line values, packed as Acc: line c of tile g at g * TL + c
    const int64_t slot = g * TL + threadIdx.x;
    if (t > 0) {
#pragma unroll
        for (int j = 0; j < LPT; ++j)
            if (act[j])
                store_partial(reinterpret_cast<Acc *>(st.aggs) + slot + j * BLOCK, tot[j]);
        wait_stores();
        __syncthreads();
        if (threadIdx.x == 0)
            __hip_atomic_store(st.flag(g), kFlagAggregate, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    Acc acc[LPT];
    const Acc init = from_bits<Acc>(a.init_bits);
#pragma unroll
    for (int j = 0; j < LPT; ++j)
        acc[j] = t == 0 ? init : Op::template identity<Acc>();
    if (t > 0) {
        int64_t top = t - 1;
        for (;;) {
            if (threadIdx.x < 64) {
                const int64_t jt = top - int64_t(threadIdx.x);
                uint64_t pm = 0;
                for (uint32_t spin = 0;; ++spin) {
                    const uint32_t f = jt >= 0 ? __hip_atomic_load(st.flag(jt * a.col_tiles + ct), __ATOMIC_RELAXED,
                                                                   __HIP_MEMORY_SCOPE_AGENT)
                                               : kFlagPrefix;
                    pm = __ballot(f == kFlagPrefix);
                    const uint64_t zm = __ballot(f == 0);
                    // done when every predecessor nearer than the first prefix has published
                    const uint64_t need = pm ? (pm & (0 - pm)) - 1 : ~uint64_t(0);
                    if ((zm & need) == 0 && !a.force_wait)
                        break;
                    if (spin >= a.spin_limit) {
                        if (threadIdx.x == 0) {
                            __hip_atomic_store(st.timeout, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            record_timeout(a.slot);
                        }
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
                if (threadIdx.x == 0)
                    s_first = pm ? __builtin_ctzll(pm) : 64;
            }
            __syncthreads();
            const int first = s_first;
            // the window's values, QB predecessors' loads in flight at a time
            constexpr int QB = 8;
            for (int q0 = 0; q0 <= first && q0 < 64 && top - q0 >= 0; q0 += QB) {
                Acc v[QB][LPT];
#pragma unroll
                for (int u = 0; u < QB; ++u) {
                    // unused slots load predecessor q0's values (in bounds, discarded)
                    const int q = q0 + u;
                    const bool use = q <= first && q < 64 && top - q >= 0;
                    const int qq = use ? q : q0;
                    const Acc *src = reinterpret_cast<const Acc *>(qq == first ? st.pres : st.aggs) +
                                     ((top - qq) * a.col_tiles + ct) * TL + threadIdx.x;
#pragma unroll
                    for (int j = 0; j < LPT; ++j) {
                        const Acc w = load_partial(src + j * BLOCK);
                        v[u][j] = use && act[j] ? w : Op::template identity<Acc>();
                    }
                }
#pragma unroll
                for (int u = 0; u < QB; ++u)
#pragma unroll
                    for (int j = 0; j < LPT; ++j)
                        acc[j] = Op::apply(v[u][j], acc[j]);
            }
            __syncthreads();                   // s_first is written again by the next window
            if (first < 64)
                break;
            top -= 64;
        }
    }
#pragma unroll
    for (int j = 0; j < LPT; ++j)
        if (act[j])
            store_partial(reinterpret_cast<Acc *>(st.pres) + slot + j * BLOCK, Op::apply(acc[j], tot[j]));
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0)
        __hip_atomic_store(st.flag(g), kFlagPrefix, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // outputs into this thread's own slots
#pragma unroll
    for (int j = 0; j < LPT; ++j) {
        const int c = int(threadIdx.x) + j * BLOCK, ia = c % TA, ib = c / TA;
        Acc run = acc[j];
#pragma unroll
        for (int p = 0; p < TP; ++p) {
            const Acc e = InTraits<In>::template one<Acc>(vals[j][p]);
            Acc o;
            if (a.inclusive) {
                run = Op::apply(run, e);
                o = run;
            } else {
                o = run;
                run = Op::apply(run, e);
            }
            slot_put<Acc>(tile[at(ia, ib, p)], o);
        }
    }
    __syncthreads();

    // stores: the output's contiguous axis fastest (p in mode 2, b otherwise;
    // that axis has output stride 1), SBATCH slots read from LDS ahead of
    // their stores, the output type fixed outside the loop
    auto store_tile = [&](auto od) {
        constexpr int OD = decltype(od)::value;
        constexpr int SBATCH = 16;
#pragma unroll
        for (int k0 = 0; k0 < EPT; k0 += SBATCH) {
            Acc o[SBATCH];
#pragma unroll
            for (int u = 0; u < SBATCH; ++u) {
                const int e = int(threadIdx.x) + (k0 + u) * BLOCK;
                const int ip = MODE == 2 ? e % TP : e / TL;
                const int ia = MODE == 2 ? e / TP : (e / TB) % TA;
                const int ib = MODE == 2 ? 0 : e % TB;
                o[u] = slot_get<Acc>(tile[at(ia, ib, ip)]);
            }
#pragma unroll
            for (int u = 0; u < SBATCH; ++u) {
                const int e = int(threadIdx.x) + (k0 + u) * BLOCK;
                const int ip = MODE == 2 ? e % TP : e / TL;
                const int ia = MODE == 2 ? e / TP : (e / TB) % TA;
                const int ib = MODE == 2 ? 0 : e % TB;
                if (ia < na && ib < nb && ip < np) {
                    const Acc w[1] = {o[u]};
                    const int64_t off = MODE == 2 ? ip + ia * sa_out : ib + ia * sa_out + ip * a.s_out;
                    store_run_as<OD, Acc, 1, true>(a.out, ob + off, w);
                }
            }
        }
    };
    if constexpr (std::is_floating_point_v<Acc>) {
        switch (a.out_dtype) {
        case F32: store_tile(std::integral_constant<int, F32>{}); break;
        case F64: store_tile(std::integral_constant<int, F64>{}); break;
        case BF16: store_tile(std::integral_constant<int, BF16>{}); break;
        case F16: store_tile(std::integral_constant<int, F16>{}); break;
        default: break;
        }
    } else {
        switch (a.out_dtype) {
        case I32: store_tile(std::integral_constant<int, I32>{}); break;
        case I64: store_tile(std::integral_constant<int, I64>{}); break;
        default: break;
        }
    }
    scan_release(st, a.ws, a.tiles);
}

// ---------------------------------------------------------------- launchers

// Zero the first `words` 32-bit words of the workspace: the look-back
// state's counter, timeout word and flags (workspace state).
inline void clear_state(const ScanArgs &a, int64_t words, hipStream_t st)
{
    const unsigned cg = (unsigned)std::min<int64_t>((words + 255) / 256, 1024);
    hipLaunchKernelGGL(k_scan_clear<256>, dim3(cg), dim3(256), 0, st, static_cast<uint32_t *>(a.ws), words);
}

template <class In, class Acc, class Op>
int run_scan_typed(const ScanLaunch &L)
{
    hipStream_t st = static_cast<hipStream_t>(L.stream);
    const dim3 grid((unsigned)L.grid), block((unsigned)L.block);
    constexpr int B = tune::kScanBlock;
    constexpr int BT = tune::kScanTileBlock;
    constexpr int U = tune::kScanUnroll;
    constexpr int UT = tune::kScanTileUnroll;
    constexpr int UW = tune::kScanWaveUnroll;
    constexpr int BC = tune::kScanColBlock;
    if (L.kernel == SK_COLUMNS ? L.block != BC
        : L.kernel == SK_TRANSPOSE ? L.block != tune::kScanTrBlock
                                   : (L.block != B && !(L.kernel == SK_TILE && L.block == BT)))
        return ST_INVALID;
    // a ScanLaunch carries no Launch; launch_first only reads the events
    Launch ev;
    ev.ev_begin = L.ev_begin;
    ev.ev_end = L.ev_end;
    // elements per lane of the tile and row-wave kernels: the input's 16-byte
    // vector, the accumulator's (outputs wider than inputs), or one
    constexpr int VV = InTraits<In>::vec;
    constexpr int VW = int(16 / sizeof(Acc)) < VV ? int(16 / sizeof(Acc)) : VV;
    const int vl = L.vec;
    if (vl != 1 && vl != VV && vl != VW)
        return ST_INVALID;
    switch (L.kernel) {
    case SK_TILE: {
        if (L.args.slot < 0)
            clear_state(L.args, scan_tile_state_bytes(L.args.tiles) / 4, st);
#define RK_SCAN_TILE(BK, UK, VLN) launch_first(&k_scan_tile<In, Acc, Op, BK, UK, VLN, true>, grid, block, st, ev, L.args)
#define RK_SCAN_TILE_STR(BK, UK, VLN, SK)                                                                     \
    launch_first(&k_scan_tile<In, Acc, Op, BK, UK, VLN, true, SK>, grid, block, st, ev, L.args)
        if (L.tstr == 1) {                       // strided outputs: the input's vector or element loads
            // large tiles only while a lane's vector of accumulators stays within 32 bytes
            // (bf16 or f16 into f64 went to scratch memory there)
            constexpr bool large_ok = VV * sizeof(Acc) <= 32;
            if (L.block == B && vl == VV) RK_SCAN_TILE_STR(B, U, VV, 1);
            else if (L.block == B && vl == 1) RK_SCAN_TILE_STR(B, U, 1, 1);
            else if (L.block == BT && vl == VV) {
                if constexpr (large_ok) RK_SCAN_TILE_STR(BT, UT, VV, 1);
                else return ST_INVALID;
            } else {
                return ST_INVALID;
            }
        } else if (L.tstr == 2) {                // strided inputs: element loads, small tiles
            if (L.block == B && vl == 1) RK_SCAN_TILE_STR(B, U, 1, 2);
            else return ST_INVALID;
        } else if (L.block == BT) {
            if (vl == VV) RK_SCAN_TILE(BT, UT, VV);
            else if (vl == VW) RK_SCAN_TILE(BT, UT, VW);
            else return ST_INVALID;             // element loads take the small tiles
        } else {
            if (vl == VV) RK_SCAN_TILE(B, U, VV);
            else if (vl == VW) RK_SCAN_TILE(B, U, VW);
            else RK_SCAN_TILE(B, U, 1);
        }
#undef RK_SCAN_TILE
#undef RK_SCAN_TILE_STR
        break;
    }
    case SK_ROWWAVE:
        if (vl == VV)
            launch_first(&k_scan_rowwave<In, Acc, Op, B, UW, VV>, grid, block, st, ev, L.args);
        else if (vl == VW)
            launch_first(&k_scan_rowwave<In, Acc, Op, B, UW, VW>, grid, block, st, ev, L.args);
        else
            launch_first(&k_scan_rowwave<In, Acc, Op, B, U, 1>, grid, block, st, ev, L.args);
        break;
    case SK_LINES:
        if (scan_lines_packed(L.args.s_in, L.args.s_out, L.args.m)) {
            constexpr int UL = tune::kScanPackedUnroll;
            const bool l32 = L.args.lines <= int64_t(UINT32_MAX);
#define RK_PACKED(UK, EK)                                                                                    \
    (l32 ? launch_first(&k_scan_packed<In, Acc, Op, B, UK, EK, true>, grid, block, st, ev, L.args)             \
         : launch_first(&k_scan_packed<In, Acc, Op, B, UK, EK, false>, grid, block, st, ev, L.args))
            switch (scan_packed_width(L.args.m)) {
            case 1: RK_PACKED(UL, 1); break;
            case 2: RK_PACKED(UL, 2); break;
            default: RK_PACKED(UL / 2, 4); break;
            }
#undef RK_PACKED
        } else
            launch_first(&k_scan_lines<In, Acc, Op, B, tune::kScanLinesUnroll>, grid, block, st, ev, L.args);
        break;
    case SK_COLUMNS: {
        if (vl != 1 && vl != VV)
            return ST_INVALID;
        if (L.args.slot < 0)
            clear_state(L.args, 64 + scan_flag_lines(L.args.tiles) * 32, st);
        if (vl == VV)
            launch_first(&k_scan_columns<In, Acc, Op, BC, tune::kScanColLanes, tune::kScanColRows, true>, grid,
                         block, st, ev, L.args);
        else
            launch_first(&k_scan_columns<In, Acc, Op, BC, tune::kScanColLanesScalar, tune::kScanColRows, false>,
                         grid, block, st, ev, L.args);
        break;
    }
    case SK_TRANSPOSE:
        if (vl != 1)
            return ST_INVALID;
        if (L.args.slot < 0)
            clear_state(L.args, 64 + scan_flag_lines(L.args.tiles) * 32, st);
        switch (L.tmode) {
        case 0: launch_first(&k_scan_transpose<In, Acc, Op, 0>, grid, block, st, ev, L.args); break;
        case 1: launch_first(&k_scan_transpose<In, Acc, Op, 1>, grid, block, st, ev, L.args); break;
        case 2: launch_first(&k_scan_transpose<In, Acc, Op, 2>, grid, block, st, ev, L.args); break;
        default: return ST_INVALID;
        }
        break;
    default:
        return ST_INVALID;
    }
    return hipGetLastError() == hipSuccess ? ST_OK : ST_HIP;
}

template <class In, class Acc>
int run_scan_acc(const ScanLaunch &L)
{
    switch (L.op) {
    case 0: return run_scan_typed<In, Acc, OpSum>(L);
    case 1: return run_scan_typed<In, Acc, OpMax>(L);
    case 2: return run_scan_typed<In, Acc, OpMin>(L);
    }
    return ST_INVALID;
}

template <class In>
int run_scan_in(const ScanLaunch &L)
{
    if (L.kernel == SK_TAKE_TIMEOUTS)           // this translation unit's counts (the stream has drained)
        return RK_UNIT::take_timeouts<false>(L.args.slot, static_cast<uint64_t *>(L.args.ws), false);
    if constexpr (std::is_same_v<In, float> || std::is_same_v<In, bf16_in> || std::is_same_v<In, f16_in>) {
        if (L.acc == F32) return run_scan_acc<In, float>(L);
        if (L.acc == F64) return run_scan_acc<In, double>(L);
    } else if constexpr (std::is_same_v<In, double>) {
        if (L.acc == F64) return run_scan_acc<In, double>(L);
    } else if constexpr (std::is_same_v<In, int32_t>) {
        if (L.acc == I32) return run_scan_acc<In, int32_t>(L);
        if (L.acc == I64) return run_scan_acc<In, int64_t>(L);
    } else if constexpr (std::is_same_v<In, int64_t>) {
        if (L.acc == I64) return run_scan_acc<In, int64_t>(L);
    }
    return ST_UNSUPPORTED;
}

}  // namespace rk
