// rk_device.hpp -- gfx950 (CDNA4) device primitives for the reductions.
//
// Element decoding from 16-byte loads, the ops and maps, wave64 reductions
// built from DPP and ds_swizzle lane moves, block reductions through LDS, the
// XCD-aware block order, and the finishing store that every last pass uses
// (AcceleratedKernels.jl PR #139, "What changes": each pass stores through
// one finishing step that applies init, or folds into the output's previous
// value, or leaves a bare partial; "Compatibility": partials keep the
// accumulator type until that single final conversion).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <limits>
#include <type_traits>

#include "rk_launch.hpp"
#include "rk_plan.hpp"

// Every kernel translation unit defines RK_UNIT, a name of its own, before
// including this header.  The library state each unit keeps in device memory
// (the tables below) lives in a namespace of that name, so its device symbols
// differ from unit to unit: the runtime finds a symbol the host names by
// its device name, and equal names would all resolve to one unit's copy.
#ifndef RK_UNIT
#error "define RK_UNIT (a name unique to the translation unit) before including rk_device.hpp"
#endif

namespace rk {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <class To, class From>
__device__ __forceinline__ To bitcast(From v)
{
    static_assert(sizeof(To) == sizeof(From), "size mismatch");
    return __builtin_bit_cast(To, v);
}

// ------------------------------------------------------------ input types

struct bf16_in {};   // tag: bfloat16 input, stored as uint16_t
struct f16_in {};    // tag: IEEE half input, stored as uint16_t

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h16) { return bitcast<float>(h16 << 16); }
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h16)
{
    return (float)bitcast<_Float16>((uint16_t)h16);
}

// InTraits<In>: storage type, elements per 16-byte vector, and widening of
// one element / one vector to the accumulator type.
template <class In> struct InTraits;

template <> struct InTraits<float> {
    using S = float;
    static constexpr int vec = 4;
    template <class Acc> __device__ static Acc one(S v) { return (Acc)v; }
    template <class Acc> __device__ static void decode(u32x4 w, Acc *e)
    {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            e[i] = (Acc)bitcast<float>(w[i]);
    }
};

template <> struct InTraits<bf16_in> {
    using S = uint16_t;
    static constexpr int vec = 8;
    template <class Acc> __device__ static Acc one(S v) { return (Acc)bf16_bits_to_f32(v); }
    template <class Acc> __device__ static void decode(u32x4 w, Acc *e)
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            e[2 * i] = (Acc)bitcast<float>(w[i] << 16);
            e[2 * i + 1] = (Acc)bitcast<float>(w[i] & 0xffff0000u);
        }
    }
};

template <> struct InTraits<f16_in> {
    using S = uint16_t;
    static constexpr int vec = 8;
    template <class Acc> __device__ static Acc one(S v) { return (Acc)f16_bits_to_f32(v); }
    template <class Acc> __device__ static void decode(u32x4 w, Acc *e)
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            e[2 * i] = (Acc)f16_bits_to_f32(w[i] & 0xffffu);
            e[2 * i + 1] = (Acc)f16_bits_to_f32(w[i] >> 16);
        }
    }
};

template <> struct InTraits<double> {
    using S = double;
    static constexpr int vec = 2;
    template <class Acc> __device__ static Acc one(S v) { return (Acc)v; }
    template <class Acc> __device__ static void decode(u32x4 w, Acc *e)
    {
#pragma unroll
        for (int i = 0; i < 2; ++i)
            e[i] = (Acc)bitcast<double>(((uint64_t)w[2 * i + 1] << 32) | w[2 * i]);
    }
};

template <> struct InTraits<int32_t> {
    using S = int32_t;
    static constexpr int vec = 4;
    template <class Acc> __device__ static Acc one(S v) { return (Acc)v; }
    template <class Acc> __device__ static void decode(u32x4 w, Acc *e)
    {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            e[i] = (Acc)(int32_t)w[i];
    }
};

template <> struct InTraits<int64_t> {
    using S = int64_t;
    static constexpr int vec = 2;
    template <class Acc> __device__ static Acc one(S v) { return (Acc)v; }
    template <class Acc> __device__ static void decode(u32x4 w, Acc *e)
    {
#pragma unroll
        for (int i = 0; i < 2; ++i)
            e[i] = (Acc)(int64_t)(((uint64_t)w[2 * i + 1] << 32) | w[2 * i]);
    }
};

// -------------------------------------------------------------- maps, ops
// Integer maps and sums wrap (two's complement) in the accumulator type.

struct MapIdentity {
    template <class T> __device__ __forceinline__ static T apply(T v) { return v; }
};

struct MapSquare {
    template <class T> __device__ __forceinline__ static T apply(T v)
    {
        if constexpr (std::is_integral_v<T>) {
            using U = std::make_unsigned_t<T>;
            return (T)((U)v * (U)v);
        } else {
            return v * v;     // built with -ffp-contract=off: never fused into the fold
        }
    }
};

struct MapAbs {
    template <class T> __device__ __forceinline__ static T apply(T v)
    {
        if constexpr (std::is_integral_v<T>) {
            using U = std::make_unsigned_t<T>;
            return v < 0 ? (T)((U)0 - (U)v) : v;
        } else {
            return __builtin_fabs(v);
        }
    }
};

// Two-input maps f(a, b) of a fused source, evaluated after widening both
// elements to the accumulator type; integer forms wrap in that type.
struct Map2Mul {
    template <class T> __device__ __forceinline__ static T apply(T a, T b)
    {
        if constexpr (std::is_integral_v<T>) {
            using U = std::make_unsigned_t<T>;
            return (T)((U)a * (U)b);
        } else {
            return a * b;
        }
    }
};

struct Map2SqDiff {
    template <class T> __device__ __forceinline__ static T apply(T a, T b)
    {
        if constexpr (std::is_integral_v<T>) {
            using U = std::make_unsigned_t<T>;
            const U d = (U)a - (U)b;
            return (T)(d * d);
        } else {
            const T d = a - b;
            return d * d;
        }
    }
};

struct Map2AbsDiff {
    template <class T> __device__ __forceinline__ static T apply(T a, T b)
    {
        if constexpr (std::is_integral_v<T>) {
            using U = std::make_unsigned_t<T>;
            const T d = (T)((U)a - (U)b);
            return d < 0 ? (T)((U)0 - (U)d) : d;
        } else {
            return __builtin_fabs(a - b);
        }
    }
};

struct OpSum {
    template <class T> __device__ __forceinline__ static T identity() { return T(0); }
    template <class T> __device__ __forceinline__ static T apply(T a, T b)
    {
        if constexpr (std::is_integral_v<T>) {
            using U = std::make_unsigned_t<T>;
            return (T)((U)a + (U)b);
        } else {
            return a + b;
        }
    }
};

// max/min propagate NaN: the result is NaN when either operand is.  For
// floats this is IEEE 754-2019 maximum/minimum, which gfx950 executes as one
// instruction (v_maximum3_f32 / v_minimum3_f32); ties of -0 and +0 may take
// either sign.
struct OpMax {
    template <class T> __device__ __forceinline__ static T identity()
    {
        if constexpr (std::is_integral_v<T>)
            return std::numeric_limits<T>::min();
        else
            return -std::numeric_limits<T>::infinity();
    }
    template <class T> __device__ __forceinline__ static T apply(T a, T b)
    {
        if constexpr (std::is_integral_v<T>)
            return a > b ? a : b;
        else
            return __builtin_elementwise_maximum(a, b);
    }
};

struct OpMin {
    template <class T> __device__ __forceinline__ static T identity()
    {
        if constexpr (std::is_integral_v<T>)
            return std::numeric_limits<T>::max();
        else
            return std::numeric_limits<T>::infinity();
    }
    template <class T> __device__ __forceinline__ static T apply(T a, T b)
    {
        if constexpr (std::is_integral_v<T>)
            return a < b ? a : b;
        else
            return __builtin_elementwise_minimum(a, b);
    }
};

// ------------------------------------------------------------ lane moves
// wave64 cross-lane moves: DPP within a 16-lane row (quad permutes and
// mirrors), ds_swizzle (bit-mask mode) within 32 lanes, ds_bpermute across
// the halves.  64-bit values move as two 32-bit halves.

template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xf, 0xf, false);
}

template <int PATTERN>
__device__ __forceinline__ uint32_t swizzle32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, PATTERN);
}

__device__ __forceinline__ uint32_t bpermute32(uint32_t v, int src_lane)
{
    return (uint32_t)__builtin_amdgcn_ds_bpermute(src_lane << 2, (int)v);
}

template <class T, class F>
__device__ __forceinline__ T move_words(T v, F &&f)
{
    if constexpr (sizeof(T) == 4) {
        return bitcast<T>(f(bitcast<uint32_t>(v)));
    } else {
        static_assert(sizeof(T) == 8, "4- or 8-byte values");
        const uint64_t u = bitcast<uint64_t>(v);
        const uint32_t lo = f((uint32_t)u), hi = f((uint32_t)(u >> 32));
        return bitcast<T>(((uint64_t)hi << 32) | lo);
    }
}

// DPP controls (GFX9 encoding)
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL, class T>
__device__ __forceinline__ T dpp_move(T v)
{
    return move_words(v, [](uint32_t w) { return dpp32<CTRL>(w); });
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

// value of lane (this lane ^ X)
template <int X, class T>
__device__ __forceinline__ T lane_xor(T v)
{
    if constexpr (X == 1) {
        return dpp_move<kDppQuadXor1>(v);
    } else if constexpr (X == 2) {
        return dpp_move<kDppQuadXor2>(v);
    } else if constexpr (X < 32) {
        // ds_swizzle bit-mask mode: lane' = ((lane & 0x1f) | 0) ^ X within 32 lanes
        return move_words(v, [](uint32_t w) { return swizzle32<(X << 10) | 0x1f>(w); });
    } else {
        const int src = lane_id() ^ X;
        return move_words(v, [src](uint32_t w) { return bpermute32(w, src); });
    }
}

template <class T>
__device__ __forceinline__ T read_lane(T v, int lane)
{
    return move_words(v, [lane](uint32_t w) {
        return (uint32_t)__builtin_amdgcn_readlane((int)w, lane);
    });
}

// Reduce over all 64 lanes; every lane gets the (wave-uniform) result.
// All 64 lanes must be active.
template <class Op, class T>
__device__ __forceinline__ T wave_reduce(T v)
{
    v = Op::apply(v, dpp_move<kDppQuadXor1>(v));
    v = Op::apply(v, dpp_move<kDppQuadXor2>(v));
    v = Op::apply(v, dpp_move<kDppRowHalfMirror>(v));   // the two quads of a half-row
    v = Op::apply(v, dpp_move<kDppRowMirror>(v));       // the two halves of a row
    // every lane of a 16-lane row now holds that row's result
    return Op::apply(Op::apply(read_lane(v, 0), read_lane(v, 16)),
                     Op::apply(read_lane(v, 32), read_lane(v, 48)));
}

// Reduce over the lanes that share (lane % CL), i.e. the 64/CL rows of a
// wave that hold the same tile column; every lane gets its column's result.
template <int CL, class Op, class T>
__device__ __forceinline__ T wave_reduce_columns(T v)
{
    if constexpr (CL <= 1) v = Op::apply(v, lane_xor<1>(v));
    if constexpr (CL <= 2) v = Op::apply(v, lane_xor<2>(v));
    if constexpr (CL <= 4) v = Op::apply(v, lane_xor<4>(v));
    if constexpr (CL <= 8) v = Op::apply(v, lane_xor<8>(v));
    if constexpr (CL <= 16) v = Op::apply(v, lane_xor<16>(v));
    if constexpr (CL <= 32) v = Op::apply(v, lane_xor<32>(v));
    return v;
}

// Whole-block reduction; the result is valid in wave 0 (thread 0 stores it).
// Uses LDS: a caller that reduces again must __syncthreads() first.
template <class Op, int BLOCK, class T>
__device__ __forceinline__ T block_reduce(T v)
{
    constexpr int NW = BLOCK / 64;
    static_assert(BLOCK % 64 == 0, "blocks are whole waves");
    v = wave_reduce<Op>(v);
    if constexpr (NW == 1) {
        return v;
    } else {
        __shared__ T part[NW];
        const int w = (int)(threadIdx.x >> 6);
        if (lane_id() == 0)
            part[w] = v;
        __syncthreads();
        T r = Op::template identity<T>();
        if (w == 0) {
            r = lane_id() < NW ? part[lane_id()] : r;
            r = wave_reduce<Op>(r);
        }
        return r;
    }
}

// ------------------------------------------------------- XCD block order
// MI355X dispatches consecutive workgroups round-robin over its 8 XCDs, each
// with a private L2.  This permutation gives every XCD one contiguous range
// of logical block ids, so neighbouring tiles that share cache lines are
// served by the same L2.  It is a bijection for any grid size.
constexpr uint32_t kXcds = 8;

__device__ __forceinline__ uint32_t xcd_block(uint32_t bid, uint32_t nblocks)
{
    const uint32_t q = nblocks / kXcds, r = nblocks % kXcds;
    const uint32_t xcd = bid % kXcds, local = bid / kXcds;
    return xcd * q + (xcd < r ? xcd : r) + local;
}

// ----------------------------------------------------------- conversions

// float -> bfloat16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u = bitcast<uint32_t>(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// double -> float rounded to odd: truncate, then set the last bit when the
// conversion was inexact.  Rounding that float once more to a format of at
// most 22 significant bits gives the correctly rounded double result
// (rounding to odd as an intermediate step, Boldo and Melquiond 2008).
__device__ __forceinline__ float f64_to_f32_odd(double d)
{
    float f = (float)d;
    if (d != d)
        return f;
    if (__builtin_isinf(f) && !__builtin_isinf(d))
        return d > 0 ? 3.40282347e38f : -3.40282347e38f;
    const double back = (double)f;
    if (back != d) {
        uint32_t b = bitcast<uint32_t>(f);
        if (__builtin_fabs(back) > __builtin_fabs(d))
            b -= 1;                    // one step toward zero
        f = bitcast<float>(b | 1u);
    }
    return f;
}

template <class Acc>
__device__ __forceinline__ void store_out(void *out, int64_t o, int out_dtype, Acc v)
{
    if constexpr (std::is_floating_point_v<Acc>) {
        switch (out_dtype) {
        case F32: static_cast<float *>(out)[o] = (float)v; break;
        case F64: static_cast<double *>(out)[o] = (double)v; break;
        case BF16:
            if constexpr (std::is_same_v<Acc, double>)
                static_cast<uint16_t *>(out)[o] = f32_to_bf16_rne(f64_to_f32_odd(v));
            else
                static_cast<uint16_t *>(out)[o] = f32_to_bf16_rne(v);
            break;
        case F16: {
            float f;
            if constexpr (std::is_same_v<Acc, double>)
                f = f64_to_f32_odd(v);
            else
                f = v;
            static_cast<uint16_t *>(out)[o] = bitcast<uint16_t>((_Float16)f);
            break;
        }
        default: break;
        }
    } else {
        switch (out_dtype) {
        case I32: static_cast<int32_t *>(out)[o] = (int32_t)(uint32_t)(uint64_t)v; break;
        case I64: static_cast<int64_t *>(out)[o] = (int64_t)v; break;
        default: break;
        }
    }
}

// Previous output value, read back into the accumulator type (fold mode).
template <class Acc>
__device__ __forceinline__ Acc load_out(const void *out, int64_t o, int out_dtype)
{
    if constexpr (std::is_floating_point_v<Acc>) {
        switch (out_dtype) {
        case F32: return (Acc) static_cast<const float *>(out)[o];
        case F64: return (Acc) static_cast<const double *>(out)[o];
        case BF16: return (Acc)bf16_bits_to_f32(static_cast<const uint16_t *>(out)[o]);
        case F16: return (Acc)f16_bits_to_f32(static_cast<const uint16_t *>(out)[o]);
        default: return Acc(0);
        }
    } else {
        switch (out_dtype) {
        case I32: return (Acc) static_cast<const int32_t *>(out)[o];
        case I64: return (Acc) static_cast<const int64_t *>(out)[o];
        default: return Acc(0);
        }
    }
}

template <class Acc>
__device__ __forceinline__ Acc from_bits(uint64_t b)
{
    if constexpr (sizeof(Acc) == 4)
        return bitcast<Acc>((uint32_t)b);
    else
        return bitcast<Acc>(b);
}

// Host mode: the bare result goes straight to the library's pinned host
// buffer (f.out) with a system-scope store, followed -- once that store has
// completed -- by the call's sequence number at byte 8, which the host waits
// for.  Without such a buffer the result goes to ws[grid] and the sequence
// number to host_seq_offset, both copied back once the stream has drained.
template <class Acc>
__device__ __forceinline__ void store_host_result(const Finish &f, Acc *ws, int grid, Acc v)
{
    if (f.out) {
        if constexpr (sizeof(Acc) == 4)
            __hip_atomic_store(static_cast<uint32_t *>(f.out), bitcast<uint32_t>(v), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_SYSTEM);
        else
            __hip_atomic_store(static_cast<uint64_t *>(f.out), bitcast<uint64_t>(v), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_SYSTEM);
        __builtin_amdgcn_s_waitcnt(0);
        __hip_atomic_store(reinterpret_cast<uint32_t *>(static_cast<char *>(f.out) + 8), f.host_seq,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    } else {
        ws[grid] = v;
        *reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(ws) + host_seq_offset(grid, sizeof(Acc))) =
            f.host_seq;
    }
}

__device__ __forceinline__ int64_t div_nonneg(int64_t a, int64_t b);

// Where output o (in the kernel's numbering) sits in the output: o itself,
// or, under an output map, its digits over m.ext times m.str.
__device__ __forceinline__ int64_t out_index(const OutMap &m, int64_t o)
{
    if (m.nd == 0)
        return o;
    int64_t r = 0;
    for (int k = 0; k + 1 < m.nd; ++k) {
        const int64_t q = div_nonneg(o, m.ext[k]);
        r += (o - q * m.ext[k]) * m.str[k];
        o = q;
    }
    return r + o * m.str[m.nd - 1];
}

// The one finishing step of every last pass, for output o.
//   OVERWRITE: out[o] = convert(op(init, v))
//   FOLD:      out[o] = convert(op(widen(out[o]), v))
// (HOST and PARTIAL store bare accumulators; the callers do that.)
template <class Op, class Acc>
__device__ __forceinline__ void finish_store(const Finish &f, int64_t o, Acc v)
{
    Acc s = f.mode == FIN_FOLD ? load_out<Acc>(f.out, o, f.out_dtype) : from_bits<Acc>(f.init_bits);
    store_out<Acc>(f.out, o, f.out_dtype, Op::apply(s, v));
}

// ------------------------------------------------- waits that give up
// Every wait of one block on others is bounded.  One that gives up (never in
// a normal run: no block waits on the block that waits) is counted here, per
// stream slot, plus one entry shared by calls on streams without a slot; the
// host reads and clears the counts (rk_stream_timeouts).  Each translation
// unit has its own table, as it has its own slots.
namespace RK_UNIT {
static __device__ __attribute__((aligned(128))) uint32_t g_timeouts[kTimeoutEntries];
}
using RK_UNIT::g_timeouts;

__device__ __forceinline__ void record_timeout(int slot)
{
    __hip_atomic_fetch_add(&g_timeouts[slot >= 0 && slot < kArriveSlots ? slot : kArriveSlots], 1u,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------- finishing in one launch
// The blocks that share an output store their partials, and the last one to
// arrive folds them and finishes: one launch instead of a second pass.  The
// counters belong to the library, are zero when the code object loads, and
// atomicInc's wrap-around (n - 1 -> 0) leaves each one at zero again after
// its n arrivals, so nothing has to be cleared between calls.  Each stream
// gets its own slot of counters, so calls that may overlap never share one.
// Counter c of a slot sits in line c % kArriveLines, word c / kArriveLines,
// so consecutive counters never share a 128-byte line.
namespace RK_UNIT {
static __device__ __attribute__((aligned(128))) uint32_t g_arrive[kArriveSlots * kArriveCapacity];
}
using RK_UNIT::g_arrive;
constexpr int kArriveLineWords = 32;
constexpr int kArriveLines = kArriveCapacity / kArriveLineWords;

// Partials cross XCDs, each with a private L2.  They are written with
// device-scope atomic stores, which write through to the device's point of
// coherence (`sc1` stores on gfx950), and read with device-scope atomic
// loads, which do not hit a stale L2 line (`sc1` loads).  So handing them
// over needs no L2 writeback or invalidation -- which is what a device-scope
// release/acquire fence would add (buffer_wbl2 / buffer_inv), at a cost of
// tens of microseconds over a 1024-block grid -- only that each store has
// completed before its block's arrival is counted (wait_stores).
template <class T>
__device__ __forceinline__ void store_partial(T *p, T v)
{
    if constexpr (sizeof(T) == 4)
        __hip_atomic_store(reinterpret_cast<uint32_t *>(p), bitcast<uint32_t>(v), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    else
        __hip_atomic_store(reinterpret_cast<uint64_t *>(p), bitcast<uint64_t>(v), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

template <class T>
__device__ __forceinline__ T load_partial(const T *p)
{
    if constexpr (sizeof(T) == 4)
        return bitcast<T>(__hip_atomic_load(reinterpret_cast<const uint32_t *>(p), __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT));
    else
        return bitcast<T>(__hip_atomic_load(reinterpret_cast<const uint64_t *>(p), __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT));
}

// Take wave-uniform values -- kernel arguments, addresses of library
// memory -- into scalar registers here, all together.  Left to itself the
// compiler loads a kernel's arguments in several dependent batches, each a
// memory round trip, before a block issues its first data load.
// (One asm statement for all of them: with several, the compiler may wait for
// the first statement's loads before it issues the next statement's.)
template <class T0, class T1, class T2, class T3, class T4, class T5, class T6, class T7, class T8, class T9,
          class T10, class T11, class T12, class T13, class T14, class T15, class T16, class T17, class T18, class T19>
__device__ __forceinline__ void sgpr_ready(const T0 &v0, const T1 &v1, const T2 &v2, const T3 &v3, const T4 &v4,
                                           const T5 &v5, const T6 &v6, const T7 &v7, const T8 &v8, const T9 &v9,
                                           const T10 &v10, const T11 &v11, const T12 &v12, const T13 &v13,
                                           const T14 &v14, const T15 &v15, const T16 &v16, const T17 &v17,
                                           const T18 &v18, const T19 &v19)
{
    asm volatile("" ::"s"(v0), "s"(v1), "s"(v2), "s"(v3), "s"(v4), "s"(v5), "s"(v6), "s"(v7), "s"(v8), "s"(v9),
                 "s"(v10), "s"(v11), "s"(v12), "s"(v13), "s"(v14), "s"(v15), "s"(v16), "s"(v17), "s"(v18), "s"(v19));
}

// Keep every load of an unrolled group ahead of the arithmetic that consumes
// it: without this the scheduler may interleave a wait (and cut the loads in
// flight) to pair loads up for v_max3 and the like.
__device__ __forceinline__ void issue_barrier() { __builtin_amdgcn_sched_barrier(0); }

// Wait until this thread's outstanding memory operations have completed
// (s_waitcnt with every counter at zero).
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0); }

// One arrival on counter c of a slot; true for the n-th (last) one.
__device__ __forceinline__ bool count_arrival(int slot, int64_t c, uint32_t n)
{
    uint32_t *p = &g_arrive[int64_t(slot) * kArriveCapacity + (c % kArriveLines) * kArriveLineWords
                            + c / kArriveLines];
    return __builtin_amdgcn_atomic_inc32(p, n - 1, __ATOMIC_RELAXED, "agent") == n - 1;
}

// Count the arrival of `member` (0 <= member < n) of output idx's n
// contributors; true for the last of all n.  Up to kArriveGroup arrivals go
// to the output's one counter; more are counted per group first, and only
// the last of each group counts on the top counter.  Every thread that
// stored a partial must have called wait_stores() and met the caller at a
// barrier first.  A group's last arrival has seen every arrival of its
// group, each made after that member's stores completed, so the top
// counter's last arrival follows every member's stores.
__device__ __forceinline__ bool arrive_last(int slot, int64_t idx, uint32_t member, uint32_t n)
{
    wait_stores();
    const int64_t top = idx * arrive_counters(n);
    if (n <= uint32_t(kArriveGroup))
        return count_arrival(slot, top, n);
    const uint32_t g = member / kArriveGroup;
    const uint32_t in_group = n - g * kArriveGroup < uint32_t(kArriveGroup) ? n - g * kArriveGroup
                                                                            : uint32_t(kArriveGroup);
    if (!count_arrival(slot, top + 1 + g, in_group))
        return false;
    return count_arrival(slot, top, (n + kArriveGroup - 1) / kArriveGroup);
}

// --------------------------------------- whole-array finish by collection
// A whole-array pass needs its blocks' partials in one place, and counting
// arrivals puts a chain of dependent memory round trips behind the last
// block (store and wait, group counter, top counter, loads).  Instead every
// block stores its partial with the call's tag in the same 64-bit word (one
// device-scope store, no wait; 8-byte partials take two words, a tagged
// half each), and block 0, after its own tiles, polls the words until every
// one carries the tag, folds them in block order -- the order of the second
// launch -- and finishes.  No block waits on block 0, so the poll always
// ends; a bounded spin is the safety net.
//
// Tags: each stream slot keeps the last call's tag E; a call's tag is E + 1,
// read by every block when it starts, and block 0 stores it back into E when
// it is done, so the next call on the stream (a graph replay included) gets
// a fresh one.  E is kept in kFinalTagCopies copies, a 128-byte line each,
// and block b reads copy b mod kFinalTagCopies: a thousand blocks reading one
// line would queue where device-scope accesses are performed.  Tags run
// 1 .. 2^32 - 1; the call that reaches 2^32 - 1 zeroes every word of the
// slot and sets E to 0, so a word never carries a stale tag that equals the
// current one.
constexpr int kFinalTagCopies = 32;
constexpr int kFinalHeaderWords = 16 * kFinalTagCopies;
constexpr int kFinalSlotWords = kFinalHeaderWords + 2 * kFinalCapacity;
namespace RK_UNIT {
static __device__ __attribute__((aligned(128))) uint64_t g_final[kArriveSlots * kFinalSlotWords];
}
using RK_UNIT::g_final;

// The slot's last tag E (read when a block starts; thread 0 only): the
// call's tag is E + 1.  Callers add the 1 only where they use the tag, at the
// block's end, so nothing waits for this load before the block's first tiles
// are loaded: it returns while they are in flight.
__device__ __forceinline__ uint32_t last_tag(int slot)
{
    // the low 32 bits of the 64-bit word (tags fit 32 bits): a 64-bit load
    // would leave a dead half whose register reuse waits for the load
    const int64_t copy = int64_t(blockIdx.x % kFinalTagCopies) * 16;
    return __hip_atomic_load(reinterpret_cast<const uint32_t *>(&g_final[int64_t(slot) * kFinalSlotWords + copy]),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class Acc>
__device__ __forceinline__ void publish_tagged(int slot, int b, Acc v, uint32_t tag)
{
    uint64_t *w = &g_final[int64_t(slot) * kFinalSlotWords + kFinalHeaderWords];
    const uint64_t t = uint64_t(tag) << 32;
    if constexpr (sizeof(Acc) == 4) {
        __hip_atomic_store(w + b, t | bitcast<uint32_t>(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        const uint64_t bits = bitcast<uint64_t>(v);
        __hip_atomic_store(w + 2 * b, t | (bits & 0xffffffffu), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(w + 2 * b + 1, t | (bits >> 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Block 0: wait until all `grid` partials carry `tag`, then fold thread t's
// partials t, t + BLOCK, ... in that order (every thread's result, before
// the block reduction).  Called by every thread of block 0.  Each thread
// polls its own words until they all carry the tag, and the block meets
// once, at the end: a barrier per poll would hold every thread to the
// slowest one's round trip (the 10^8 f32 sum measured 0.5 us faster so).
// A thread that reaches `spin_limit` polls without every tag gives up, and
// then the block returns false in `*ok` (the same in every thread): the
// fold is incomplete.
template <class Acc, class Op, int BLOCK>
__device__ Acc collect_tagged(int slot, int grid, uint32_t tag, uint32_t spin_limit, bool *ok_out)
{
    const uint64_t *w = &g_final[int64_t(slot) * kFinalSlotWords + kFinalHeaderWords];
    __shared__ int s_ready;
    Acc v = Op::template identity<Acc>();
    bool ok = true;
    for (uint32_t spin = 0;; ++spin) {
        ok = true;
        v = Op::template identity<Acc>();
        for (int k = threadIdx.x; k < grid; k += BLOCK) {
            if constexpr (sizeof(Acc) == 4) {
                const uint64_t x = __hip_atomic_load(w + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                ok = ok && uint32_t(x >> 32) == tag;
                v = Op::apply(v, bitcast<Acc>(uint32_t(x)));
            } else {
                const uint64_t lo = __hip_atomic_load(w + 2 * k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const uint64_t hi = __hip_atomic_load(w + 2 * k + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                ok = ok && uint32_t(lo >> 32) == tag && uint32_t(hi >> 32) == tag;
                v = Op::apply(v, bitcast<Acc>((lo & 0xffffffffu) | (hi << 32)));
            }
        }
        if (ok || spin >= spin_limit)
            break;
        __builtin_amdgcn_s_sleep(1);
    }
    if (threadIdx.x == 0)
        s_ready = 1;
    __syncthreads();
    if (!ok)
        s_ready = 0;
    __syncthreads();
    *ok_out = s_ready != 0;
    return v;
}

// Block 0, once the result is stored (or its collection gave up): hand the
// next call its tag base.  Called by every thread of block 0.  After a
// collection that gave up, the tag still moves on: blocks that have started
// carry the old tag, which no later call's collection takes for its own.
template <int BLOCK>
__device__ __forceinline__ void advance_tag(int slot, uint32_t tag)
{
    static_assert(BLOCK >= kFinalTagCopies, "one thread per copy of the tag");
    uint64_t *s = &g_final[int64_t(slot) * kFinalSlotWords];
    uint64_t next = tag;
    if (tag == 0xffffffffu) {                  // wrap: no word may keep an old tag
        for (int i = threadIdx.x; i < 2 * kFinalCapacity; i += BLOCK)
            __hip_atomic_store(s + kFinalHeaderWords + i, uint64_t(0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        next = 0;
    }
    if (threadIdx.x < kFinalTagCopies)
        __hip_atomic_store(s + threadIdx.x * 16, next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Test hook: make the slot's last tag `e` (every copy), so a test can run
// calls across the wrap of the tags.  One block of kFinalTagCopies threads.
// In the unit's own namespace: it writes this unit's g_final, and a kernel of
// one name in every unit would be launched through one host stub, the
// linker's pick, and so always reach one unit's copy.  A template, as is
// every other use of g_final, so that the units that never instantiate one
// (the scan units) hold no copy of the array.
namespace RK_UNIT {
template <int = 0>
__global__ void k_set_final_tag(int slot, uint32_t e)
{
    if (threadIdx.x < kFinalTagCopies)
        __hip_atomic_store(&g_final[int64_t(slot) * kFinalSlotWords + threadIdx.x * 16], uint64_t(e), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
}  // namespace RK_UNIT

// ------------------------------------------------------------------ misc

// Offset of linear index idx (below the product of the extents) in a
// column-major layout of nd <= 4 dims.  The last dim takes what is left of
// idx without a division: a 64-bit division is a long VALU sequence, and the
// kernels form these offsets before their first loads.
__device__ __forceinline__ int64_t layout_offset(int nd, const int64_t *ext, const int64_t *str,
                                                 int64_t idx)
{
    int64_t off = 0;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        if (d + 1 < nd) {
            const int64_t q = idx / ext[d];
            off += (idx - q * ext[d]) * str[d];
            idx = q;
        } else if (d + 1 == nd) {
            off += idx * str[d];
        }
    }
    return off;
}

// The same for an index below 2^32 (so is every extent it divides by):
// 32-bit divisions, a handful of instructions each.
__device__ __forceinline__ int64_t layout_offset32(int nd, const int64_t *ext, const int64_t *str, uint32_t idx)
{
    int64_t off = 0;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        if (d + 1 < nd) {
            const uint32_t e = uint32_t(ext[d]);
            const uint32_t q = idx / e;
            off += int64_t(idx - q * e) * str[d];
            idx = q;
        } else if (d + 1 == nd) {
            off += int64_t(idx) * str[d];
        }
    }
    return off;
}

// a / b for 0 <= a and 0 < b, in 32-bit arithmetic when both fit.
__device__ __forceinline__ int64_t div_nonneg(int64_t a, int64_t b)
{
    if (uint64_t(a) <= 0xffffffffu && uint64_t(b) <= 0xffffffffu)
        return uint32_t(a) / uint32_t(b);
    return a / b;
}

// A position in a column-major layout of nd <= 4 dims that moves forward by
// a fixed number of elements without dividing: the position is kept as
// mixed-radix digits, and a step adds the step's own digits with carries.
// Set up once per thread (one division per dim), then advance() costs a few
// adds and compares per dim.
struct Walk {
    int64_t idx[4];     // digits of the current linear index
    int64_t off;        // its element offset
    int64_t dig[4];     // digits of the step
    int64_t step_off;   // offset change of the step without carries
    int64_t wrap[4];    // offset change when digit d wraps: str[d+1] - ext[d] * str[d]

    __device__ __forceinline__ void init(int nd, const int64_t *ext, const int64_t *str, int64_t first,
                                         int64_t step)
    {
        off = 0;
        step_off = 0;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            idx[d] = 0;
            dig[d] = 0;
            wrap[d] = 0;
            if (d < nd) {
                const int64_t q = first / ext[d];
                idx[d] = first - q * ext[d];
                first = q;
                off += idx[d] * str[d];
                const int64_t qs = step / ext[d];
                dig[d] = step - qs * ext[d];
                step = qs;
                step_off += dig[d] * str[d];
                wrap[d] = (d + 1 < nd ? str[d + 1] : 0) - ext[d] * str[d];
            }
        }
    }

    __device__ __forceinline__ void advance(int nd, const int64_t *ext)
    {
        off += step_off;
        int64_t carry = 0;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            if (d < nd) {
                idx[d] += dig[d] + carry;
                carry = idx[d] >= ext[d];
                if (carry) {
                    idx[d] -= ext[d];
                    off += wrap[d];
                }
            }
        }
    }
};

// Loads.  Streaming kernels read every input byte exactly once and pass
// NT = true: the non-temporal hint keeps the lines from displacing useful
// cache contents, and on MI355X lifts a streaming read from about 6.1 to
// about 6.8 TB/s.  Tiles whose rows are narrower than a 128-byte line pass
// NT = false, because the neighbouring tile (placed on the same XCD) reads
// the rest of each line from L2.
#ifndef RK_NONTEMPORAL_LOADS
#define RK_NONTEMPORAL_LOADS 1
#endif
constexpr bool kStreamNT = RK_NONTEMPORAL_LOADS != 0;

template <bool NT = kStreamNT>
__device__ __forceinline__ u32x4 load16(const u32x4 *p)
{
    if constexpr (NT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

template <bool NT = kStreamNT, class S>
__device__ __forceinline__ S load1(const S *p)
{
    if constexpr (NT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

}  // namespace rk
