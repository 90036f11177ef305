// rk_kernels.hpp -- the HIP kernels and their typed launchers (gfx950).
//
// Whole array (AcceleratedKernels.jl PR #139, "What changes"): a first pass
// of at most a grid cap of blocks, each striding over tiles of the input with
// several 16-byte loads in flight per thread; block 0 collects the blocks'
// tagged partials and finishes (a one-block second pass when the stream has
// no slot); an input that fits one block finishes in the first pass.  A fused
// two-input source f(x_i, y_i) takes the same passes with two loads per step.
//
// Strided dims (PR #176, "This PR"): one tile kernel serves the selector's
// three shapes -- one thread per output (a tile one row tall), the narrow
// tiled block (one pass) and the wide columns block (split along the reduced
// dim, finished by the last block to arrive or a second pass) -- over runs of
// contiguous outputs placed by the other kept dims (the middle dim of 3-d
// arrays); further reduced dims index segments of rows.  A contiguous reduced
// dim takes the row kernel (one wave per output); any other layout the
// generic kernel (blocks over (output, chunk) units).
//
// Every last pass stores through finish_store().  No kernel reads workspace
// it did not write in the same call, so a workspace is reusable as is.
#pragma once

#include <hip/hip_ext.h>

#include <algorithm>

#include "rk_device.hpp"

namespace rk {

template <class Acc, class Op, int V>
__device__ __forceinline__ void set_identity(Acc (&a)[V])
{
#pragma unroll
    for (int i = 0; i < V; ++i)
        a[i] = Op::template identity<Acc>();
}

template <class In, class Acc, class Op, class Map, int V>
__device__ __forceinline__ void fold_vec(Acc (&a)[V], u32x4 w)
{
    Acc e[V];
    InTraits<In>::template decode<Acc>(w, e);
#pragma unroll
    for (int i = 0; i < V; ++i)
        a[i] = Op::apply(a[i], Map::apply(e[i]));
}

template <class Acc, class Op, int V>
__device__ __forceinline__ Acc fold_all(const Acc (&a)[V])
{
    // pairwise, so the per-thread tree stays shallow
    Acc t[V];
#pragma unroll
    for (int i = 0; i < V; ++i)
        t[i] = a[i];
#pragma unroll
    for (int w = V / 2; w >= 1; w /= 2)
#pragma unroll
        for (int i = 0; i < w; ++i)
            t[i] = Op::apply(t[i], t[i + w]);
    return t[0];
}

// ================================================================ whole array

// Fold a whole-array call's `grid` block partials and finish: store into
// the output, or leave the bare result in ws[grid] for the host.  Run by one
// block (the second launch, or the last block to arrive when a grid is too
// large for collection).
// Fold `count` partials p[first + k * stride], k < count, issuing up to 8
// loads at a time: the partials come from memory, and one round trip per
// partial would dominate the finishing step.
template <class Acc, class Op>
__device__ __forceinline__ Acc fold_partials(const Acc *p, int64_t first, int64_t count, int64_t stride)
{
    constexpr int P = 8;
    Acc v = Op::template identity<Acc>();
    for (int64_t k0 = 0; k0 < count; k0 += P) {
        Acc w[P];
#pragma unroll
        for (int u = 0; u < P; ++u)
            w[u] = k0 + u < count ? load_partial(p + first + (k0 + u) * stride) : Op::template identity<Acc>();
#pragma unroll
        for (int u = 0; u < P; ++u)
            v = Op::apply(v, w[u]);
    }
    return v;
}

template <class Acc, class Op, int BLOCK>
__device__ __forceinline__ void fold_partials_and_finish(Acc *ws, int grid, const Finish &fin)
{
    // thread t folds partials t, t + BLOCK, ...
    const int64_t mine = threadIdx.x < grid ? (grid - 1 - threadIdx.x) / BLOCK + 1 : 0;
    Acc v = fold_partials<Acc, Op>(ws, threadIdx.x, mine, BLOCK);
    v = block_reduce<Op, BLOCK>(v);
    if (threadIdx.x == 0) {
        if (fin.mode == FIN_HOST)
            store_host_result(fin, ws, grid, v);
        else
            finish_store<Op>(fin, 0, v);
    }
}

// Start of a first-pass block: the slot's last tag E, used when the call
// finishes by collection (read early, so the load is long done by the end;
// the call's tag is E + 1, formed in the epilogue).  Every thread loads it,
// unconditionally: a load made in a branch is waited for where the branch
// ends, which would hold the block's first tile loads behind a device-scope
// round trip.  (One load per wave; calls without a slot read slot 0's copy
// and never use it.)
__device__ __forceinline__ uint32_t whole_prologue(const AllArgs &a)
{
    return last_tag(a.arrive_slot >= 0 ? a.arrive_slot : 0);
}

// End of a first-pass block holding its reduced value v (valid in thread 0)
// and the slot's last tag E from whole_prologue (thread 0).
template <class Acc, class Op, int BLOCK>
__device__ __forceinline__ void whole_epilogue(const AllArgs &a, Acc v, uint32_t last_e)
{
    const uint32_t tag = last_e + 1u;
    Acc *ws = static_cast<Acc *>(a.ws);
    if (a.grid == 1) {                          // the whole input in one block
        if (threadIdx.x == 0) {
            if (a.fin.mode == FIN_HOST)
                store_host_result(a.fin, ws, 1, v);   // bare result for the host to finish
            else
                finish_store<Op>(a.fin, 0, v);
        }
        return;
    }
    if (a.arrive_slot < 0) {                    // a second launch folds the partials
        if (threadIdx.x == 0)
            ws[blockIdx.x] = v;
        return;
    }
    if (a.grid <= kFinalCapacity) {             // tagged partials, collected by block 0
        if (threadIdx.x == 0)
            publish_tagged(a.arrive_slot, blockIdx.x, v, tag);
        if (blockIdx.x != 0)
            return;
        __shared__ uint32_t s_tag;
        if (threadIdx.x == 0)
            s_tag = tag;
        __syncthreads();
        const uint32_t t = s_tag;
        bool ok = false;
        Acc r = collect_tagged<Acc, Op, BLOCK>(a.arrive_slot, a.grid, t ^ a.tag_xor, a.spin_limit, &ok);
        r = block_reduce<Op, BLOCK>(r);
        if (threadIdx.x == 0) {
            if (!ok)                            // an incomplete fold is no result: store nothing
                record_timeout(a.arrive_slot);
            else if (a.fin.mode == FIN_HOST)
                store_host_result(a.fin, ws, a.grid, r);
            else
                finish_store<Op>(a.fin, 0, r);
        }
        advance_tag<BLOCK>(a.arrive_slot, t);
        return;
    }
    __shared__ int last;
    if (threadIdx.x == 0) {
        store_partial(ws + blockIdx.x, v);
        last = arrive_last(a.arrive_slot, 0, blockIdx.x, (uint32_t)a.grid);
    }
    __syncthreads();
    if (!last)
        return;
    fold_partials_and_finish<Acc, Op, BLOCK>(ws, a.grid, a.fin);
}

template <class In, class Acc, class Op, class Map, int BLOCK, int UNROLL>
__global__ __launch_bounds__(BLOCK) void k_all_pass1(AllArgs a)
{
    using S = typename InTraits<In>::S;
    constexpr int V = InTraits<In>::vec;
    sgpr_ready(a.x, a.head, a.nvec, a.tail, a.arrive_slot, gridDim.x, static_cast<const void *>(g_final), a.grid,
               a.ws, a.fin.out, a.fin.init_bits, a.fin.mode, a.fin.out_dtype, a.fin.host_seq, a.spin_limit, a.tag_xor,
               a.n, a.y, blockIdx.x, a.nd);
    const uint32_t last_e = whole_prologue(a);
    const S *x = static_cast<const S *>(a.x);
    const u32x4 *body = reinterpret_cast<const u32x4 *>(x + a.head);

    Acc acc0[V], acc1[V];
    set_identity<Acc, Op>(acc0);
    set_identity<Acc, Op>(acc1);

    // Full tiles of BLOCK * UNROLL vectors; block b takes tiles b, b + G, ...
    // One wave instruction reads 64 * 16 = 1 KiB of consecutive bytes.
    constexpr int64_t kTile = int64_t(BLOCK) * UNROLL;
    const int64_t full = a.nvec / kTile;
    for (int64_t t = blockIdx.x; t < full; t += gridDim.x) {
        const u32x4 *p = body + t * kTile + threadIdx.x;
        u32x4 w[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            w[u] = load16(p + u * BLOCK);
        issue_barrier();
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            if (u & 1)
                fold_vec<In, Acc, Op, Map, V>(acc1, w[u]);
            else
                fold_vec<In, Acc, Op, Map, V>(acc0, w[u]);
        }
    }
    // the last, partial tile is spread over the whole grid
    const int64_t gtid = int64_t(blockIdx.x) * BLOCK + threadIdx.x;
    const int64_t gthreads = int64_t(gridDim.x) * BLOCK;
    for (int64_t i = full * kTile + gtid; i < a.nvec; i += gthreads)
        fold_vec<In, Acc, Op, Map, V>(acc0, load16(body + i));
    // scalars before the first 16-byte boundary and after the last vector
    Acc s = Op::template identity<Acc>();
    if (gtid < a.head)
        s = Op::apply(s, Map::apply(InTraits<In>::template one<Acc>(load1(x + gtid))));
    if (gtid < a.tail)
        s = Op::apply(s, Map::apply(InTraits<In>::template one<Acc>(load1(x + a.head + a.nvec * V + gtid))));

#pragma unroll
    for (int i = 0; i < V; ++i)
        acc0[i] = Op::apply(acc0[i], acc1[i]);
    Acc v = Op::apply(fold_all<Acc, Op, V>(acc0), s);
    v = block_reduce<Op, BLOCK>(v);
    whole_epilogue<Acc, Op, BLOCK>(a, v, last_e);
}

// Single output over a non-contiguous view: element i lives at
// layout_offset(i); scalar loads, several in flight per thread.
template <class In, class Acc, class Op, class Map, int BLOCK, int UNROLL>
__global__ __launch_bounds__(BLOCK) void k_all_pass1_strided(AllArgs a)
{
    using S = typename InTraits<In>::S;
    const uint32_t last_e = whole_prologue(a);
    const S *x = static_cast<const S *>(a.x);
    Acc acc[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
        acc[u] = Op::template identity<Acc>();
    const int64_t step = int64_t(gridDim.x) * BLOCK * UNROLL;
    for (int64_t base = int64_t(blockIdx.x) * BLOCK * UNROLL + threadIdx.x; base < a.n; base += step) {
        S w[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int64_t i = base + int64_t(u) * BLOCK;
            if (i < a.n)
                w[u] = load1(x + layout_offset(a.nd, a.ext, a.str, i));
        }
        issue_barrier();
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int64_t i = base + int64_t(u) * BLOCK;
            if (i < a.n)
                acc[u] = Op::apply(acc[u], Map::apply(InTraits<In>::template one<Acc>(w[u])));
        }
    }
    Acc v = fold_all<Acc, Op, UNROLL>(acc);
    v = block_reduce<Op, BLOCK>(v);
    whole_epilogue<Acc, Op, BLOCK>(a, v, last_e);
}

template <class Acc, class Op, int BLOCK>
__global__ __launch_bounds__(BLOCK) void k_all_pass2(Acc *ws, int grid, Finish fin)
{
    fold_partials_and_finish<Acc, Op, BLOCK>(ws, grid, fin);
}

// ========================================================= two-input source

template <class In, class Acc, class Op, class Map2, int V>
__device__ __forceinline__ void fold_vec2(Acc (&acc)[V], u32x4 wa, u32x4 wb)
{
    Acc ea[V], eb[V];
    InTraits<In>::template decode<Acc>(wa, ea);
    InTraits<In>::template decode<Acc>(wb, eb);
#pragma unroll
    for (int i = 0; i < V; ++i)
        acc[i] = Op::apply(acc[i], Map2::apply(ea[i], eb[i]));
}

template <class In, class Acc, class Map2>
__device__ __forceinline__ Acc map2_one(typename InTraits<In>::S a, typename InTraits<In>::S b)
{
    return Map2::apply(InTraits<In>::template one<Acc>(a), InTraits<In>::template one<Acc>(b));
}

// The 16 bytes that start K * 4 + r bytes into the 32 bytes c0:c1: whole
// dwords picked at compile time, then (2-byte elements only: r = 2) a byte
// funnel shift per dword.
template <int K, bool HALF>
__device__ __forceinline__ u32x4 join_shifted(u32x4 c0, u32x4 c1, uint32_t r)
{
    const uint32_t w[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        o[j] = HALF ? __builtin_amdgcn_alignbyte(w[j + K + 1], w[j + K], r) : w[j + K];
    return o;
}

// Lane l's value from lane (l + 1) mod 64: a DPP wavefront rotate.
__device__ __forceinline__ u32x4 from_next_lane(u32x4 v)
{
    constexpr int kWaveRol1 = 0x134;
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        o[j] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v[j], kWaveRol1, 0xf, 0xf, false);
    return o;
}

// Two-input load modes: every element on its own; both inputs in 16-byte
// vectors (same offset from a 16-byte boundary); x in vectors and y in
// aligned 16-byte chunks shifted into place (different offsets).
enum All2Mode { ALL2_ELEMENTS = 0, ALL2_VECTORS = 1, ALL2_SHIFTED = 2 };

// First pass over a fused two-input source f(x_i, y_i) (PR #139: the source
// may be a lazy broadcast).  ALL2_VECTORS: both bodies take the one-input
// kernel's tiles with UNROLL 16-byte loads of each input in flight.
// ALL2_SHIFTED: the body starts where x is 16-byte aligned and y is not;
// a wave covers UNROLL * 64 consecutive vectors (load u of lane l: vector
// 64 u + l of the wave's span), every lane loads x's vector and the aligned
// 16-byte chunk of y holding the start of its y elements, takes the
// following chunk from the next lane by a wavefront rotate (lane 63: lane
// 0's chunk of the next load, or, after the last, one more chunk it loads),
// and shifts the pair into place -- every byte of both inputs is loaded
// once, in 16-byte loads.  ALL2_ELEMENTS: every element is
// loaded on its own, 2 * UNROLL per input in flight, each wave instruction
// still reading consecutive elements.  Same grid, epilogue and workspace as
// the one-input pass.
template <class In, class Acc, class Op, class Map2, int BLOCK, int UNROLL, int MODE, int K = 0>
__global__ __launch_bounds__(BLOCK) void k_all2_pass1(AllArgs a)
{
    using S = typename InTraits<In>::S;
    sgpr_ready(a.x, a.y, a.head, a.nvec, a.tail, a.arrive_slot, gridDim.x, static_cast<const void *>(g_final),
               a.grid, a.ws, a.fin.out, a.fin.init_bits, a.fin.mode, a.fin.out_dtype, a.fin.host_seq, a.spin_limit,
               a.tag_xor, a.n, blockIdx.x, a.nd);
    const uint32_t last_e = whole_prologue(a);
    constexpr bool VECTOR = MODE != ALL2_ELEMENTS;
    constexpr int V = VECTOR ? InTraits<In>::vec : 1;
    const S *x = static_cast<const S *>(a.x);
    const S *y = static_cast<const S *>(a.y);

    Acc acc0[V], acc1[V];
    set_identity<Acc, Op>(acc0);
    set_identity<Acc, Op>(acc1);
    Acc s = Op::template identity<Acc>();
    const int64_t gtid = int64_t(blockIdx.x) * BLOCK + threadIdx.x;
    const int64_t gthreads = int64_t(gridDim.x) * BLOCK;

    if constexpr (MODE == ALL2_SHIFTED) {
        // y's elements of x's vector i: bytes sb + 16 i .. sb + 16 i + 15 of
        // y's aligned chunk stream, i.e. the end of chunk i and the start of
        // chunk i + 1.  The plan stops the body one chunk before y's last
        // whole one, so chunk i + 1 always lies inside y.
        const u32x4 *bx = reinterpret_cast<const u32x4 *>(x + a.head);
        const S *yh = y + a.head;
        // sb = K * 4 + r bytes: K whole dwords (a template argument), r = 2
        // only for 2-byte elements.  The aligned base comes from pointer
        // arithmetic, not from an integer: a pointer rebuilt from an integer
        // loses its global address space, and its loads compile to flat ones.
        const int sb = (int)(reinterpret_cast<uintptr_t>(yh) & 15);
        const u32x4 *by = reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(yh) - sb);
        constexpr bool HALF = sizeof(S) == 2;
        const uint32_t r = uint32_t(sb & 3);
        const int lane = (int)(threadIdx.x & 63);
        const bool last_lane = lane == 63;
        constexpr int64_t kTile = int64_t(BLOCK) * UNROLL;
        const int64_t full = a.nvec / kTile;
        for (int64_t t = blockIdx.x; t < full; t += gridDim.x) {
            const int64_t span = t * kTile + int64_t(threadIdx.x >> 6) * 64 * UNROLL;   // the wave's vectors
            u32x4 wx[UNROLL], wy[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                wx[u] = load16(bx + span + u * 64 + lane);
                wy[u] = load16(by + span + u * 64 + lane);
            }
            const u32x4 after = last_lane ? load16(by + span + UNROLL * 64) : u32x4{0u, 0u, 0u, 0u};
            issue_barrier();
            u32x4 rot = from_next_lane(wy[0]);
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const u32x4 rot_next = u + 1 < UNROLL ? from_next_lane(wy[u + 1 < UNROLL ? u + 1 : u]) : after;
                const u32x4 ys = join_shifted<K, HALF>(wy[u], last_lane ? rot_next : rot, r);
                rot = rot_next;
                if (u & 1)
                    fold_vec2<In, Acc, Op, Map2, V>(acc1, wx[u], ys);
                else
                    fold_vec2<In, Acc, Op, Map2, V>(acc0, wx[u], ys);
            }
        }
        for (int64_t i = full * kTile + gtid; i < a.nvec; i += gthreads)
            fold_vec2<In, Acc, Op, Map2, V>(acc0, load16(bx + i),
                                            join_shifted<K, HALF>(load16(by + i), load16(by + i + 1), r));
        if (gtid < a.head)
            s = Op::apply(s, map2_one<In, Acc, Map2>(load1(x + gtid), load1(y + gtid)));
        const int64_t t0 = a.head + a.nvec * InTraits<In>::vec;
        if (gtid < a.tail)
            s = Op::apply(s, map2_one<In, Acc, Map2>(load1(x + t0 + gtid), load1(y + t0 + gtid)));
    } else if constexpr (VECTOR) {
        const u32x4 *bx = reinterpret_cast<const u32x4 *>(x + a.head);
        const u32x4 *by = reinterpret_cast<const u32x4 *>(y + a.head);
        constexpr int64_t kTile = int64_t(BLOCK) * UNROLL;
        const int64_t full = a.nvec / kTile;
        for (int64_t t = blockIdx.x; t < full; t += gridDim.x) {
            const int64_t off = t * kTile + threadIdx.x;
            u32x4 wx[UNROLL], wy[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                wx[u] = load16(bx + off + u * BLOCK);
                wy[u] = load16(by + off + u * BLOCK);
            }
            issue_barrier();
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                if (u & 1)
                    fold_vec2<In, Acc, Op, Map2, V>(acc1, wx[u], wy[u]);
                else
                    fold_vec2<In, Acc, Op, Map2, V>(acc0, wx[u], wy[u]);
            }
        }
        for (int64_t i = full * kTile + gtid; i < a.nvec; i += gthreads)
            fold_vec2<In, Acc, Op, Map2, V>(acc0, load16(bx + i), load16(by + i));
        if (gtid < a.head)
            s = Op::apply(s, map2_one<In, Acc, Map2>(load1(x + gtid), load1(y + gtid)));
        const int64_t t0 = a.head + a.nvec * InTraits<In>::vec;
        if (gtid < a.tail)
            s = Op::apply(s, map2_one<In, Acc, Map2>(load1(x + t0 + gtid), load1(y + t0 + gtid)));
    } else {
        constexpr int U = 2 * UNROLL;
        const int64_t step = gthreads * U;
        for (int64_t base = int64_t(blockIdx.x) * BLOCK * U + threadIdx.x; base < a.n; base += step) {
            S wx[U], wy[U];
            const bool whole = base + int64_t(U - 1) * BLOCK < a.n;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = base + int64_t(u) * BLOCK;
                if (whole || i < a.n) {
                    wx[u] = load1(x + i);
                    wy[u] = load1(y + i);
                }
            }
            issue_barrier();
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = base + int64_t(u) * BLOCK;
                if (whole || i < a.n) {
                    const Acc e = map2_one<In, Acc, Map2>(wx[u], wy[u]);
                    if (u & 1)
                        acc1[0] = Op::apply(acc1[0], e);
                    else
                        acc0[0] = Op::apply(acc0[0], e);
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < V; ++i)
        acc0[i] = Op::apply(acc0[i], acc1[i]);
    Acc v = Op::apply(fold_all<Acc, Op, V>(acc0), s);
    v = block_reduce<Op, BLOCK>(v);
    whole_epilogue<Acc, Op, BLOCK>(a, v, last_e);
}

// ======================================================================= dims

// Tile kernel.  A block covers W = CL * V contiguous outputs of one run and
// RG = BLOCK / CL row groups; lane c of a row group loads V outputs' worth of
// one row (one 16-byte load when V > 1), so a wave reads 64 / CL rows of
// W * sizeof(In) bytes per instruction.  Row groups stride over the reduced
// dim with UNROLL loads in flight, then fold together (in-wave lane moves,
// then LDS across waves).  CL == BLOCK is the thread-per-output shape.
// PLAIN: one reduced dim (no segments) and at most one kept dim after the
// run's -- a 2-d array, or the middle dim of a 3-d one.  The block then finds
// its place from a few arguments: the general form keeps the segment and
// run layouts in scalar registers, whose loads the compiler spreads over
// several dependent batches before the first data load.
template <class In, class Acc, class Op, class Map, bool VECTOR, int CL, int BLOCK, int UNROLL, bool NT,
          bool PLAIN = false>
__global__ __launch_bounds__(BLOCK) void k_dims_tile(DimsArgs a)
{
    using S = typename InTraits<In>::S;
    constexpr int V = VECTOR ? InTraits<In>::vec : 1;
    constexpr int W = CL * V;
    constexpr int RG = BLOCK / CL;
    constexpr int NW = BLOCK / 64;
    static_assert(CL == BLOCK || CL <= 64, "a row group is within one wave, or the whole block");

    const int c = (int)(threadIdx.x % CL);
    const int rg = (int)(threadIdx.x / CL);
    if constexpr (PLAIN)
        sgpr_ready(a.x, a.tiles, a.tiles_per_run, a.run_len, a.s_red, a.row_len, a.rows_per_split, a.outer_str[0],
                   a.split, a.ws, a.n_out, a.arrive_slot, a.segs, a.fin.out, a.fin.init_bits, a.fin.mode,
                   a.fin.out_dtype, blockIdx.x, gridDim.x, a.splits_per_seg);
    // neighbouring tiles on one XCD share its L2 where a tile row is narrower
    // than a line (the tiled shape); columns tiles read whole lines, and
    // spread round-robin over the XCDs they measured 0.5-2% faster
    constexpr bool kColumns = NT && CL < BLOCK;
    const uint32_t b = kColumns ? blockIdx.x : xcd_block(blockIdx.x, gridDim.x);
    // tiles, runs and splits number below 2^31 (the grid does): 32-bit
    // arithmetic for the block's place, before its first loads
    const uint32_t tiles32 = uint32_t(a.tiles), tpr32 = uint32_t(a.tiles_per_run);
    const uint32_t tile32 = b % tiles32;
    const int64_t tile = tile32;
    const int sp = (int)(b / tiles32);
    const uint32_t run32 = tile32 / tpr32;
    const int64_t run = run32;
    const int64_t col0 = int64_t(tile32 - run32 * tpr32) * W;
    const int64_t col = col0 + int64_t(c) * V;
    const bool active = col < a.run_len;       // vector loads: run_len % V == 0
    const int64_t in_base =
        (PLAIN ? int64_t(run32) * a.outer_str[0] : layout_offset32(a.outer_nd, a.outer_ext, a.outer_str, run32)) + col;
    // this block's share of the reduced dims: segments [k0, k1) and, in
    // each, rows [j0, j1) of its row sequence (every row of the row dim, or
    // in the plain form every split-th row from row sp)
    int64_t k0, k1, j0, j1;
    if (PLAIN) {
        // one segment, whose rows the split units share interleaved: unit sp
        // takes rows sp, sp + split, ...  With a contiguous band of rows per
        // unit, the units' concurrent streams sat a power of two apart (64 MB
        // for 8192^2 f32), likely on the same memory channels and banks: that
        // geometry read in 40.0-40.6 us, the interleaved one in 37.9-38.6.
        k0 = 0;
        k1 = a.segs;                            // 1; left to the argument, the tail group below keeps
                                                // the general form's registers (known to be 1 it took 236 VGPRs)
        j0 = 0;
        j1 = div_nonneg(a.row_len - sp + a.split - 1, a.split);
    } else if (a.splits_per_seg > 1) {
        k0 = uint32_t(sp) / uint32_t(a.splits_per_seg);
        k1 = k0 + 1;
        j0 = (sp - k0 * a.splits_per_seg) * a.rows_per_split;
        j1 = j0 + a.rows_per_split < a.row_len ? j0 + a.rows_per_split : a.row_len;
    } else {
        k0 = int64_t(sp) * a.segs_per_split;
        k1 = k0 + a.segs_per_split < a.segs ? k0 + a.segs_per_split : a.segs;
        j0 = 0;
        j1 = a.row_len;
    }
    const S *xt = static_cast<const S *>(a.x) + in_base + (PLAIN ? int64_t(sp) * a.s_red : 0);
    const int64_t s = PLAIN ? a.s_red * a.split : a.s_red;

    Acc acc0[V], acc1[V];
    set_identity<Acc, Op>(acc0);
    set_identity<Acc, Op>(acc1);
    for (int64_t k = k0; active && k < k1; ++k) {
        const S *x = PLAIN ? xt : xt + layout_offset(a.seg_nd, a.seg_ext, a.seg_str, k);
        int64_t j = j0 + rg;
        // full groups of UNROLL rows per thread, every load issued first
        for (; j + int64_t(UNROLL - 1) * RG < j1; j += int64_t(UNROLL) * RG) {
            if constexpr (VECTOR) {
                u32x4 w[UNROLL];
#pragma unroll
                for (int u = 0; u < UNROLL; ++u)
                    w[u] = load16<NT>(reinterpret_cast<const u32x4 *>(x + (j + int64_t(u) * RG) * s));
                issue_barrier();
#pragma unroll
                for (int u = 0; u < UNROLL; ++u) {
                    if (u & 1)
                        fold_vec<In, Acc, Op, Map, V>(acc1, w[u]);
                    else
                        fold_vec<In, Acc, Op, Map, V>(acc0, w[u]);
                }
            } else {
                S w[UNROLL];
#pragma unroll
                for (int u = 0; u < UNROLL; ++u)
                    w[u] = load1<NT>(x + (j + int64_t(u) * RG) * s);
                issue_barrier();
#pragma unroll
                for (int u = 0; u < UNROLL; ++u) {
                    Acc e = Map::apply(InTraits<In>::template one<Acc>(w[u]));
                    if (u & 1)
                        acc1[0] = Op::apply(acc1[0], e);
                    else
                        acc0[0] = Op::apply(acc0[0], e);
                }
            }
        }
        // the last, partial group (fewer than UNROLL rows left per thread),
        // still with all of its loads in flight together
        if (j < j1) {
            // this thread's rows in the group, a count rather than a 64-bit
            // index per load; registers zeroed where a load is skipped, so the
            // group shares the registers of the full ones (f32: 56 VGPRs against
            // 88).  Not with 64 bytes of accumulators per lane (2-byte inputs
            // into 8-byte ones), where zeroing spilled instead.
            const int nu = (int)((j1 - j + RG - 1) / RG);
            if constexpr (VECTOR) {
                constexpr bool kZero = V * sizeof(Acc) <= 32;
                u32x4 w[UNROLL];
#pragma unroll
                for (int u = 0; u < UNROLL; ++u) {
                    if constexpr (kZero)
                        w[u] = u32x4{0u, 0u, 0u, 0u};
                    if (u < nu)
                        w[u] = load16<NT>(reinterpret_cast<const u32x4 *>(x + (j + int64_t(u) * RG) * s));
                }
                issue_barrier();
#pragma unroll
                for (int u = 0; u < UNROLL; ++u)
                    if (u < nu)
                        fold_vec<In, Acc, Op, Map, V>(acc0, w[u]);
            } else {
                S w[UNROLL];
#pragma unroll
                for (int u = 0; u < UNROLL; ++u) {
                    w[u] = S{};
                    if (u < nu)
                        w[u] = load1<NT>(x + (j + int64_t(u) * RG) * s);
                }
                issue_barrier();
#pragma unroll
                for (int u = 0; u < UNROLL; ++u)
                    if (u < nu)
                        acc0[0] = Op::apply(acc0[0], Map::apply(InTraits<In>::template one<Acc>(w[u])));
            }
        }
    }
#pragma unroll
    for (int i = 0; i < V; ++i)
        acc0[i] = Op::apply(acc0[i], acc1[i]);

    const int64_t o_tile = run * a.run_len + col0;     // output index of the tile's first column
    const int64_t outs_left = a.run_len - col0;        // outputs of this tile inside the run
    Acc *ws = static_cast<Acc *>(a.ws);

    if constexpr (CL == BLOCK) {
        // one row group: this thread owns its V outputs
        if (active) {
#pragma unroll
            for (int i = 0; i < V; ++i) {
                const int64_t o = o_tile + int64_t(c) * V + i;
                if (a.split > 1)
                    ws[int64_t(sp) * a.n_out + o] = acc0[i];
                else
                    finish_store<Op>(a.fin, out_index(a.omap, o), acc0[i]);
            }
        }
    } else {
        // fold the 64 / CL row groups of each wave, then the NW waves
#pragma unroll
        for (int i = 0; i < V; ++i)
            acc0[i] = wave_reduce_columns<CL, Op>(acc0[i]);
        __shared__ Acc part[NW][W];
        const int w = (int)(threadIdx.x >> 6);
        if (lane_id() < CL) {
#pragma unroll
            for (int i = 0; i < V; ++i)
                part[w][lane_id() * V + i] = acc0[i];
        }
        __syncthreads();
        const bool mine = threadIdx.x < W && int64_t(threadIdx.x) < outs_left;
        const int64_t o = o_tile + threadIdx.x;
        Acc v = Op::template identity<Acc>();
        if (mine) {
            v = part[0][threadIdx.x];
#pragma unroll
            for (int k = 1; k < NW; ++k)
                v = Op::apply(v, part[k][threadIdx.x]);
        }
        if (a.split == 1) {
            if (mine)
                finish_store<Op>(a.fin, out_index(a.omap, o), v);
            return;
        }
        if (a.arrive_slot < 0) {                // a second launch folds the splits
            if (mine)
                ws[int64_t(sp) * a.n_out + o] = v;
            return;
        }
        // the last of the tile's `split` blocks to arrive folds and finishes
        if (mine) {
            store_partial(ws + int64_t(sp) * a.n_out + o, v);
            wait_stores();
        }
        __shared__ int last;
        __syncthreads();
        if (threadIdx.x == 0)
            last = arrive_last(a.arrive_slot, tile, (uint32_t)sp, (uint32_t)a.split);
        __syncthreads();
        if (!last)
            return;
        if (mine)
            finish_store<Op>(a.fin, out_index(a.omap, o), fold_partials<Acc, Op>(ws, o, a.split, a.n_out));
    }
}

// Row kernel: one wave per (output, chunk) over a contiguous reduced dim.
// With several reduced dims the others index segments of such rows; a chunk
// is every split-th segment or a piece of one segment's row.  Each row piece
// takes a scalar head up to its first 16-byte boundary, 16-byte loads
// (UNROLL in flight per lane) and a scalar tail.
template <class In, class Acc, class Op, class Map, int BLOCK, int UNROLL>
__global__ __launch_bounds__(BLOCK) void k_dims_row(DimsArgs a)
{
    using S = typename InTraits<In>::S;
    constexpr int V = InTraits<In>::vec;
    const int lane = lane_id();
    // the wave's number, read as uniform so that the index arithmetic below
    // runs on the scalar unit
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    sgpr_ready(a.x, a.n_out, a.split, a.splits_per_seg, a.rows_per_split, a.row_len, a.segs_per_split, a.segs,
               a.kept_nd, a.kept_ext[0], a.kept_str[0], a.seg_nd, a.arrive_slot, a.ws, a.fin.out, a.fin.mode,
               a.fin.init_bits, a.fin.out_dtype, a.kept_ext[1], a.kept_str[1]);
    const int64_t unit = int64_t(blockIdx.x) * (BLOCK / 64) + wave;
    if (unit >= a.n_out * a.split)
        return;                                 // whole wave; no block barrier below
    const int64_t o = a.split == 1 ? unit : div_nonneg(unit, a.split);
    const int sp = (int)(unit - o * a.split);
    int64_t k0, k1, kstep = 1, j0, j1;
    if (a.splits_per_seg > 1) {
        k0 = uint32_t(sp) / uint32_t(a.splits_per_seg);
        k1 = k0 + 1;
        j0 = (sp - k0 * a.splits_per_seg) * a.rows_per_split;
        j1 = j0 + a.rows_per_split < a.row_len ? j0 + a.rows_per_split : a.row_len;
    } else {
        // split units take whole segments, interleaved: unit sp takes
        // segments sp, sp + split, ...  (3136x256x84 f32 dims=(1,3), split 8:
        // 42.3-42.5 us against 43.3-43.5 for runs of consecutive segments)
        k0 = sp;
        k1 = a.segs;
        kstep = a.split;
        j0 = 0;
        j1 = a.row_len;
    }
    const S *base = static_cast<const S *>(a.x) + layout_offset(a.kept_nd, a.kept_ext, a.kept_str, o) + j0;
    const int64_t len = j1 - j0;

    Acc acc0[V], acc1[V];
    set_identity<Acc, Op>(acc0);
    set_identity<Acc, Op>(acc1);
    Acc s = Op::template identity<Acc>();
    for (int64_t k = k0; k < k1; k += kstep) {
        const S *row = base + layout_offset(a.seg_nd, a.seg_ext, a.seg_str, k);
        // scalar head up to the first 16-byte boundary, vector body, scalar tail
        int64_t head = (int64_t)(((16u - ((uintptr_t)row & 15u)) & 15u) / sizeof(S));
        head = head < len ? head : len;
        const int64_t nv = (len - head) / V;
        const int64_t tail = len - head - nv * V;
        const u32x4 *body = reinterpret_cast<const u32x4 *>(row + head);
        int64_t i = lane;
        for (; i + int64_t(UNROLL - 1) * 64 < nv; i += int64_t(UNROLL) * 64) {
            u32x4 w[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u)
                w[u] = load16(body + i + u * 64);
            issue_barrier();
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                if (u & 1)
                    fold_vec<In, Acc, Op, Map, V>(acc1, w[u]);
                else
                    fold_vec<In, Acc, Op, Map, V>(acc0, w[u]);
            }
        }
        if (i < nv) {                           // last, partial group, loads together
            // this lane's loads in the group, one count rather than a 64-bit
            // index per load.  Each vector holds zero where its load is
            // skipped: left undefined there, every one kept registers of its
            // own (170 VGPRs in all, against 91).  No load is issued twice: the
            // loads bypass the cache, so a repeat is fetched from memory again.
            const int nu = (int)((nv - i + 63) / 64);
            u32x4 w[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                w[u] = u32x4{0u, 0u, 0u, 0u};
                if (u < nu)
                    w[u] = load16(body + i + u * 64);
            }
            issue_barrier();
#pragma unroll
            for (int u = 0; u < UNROLL; ++u)
                if (u < nu)
                    fold_vec<In, Acc, Op, Map, V>(acc0, w[u]);
        }
        if (lane < head)
            s = Op::apply(s, Map::apply(InTraits<In>::template one<Acc>(load1(row + lane))));
        if (lane < tail)
            s = Op::apply(s, Map::apply(InTraits<In>::template one<Acc>(load1(row + head + nv * V + lane))));
    }
#pragma unroll
    for (int k = 0; k < V; ++k)
        acc0[k] = Op::apply(acc0[k], acc1[k]);
    Acc v = wave_reduce<Op>(Op::apply(fold_all<Acc, Op, V>(acc0), s));
    Acc *ws = static_cast<Acc *>(a.ws);
    if (a.split == 1) {
        if (lane == 0)
            finish_store<Op>(a.fin, o, v);
        return;
    }
    if (a.arrive_slot < 0) {                    // a second launch folds the chunks
        if (lane == 0)
            ws[int64_t(sp) * a.n_out + o] = v;
        return;
    }
    // the last of the output's `split` waves to arrive folds and finishes
    int last = 0;
    if (lane == 0) {
        store_partial(ws + int64_t(sp) * a.n_out + o, v);
        last = arrive_last(a.arrive_slot, o, (uint32_t)sp, (uint32_t)a.split);
    }
    last = __builtin_amdgcn_readfirstlane(last);
    if (!last)
        return;
    Acc r = Op::template identity<Acc>();
    for (int k = lane; k < a.split; k += 64)
        r = Op::apply(r, load_partial(ws + int64_t(k) * a.n_out + o));
    r = wave_reduce<Op>(r);
    if (lane == 0)
        finish_store<Op>(a.fin, o, r);
}

// Generic kernel: any layout.  A unit is (output, chunk of its reduced
// elements); blocks take units grid-stride.  The block's threads share the
// chunk, element j at layout offset walked from j - BLOCK without a
// division, UNROLL loads in flight per thread.  VECTOR: the innermost
// reduced dim is contiguous and every reduced row starts 16-byte aligned, so
// the units are 16-byte vectors (the planner scales the reduced layout and
// the chunk to vectors).  A split output is finished by the last of its
// chunks to arrive, or by a second launch.
template <class In, class Acc, class Op, class Map, int BLOCK, int UNROLL, bool VECTOR>
__global__ __launch_bounds__(BLOCK) void k_dims_generic(DimsArgs a)
{
    using S = typename InTraits<In>::S;
    constexpr int V = VECTOR ? InTraits<In>::vec : 1;
    const S *x = static_cast<const S *>(a.x);
    Acc *ws = static_cast<Acc *>(a.ws);
    const int64_t units = a.n_out * a.split;
    const int64_t len = a.m / V;               // reduced length in load units
    for (int64_t unit = blockIdx.x; unit < units; unit += gridDim.x) {
        const int64_t o = a.split == 1 ? unit : div_nonneg(unit, a.split);
        const int sp = (int)(unit - o * a.split);
        const int64_t j0 = int64_t(sp) * a.rows_per_split;
        const int64_t j1 = j0 + a.rows_per_split < len ? j0 + a.rows_per_split : len;
        const S *xo = x + layout_offset(a.kept_nd, a.kept_ext, a.kept_str, o);
        Acc acc0[V], acc1[V];
        set_identity<Acc, Op>(acc0);
        set_identity<Acc, Op>(acc1);
        Walk w;
        w.init(a.red_nd, a.red_ext, a.red_str, j0 + threadIdx.x, BLOCK);
        for (int64_t j = j0 + threadIdx.x; j < j1; j += int64_t(BLOCK) * UNROLL) {
            if constexpr (VECTOR) {
                u32x4 v[UNROLL];
#pragma unroll
                for (int u = 0; u < UNROLL; ++u) {
                    if (j + int64_t(u) * BLOCK < j1)
                        v[u] = load16(reinterpret_cast<const u32x4 *>(xo + w.off));
                    w.advance(a.red_nd, a.red_ext);
                }
                issue_barrier();
#pragma unroll
                for (int u = 0; u < UNROLL; ++u) {
                    if (j + int64_t(u) * BLOCK < j1) {
                        if (u & 1)
                            fold_vec<In, Acc, Op, Map, V>(acc1, v[u]);
                        else
                            fold_vec<In, Acc, Op, Map, V>(acc0, v[u]);
                    }
                }
            } else {
                S v[UNROLL];
#pragma unroll
                for (int u = 0; u < UNROLL; ++u) {
                    if (j + int64_t(u) * BLOCK < j1)
                        v[u] = load1(xo + w.off);
                    w.advance(a.red_nd, a.red_ext);
                }
                issue_barrier();
#pragma unroll
                for (int u = 0; u < UNROLL; ++u) {
                    if (j + int64_t(u) * BLOCK < j1) {
                        const Acc e = Map::apply(InTraits<In>::template one<Acc>(v[u]));
                        if (u & 1)
                            acc1[0] = Op::apply(acc1[0], e);
                        else
                            acc0[0] = Op::apply(acc0[0], e);
                    }
                }
            }
        }
#pragma unroll
        for (int i = 0; i < V; ++i)
            acc0[i] = Op::apply(acc0[i], acc1[i]);
        Acc v = block_reduce<Op, BLOCK>(fold_all<Acc, Op, V>(acc0));
        if (a.split == 1) {
            if (threadIdx.x == 0)
                finish_store<Op>(a.fin, o, v);
        } else if (a.arrive_slot < 0) {         // a second launch folds the chunks
            if (threadIdx.x == 0)
                ws[int64_t(sp) * a.n_out + o] = v;
        } else {                                // the last chunk to arrive finishes
            __shared__ int last;
            if (threadIdx.x == 0) {
                store_partial(ws + int64_t(sp) * a.n_out + o, v);
                last = arrive_last(a.arrive_slot, o, (uint32_t)sp, (uint32_t)a.split);
            }
            __syncthreads();
            // in split order, as the second launch folds them
            if (last && threadIdx.x == 0)
                finish_store<Op>(a.fin, o, fold_partials<Acc, Op>(ws, o, a.split, a.n_out));
        }
        __syncthreads();                        // LDS of block_reduce and `last` are reused
    }
}

// Second pass of a split dims reduction: fold split partials per output.
template <class Acc, class Op, int BLOCK>
__global__ __launch_bounds__(BLOCK) void k_split_finish(const Acc *ws, int64_t n_out, int split, Finish fin,
                                                        OutMap omap)
{
    const int64_t o = int64_t(blockIdx.x) * BLOCK + threadIdx.x;
    if (o >= n_out)
        return;
    Acc v = ws[o];
    for (int k = 1; k < split; ++k)
        v = Op::apply(v, ws[int64_t(k) * n_out + o]);
    finish_store<Op>(fin, out_index(omap, o), v);
}

// ================================================================== launchers

// Launch a call's first kernel.  With a timing event pair the events ride
// on the kernel's own dispatch packet (hipExtLaunchKernel), so they bracket
// exactly that kernel and add no packets of their own to the stream.
template <class... KArgs, class... Args>
void launch_first(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t st, const Launch &L,
                  Args... args)
{
    hipEvent_t b = static_cast<hipEvent_t>(L.ev_begin), e = static_cast<hipEvent_t>(L.ev_end);
    if (b && e)
        hipExtLaunchKernelGGL(kernel, grid, block, 0, st, b, e, 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
}

// Launch the tile kernel shape the planner chose (kernel, vector width,
// lanes per tile row).  Returns false for a shape that has no instantiation.
template <class In, class Acc, class Op, class Map>
bool launch_tile(const Launch &L, dim3 grid, hipStream_t st)
{
    constexpr int V = InTraits<In>::vec;
    constexpr int U = tune::kDimsUnroll;
    const bool vec = L.vec > 1;
    if (vec && L.vec != V)
        return false;
    const DimsArgs &a = L.dims;
#define RK_TILE(VECTOR, CL, B, NT) \
    launch_first(&k_dims_tile<In, Acc, Op, Map, VECTOR, CL, B, U, NT>, grid, dim3(B), st, L, a)
    if (L.kernel == K_THREAD) {
        constexpr int B = tune::kThreadBlock;
        if (L.lanes != B || L.block != B)
            return false;
        if (vec)
            RK_TILE(true, B, B, true);
        else
            RK_TILE(false, B, B, true);
        return true;
    }
    if (L.kernel == K_TILED) {
        constexpr int B = tune::kTiledBlock;
        constexpr int CLV = tune::kTiledOutputs / V, CLS = tune::kTiledOutputs;
        if (L.block != B || L.lanes != (vec ? CLV : CLS))
            return false;
        if (vec)
            RK_TILE(true, CLV, B, false);
        else
            RK_TILE(false, CLS, B, false);
        return true;
    }
    constexpr int B = tune::kColumnsBlock;
    if (L.block != B)
        return false;
    if (!vec) {
        if (L.lanes != tune::kColumnsScalarLanes)
            return false;
        RK_TILE(false, tune::kColumnsScalarLanes, B, true);
        return true;
    }
    // one reduced dim and at most one kept dim after the run's: the plain form
    const bool plain = a.seg_nd == 0 && a.segs == 1 && a.outer_nd <= 1 && (a.split == 1 || a.splits_per_seg == a.split);
#define RK_COLS(CL)                                                                                         \
    (plain ? launch_first(&k_dims_tile<In, Acc, Op, Map, true, CL, B, U, true, true>, grid, dim3(B), st, L, a) \
           : launch_first(&k_dims_tile<In, Acc, Op, Map, true, CL, B, U, true>, grid, dim3(B), st, L, a))
    switch (L.lanes) {          // tile rows of 16 * lanes bytes
    case 8: RK_COLS(8); return true;
    case 16: RK_COLS(16); return true;
    case 32: RK_COLS(32); return true;
    }
#undef RK_COLS
#undef RK_TILE
    return false;
}

// Run the call's kernels for one (In, Acc, Op, Map).
template <class In, class Acc, class Op, class Map>
int run_typed(const Launch &L)
{
    hipStream_t st = static_cast<hipStream_t>(L.stream);
    const dim3 grid((unsigned)L.grid), block((unsigned)L.block);

    int split = 1;
    switch (L.kernel) {
    case K_ALL:
        launch_first(&k_all_pass1<In, Acc, Op, Map, tune::kAllBlock, tune::kAllUnroll>, grid,
                     dim3(tune::kAllBlock), st, L, L.all);
        break;
    case K_ALL_STRIDED:
        launch_first(&k_all_pass1_strided<In, Acc, Op, Map, tune::kAllBlock, tune::kAllUnroll>, grid,
                     dim3(tune::kAllBlock), st, L, L.all);
        break;
    case K_THREAD: case K_TILED: case K_COLUMNS: {
        if (!launch_tile<In, Acc, Op, Map>(L, grid, st))
            return ST_INVALID;
        split = L.dims.split;
        break;
    }
    case K_ROW: {
        constexpr int RU = sizeof(Acc) == 8 && sizeof(typename InTraits<In>::S) == 2 ? tune::kRowUnrollHalfToWide
                                                                                    : tune::kRowUnroll;
        launch_first(&k_dims_row<In, Acc, Op, Map, tune::kDimsBlock, RU>, grid, block, st, L, L.dims);
        split = L.dims.split;
        break;
    }
    case K_GENERIC:
        if (L.vec > 1) {
            if (L.vec != InTraits<In>::vec)
                return ST_INVALID;
            launch_first(&k_dims_generic<In, Acc, Op, Map, tune::kDimsBlock, tune::kGenericUnroll, true>, grid,
                         block, st, L, L.dims);
        } else {
            launch_first(&k_dims_generic<In, Acc, Op, Map, tune::kDimsBlock, tune::kGenericUnroll, false>, grid,
                         block, st, L, L.dims);
        }
        split = L.dims.split;
        break;
    default:
        return ST_INVALID;
    }
    if (hipGetLastError() != hipSuccess)
        return ST_HIP;

    // second launches, unless the call finished inside its first launch
    if ((L.kernel == K_ALL || L.kernel == K_ALL_STRIDED) && L.all.grid > 1 && L.all.arrive_slot < 0) {
        hipLaunchKernelGGL((k_all_pass2<Acc, Op, tune::kPass2Block>), dim3(1), dim3(tune::kPass2Block), 0,
                           st, static_cast<Acc *>(L.all.ws), L.all.grid, L.all.fin);
    } else if (split > 1 && L.dims.arrive_slot < 0) {
        constexpr int B = 256;
        const unsigned g = (unsigned)((L.dims.n_out + B - 1) / B);
        hipLaunchKernelGGL((k_split_finish<Acc, Op, B>), dim3(g), dim3(B), 0, st,
                           static_cast<const Acc *>(L.dims.ws), L.dims.n_out, split, L.dims.fin, L.dims.omap);
    } else {
        return ST_OK;
    }
    return hipGetLastError() == hipSuccess ? ST_OK : ST_HIP;
}

// Run a two-input call for one (In, Acc, Op, Map2).
template <class In, class Acc, class Op, class Map2>
int run_typed2(const Launch &L)
{
    hipStream_t st = static_cast<hipStream_t>(L.stream);
    const dim3 grid((unsigned)L.grid), block(tune::kAllBlock);
    using S = typename InTraits<In>::S;
    const bool same_phase = ((reinterpret_cast<uintptr_t>(static_cast<const S *>(L.all.x) + L.all.head) ^
                              reinterpret_cast<uintptr_t>(static_cast<const S *>(L.all.y) + L.all.head)) & 15) == 0;
    if (L.vec > 1 && same_phase)
        launch_first(&k_all2_pass1<In, Acc, Op, Map2, tune::kAllBlock, tune::kAllUnroll, ALL2_VECTORS>, grid,
                     block, st, L, L.all);
    else if (L.vec > 1) {
        // whole dwords of y's phase: 1..3 for 4-byte elements, 2 for 8-byte
        // ones, 0..3 for 2-byte ones
        const int k = int((reinterpret_cast<uintptr_t>(static_cast<const S *>(L.all.y) + L.all.head) & 15) >> 2);
#define RK_ALL2_SHIFTED(KK) launch_first(&k_all2_pass1<In, Acc, Op, Map2, tune::kAllBlock, tune::kAllUnroll, \
                                                       ALL2_SHIFTED, KK>, grid, block, st, L, L.all)
        if constexpr (sizeof(S) == 8) {
            RK_ALL2_SHIFTED(2);
        } else {
            if (k == 0) {
                if constexpr (sizeof(S) == 2)
                    RK_ALL2_SHIFTED(0);
                else
                    return ST_INVALID;          // 4-byte phases differ by whole dwords
            } else if (k == 1) {
                RK_ALL2_SHIFTED(1);
            } else if (k == 2) {
                RK_ALL2_SHIFTED(2);
            } else {
                RK_ALL2_SHIFTED(3);
            }
        }
#undef RK_ALL2_SHIFTED
    }
    else
        launch_first(&k_all2_pass1<In, Acc, Op, Map2, tune::kAllBlock, tune::kAllUnroll, ALL2_ELEMENTS>, grid,
                     block, st, L, L.all);
    if (hipGetLastError() != hipSuccess)
        return ST_HIP;
    if (L.all.grid > 1 && L.all.arrive_slot < 0) {
        hipLaunchKernelGGL((k_all_pass2<Acc, Op, tune::kPass2Block>), dim3(1), dim3(tune::kPass2Block), 0, st,
                           static_cast<Acc *>(L.all.ws), L.all.grid, L.all.fin);
        if (hipGetLastError() != hipSuccess)
            return ST_HIP;
    }
    return ST_OK;
}

template <class In, class Acc, class Op>
int run_op2(const Launch &L)
{
    switch (L.map) {
    case 0: return run_typed2<In, Acc, Op, Map2Mul>(L);
    case 1: return run_typed2<In, Acc, Op, Map2SqDiff>(L);
    case 2: return run_typed2<In, Acc, Op, Map2AbsDiff>(L);
    }
    return ST_INVALID;
}

template <class In, class Acc>
int run_acc(const Launch &L)
{
    if (L.kernel == K_ALL2) {
        switch (L.op) {
        case 0: return run_op2<In, Acc, OpSum>(L);
        case 1: return run_op2<In, Acc, OpMax>(L);
        case 2: return run_op2<In, Acc, OpMin>(L);
        }
        return ST_INVALID;
    }
    switch (L.op) {
    case 0:
        switch (L.map) {
        case 0: return run_typed<In, Acc, OpSum, MapIdentity>(L);
        case 1: return run_typed<In, Acc, OpSum, MapSquare>(L);
        case 2: return run_typed<In, Acc, OpSum, MapAbs>(L);
        }
        break;
    case 1:
        switch (L.map) {
        case 0: return run_typed<In, Acc, OpMax, MapIdentity>(L);
        case 1: return run_typed<In, Acc, OpMax, MapSquare>(L);
        case 2: return run_typed<In, Acc, OpMax, MapAbs>(L);
        }
        break;
    case 2:
        switch (L.map) {
        case 0: return run_typed<In, Acc, OpMin, MapIdentity>(L);
        case 1: return run_typed<In, Acc, OpMin, MapSquare>(L);
        case 2: return run_typed<In, Acc, OpMin, MapAbs>(L);
        }
        break;
    }
    return ST_INVALID;
}

// Add this unit's count of waits that gave up on `slot` (slot < 0: the
// entry of calls without a slot) and on the shared entry to *count, and
// clear both.  With `repair` and a count, also zero the slot's tagged words:
// a block that had not even started when its collection gave up publishes
// under the next call's tag, and the drained stream guarantees every such
// block has ended.  Synchronous (hipMemcpy to and from the tables).  In the
// unit's own namespace: an inline function of one name in every unit is
// merged by the linker into one copy, which would only see that unit's tables.
// REPAIR: the unit holds whole-array tagged words (the scan units hold none).
namespace RK_UNIT {
template <bool REPAIR>
inline int take_timeouts(int slot, uint64_t *count, bool repair)
{
    uint32_t t[kTimeoutEntries];
    if (hipMemcpyFromSymbol(t, HIP_SYMBOL(g_timeouts), sizeof t, 0, hipMemcpyDeviceToHost) != hipSuccess)
        return ST_HIP;
    const int e = slot >= 0 && slot < kArriveSlots ? slot : kArriveSlots;
    const uint64_t n = uint64_t(t[e]) + (e != kArriveSlots ? t[kArriveSlots] : 0u);
    const uint32_t zero = 0;
    if ((t[e] && hipMemcpyToSymbol(HIP_SYMBOL(g_timeouts), &zero, 4, size_t(e) * 4, hipMemcpyHostToDevice) != hipSuccess) ||
        (t[kArriveSlots] && hipMemcpyToSymbol(HIP_SYMBOL(g_timeouts), &zero, 4, size_t(kArriveSlots) * 4,
                                              hipMemcpyHostToDevice) != hipSuccess))
        return ST_HIP;
    if constexpr (REPAIR) {
        if (repair && t[e] && e != kArriveSlots) {
            static const uint64_t zeros[2 * kFinalCapacity] = {};
            const size_t off = (size_t(e) * kFinalSlotWords + kFinalHeaderWords) * sizeof(uint64_t);
            if (hipMemcpyToSymbol(HIP_SYMBOL(g_final), zeros, sizeof zeros, off, hipMemcpyHostToDevice) != hipSuccess)
                return ST_HIP;
        }
    }
    *count += n;
    return ST_OK;
}
}  // namespace RK_UNIT

// Accumulators a given input type may use (the public dtype table).
template <class In>
int run_in(const Launch &L)
{
    if (L.kernel == K_SET_TAG) {                // this translation unit's copy of the slot
        hipLaunchKernelGGL(RK_UNIT::k_set_final_tag<>, dim3(1), dim3(kFinalTagCopies), 0,
                           static_cast<hipStream_t>(L.stream), L.all.arrive_slot, uint32_t(L.all.n));
        return hipGetLastError() == hipSuccess ? ST_OK : ST_HIP;
    }
    if (L.kernel == K_TAKE_TIMEOUTS)            // this translation unit's counts (the stream has drained)
        return RK_UNIT::take_timeouts<true>(L.all.arrive_slot, static_cast<uint64_t *>(L.all.ws), L.all.n != 0);
    if constexpr (std::is_same_v<In, float> || std::is_same_v<In, bf16_in> || std::is_same_v<In, f16_in>) {
        if (L.acc == F32) return run_acc<In, float>(L);
        if (L.acc == F64) return run_acc<In, double>(L);
    } else if constexpr (std::is_same_v<In, double>) {
        if (L.acc == F64) return run_acc<In, double>(L);
    } else if constexpr (std::is_same_v<In, int32_t>) {
        if (L.acc == I32) return run_acc<In, int32_t>(L);
        if (L.acc == I64) return run_acc<In, int64_t>(L);
    } else if constexpr (std::is_same_v<In, int64_t>) {
        if (L.acc == I64) return run_acc<In, int64_t>(L);
    }
    return ST_UNSUPPORTED;
}

}  // namespace rk
