// rk_launch.hpp -- what the C ABI hands to the kernel translation units.
//
// Plain structs passed by value as kernel arguments, plus one launcher entry
// per input dtype (each lives in its own .hip file so they compile in
// parallel).  No HIP types appear here.
#pragma once

#include <cstdint>

namespace rk {

// Finishing modes of the last pass: the three public modes plus PARTIAL,
// which stores a bare accumulator per block for a following pass.
enum FinishMode { FIN_OVERWRITE = 0, FIN_FOLD = 1, FIN_HOST = 2, FIN_PARTIAL = 3 };

// Arrival counters for finishing in the last block to arrive (no second
// launch).  Each stream slot owns kArriveCapacity counters; a plan whose
// counters would not fit takes the two-launch path.
constexpr int kArriveSlots = 32;
constexpr int kArriveCapacity = 4096;
// Atomics on one 128-byte line are serialised where device-scope atomics are
// performed, about 10 ns each on MI355X: 1024 blocks counting themselves on
// one counter queue for ~10 us when they end together.  So n > kArriveGroup
// arrivals are counted in groups of kArriveGroup consecutive members, each
// group on a counter of its own, and the last of each group counts the
// group on the output's top counter.
constexpr int kArriveGroup = 32;

// Counters one output takes for n arrivals: the top one, plus one per group.
constexpr int64_t arrive_counters(int64_t n)
{
    return n > kArriveGroup ? 1 + (n + kArriveGroup - 1) / kArriveGroup : 1;
}

// A whole-array pass of up to kFinalCapacity blocks finishes without
// counters: every block stores its partial tagged with the call's number,
// and block 0 collects them (see rk_device.hpp).
constexpr int kFinalCapacity = 2048;
constexpr uint32_t kFinalSpinLimit = 1u << 24;   // block 0's polls (with a short sleep each): far beyond any run

// Waits that give up (block 0's collection, a scan's look-back) are counted
// per stream slot, plus one shared entry for calls on streams without a
// slot, in each translation unit's own table; the host reads and clears
// them (rk_stream_timeouts).
constexpr int kTimeoutEntries = kArriveSlots + 1;

// Host mode without the pinned result buffer: the bare result goes to
// ws[grid] and the call's sequence number to the 4 bytes at this byte offset
// of the workspace, so the host can tell a result of this call from stale
// bytes after copying both back.
constexpr int64_t host_seq_offset(int64_t grid, int acc_size) { return ((grid + 1) * acc_size + 7) / 8 * 8; }

struct Finish {
    void *out;            // device output (OVERWRITE / FOLD); HOST: pinned host result buffer or NULL
    int out_dtype;
    int mode;             // FinishMode
    uint64_t init_bits;   // starting value, accumulator bits (identity when no init)
    uint32_t host_seq;    // HOST: stored after the result (result buffer: at byte 8;
                          // workspace: at host_seq_offset)
};

// Outputs numbered in storage order instead of the output's own (a tile
// kernel over kept dims that only run contiguously in another order): output
// o goes to sum_k digit_k(o) * str[k], o's digits taken over ext in order.
// nd 0: output o is out[o].  Only the dims arguments carry one; the
// whole-array arguments and their kernels' code stay as they are.
struct OutMap {
    int nd;
    int64_t ext[4];
    int64_t str[4];
};

struct AllArgs {
    const void *x;        // first element
    const void *y;        // two-input source: first element of the second input
    int64_t n;            // elements
    int64_t head;         // scalars before the 16-byte-aligned body
    int64_t nvec;         // 16-byte vectors in the body (strided variant: elements)
    int64_t tail;         // scalars after the body
    int nd;               // strided variant: element i sits at sum_d ((i / prod ext[<d]) % ext[d]) * str[d]
    int64_t ext[4];
    int64_t str[4];
    void *ws;             // grid + 1 accumulators, then (host mode, copied back) the sequence word
    int grid;
    int arrive_slot;      // >= 0: the last block to arrive finishes (one launch)
    uint32_t spin_limit;  // block 0's polls before its collection gives up
    uint32_t tag_xor;     // 0; nonzero only to make block 0 wait for a tag no block carries (a test hook)
    Finish fin;
};

struct DimsArgs {
    const void *x;        // element (0, ..., 0)
    void *ws;             // split * n_out accumulators when split > 1
    int64_t n_out;
    int64_t m;            // elements per output
    int64_t s_red;        // tile kernels: stride of the row dim (one of the reduced dims)
    int64_t row_len;      // tile kernels: extent of the row dim
    int seg_nd;           // tile kernels: the other reduced dims; each index of them is a segment
    int64_t seg_ext[3];
    int64_t seg_str[3];
    int64_t segs;         // segments (1 when the row dim is the only reduced dim)
    int64_t segs_per_split;   // splits_per_seg == 1: whole segments per split unit
    int64_t splits_per_seg;   // > 1: split units per segment, rows_per_split rows each
    int64_t run_len;      // contiguous outputs per run (tile kernels)
    int64_t tiles_per_run;
    int64_t tiles;
    int64_t rows_per_split;   // row kernel: reduced elements per split unit; generic: load units
    int split;
    int outer_nd;         // kept dims after the first (tile kernels): run offsets
    int64_t outer_ext[3];
    int64_t outer_str[3];
    int kept_nd;          // all kept dims (row and generic kernels)
    int64_t kept_ext[4];
    int64_t kept_str[4];
    int red_nd;           // reduced dims (generic kernel)
    int64_t red_ext[4];
    int64_t red_str[4];
    int arrive_slot;      // >= 0 with split > 1: the last block (or wave) of each output finishes
    Finish fin;
    OutMap omap;          // tile kernels: where each output goes (nd 0: in order)
};

struct Launch {
    int kernel;           // rk::Kernel
    int acc, op, map;     // accumulator dtype, op and map codes (K_ALL2: the two-input map)
    int vec;              // elements per load of the first launch
    int lanes;            // tile kernels: lanes across a tile row
    int64_t grid;
    int block;
    AllArgs all;          // K_ALL, K_ALL_STRIDED, K_ALL2
    DimsArgs dims;        // other kernels
    void *stream;         // hipStream_t
    void *ev_begin;       // optional hipEvent_t pair around the first launch
    void *ev_end;
};

int launch_in_f32(const Launch &L);
int launch_in_bf16(const Launch &L);
int launch_in_f16(const Launch &L);
int launch_in_f64(const Launch &L);
int launch_in_i32(const Launch &L);
int launch_in_i64(const Launch &L);

}  // namespace rk
