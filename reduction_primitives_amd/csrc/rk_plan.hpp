// rk_plan.hpp -- host-side planning of whole-array and dims reductions.
//
// Pure C++ (no HIP): it turns a call's dtypes, shape, strides and alignment
// into a launch plan -- which kernel, grid, split and workspace -- so the
// same decisions can be unit-tested on a machine without a GPU.  All tuning
// values live in the one table below; the dims kernel choice is made in one
// place, select_strided_kernel() (AcceleratedKernels.jl PR #176, section
// "This PR" item 1).
#pragma once

#include <cstddef>
#include <cstdint>

#include "rk_launch.hpp"

namespace rk {

enum Dtype { F32 = 0, BF16 = 1, F16 = 2, F64 = 3, I32 = 4, I64 = 5 };
enum Mode { OVERWRITE = 0, FOLD = 1, HOST = 2 };
enum Kernel {
    K_NONE = 0, K_ALL = 1, K_ALL_STRIDED = 2, K_THREAD = 3, K_TILED = 4,
    K_COLUMNS = 5, K_ROW = 6, K_GENERIC = 7, K_ALL2 = 8,
    K_SET_TAG = 100,              // test hook: set a slot's whole-array tag (no reduction)
    K_TAKE_TIMEOUTS = 101         // read and clear a slot's count of waits that gave up (no reduction)
};

int dtype_size(int d);            // bytes per element, 0 for an unknown code
bool dtype_is_fp(int d);
bool dtype_known(int d);
// input/accumulator/output combination of the public dtype table
bool dtype_combo_ok(int in, int acc, int out);

// ---------------------------------------------------------------- tuning
// gfx950 values, set from measurements on MI355X (256 CUs, 8 XCDs, 128-byte
// L2 lines).  The pages' own numbers -- 256 target blocks, 64 bytes of
// accumulator per thread, 8-output tiled blocks, 32-output column tiles, a
// 64 KiB row threshold -- were tuned for other GPUs and are not used as is:
//  * an 8-output tile reads 32-byte row pieces and wastes most of each
//    128-byte line (1.5-2.7x slower than the best shape on every shape
//    measured), so the one-pass tiled kernel takes 32 outputs per block;
//  * a split tile streams best with 512-byte rows and about one block per
//    CU, so the columns kernel takes 512 bytes of outputs (256 or 128 bytes
//    when a run of outputs is shorter);
//  * one thread per output keeps only a few bytes in flight per thread, so it
//    needs a row of outputs of 4 MiB before it can keep HBM busy.
namespace tune {
// whole-array first pass
constexpr int kAllBlock = 256;            // threads per block
constexpr int kAllUnroll = 8;             // 16-byte loads in flight per thread
constexpr int kAllBlocksPerCu = 4;        // grid cap = CUs * this
constexpr int kAllSingleLaunchTiles = 2;  // <= this many tiles: one launch
constexpr int kPass2Block = 256;          // threads of the one-block second pass
// dims
constexpr int kDimsBlock = 256;           // row and generic kernels
constexpr int kDimsUnroll = 8;            // loads in flight per thread (tile kernels)
// Loads in flight per lane (row kernel).  8 takes the f32 kernel to 58 VGPRs,
// so all 8 waves per SIMD are resident (16: 91, five); against 16 it measured
// 0.6-0.9 us faster on 3136x256x84 dims=(1,3), 0.2-0.3 on 3072x2048 and 0.2
// on 8192^2 dims=1.  2-byte inputs into 8-byte accumulators keep 16: with 8
// the compiler takes their sums to 135-145 VGPRs, past the 128 of 4 waves.
constexpr int kRowUnroll = 8;
constexpr int kRowUnrollHalfToWide = 16;
constexpr int kThreadBlock = 256;         // thread-per-output kernel
constexpr int kTiledBlock = 1024;         // one-pass tiled kernel: 16 waves share a tile
constexpr int kColumnsBlock = 256;        // split columns kernel
constexpr int64_t kThreadRowBytes = 4 * 1024 * 1024;  // rule 1: row of outputs this wide -> thread kernel
constexpr int64_t kMinReduceLen = 32;                 // rule 1: shorter reductions -> thread kernel
constexpr int kTiledOutputs = 32;                     // tiled kernel: outputs per block
constexpr int kColumnsRowBytes = 512;                 // columns kernel: bytes of outputs per block (max)
constexpr int kColumnsMinRowBytes = 128;              //   ... and the narrowest it goes for short runs
constexpr int kColumnsScalarLanes = 64;               // columns tile without 16-byte loads: 64 outputs
constexpr int kFillTilesPerCu = 1;        // rule 2: tiled while its tiles number fewer than CUs * this
constexpr int kColumnsBlocksPerCu = 1;    // columns split target: CUs * this blocks
constexpr int64_t kColumnsMinRows = 128;  // rows per split chunk, at least
constexpr int kTiledBlocksPerCu = 0;      // tiled split target (0: the tiled kernel is not split)
constexpr int64_t kTiledMinRows = 256;    //   ... rows per split chunk, at least
constexpr int kRowWavesPerCu = 8;         // row kernel split target (3136x256x84 f32 dims=(1,3): 42.4 us;
                                          // 16, 32, 64 per CU: 46.5, 49.7, 48.0)
constexpr int64_t kRowMinChunk = 2048;    // elements per row chunk, at least
constexpr int64_t kRowSegMinBytes = 4096; // row kernel over several reduced dims: contiguous rows this long
constexpr int kGenericBlocksPerCu = 8;   // generic kernel: grid cap, and split target
constexpr int kGenericUnroll = 8;        // generic kernel: element loads in flight per thread
constexpr int64_t kGenericMinChunk = 4096;   // generic kernel: reduced elements per split unit, at least
constexpr int kDefaultCus = 256;          // MI355X
}  // namespace tune

constexpr int kMaxDims = 4;

struct Layout {                   // column-major dims, innermost first
    int nd = 0;
    int64_t ext[kMaxDims] = {0, 0, 0, 0};
    int64_t str[kMaxDims] = {0, 0, 0, 0};
};

struct AllPlan {
    int64_t n = 0;
    int vec = 1;            // elements per 16-byte load
    int64_t head = 0;       // scalar elements before the first 16-byte boundary
    int64_t nvec = 0;       // 16-byte vectors of the aligned body
    int64_t tail = 0;       // scalar elements after the body
    int64_t tiles = 0;      // tiles of block * unroll vectors
    int grid = 1;           // first-pass blocks
    int block = tune::kAllBlock;
    int launches = 1;       // with a second pass; 1 when the last block finishes
    size_t ws_bytes = 0;
};

struct DimsPlan {
    int kernel = K_NONE;
    int launches = 0;
    int64_t n_out = 0;      // outputs
    int64_t m = 0;          // elements folded into each output
    Layout kept;            // normalised kept dims (output order; storage order under out_map)
    // Tile kernels over kept dims that run contiguously only in storage
    // order: `kept` is then in that order, and output k of that numbering is
    // stored at sum_i digit_i(k) * out_map.str[i], k's digits taken over
    // out_map.ext (the kept dims in storage order, unmerged).  nd 0: no map.
    Layout out_map;
    Layout red;             // normalised reduced dims
    AllPlan all;            // K_ALL / K_ALL_STRIDED
    // tile kernels (THREAD / TILED / COLUMNS): outputs come in runs of
    // run_len contiguous elements (kept.ext[0], stride 1); the other kept
    // dims (`outer`) place the runs.
    int64_t run_len = 0;
    int64_t runs = 0;
    int64_t s_red = 0;      // stride of the row dim: the reduced dim of largest extent
    int64_t row_len = 0;    // its extent
    Layout seg;             // the other reduced dims; one segment per index
    int64_t segs = 1;
    int64_t segs_per_split = 1;   // see DimsArgs
    int64_t splits_per_seg = 1;
    Layout outer;
    int vec = 1;            // elements per load
    int lanes = 1;          // lanes across one row of a tile
    int tile_outputs = 1;
    int64_t tiles_per_run = 0;
    int64_t tiles = 0;
    int split = 1;          // blocks (tile kernels) or waves (row) per output
    int64_t rows_per_split = 0;
    int64_t grid = 0;
    int block = tune::kDimsBlock;
    size_t ws_bytes = 0;
    // split reductions can finish in the last block to arrive when their
    // arrival counters fit one slot (see rk_launch.hpp)
    bool fused_ok = false;
};

// Status codes as in the public header.
enum { ST_OK = 0, ST_INVALID = 1, ST_UNSUPPORTED = 2, ST_HIP = 3 };

// Whole-array plan: n elements at address `addr`.
int plan_all(int in_dtype, int acc_dtype, uintptr_t addr, int64_t n, int num_cus, AllPlan *p);

// Whole-array plan of a two-input source: n elements at addr_a and at
// addr_b.  The grid and workspace are those of plan_all() for the first
// input.  When the two inputs sit at the same offset from a 16-byte
// boundary both use 16-byte loads with the same head; otherwise the plan
// takes element loads (vec = 1, no head or tail).
int plan_all2(int in_dtype, int acc_dtype, uintptr_t addr_a, uintptr_t addr_b, int64_t n, int num_cus,
              AllPlan *p);

// Dims plan: validates the layout (1..4 dims, non-negative extents and
// strides, mask within ndim) and normalises it before choosing a kernel.
int plan_dims(int in_dtype, int acc_dtype, uintptr_t addr, int ndim, const int64_t *shape,
              const int64_t *strides, uint32_t mask, int num_cus, DimsPlan *p);

// The selector for a strided reduced dim with contiguous runs of outputs.
int select_strided_kernel(int64_t run_len, int64_t n_out, int64_t m, int in_size, int num_cus);

size_t round_up_256(size_t b);

// Whether a view's counts and offsets stay below 2^62: extents and strides,
// outputs (the kept dims' product, at up to 8 bytes each), elements and
// bytes (at isz bytes each) from the first element to the last.  Bit d of
// mask marks dim d as reduced (0 for a scan: every element is an output).
bool view_fits(int ndim, const int64_t *shape, const int64_t *strides, uint32_t mask, int isz);

}  // namespace rk
