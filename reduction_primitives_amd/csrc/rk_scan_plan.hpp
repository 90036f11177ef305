// rk_scan_plan.hpp -- host-side planning of scans and what the C ABI hands
// to the scan translation units (plain structs, no HIP types).
//
// Scans along one dim (AcceleratedKernels.jl PR #202, opening paragraph):
// every line -- all indices fixed but the scan dim's -- is scanned on its own.
// Kept apart from the reductions' plan and launch headers so that the two
// families change independently.
#pragma once

#include <cstddef>
#include <cstdint>

#include "rk_plan.hpp"

namespace rk {

// Scan kernels (rk_scan.hpp).
enum ScanKernel { SK_NONE = 0, SK_TILE = 1, SK_ROWWAVE = 2, SK_LINES = 3, SK_COLUMNS = 4, SK_TRANSPOSE = 5,
                  SK_TAKE_TIMEOUTS = 100 };   // read and clear the count of waits that gave up (no scan)

namespace tune {
constexpr int kScanBlock = 256;           // threads per block of the row-wave and lines kernels
constexpr int kScanTileBlock = 1024;      // tile kernel: 16 waves share a tile (fewer, larger tiles
                                          // amortise the look-back; 1e8 f32: 177 us vs 236 us at 256);
                                          // kScanBlock-thread tiles when the large ones number < CUs
constexpr int kScanTileUnroll = 16;       // 16-byte chunks per lane of a large tile (10^8 f32 cumsum: 151.7 us
                                          // against 165.7 at 8 and 157.5 at 24; the look-back costs per tile)
constexpr int kScanMaxChunks = 32;        // chunks a lane holds with vector loads: 64 (bf16 -> f64 at
                                          // 16 chunks) went to scratch memory
constexpr int kScanWaveUnroll = 16;       // chunks in flight per lane, row-wave kernel with vector loads (16
                                          // bytes of input or of output; 8192x8192 f32 dims=1: 93.0 us
                                          // against 104.0 at 8)
constexpr int kScanUnroll = 8;            // 16-byte chunks in flight per lane (256-thread tiles; row-wave
                                          // kernel with element loads)
constexpr int kScanLinesUnroll = 8;       // elements in flight per thread (lines kernel)
constexpr int kScanLinesBlocksPerCu = 8;  // lines kernel grid cap
// Contiguous lines at least this long take a wave each (or tiles); shorter
// ones from 16 elements are packed whole into waves (scan_lines_packed).  f32
// cumsum along dim 1, about 5 million elements: lines of 200 22.2 us packed,
// 28.9 a wave each, 119.3 a thread each; lines of 100 28.9, 50.5 and 77.4.
constexpr int64_t kScanWaveMinLen = 256;
constexpr int64_t kScanTileFewLines = 4;  // fewer lines than CUs * this, each >= kScanTileMinLen: tiles
constexpr int64_t kScanTileMinLen = 4096;
constexpr int kScanSpinLimit = 1 << 24;   // look-back: sleeps per wait before giving up (about a second)
// columns scan (strided scan dim, contiguous lines): a tile is W lines x R
// scan positions; W = lanes * elements per 16-byte load
constexpr int kScanColBlock = 512;        // threads per block (8192x8192 f32 dims=2: 105.4 us against
                                          // 110.6 us at 256 threads and 110.7 us at 1024)
constexpr int kScanColLanes = 32;         // lanes across a tile row with 16-byte loads (512-byte rows)
constexpr int kScanColLanesScalar = 64;   //   ... with element loads
constexpr int kScanColRows = 16;          // consecutive scan positions per thread (8: 125.7 us at 1024 threads)
constexpr int64_t kScanColMinRun = 16;    // runs of lines narrower than this take the lines kernel
constexpr int kScanPackedBlocksPerCu = 8; // lines kernel, packed form: grid cap
constexpr int kScanPackedUnroll = 8;      //   ... and groups of lines a round (half with 4 elements a lane;
                                          // 16: lines of 50 32.3 against 30.1 us, of 100 30.8 against 25.4)
constexpr int kScanTrBlock = 256;         // transposing scan: threads per block
// LDS per tile of the transposing scan when the scan dim is the output's
// contiguous one (mode 2): 32 KB tiles fit four blocks to a CU (92 VGPRs),
// 140-145 us against 155-172 at 64 KB on row-major 8192x8192 f32 along dim 1.
// The other modes keep 64 KB: at 32 KB the scan dim contiguous in the input
// took 174 us against 157 (three blocks to a CU, 135 VGPRs; 198 us at four,
// with the registers held to 128), the permuted view 200 against 167.
constexpr int kScanTrTileKBScanOut = 32;
constexpr int64_t kScanTrMinRun = 16;     // its two contiguous axes span at least this many elements
// With the scan dim contiguous on one side, the transposing tiles need this
// many lines; fewer take the tile kernel, the other side's elements moved one
// by one.
// 8 Mi f32 as L row-major rows along their rows, us transposing / tile: L = 16
// 357 / 103, 32 194 / 122, 64 113 / 118, 128 70 / 116, 256 46 / 60.
constexpr int64_t kScanTrMinLines = 64;
}  // namespace tune

// The lines kernel's packed form: lines contiguous along the scan dim in
// input and output, from a quarter wave long up to the row-wave length (at
// most 4 waves), go whole to waves, each lane holding scan_packed_width(m)
// consecutive elements.  Against a thread per line (f32, about 5 million
// elements, before its lane moves were issued for all groups at once): lines
// of 50 88.8 -> 36.3 us, of 24 47.2 -> 34.1; lines of 10
// stay with a thread each (27.8 against 30.6 packed), whose neighbours share
// its cache lines.  One test for the planner and the launch.
constexpr bool scan_lines_packed(int64_t s_in, int64_t s_out, int64_t m)
{
    return s_in == 1 && s_out == 1 && m >= 16 && m < 256 && m < tune::kScanWaveMinLen;
}
// Elements a lane holds in the packed form: 1 below 64, 2 below 128, else 4.
constexpr int scan_packed_width(int64_t m) { return m < 64 ? 1 : m < 128 ? 2 : 4; }

// Scans (prefix folds) along one dim: every line -- all indices fixed but
// the scan dim's -- is scanned on its own.  Line l starts at input element
// layout_offset(kept_in, l) and output element layout_offset(kept_out, l);
// element k of a line is s_in * k / s_out * k further on.
struct ScanArgs {
    const void *x;
    void *out;
    void *ws;             // tile kernel: [counter | flags[tiles] | aggregates[tiles] | prefixes[tiles]]
    int64_t m;            // elements per line
    int64_t lines;
    int kept_nd;
    int64_t kept_ext[4];
    int64_t kept_in[4];
    int64_t kept_out[4];
    int64_t s_in, s_out;  // scan-dim strides in elements
    int64_t tiles_per_line;   // tile kernel
    int64_t tiles;            // tile and columns kernels
    int64_t col_tiles_per_run;    // columns kernel: tiles across one run of lines (kept dim 0);
                                  // transposing kernel: across kept dims 0 and 1 (its a and b)
    int64_t col_tiles;            //   ... across all runs; tiles = col_tiles * chunks of the scan dim
    int inclusive;
    int out_dtype;
    uint64_t init_bits;   // starting value, accumulator bits
    int slot;             // >= 0: look-back state in the library's slot (reset by the last
                          // block); < 0: in the workspace, cleared by a fill launch first
    uint32_t spin_limit;  // look-back: polls of one window before the wait gives up
    uint32_t force_wait;  // 0; nonzero only to make every look-back wait until it gives up (a test hook)
};

// Transposing scan (k_scan_transpose): the input is contiguous along one
// axis of a line x position tile and the output along another, so a tile
// goes through LDS between its loads and its stores.  Its axes: a, a kept dim
// with input stride 1; b, a kept dim with output stride 1; p, the scan
// positions.  Mode 0: the scan dim is the input's contiguous one (a row-major
// matrix scanned along its rows, say), a tile is 256 b x 64 p; mode 1: a and
// b are different kept dims (a permuted view), 32 a x 32 b x 16 p; mode 2:
// the scan dim is the output's contiguous one, 256 a x 32 p.  Each side then
// moves runs of 32 or more consecutive elements (16 for 8-byte slots in mode
// 2).  A slot is the larger of the input and accumulator elements, 4 or 8
// bytes; 8-byte slots halve the positions.  A tile takes 64 KB of LDS, 32 KB
// in mode 2.
constexpr int scan_tr_ta(int mode) { return mode == 0 ? 1 : mode == 1 ? 32 : 256; }
constexpr int scan_tr_tb(int mode) { return mode == 0 ? 256 : mode == 1 ? 32 : 1; }
constexpr int scan_tr_tp(int mode, int slot_bytes)
{
    return mode == 1 ? 16 * 4 / slot_bytes
           : mode == 0 ? 64 * 4 / slot_bytes
                       : 64 * 4 / slot_bytes * tune::kScanTrTileKBScanOut / 64;
}

// Columns-scan state: a 256-byte header (as the tile scan's), the flags --
// 32-bit words, the flag of tile g at word (g % lines) * 32 + g / lines,
// lines = ceil(tiles / 32), so consecutive tiles sit in different 128-byte
// lines -- then room for `width` 8-byte aggregates per tile and as many
// prefixes.  The kernel packs them at its accumulator's width, a tile's
// values in line order of the threads that store them.
constexpr int kScanFlagCapacity = 8192;  // tiles whose flags fit one library slot
constexpr int64_t scan_flag_lines(int64_t tiles) { return (tiles + 31) / 32; }
constexpr int64_t scan_columns_state_bytes(int64_t tiles, int64_t width)
{
    return 256 + scan_flag_lines(tiles) * 128 + tiles * width * 16;
}

// Tile-scan state: a 256-byte header (line 0: tile counter, timeout word;
// line 1: blocks done) and one 32-byte record per tile {flag, -, aggregate,
// inclusive prefix, -}, four records to a 128-byte line.  Record of tile g:
// number (g % lines) * 4 + g / lines, lines = ceil(tiles / 4), so
// consecutive tiles sit in different lines.
constexpr int kScanHeaderBytes = 256;
constexpr int kScanRecBytes = 32;
constexpr int kScanRecCapacity = 4096;   // tiles whose records fit one library slot
constexpr int64_t scan_rec_lines(int64_t tiles) { return (tiles + 3) / 4; }
constexpr int64_t scan_tile_state_bytes(int64_t tiles)
{
    return kScanHeaderBytes + scan_rec_lines(tiles) * 4 * kScanRecBytes;
}

struct ScanLaunch {
    int kernel;           // rk::ScanKernel
    int acc, op;
    int vec;              // elements per load (1: element loads)
    int tmode;            // transposing kernel: its mode
    int tstr;             // tile kernel: 1 outputs s_out apart, 2 inputs s_in apart
    int64_t grid;
    int block;
    ScanArgs args;
    void *stream;
    void *ev_begin;       // optional hipEvent_t pair around the scan kernel
    void *ev_end;
};

int launch_scan_in_f32(const ScanLaunch &L);
int launch_scan_in_bf16(const ScanLaunch &L);
int launch_scan_in_f16(const ScanLaunch &L);
int launch_scan_in_f64(const ScanLaunch &L);
int launch_scan_in_i32(const ScanLaunch &L);
int launch_scan_in_i64(const ScanLaunch &L);

// Scan along one dim.  Lines are the indices of the other dims (extent-1
// dims dropped, neighbours merged when both their input and output strides
// chain), numbered column-major; the output is the view's shape stored
// contiguously in column-major order.
struct ScanPlan {
    int kernel = SK_NONE;
    int64_t m = 0;          // elements per line
    int64_t lines = 0;
    Layout kept_in;         // line -> input offset
    int64_t kept_out[kMaxDims] = {0, 0, 0, 0};   // line -> output offset (extents of kept_in)
    int64_t s_in = 0, s_out = 0;
    int vec = 1;
    int64_t tile_elems = 0; // elements per tile (tile and columns kernels)
    int64_t tiles_per_line = 0;
    int64_t tiles = 0;
    int64_t col_tiles_per_run = 0;   // columns and transposing kernels
    int64_t col_tiles = 0;
    int tmode = 0;                   // transposing kernel: its mode
    int tstr = 0;                    // tile kernel: 1 outputs s_out apart, 2 inputs s_in apart
    int64_t chunks = 0;
    int64_t grid = 0;
    int block = tune::kScanBlock;
    size_t ws_bytes = 0;
};

// Elements of one scan tile for an input dtype, tile-kernel block size and
// lane load width vl (elements).
// Chunks per lane of the tile and row-wave kernels: U chunks of the input's
// 16-byte vector, counted in loads of vl elements, at most kScanMaxChunks
// with vector loads.  Shared by the kernels and the plan's tile size.
constexpr int scan_lane_chunks(int unroll, int vec, int vl)
{
    return vl > 1 && unroll * (vec / vl) > tune::kScanMaxChunks ? tune::kScanMaxChunks : unroll * (vec / vl);
}
int64_t scan_tile_elems(int in_dtype, int block, int vl);

// Scan plan: `dim` is 0-based; addresses only matter through alignment.
int plan_scan(int in_dtype, int acc_dtype, int out_dtype, uintptr_t in_addr, uintptr_t out_addr, int ndim,
              const int64_t *shape, const int64_t *strides, int dim, int num_cus, ScanPlan *p);

}  // namespace rk
