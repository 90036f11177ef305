// rk_plan.cpp -- host-side planning (no HIP; unit-tested on the CPU).
#include "rk_plan.hpp"
#include "rk_scan_plan.hpp"

#include <algorithm>
#include <cstdint>

namespace rk {

int dtype_size(int d)
{
    switch (d) {
    case F32: case I32: return 4;
    case BF16: case F16: return 2;
    case F64: case I64: return 8;
    }
    return 0;
}

bool dtype_known(int d) { return dtype_size(d) != 0; }
bool dtype_is_fp(int d) { return d == F32 || d == BF16 || d == F16 || d == F64; }

bool dtype_combo_ok(int in, int acc, int out)
{
    if (!dtype_known(in) || !dtype_known(acc) || !dtype_known(out))
        return false;
    if (dtype_is_fp(in) != dtype_is_fp(acc) || dtype_is_fp(acc) != dtype_is_fp(out))
        return false;
    if (acc == BF16 || acc == F16)          // accumulators are f32, f64, i32 or i64
        return false;
    return dtype_size(acc) >= dtype_size(in);
}

size_t round_up_256(size_t b) { return (b + 255) & ~size_t(255); }

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool view_fits(int ndim, const int64_t *shape, const int64_t *strides, uint32_t mask, int isz)
{
    // Every element count, offset and byte count the planner and the kernels
    // form from a view stays below 2^62: extents and strides are each below
    // it, and so are the outputs (at 8 bytes each), the elements, and the
    // bytes from the first element to the last, all computed with overflow
    // checks (128-bit products).
    constexpr __int128 kLimit = __int128(1) << 62;
    __int128 n_out = 1, m = 1, span = 0;
    for (int i = 0; i < ndim; ++i) {
        if (shape[i] < 0 || strides[i] < 0 || shape[i] >= kLimit || strides[i] >= kLimit)
            return false;
        if ((mask >> i) & 1)
            m *= shape[i];
        else
            n_out *= shape[i];
        if (n_out >= kLimit / 8 || m >= kLimit)      // both stay below 2^62: their product fits 128 bits
            return false;
        if (shape[i] > 0)
            span += __int128(shape[i] - 1) * strides[i];
        if (span >= kLimit)
            return false;
    }
    if (n_out * m == 0)
        return true;                                 // nothing is read
    return n_out * m * isz < kLimit && (span + 1) * isz < kLimit;
}

int plan_all(int in_dtype, int acc_dtype, uintptr_t addr, int64_t n, int num_cus, AllPlan *p)
{
    if (!p || n < 0 || !dtype_known(in_dtype) || !dtype_known(acc_dtype))
        return ST_INVALID;
    if (num_cus <= 0)
        num_cus = tune::kDefaultCus;
    const int isz = dtype_size(in_dtype);
    if (n >= (int64_t(1) << 62) / isz)
        return ST_INVALID;                  // bytes of the input beyond 2^62
    AllPlan a;
    a.n = n;
    a.vec = 16 / isz;
    // Peel scalars up to the first 16-byte boundary so the body can use
    // dwordx4 loads (offset views need not be aligned).
    const uintptr_t mis = addr & 15;
    a.head = mis ? std::min<int64_t>(n, int64_t((16 - mis) / isz)) : 0;
    const int64_t body = n - a.head;
    a.nvec = body / a.vec;
    a.tail = body - a.nvec * a.vec;
    const int64_t tile_vecs = int64_t(tune::kAllBlock) * tune::kAllUnroll;
    a.tiles = ceil_div(a.nvec, tile_vecs);
    a.block = tune::kAllBlock;
    if (a.tiles <= tune::kAllSingleLaunchTiles) {
        a.grid = 1;                         // fits one block: one launch
    } else {
        a.grid = int(std::min<int64_t>(a.tiles, int64_t(num_cus) * tune::kAllBlocksPerCu));
    }
    a.launches = a.grid == 1 ? 1 : 2;
    // pass-1 partials, one slot for the bare final partial, and the host-mode
    // sequence word after it
    a.ws_bytes = round_up_256(size_t(host_seq_offset(a.grid, dtype_size(acc_dtype))) + 4);
    *p = a;
    return ST_OK;
}

int plan_all2(int in_dtype, int acc_dtype, uintptr_t addr_a, uintptr_t addr_b, int64_t n, int num_cus,
              AllPlan *p)
{
    AllPlan a;
    const int rc = plan_all(in_dtype, acc_dtype, addr_a, n, num_cus, &a);
    if (rc)
        return rc;
    if (a.vec > 1 && ((addr_a ^ addr_b) & 15) != 0) {
        // different offsets from a 16-byte boundary: x in vectors from its
        // head on; y read as aligned 16-byte chunks, vector i needing chunks
        // i and i + 1, so the body ends one chunk before y's last whole one
        const int64_t es = dtype_size(in_dtype);
        const int64_t yphase = int64_t((addr_b + uintptr_t(a.head * es)) & 15);
        // y's first chunk must not start before y: one more vector of head
        // scalars when x's head is shorter than y's phase
        if (a.head * es < yphase)
            a.head = std::min<int64_t>(n, a.head + a.vec);
        const int64_t rest = (n - a.head) * es;
        const int64_t nv = std::min<int64_t>(rest / 16, (yphase + rest) / 16 - 1);
        if (nv >= 1) {
            a.nvec = nv;
            a.tail = n - a.head - nv * a.vec;
        } else {
            a.vec = 1;
            a.head = 0;
            a.nvec = n;
            a.tail = 0;
        }
    }
    *p = a;
    return ST_OK;
}

int select_strided_kernel(int64_t run_len, int64_t n_out, int64_t m, int in_size, int num_cus)
{
    // Rule 1: one thread per output when a row of outputs is already wide
    // enough to keep the device busy, or when the reduction is too short to
    // be worth sharing among threads.
    if (run_len * in_size >= tune::kThreadRowBytes || m < tune::kMinReduceLen)
        return K_THREAD;
    // Rule 2: the narrow one-pass tile when there are at least as many
    // outputs as elements per output and its tiles would not fill the GPU
    // (so wide tiles would need a split and a second launch).
    const int64_t narrow_tiles = ceil_div(n_out, tune::kTiledOutputs);
    if (n_out >= m && narrow_tiles < int64_t(num_cus) * tune::kFillTilesPerCu)
        return K_TILED;
    // Rule 3: wide tiles, split along the reduced dim when they are too few.
    return K_COLUMNS;
}

// Drop extent-1 dims and merge neighbouring dims of the same class (both
// kept or both reduced) whose strides chain, keeping column-major order.
static void push_dim(Layout &l, int64_t e, int64_t s)
{
    if (l.nd > 0) {
        const int i = l.nd - 1;
        if (__int128(s) == __int128(l.str[i]) * l.ext[i]) {   // exact, for any strides view_fits accepts
            l.ext[i] *= e;
            return;
        }
    }
    l.ext[l.nd] = e;
    l.str[l.nd] = s;
    ++l.nd;
}

// Kept dims (output order, merged) that are contiguous in storage only in
// another order: the order of increasing stride (broadcast dims last).  When
// the first of them then has stride 1, `sorted` gets them in that order
// (merged where chained) and `map` the unmerged dims in that order with each
// one's stride in the output (the product of the extents before it in output
// order); returns false otherwise and leaves both untouched.
static bool storage_order_runs(const Layout &kept, Layout *sorted, Layout *map)
{
    int idx[kMaxDims];
    for (int i = 0; i < kept.nd; ++i)
        idx[i] = i;
    auto key = [&](int i) { return kept.str[i] == 0 ? INT64_MAX : kept.str[i]; };
    std::stable_sort(idx, idx + kept.nd, [&](int x, int y) { return key(x) < key(y); });
    if (kept.nd < 2 || kept.str[idx[0]] != 1)
        return false;
    int64_t ostr[kMaxDims];
    int64_t acc = 1;
    for (int i = 0; i < kept.nd; ++i) {
        ostr[i] = acc;
        acc *= kept.ext[i];
    }
    Layout s, mp;
    for (int k = 0; k < kept.nd; ++k) {
        push_dim(s, kept.ext[idx[k]], kept.str[idx[k]]);
        mp.ext[mp.nd] = kept.ext[idx[k]];
        mp.str[mp.nd] = ostr[idx[k]];
        ++mp.nd;
    }
    *sorted = s;
    *map = mp;
    return true;
}

int plan_dims(int in_dtype, int acc_dtype, uintptr_t addr, int ndim, const int64_t *shape,
              const int64_t *strides, uint32_t mask, int num_cus, DimsPlan *p)
{
    if (!p || !shape || !strides || ndim < 1 || ndim > kMaxDims)
        return ST_INVALID;
    if (!dtype_known(in_dtype) || !dtype_known(acc_dtype))
        return ST_INVALID;
    if (mask >> ndim)
        return ST_INVALID;
    if (num_cus <= 0)
        num_cus = tune::kDefaultCus;
    const int isz = dtype_size(in_dtype);
    const int asz = dtype_size(acc_dtype);
    if (!view_fits(ndim, shape, strides, mask, isz))
        return ST_INVALID;

    DimsPlan d;
    int64_t n_out = 1, m = 1;
    for (int i = 0; i < ndim; ++i) {
        if (shape[i] < 0 || strides[i] < 0)
            return ST_INVALID;
        if ((mask >> i) & 1)
            m *= shape[i];
        else
            n_out *= shape[i];
    }
    d.n_out = n_out;
    d.m = m;
    if (n_out == 0) {                   // nothing to store
        d.kernel = K_NONE;
        *p = d;
        return ST_OK;
    }
    if (m == 0) {
        // Every output is its starting value: a zero-length generic fold.
        for (int i = 0; i < ndim; ++i)
            if (!((mask >> i) & 1) && shape[i] != 1)
                push_dim(d.kept, shape[i], strides[i]);
        d.red = Layout();
        d.kernel = K_GENERIC;
    } else {
        for (int i = 0; i < ndim; ++i) {
            if (shape[i] == 1)
                continue;
            if ((mask >> i) & 1)
                push_dim(d.red, shape[i], strides[i]);
            else
                push_dim(d.kept, shape[i], strides[i]);
        }
        if (d.kept.nd == 0) {
            // A single output.  A contiguous source takes the whole-array
            // path (PR #139, "What changes", last paragraph).
            if (d.red.nd == 0 || (d.red.nd == 1 && d.red.str[0] == 1))
                d.kernel = K_ALL;
            else
                d.kernel = K_ALL_STRIDED;
        } else if (d.red.nd == 0) {
            d.kernel = K_GENERIC;           // nothing to reduce: f applied per element
        } else if (d.red.str[0] == 1 && (d.red.nd == 1 || d.red.ext[0] * isz >= tune::kRowSegMinBytes)) {
            // a contiguous reduced dim: rows, and with several reduced dims
            // the others index segments of such rows
            d.kernel = K_ROW;
        } else if (d.kept.str[0] == 1) {
            // contiguous runs of outputs over any reduced dims (PR #176's
            // selector; several reduced dims become segments of rows)
            d.kernel = select_strided_kernel(d.kept.ext[0], n_out, m, isz, num_cus);
        } else if (storage_order_runs(d.kept, &d.kept, &d.out_map)) {
            // the kept dims run contiguously in storage order (a permuted
            // view): the same tile kernels, numbering outputs in that order
            d.kernel = select_strided_kernel(d.kept.ext[0], n_out, m, isz, num_cus);
        } else {
            d.kernel = K_GENERIC;
        }
    }

    switch (d.kernel) {
    case K_ALL: {
        int rc = plan_all(in_dtype, acc_dtype, addr, m, num_cus, &d.all);
        if (rc)
            return rc;
        d.launches = d.all.launches;
        d.grid = d.all.grid;
        d.block = d.all.block;
        d.vec = d.all.vec;
        d.ws_bytes = d.all.ws_bytes;
        d.fused_ok = d.all.grid > 1;
        break;
    }
    case K_ALL_STRIDED: {
        AllPlan a;
        a.n = m;
        a.vec = 1;
        a.nvec = m;                         // scalar "vectors", addressed through `red`
        const int64_t tile = int64_t(tune::kAllBlock) * tune::kAllUnroll;
        a.tiles = ceil_div(m, tile);
        a.grid = a.tiles <= tune::kAllSingleLaunchTiles
                     ? 1
                     : int(std::min<int64_t>(a.tiles, int64_t(num_cus) * tune::kAllBlocksPerCu));
        a.launches = a.grid == 1 ? 1 : 2;
        a.ws_bytes = round_up_256(size_t(host_seq_offset(a.grid, asz)) + 4);
        d.all = a;
        d.launches = a.launches;
        d.grid = a.grid;
        d.block = a.block;
        d.ws_bytes = a.ws_bytes;
        d.fused_ok = a.grid > 1;
        break;
    }
    case K_THREAD: case K_TILED: case K_COLUMNS: {
        d.run_len = d.kept.ext[0];
        d.runs = n_out / d.run_len;
        // rows run along the reduced dim of largest extent; the others
        // index segments of such rows
        int r = 0;
        for (int i = 1; i < d.red.nd; ++i)
            if (d.red.ext[i] > d.red.ext[r])
                r = i;
        d.s_red = d.red.str[r];
        d.row_len = d.red.ext[r];
        d.seg = Layout();
        for (int i = 0; i < d.red.nd; ++i) {
            if (i == r)
                continue;
            d.seg.ext[d.seg.nd] = d.red.ext[i];
            d.seg.str[d.seg.nd] = d.red.str[i];
            ++d.seg.nd;
        }
        d.segs = m / d.row_len;
        d.outer = Layout();
        for (int i = 1; i < d.kept.nd; ++i) {
            d.outer.ext[d.outer.nd] = d.kept.ext[i];
            d.outer.str[d.outer.nd] = d.kept.str[i];
            ++d.outer.nd;
        }
        // 16-byte loads when every row of every run starts 16-byte aligned
        const int v = 16 / isz;
        bool vec_ok = (addr % 16) == 0 && d.run_len % v == 0 && (d.s_red * isz) % 16 == 0;
        for (int i = 0; i < d.outer.nd; ++i)
            vec_ok = vec_ok && (d.outer.str[i] * isz) % 16 == 0;
        for (int i = 0; i < d.seg.nd; ++i)
            vec_ok = vec_ok && (d.seg.str[i] * isz) % 16 == 0;
        d.vec = vec_ok ? v : 1;
        if (d.kernel == K_THREAD) {
            d.block = tune::kThreadBlock;
            d.lanes = d.block;
        } else if (d.kernel == K_TILED) {
            d.block = tune::kTiledBlock;
            d.lanes = tune::kTiledOutputs / d.vec;
        } else {
            d.block = tune::kColumnsBlock;
            if (d.vec > 1) {
                // widest row of 128, 256 or 512 bytes the runs can fill
                int bytes = tune::kColumnsRowBytes;
                while (bytes > tune::kColumnsMinRowBytes && d.run_len * isz <= bytes / 2)
                    bytes /= 2;
                d.lanes = bytes / 16;
            } else {
                d.lanes = tune::kColumnsScalarLanes;
            }
        }
        d.tile_outputs = d.lanes * d.vec;
        d.tiles_per_run = ceil_div(d.run_len, d.tile_outputs);
        d.tiles = d.runs * d.tiles_per_run;
        // split units: whole segments each, or pieces of rows_per_split
        // rows of one segment
        d.split = 1;
        d.rows_per_split = d.row_len;
        d.segs_per_split = d.segs;
        d.splits_per_seg = 1;
        const bool split_tiles = d.kernel == K_COLUMNS || (d.kernel == K_TILED && tune::kTiledBlocksPerCu > 0);
        if (split_tiles) {
            const bool cols = d.kernel == K_COLUMNS;
            const int64_t target = int64_t(num_cus) * (cols ? tune::kColumnsBlocksPerCu : tune::kTiledBlocksPerCu);
            const int64_t min_rows = cols ? tune::kColumnsMinRows : tune::kTiledMinRows;
            int64_t s = std::max<int64_t>(1, ceil_div(target, d.tiles));
            s = std::min<int64_t>(s, std::max<int64_t>(1, m / min_rows));
            if (s <= d.segs) {
                d.segs_per_split = ceil_div(d.segs, s);
                d.split = int(ceil_div(d.segs, d.segs_per_split));
            } else {
                int64_t per = std::min<int64_t>(ceil_div(s, d.segs), std::max<int64_t>(1, d.row_len / min_rows));
                d.rows_per_split = ceil_div(d.row_len, per);
                per = ceil_div(d.row_len, d.rows_per_split);
                d.segs_per_split = 1;
                d.splits_per_seg = per;
                d.split = int(d.segs * per);
            }
        }
        d.grid = d.tiles * d.split;
        d.launches = d.split > 1 ? 2 : 1;
        d.ws_bytes = d.split > 1 ? round_up_256(size_t(d.split) * n_out * asz) : 0;
        d.fused_ok = d.split > 1 && d.tiles * arrive_counters(d.split) <= kArriveCapacity;   // per tile
        break;
    }
    case K_ROW: {
        d.vec = 16 / isz;
        d.row_len = d.red.ext[0];
        d.seg = Layout();
        for (int i = 1; i < d.red.nd; ++i) {
            d.seg.ext[d.seg.nd] = d.red.ext[i];
            d.seg.str[d.seg.nd] = d.red.str[i];
            ++d.seg.nd;
        }
        d.segs = m / d.row_len;
        const int64_t waves_target = int64_t(num_cus) * tune::kRowWavesPerCu;
        int64_t s = 1;
        if (n_out < waves_target)
            s = std::min<int64_t>(ceil_div(waves_target, n_out),
                                  std::max<int64_t>(1, m / tune::kRowMinChunk));
        // split units: whole segments each, or pieces of one segment's row
        d.rows_per_split = d.row_len;
        d.segs_per_split = d.segs;
        d.splits_per_seg = 1;
        if (s <= d.segs) {
            d.segs_per_split = ceil_div(d.segs, s);
            d.split = int(ceil_div(d.segs, d.segs_per_split));
        } else {
            int64_t per = std::min<int64_t>(ceil_div(s, d.segs), std::max<int64_t>(1, d.row_len / tune::kRowMinChunk));
            int64_t rows = ceil_div(d.row_len, per);
            rows = ceil_div(rows, d.vec) * d.vec;   // pieces keep the row's 16-byte phase
            d.rows_per_split = rows;
            per = ceil_div(d.row_len, rows);
            d.segs_per_split = 1;
            d.splits_per_seg = per;
            d.split = int(d.segs * per);
        }
        const int waves_per_block = tune::kDimsBlock / 64;
        d.block = tune::kDimsBlock;
        d.grid = ceil_div(n_out * d.split, waves_per_block);
        d.launches = d.split > 1 ? 2 : 1;
        d.ws_bytes = d.split > 1 ? round_up_256(size_t(d.split) * n_out * asz) : 0;
        d.fused_ok = d.split > 1 && n_out * arrive_counters(d.split) <= kArriveCapacity;   // per output
        break;
    }
    case K_GENERIC: {
        // units of (output, chunk of reduced elements): split an output over
        // several blocks when the outputs alone would not fill the GPU
        // 16-byte loads when the innermost reduced dim is contiguous and
        // every reduced row and every output's base stay 16-byte aligned:
        // the kernel then walks the reduced layout in vectors
        d.vec = 1;
        {
            const int v = 16 / isz;
            bool vec_ok = m > 0 && d.red.nd >= 1 && d.red.str[0] == 1 && d.red.ext[0] % v == 0 && addr % 16 == 0;
            for (int i = 1; i < d.red.nd; ++i)
                vec_ok = vec_ok && (d.red.str[i] * isz) % 16 == 0;
            for (int i = 0; i < d.kept.nd; ++i)
                vec_ok = vec_ok && (d.kept.str[i] * isz) % 16 == 0;
            if (vec_ok) {
                d.vec = v;
                d.red.ext[0] /= v;
                d.red.str[0] = v;
            }
        }
        const int64_t units = m / d.vec;            // reduced length in load units
        d.block = tune::kDimsBlock;
        const int64_t target = int64_t(num_cus) * tune::kGenericBlocksPerCu;
        int64_t s = 1;
        if (n_out < target && m > 0)
            s = std::min<int64_t>(ceil_div(target, n_out),
                                  std::max<int64_t>(1, units * d.vec / tune::kGenericMinChunk));
        d.rows_per_split = m > 0 ? ceil_div(units, s) : 0;
        d.split = m > 0 ? int(ceil_div(units, d.rows_per_split)) : 1;
        d.grid = std::min<int64_t>(n_out * d.split, target);
        d.launches = d.split > 1 ? 2 : 1;
        d.ws_bytes = d.split > 1 ? round_up_256(size_t(d.split) * n_out * asz) : 0;
        d.fused_ok = d.split > 1 && n_out * arrive_counters(d.split) <= kArriveCapacity;   // per output
        break;
    }
    default:
        break;
    }
    *p = d;
    return ST_OK;
}

// ------------------------------------------------------------------ scans

int64_t scan_tile_elems(int in_dtype, int block, int vl)
{
    const int isz = dtype_size(in_dtype);
    if (isz == 0 || vl < 1)
        return 0;
    const int unroll = block == tune::kScanTileBlock ? tune::kScanTileUnroll : tune::kScanUnroll;
    return int64_t(block / 64) * scan_lane_chunks(unroll, 16 / isz, vl) * 64 * vl;
}

// The transposing kernel, when the input and the output are contiguous along
// different axes that each span at least kScanTrMinRun elements: the scan
// dim and a kept dim with output stride 1 (mode 0), a kept dim with input
// stride 1 and another with output stride 1 (mode 1), or a kept dim with
// input stride 1 and the scan dim (mode 2).  The kept dims are reordered to
// (a, b, the rest), a missing axis taking extent 1.
static bool plan_scan_transpose(ScanPlan &d, int isz, int asz)
{
    const Layout &k = d.kept_in;
    int ia = -1, ib = -1;
    for (int i = 0; i < k.nd; ++i) {
        if (ia < 0 && k.str[i] == 1)
            ia = i;
        if (ib < 0 && d.kept_out[i] == 1)
            ib = i;
    }
    const int64_t R = tune::kScanTrMinRun;
    int mode = -1;
    if (d.s_in == 1 && d.s_out != 1 && ib >= 0 && d.m >= R && k.ext[ib] >= tune::kScanTrMinLines)
        mode = 0;
    else if (ia >= 0 && ib >= 0 && ia != ib && k.ext[ia] >= R && k.ext[ib] >= R)
        mode = 1;
    else if (ia >= 0 && d.s_out == 1 && d.s_in != 1 && d.m >= R && k.ext[ia] >= tune::kScanTrMinLines)
        mode = 2;
    if (mode < 0)
        return false;
    const int da = mode == 0 ? -1 : ia, db = mode == 2 ? -1 : ib;
    Layout t;
    int64_t to[kMaxDims] = {0, 0, 0, 0};
    auto put = [&](int i) {
        t.ext[t.nd] = i < 0 ? 1 : k.ext[i];
        t.str[t.nd] = i < 0 ? 0 : k.str[i];
        to[t.nd] = i < 0 ? 0 : d.kept_out[i];
        ++t.nd;
    };
    put(da);
    put(db);
    for (int i = 0; i < k.nd; ++i)
        if (i != da && i != db)
            put(i);
    const int slot = std::max(isz, asz) > 4 ? 8 : 4;
    const int64_t ta = scan_tr_ta(mode), tb = scan_tr_tb(mode), tp = scan_tr_tp(mode, slot);
    const int64_t per_run = ceil_div(t.ext[0], ta) * ceil_div(t.ext[1], tb);
    d.kernel = SK_TRANSPOSE;
    d.tmode = mode;
    d.kept_in = t;
    for (int i = 0; i < kMaxDims; ++i)
        d.kept_out[i] = to[i];
    d.block = tune::kScanTrBlock;
    d.vec = 1;
    d.col_tiles_per_run = per_run;
    d.col_tiles = d.lines / (t.ext[0] * t.ext[1]) * per_run;
    d.chunks = ceil_div(d.m, tp);
    d.tiles = d.col_tiles * d.chunks;
    d.tile_elems = ta * tb * tp;
    d.grid = d.tiles;
    if (d.tiles > INT32_MAX)                    // refused by the caller; no state size to form
        return true;
    d.ws_bytes = round_up_256(size_t(scan_columns_state_bytes(d.tiles, ta * tb)));
    return true;
}

int plan_scan(int in_dtype, int acc_dtype, int out_dtype, uintptr_t in_addr, uintptr_t out_addr, int ndim,
              const int64_t *shape, const int64_t *strides, int dim, int num_cus, ScanPlan *p)
{
    if (!p || !shape || !strides || ndim < 1 || ndim > kMaxDims || dim < 0 || dim >= ndim)
        return ST_INVALID;
    if (!dtype_known(in_dtype) || !dtype_known(acc_dtype) || !dtype_known(out_dtype))
        return ST_INVALID;
    if (num_cus <= 0)
        num_cus = tune::kDefaultCus;
    const int isz = dtype_size(in_dtype), osz = dtype_size(out_dtype);
    if (!view_fits(ndim, shape, strides, 0u, isz))
        return ST_INVALID;
    ScanPlan d;
    int64_t total = 1, ostr[kMaxDims];
    for (int i = 0; i < ndim; ++i) {
        if (shape[i] < 0 || strides[i] < 0)
            return ST_INVALID;
        ostr[i] = total;                        // the output is contiguous, column-major
        total *= shape[i];
    }
    d.m = shape[dim];
    d.s_in = strides[dim];
    d.s_out = ostr[dim];
    if (total == 0) {
        *p = d;
        return ST_OK;
    }
    d.lines = total / d.m;
    // kept dims: drop extent 1, merge neighbours whose input and output strides both chain
    Layout &k = d.kept_in;
    for (int i = 0; i < ndim; ++i) {
        if (i == dim || shape[i] == 1)
            continue;
        if (k.nd > 0) {
            const int j = k.nd - 1;
            if (__int128(strides[i]) == __int128(k.str[j]) * k.ext[j] && ostr[i] == d.kept_out[j] * k.ext[j]) {
                k.ext[j] *= shape[i];
                continue;
            }
        }
        k.ext[k.nd] = shape[i];
        k.str[k.nd] = strides[i];
        d.kept_out[k.nd] = ostr[i];
        ++k.nd;
    }
    const int v = 16 / isz;
    const int asz = dtype_size(acc_dtype);
    if (d.s_in == 1 && d.s_out == 1 && d.m >= tune::kScanWaveMinLen) {
        // lines contiguous along the scan dim in both input and output.  A
        // lane loads vl elements: the input's 16 bytes, or, when the outputs
        // are as wide as the accumulator and wider than the inputs, as many as
        // make 16 bytes of output, so each store stays one contiguous piece.
        const int vl = (osz > isz && osz == asz) ? 16 / osz : v;
        const int lb = vl * isz;                // bytes of one lane's load
        const int ob = std::min(16, vl * osz);  // bytes of one lane's outputs, up to 16
        bool vec_ok = in_addr % lb == 0 && d.m % vl == 0 && out_addr % ob == 0;
        for (int i = 0; i < k.nd; ++i)
            vec_ok = vec_ok && (k.str[i] * isz) % lb == 0 && (d.kept_out[i] * osz) % ob == 0;
        d.vec = vec_ok ? vl : 1;
        d.tile_elems = scan_tile_elems(in_dtype, tune::kScanTileBlock, d.vec);
        const bool few_lines = d.lines < int64_t(num_cus) * tune::kScanTileFewLines;
        if (d.m >= d.tile_elems || (few_lines && d.m >= tune::kScanTileMinLen)) {
            d.kernel = SK_TILE;
            d.block = tune::kScanTileBlock;
            // fewer large tiles than CUs: a quarter of the size keeps more CUs
            // busy; element loads take the small tiles too (the large ones
            // would need more than the 128 registers a 1024-thread block allows)
            if (d.lines * ceil_div(d.m, d.tile_elems) < num_cus || d.vec == 1) {
                d.block = tune::kScanBlock;
                d.tile_elems = scan_tile_elems(in_dtype, tune::kScanBlock, d.vec);
            }
            d.tiles_per_line = ceil_div(d.m, d.tile_elems);
            d.tiles = d.lines * d.tiles_per_line;
            if (d.tiles > INT32_MAX)            // tiles are numbered by a 32-bit counter
                return ST_INVALID;
            d.grid = d.tiles;
            // header and one record per tile (the state when no library slot takes it)
            d.ws_bytes = round_up_256(size_t(scan_tile_state_bytes(d.tiles)));
        } else {
            d.kernel = SK_ROWWAVE;
            d.block = tune::kScanBlock;
            d.grid = ceil_div(d.lines, tune::kScanBlock / 64);
        }
    } else if (k.nd >= 1 && k.str[0] == 1 && d.kept_out[0] == 1 && k.ext[0] >= tune::kScanColMinRun) {
        // contiguous runs of lines, strided scan dim: tiles of W lines x R
        // positions, look-back along the scan dim.  The workspace covers both
        // tile geometries, so its size does not depend on alignment.
        d.kernel = SK_COLUMNS;
        d.block = tune::kScanColBlock;
        const int ob = std::min(16, v * osz);
        bool vec_ok = in_addr % 16 == 0 && k.ext[0] % v == 0 && (d.s_in * isz) % 16 == 0 &&
                      out_addr % ob == 0 && (d.s_out * osz) % ob == 0;
        for (int i = 1; i < k.nd; ++i)
            vec_ok = vec_ok && (k.str[i] * isz) % 16 == 0 && (d.kept_out[i] * osz) % ob == 0;
        const int64_t runs = d.lines / k.ext[0];
        size_t ws = 0;
        for (int pass = 0; pass < 2; ++pass) {
            const bool vec = pass == 0;
            const int64_t lanes = vec ? tune::kScanColLanes : tune::kScanColLanesScalar;
            const int64_t w = lanes * (vec ? v : 1);
            const int64_t r = (tune::kScanColBlock / lanes) * tune::kScanColRows;
            const int64_t ctpr = ceil_div(k.ext[0], w), ct = runs * ctpr, ch = ceil_div(d.m, r);
            const int64_t tiles = ct * ch;
            if (tiles > INT32_MAX)              // tiles are numbered by a 32-bit counter (both
                return ST_INVALID;              // geometries: the workspace covers either)
            ws = std::max(ws, round_up_256(size_t(scan_columns_state_bytes(tiles, w))));
            if (vec == vec_ok) {
                d.vec = vec ? v : 1;
                d.col_tiles_per_run = ctpr;
                d.col_tiles = ct;
                d.chunks = ch;
                d.tiles = tiles;
                d.tile_elems = w * r;
                d.grid = tiles;
            }
        }
        d.ws_bytes = ws;
    } else if (plan_scan_transpose(d, isz, asz)) {
        if (d.tiles > INT32_MAX)                // tiles are numbered by a 32-bit counter
            return ST_INVALID;
    } else if (d.s_in == 1 && d.m >= tune::kScanWaveMinLen) {
        // lines contiguous in the input only, too few for the transposing
        // tiles (a few rows of a row-major matrix along their rows): the tile
        // kernel along each line, its outputs stored one by one
        d.kernel = SK_TILE;
        d.tstr = 1;
        bool vec_ok = in_addr % 16 == 0 && d.m % v == 0;
        for (int i = 0; i < k.nd; ++i)
            vec_ok = vec_ok && (k.str[i] * isz) % 16 == 0;
        d.vec = vec_ok ? v : 1;
        d.block = tune::kScanTileBlock;
        d.tile_elems = scan_tile_elems(in_dtype, tune::kScanTileBlock, d.vec);
        // large tiles only while a lane's vector of accumulators stays within 32 bytes
        if (d.lines * ceil_div(d.m, d.tile_elems) < num_cus || d.vec == 1 || v * asz > 32) {
            d.block = tune::kScanBlock;
            d.tile_elems = scan_tile_elems(in_dtype, tune::kScanBlock, d.vec);
        }
        d.tiles_per_line = ceil_div(d.m, d.tile_elems);
        d.tiles = d.lines * d.tiles_per_line;
        if (d.tiles > INT32_MAX)
            return ST_INVALID;
        d.grid = d.tiles;
        d.ws_bytes = round_up_256(size_t(scan_tile_state_bytes(d.tiles)));
    } else if (d.s_out == 1 && d.m >= tune::kScanWaveMinLen) {
        // the mirror: lines contiguous in the output only, too few for the
        // transposing tiles (a few columns of a row-major matrix along its
        // columns): the tile kernel, element loads s_in apart
        d.kernel = SK_TILE;
        d.tstr = 2;
        d.vec = 1;
        d.block = tune::kScanBlock;
        d.tile_elems = scan_tile_elems(in_dtype, tune::kScanBlock, 1);
        d.tiles_per_line = ceil_div(d.m, d.tile_elems);
        d.tiles = d.lines * d.tiles_per_line;
        if (d.tiles > INT32_MAX)
            return ST_INVALID;
        d.grid = d.tiles;
        d.ws_bytes = round_up_256(size_t(scan_tile_state_bytes(d.tiles)));
    } else {
        d.kernel = SK_LINES;
        d.block = tune::kScanBlock;
        d.vec = 1;
        if (scan_lines_packed(d.s_in, d.s_out, d.m)) {
            // short contiguous lines packed whole into waves
            const int64_t lanes = ceil_div(d.m, int64_t(scan_packed_width(d.m)));
            const int64_t waves = ceil_div(d.lines, 64 / lanes);
            d.grid = std::min<int64_t>(ceil_div(waves, tune::kScanBlock / 64),
                                       int64_t(num_cus) * tune::kScanPackedBlocksPerCu);
        } else {
            d.grid = std::min<int64_t>(ceil_div(d.lines, tune::kScanBlock),
                                       int64_t(num_cus) * tune::kScanLinesBlocksPerCu);
        }
    }
    *p = d;
    return ST_OK;
}

}  // namespace rk
