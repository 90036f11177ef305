"""GPU parity of the scans (rk_scan, rk_scan_dims) against the CPU oracle.

AcceleratedKernels.jl PR #202 (tile scans): accumulate! over a whole array
and along dims, inclusive and exclusive, with init; its test list scans runs
of each parity and partials of several sizes, whole and along dims.  Here:
lengths around chunk and tile boundaries, aligned and offset views, every
dtype/op combination with 4- and 8-byte partials, each scan kernel, strided
and permuted views, in-place scans, and the 10^8-element and 8192x8192 sizes.

Bar: integers, and max/min of any type, bit-exact.  A floating-point sum
output k of a line comes out of a tree of rounded additions in the
accumulator type, so |gpu - R_k| <= D_k * u * S_k with u = 2^-24 (f32) or
2^-53 (f64), S_k = |s| + sum of |x_j| up to k, and D_k the number of
additions any term passes through on its way to output k, which `_depth`
bounds for each kernel from its association order; a bf16 / f16 output adds
its own rounding (8e-3 / 1e-3 relative, as for the reductions).
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from reduction_primitives_amd import workloads as W
from tests.layouts import innermost, random_view
from tests.parity import code_of, raw_np

pytestmark = pytest.mark.gpu

DEV = "cuda"
OPS = {"sum": O.SUM, "max": O.MAX, "min": O.MIN}


def _rk():
    import reduction_primitives_amd as rk
    rk.load()
    return rk


def _abs_prefix(storage_cpu, shape, strides, dim, in_c, start, inclusive):
    """S_k per output: |s| + sum of |x_j| over the prefix (float64, a scale)."""
    raw = raw_np(storage_cpu)
    w = np.abs(O.widen(in_c, raw))
    idx = np.zeros(tuple(shape), np.int64)
    for d, (e, st) in enumerate(zip(shape, strides)):
        sh = [1] * len(shape)
        sh[d] = e
        idx = idx + (np.arange(e, dtype=np.int64) * st).reshape(sh)
    v = np.moveaxis(w[idx], dim, -1)
    c = np.cumsum(v, axis=-1)
    if not inclusive:
        c = np.concatenate([np.zeros(c.shape[:-1] + (1,)), c[..., :-1]], axis=-1)
    return np.moveaxis(c, -1, dim).reshape(-1, order="F") + abs(float(start))


def _depth(plan, k):
    """Upper bound on the rounded additions a term passes through on its way
    to output k of a line (k counts from 0 along the scan dim), from each
    kernel's association order."""
    name, blk = plan["kernel_name"], plan["block"]
    v, tile = max(plan["vec"], 1), max(plan["tile_outputs"], 1)
    if name == "scan_tile":
        e, nw = tile // blk, blk // 64          # elements per lane of a tile, waves
        # a tile's aggregate: a lane folds its e elements, 6 levels across the
        # wave, then the waves in order; the look-back adds one term per tile
        # before it; inside the tile an output takes the waves before it, the
        # prefix, the chunk totals before it (e / v), the lane offset (its
        # lanes' v elements and 6 levels) and its lane's own elements
        return k // tile + (e + 6 + nw) + (nw + 1 + e // v + (v + 6) + 1 + v)
    if name == "scan_rowwave":
        # one carry per chunk of 64 * v elements, then the lane offset and the
        # lane's own elements
        return k // (64 * v) + (v + 6) + 1 + v + 1
    if name == "scan_columns":
        lanes = 32 if v > 1 else 64
        rows = tile // (lanes * v)              # scan positions per tile
        rg = blk // lanes                       # row groups
        rpg = rows // rg                        # positions per thread
        # aggregate: a thread's positions, then the row groups in order; the
        # look-back chain; in the tile the row groups before it, the prefix and
        # the thread's positions up to k
        return k // rows + (rpg + rg) + (rg + 1 + rpg) + 1
    if name == "scan_transpose":
        # a tile's aggregate folds its positions in order (at most 64); the
        # look-back adds one term per tile before it (at least 8 positions
        # each); in the tile the prefix, then the positions up to k
        return k // 8 + 64 + 1 + 64 + 1
    return k + 1                                # lines: one thread walks the line


def scan_and_check(storage_cpu, shape=None, strides=None, dim=1, op="sum", acc=None, out_dtype=None,
                   init=None, inclusive=True, offset=0, expect_kernel=None, inplace=False, what=""):
    rk = _rk()
    in_c = code_of(storage_cpu.dtype)
    acc_c = rk.default_acc(in_c) if acc is None else code_of(acc)
    out_c = (acc_c if not O.is_fp(in_c) else in_c) if out_dtype is None else code_of(out_dtype)
    if shape is None:
        shape, strides = (storage_cpu.numel() - offset,), (1,)
    total = math.prod(shape)
    last = sum((e - 1) * s for e, s in zip(shape, strides))
    assert total == 0 or offset + last < storage_cpu.numel(), "view out of bounds"
    xd = storage_cpu.to(DEV)
    plan = rk.plan_scan(in_c, shape, strides, dim, acc=acc_c, out_dtype=out_c,
                        ptr=xd.data_ptr() + offset * xd.element_size())
    if expect_kernel is not None:
        assert plan["kernel_name"] == expect_kernel, plan
    out = xd if inplace else None
    res = rk.scan(xd, shape, strides, dim, op=op, acc=acc_c, out_dtype=out_c, init=init, inclusive=inclusive,
                  out=out, offset=offset)
    torch.cuda.synchronize()
    g = raw_np(res)[:total]
    op_c = OPS[op]
    s = init if init is not None else O.identity(op_c, acc_c)
    if not O.is_fp(acc_c):
        s = O.wrap_int(int(s), acc_c)
    R = O.scan_dims(op_c, in_c, acc_c, raw_np(storage_cpu)[offset:], shape, strides, dim - 1, s, inclusive)
    what = what or f"{plan['kernel_name']} {op} incl={inclusive} {shape} dim={dim}"
    if not O.is_fp(out_c):
        want = O.cast(out_c, R)
        bad = np.nonzero(g.astype(np.int64) != want.astype(np.int64))[0]
        assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[0]}: gpu {g[bad[0]]} want {want[bad[0]]}"
        return plan
    gw = O.widen(out_c, g)
    both_nan = np.isnan(gw) & np.isnan(R)
    if op_c != O.SUM:
        want = O.widen(out_c, O.cast(out_c, R))
        bad = np.nonzero(~((gw == want) | both_nan))[0]
        assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[0]}: gpu {gw[bad[0]]!r} want {want[bad[0]]!r}"
        return plan
    S = _abs_prefix(storage_cpu[offset:], shape, strides, dim - 1, in_c, s, inclusive)
    m = shape[dim - 1]
    k = np.moveaxis(np.broadcast_to(np.arange(m).reshape([-1 if d == dim - 1 else 1 for d in range(len(shape))]),
                                    shape), dim - 1, dim - 1).reshape(-1, order="F")
    u = 2.0**-24 if acc_c == O.F32 else 2.0**-53
    tol = _depth(plan, k) * u * S
    if out_c == O.BF16:
        tol = tol + 8e-3 * np.abs(R)
    elif out_c == O.F16:
        tol = tol + 1e-3 * np.abs(R)
    stored = O.widen(out_c, O.cast(out_c, R))
    assert not (np.isinf(stored) & ~np.isinf(R)).any(), f"{what}: expected prefixes overflow the output type"
    ok = (np.abs(gw - R) <= tol) | both_nan
    bad = np.nonzero(~ok)[0]
    assert bad.size == 0, f"{what}: {bad.size} outputs out of tolerance, first at {bad[0]}: gpu {gw[bad[0]]!r} " \
                          f"oracle {R[bad[0]]!r} tol {tol[bad[0]]:.3e}"
    return plan


TILE = 16 * 16 * 64 * 4         # f32 elements per scan tile: 16 waves x 16 chunks x 64 lanes x 4


# ------------------------------------------------------------ whole arrays

@pytest.mark.parametrize("n", [0, 1, 3, 63, 64, 65, 255, 256, 257, 1000, 2047, 2048, 2049, TILE - 1, TILE,
                               TILE + 1, 3 * TILE + 5, 10**6 + 3])
def test_whole_array_lengths(n):
    x = W.uniform(n, -1.0, 1.0, 11000 + n % 997)
    for inclusive in (True, False):
        scan_and_check(x, init=0.5, inclusive=inclusive)
    xi = W.randint(n, -10**6, 10**6, 11100 + n % 991)
    scan_and_check(xi, acc=torch.int64, out_dtype=torch.int64, inclusive=False, init=7)
    scan_and_check(xi, op="max", acc=torch.int32, out_dtype=torch.int32)
    xb = W.normal(n, 11200 + n % 983, torch.bfloat16)
    scan_and_check(xb, out_dtype=torch.float32, op="min")


@pytest.mark.parametrize("offset", [1, 2, 3])
def test_whole_array_offsets(offset):
    """Views that start off a 16-byte boundary take element loads."""
    rk = _rk()
    n = 3 * TILE + 17
    x = W.uniform(n + offset, -1.0, 1.0, 11300 + offset)
    xd = x.to(DEV)
    assert rk.plan_scan(torch.float32, (n,), (1,), 1, ptr=xd[offset:].data_ptr())["vec"] == 1
    scan_and_check(x, offset=offset, init=-1.0)
    scan_and_check(x, offset=offset, op="max", inclusive=False)
    xh = W.normal(n + offset, 11400 + offset, torch.float16)
    scan_and_check(xh, offset=offset, out_dtype=torch.float32)


@pytest.mark.parametrize("combo,n", [
    ((torch.int32, torch.int64, torch.int64), 2 * 10**7 + 2),
    ((torch.float32, torch.float64, torch.float64), 2 * 10**7 + 2),
    ((torch.bfloat16, torch.float32, torch.float32), 4 * 10**7 + 4),
    ((torch.bfloat16, torch.float64, torch.float64), 2 * 10**7 + 2)], ids=["i32-i64", "f32-f64", "bf16-f32", "bf16-f64"])
def test_large_tiles_wide_outputs(combo, n):
    """Outputs wider than the inputs on the 1024-thread tiles: a lane loads as
    many elements as make 16 bytes of output, over 300 tiles with a ragged
    last one (bf16 -> f64 holds its 32-chunk cap: half-size tiles)."""
    rk = _rk()
    tin, tacc, tout = combo
    if tin == torch.int32:
        x = W.randint(n, -10**6, 10**6, 11900)
    elif tin == torch.bfloat16:
        x = W.normal(n, 11901, torch.bfloat16)
    else:
        x = W.uniform(n, -1.0, 1.0, 11902)
    plan = scan_and_check(x, acc=tacc, out_dtype=tout, expect_kernel="scan_tile")
    assert plan["block"] == 1024 and plan["vec"] == 16 // tout.itemsize
    assert plan["split"] > 300 and n % plan["tile_outputs"] != 0
    if tin == torch.int32:
        scan_and_check(x, op="max", acc=tacc, out_dtype=tout, inclusive=False)


COMBOS = [  # (input, accumulator, output)
    (torch.float32, torch.float32, torch.float32),
    (torch.float32, torch.float64, torch.float64),
    (torch.float32, torch.float32, torch.bfloat16),
    (torch.bfloat16, torch.float32, torch.float32),
    (torch.bfloat16, torch.float32, torch.bfloat16),
    (torch.float16, torch.float32, torch.float16),
    (torch.float64, torch.float64, torch.float64),
    (torch.int32, torch.int32, torch.int32),
    (torch.int32, torch.int64, torch.int64),
    (torch.int64, torch.int64, torch.int64),
]


@pytest.mark.parametrize("combo", COMBOS, ids=lambda c: "-".join(str(t).split(".")[1] for t in c))
@pytest.mark.parametrize("op", ["sum", "max", "min"])
def test_dtype_op_matrix(combo, op):
    in_t, acc_t, out_t = combo
    n = 100003
    x = W.normal(n, 11500, in_t) if in_t.is_floating_point else W.randint(n, -2**31, 2**31 - 1, 11501, in_t)
    for inclusive in (True, False):
        scan_and_check(x, op=op, acc=acc_t, out_dtype=out_t, inclusive=inclusive,
                       init=None if op != "sum" else 1)


def test_whole_array_1e8():
    """The 10^8-element float32 scan (the whole-array reduction's size) and
    int32 -> int64, every output compared."""
    xf, perm = W.whole_large(10**8)
    scan_and_check(xf.data, expect_kernel="scan_tile")
    scan_and_check(perm.data, acc=torch.int64, out_dtype=torch.int64, inclusive=False)


# ---------------------------------------------------------------- exactness

def test_exact_results():
    rk = _rk()
    n = 10**6
    ones = torch.ones(n, device=DEV)
    c = rk.scan(ones)
    torch.cuda.synchronize()
    assert np.array_equal(raw_np(c), np.arange(1, n + 1, dtype=np.float32))   # exact below 2^24
    i = torch.arange(1, n + 1, dtype=torch.int32, device=DEV)
    c = rk.scan(i, acc=torch.int64, out_dtype=torch.int64)
    k = np.arange(1, n + 1, dtype=np.int64)
    assert np.array_equal(raw_np(c), k * (k + 1) // 2)
    p = W.randperm(n, 11600)
    c = rk.scan(p.to(DEV), op="max", acc=torch.int32, out_dtype=torch.int32)
    assert np.array_equal(raw_np(c), np.maximum.accumulate(p.numpy()))
    e = rk.scan(i, acc=torch.int64, out_dtype=torch.int64, inclusive=False, init=5)
    assert np.array_equal(raw_np(e), 5 + (k - 1) * k // 2)


def test_in_place():
    rk = _rk()
    for n in (1000, 5 * TILE + 3):
        x = W.small_ints(n, -8, 8, 11700 + n)
        xd = x.to(DEV)
        rk.scan(xd, out=xd)
        torch.cuda.synchronize()
        assert np.array_equal(raw_np(xd), np.cumsum(x.numpy().astype(np.float64)).astype(np.float32))


def test_look_back_never_times_out():
    """The tile kernel's bounded waits never run out in these scans: the
    timeout word of the workspace header stays zero."""
    rk = _rk()
    for n in (TILE + 1, 10**6, 3 * 10**7):
        x = W.uniform(n, -1.0, 1.0, 11750 + n % 7).to(DEV)
        ws = rk.workspace_for(rk.rk_scan_workspace_size(rk.RK_F32, rk.RK_F32, 1, [n], [1], 0), DEV)
        tiles = rk.plan_scan(torch.float32, (n,), (1,), 1)["grid"]
        for _ in range(3):
            rk.scan(x, workspace=ws)
            torch.cuda.synchronize()
            header = ws[:8].cpu().numpy().view(np.uint32)
            assert header[1] == 0
            assert header[0] == tiles               # every tile took one counter value


def test_integer_scans_are_deterministic():
    rk = _rk()
    x = W.randint(3 * 10**6, -10**6, 10**6, 11800).to(DEV)
    outs = [raw_np(rk.scan(x, acc=torch.int64, out_dtype=torch.int64)) for _ in range(5)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


# --------------------------------------------------------------------- dims

DIMS_CASES = [
    # (shape, strides or None, dim, expected kernel, why)
    ((TILE, 64), None, 1, "scan_tile", "one tile per contiguous line"),
    ((8192, 64), None, 1, "scan_tile", "few lines shorter than a tile"),
    ((3 * TILE + 100, 3), None, 1, "scan_tile", "several tiles per line, look-back per line"),
    ((3000, 40), None, 1, "scan_rowwave", "contiguous lines shorter than a tile"),
    ((300, 5000), None, 1, "scan_rowwave", "many short contiguous lines"),
    ((300, 200), None, 2, "scan_columns", "strided scan dim"),
    ((50, 300), None, 1, "scan_lines", "contiguous lines shorter than a wave's chunk: packed into waves"),
    ((10, 3000), None, 1, "scan_lines", "contiguous lines under a quarter wave: a thread each"),
    ((50, 700), (1, 53), 1, "scan_lines", "packed lines with gaps between them"),
    ((16, 30, 7), None, 1, "scan_lines", "packed lines at the offsets of two kept dims, four to a wave"),
    ((63, 301), None, 1, "scan_lines", "packed lines one short of a wave, last group partial"),
    ((100, 300), None, 1, "scan_lines", "contiguous lines of 100: packed, two elements to a lane"),
    ((201, 299), None, 1, "scan_lines", "contiguous lines of 201: packed, four elements to a lane"),
    ((256, 300), None, 1, "scan_rowwave", "contiguous lines of four wave chunks: a wave each"),
    ((64, 100, 8), None, 2, "scan_columns", "middle dim of a 3-d array"),
    ((64, 100, 8), None, 3, "scan_columns", "last dim of a 3-d array"),
    ((10, 100, 8), None, 2, "scan_lines", "runs of lines too narrow for tiles"),
    ((40, 3000, 5), None, 2, "scan_columns", "long strided scan: look-back across chunks"),
    ((130, 2000), (1, 131), 2, "scan_columns", "padded rows: element loads"),
    ((700, 9, 3), None, 1, "scan_rowwave", "lines at the offsets of two kept dims"),
    ((33, 5, 9, 4), None, 4, "scan_columns", "4-d"),
    ((256, 300), (300, 1), 1, "scan_transpose", "transposed view along its strided dim: scan dim contiguous in the output"),
    ((256, 300), (300, 1), 2, "scan_transpose", "transposed view along its contiguous dim: lines contiguous in the output"),
    ((512, 3000), (3000, 1), 2, "scan_transpose", "transposed view, long lines: look-back over windows of 64 tiles"),
    ((1000, 19), (19, 1), 2, "scan_transpose", "transposed view, lines of 19: one ragged chunk"),
    ((19, 1000), (1000, 1), 1, "scan_transpose", "transposed view, 19 lines: one ragged tile of lines"),
    ((64, 3000, 40), (40, 2560, 1), 2, "scan_transpose", "permuted view: input and output contiguous along different kept dims"),
    ((40, 7, 50), (350, 50, 1), 2, "scan_transpose", "permuted view, ragged tiles along both kept dims"),
    ((100, 17, 33), (561, 33, 1), 2, "scan_transpose", "scan dim contiguous in the input, an outer kept dim"),
    ((17, 33, 100), (3300, 100, 1), 1, "scan_transpose", "scan dim contiguous in the output, an outer kept dim"),
    ((10, 300), (300, 1), 2, "scan_tile", "ten row-major rows along their rows: tiles, outputs stored one by one"),
    ((8, 100_000), (100_000, 1), 2, "scan_tile", "few long row-major rows: look-back along each, strided outputs"),
    ((40, 500_000), (500_000, 1), 2, "scan_tile", "40 long row-major rows: large tiles, strided outputs"),
    ((5, 10_001), (10_001, 1), 2, "scan_tile", "few rows of odd length: element loads, strided outputs"),
    ((2, 3, 20_000), (60_000, 20_000, 1), 3, "scan_tile", "row-major 3-d along its last dim: two kept dims, strided outputs"),
    ((8, 200), (200, 1), 2, "scan_lines", "few short row-major rows: a thread each"),
    ((100_000, 8), (8, 1), 1, "scan_tile", "few row-major columns along their columns: element loads s_in apart"),
    ((10_001, 5), (5, 1), 1, "scan_tile", "few columns of odd length, strided inputs"),
    ((20_000, 3, 2), (6, 2, 1), 1, "scan_tile", "row-major 3-d along its first dim: two kept dims, strided inputs"),
]


@pytest.mark.parametrize("case", DIMS_CASES, ids=lambda c: c[4].replace(" ", "_"))
def test_scan_dims(case):
    shape, strides, dim, kern, _ = case
    strides = strides or W.cm_strides(shape)
    n = max(math.prod(shape), sum((e - 1) * st for e, st in zip(shape, strides)) + 1)
    x = W.normal(n, 11900 + n % 97)
    scan_and_check(x, shape, strides, dim, expect_kernel=kern, init=0.25)
    scan_and_check(x, shape, strides, dim, op="max", inclusive=False)
    xi = W.randint(n, -2**20, 2**20, 12000 + n % 89)
    scan_and_check(xi, shape, strides, dim, acc=torch.int64, out_dtype=torch.int64, inclusive=False, init=-3)
    xb = W.normal(n, 12100 + n % 83, torch.bfloat16)
    scan_and_check(xb, shape, strides, dim, out_dtype=torch.bfloat16)


def test_scan_dims_8192_square():
    """8192x8192 float32 along dims=1 and dims=2 (the dims reductions' size)."""
    mf, _ = W.matrix_8192()
    st = W.cm_strides(mf.shape)
    scan_and_check(mf.data, mf.shape, st, 1, expect_kernel="scan_rowwave")
    scan_and_check(mf.data, mf.shape, st, 2, expect_kernel="scan_columns")


def test_padded_view_with_offset():
    x = W.normal(40 * 60 + 7, 12200)
    scan_and_check(x, (30, 50), (1, 40), 1, offset=3, init=1.0)
    scan_and_check(x, (30, 50), (1, 40), 2, offset=3, op="min")


def test_empty_views():
    rk = _rk()
    x = W.normal(10, 12300).to(DEV)
    guard = torch.full((4,), 3.0, device=DEV)
    rk.scan(x, (0, 5), (1, 1), 2, out=guard)
    rk.scan(x, (5, 0), (1, 5), 1, out=guard)
    torch.cuda.synchronize()
    assert np.all(raw_np(guard) == 3.0)


# ------------------------------------------------------ look-back tile state

def _fused(rk, on):
    class _F:
        def __enter__(self):
            self.prev = rk.rk_debug_set_fused_finish(on)

        def __exit__(self, *exc):
            rk.rk_debug_set_fused_finish(self.prev)
    return _F()


@pytest.mark.parametrize("on", [1, 0], ids=["library_slot", "workspace_and_clear_launch"])
def test_tile_state_paths(on):
    """The look-back state lives in the library's stream slot (reset by each
    call's last block) or in the workspace (cleared by a launch first); both
    give exact integer scans, call after call with changing tile counts on
    one stream, and leave the tile count and a zero timeout word in the
    workspace header."""
    rk = _rk()
    cases = [((3 * TILE + 5,), (1,), 1), ((10**6 + 3,), (1,), 1), ((TILE,), (1,), 1),
             ((300, 2000), (1, 300), 2), ((10**8,), (1,), 1), ((5000, 2), (1, 5000), 1),
             ((300, 2000), (2000, 1), 2), ((30, 2000, 64), (128000, 64, 1), 1), ((5000, 6), (6, 1), 1)]
    with _fused(rk, on):
        for rep in range(2):
            for shape, strides, dim in cases:
                n = math.prod(shape)
                x = W.randint(n, -1000, 1000, 12400 + n % 101 + rep)
                xd = x.to(DEV)
                plan = rk.plan_scan(torch.int32, shape, strides, dim, acc=torch.int64)
                assert plan["launches"] == (1 if on else 2), plan
                nb = rk.rk_scan_workspace_size(rk.RK_I32, rk.RK_I64, len(shape), shape, strides, dim - 1)
                ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device=DEV)   # garbage on entry
                out = rk.scan(xd, shape, strides, dim, acc=torch.int64, out_dtype=torch.int64, workspace=ws)
                torch.cuda.synchronize()
                hdr = ws[:8].cpu().numpy().view(np.uint32)
                tiles = plan["split"] * (plan["grid"] // plan["split"])
                assert hdr[0] == plan["grid"] == tiles and hdr[1] == 0, (shape, hdr)
                R = O.scan_dims(O.SUM, O.I32, O.I64, raw_np(x), shape, strides, dim - 1, 0, True)
                assert np.array_equal(raw_np(out)[:n], R), (shape, dim, on, rep)


def test_tile_state_on_many_streams():
    """Look-back scans queued on 40 streams at once (more streams than
    library slots: the rest take workspace state), each with its own
    workspace: every result exact."""
    rk = _rk()
    n = 3 * TILE + 77
    xs = [W.randint(n, -1000, 1000, 12500 + i) for i in range(8)]
    xds = [x.to(DEV) for x in xs]
    nb = rk.rk_scan_workspace_size(rk.RK_I32, rk.RK_I64, 1, [n], [1], 0)
    wss = [torch.empty(nb, dtype=torch.uint8, device=DEV) for _ in range(40)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(40)]
    outs = []
    for i, s in enumerate(streams):
        with torch.cuda.stream(s):
            outs.append(rk.scan(xds[i % 8], acc=torch.int64, out_dtype=torch.int64, workspace=wss[i], init=i))
    for s in streams:
        s.synchronize()
    for i, o in enumerate(outs):
        R = O.scan(O.SUM, O.I32, O.I64, raw_np(xs[i % 8]), i, True)
        assert np.array_equal(raw_np(o), R), i


def test_beyond_2_31_elements():
    """A scan of more than 2^31 int32 ones into int64 (8.6 GB in, 17 GB out):
    more tiles than a library slot holds, so the workspace state and its
    clearing launch; output k is k + 1 (sampled).  Along dims=2 of a
    (2^16, 32769) view the last line's outputs sit past 2^31 elements, and so
    do those of the same ones read as a row-major (32769, 2^16) matrix
    scanned along its rows (the transposing tiles)."""
    rk = _rk()
    n = 2**31 + 70_000
    ones = torch.ones(n, dtype=torch.int32, device=DEV)
    plan = rk.plan_scan(torch.int32, (n,), (1,), 1, acc=torch.int64)
    assert plan["kernel_name"] == "scan_tile" and plan["launches"] == 2
    out = rk.scan(ones, acc=torch.int64, out_dtype=torch.int64)
    idx = torch.tensor([0, 1, 12345, 2**31 - 1, 2**31, n - 2, n - 1], device=DEV)
    assert out[idx].cpu().tolist() == [int(i) + 1 for i in idx.cpu().tolist()]
    del out
    L, k = 1 << 16, n // (1 << 16)
    cols = rk.scan(ones, (L, k), (1, L), 2, acc=torch.int64, out_dtype=torch.int64)
    assert rk.plan_scan(torch.int32, (L, k), (1, L), 2, acc=torch.int64)["kernel_name"] == "scan_columns"
    last = cols[(k - 1) * L:k * L]
    assert bool((last == k).all().item()) and int(cols[L - 1].item()) == 1
    del cols
    assert k == 32769 and k * L > 2**31
    assert rk.plan_scan(torch.int32, (k, L), (L, 1), 2, acc=torch.int64)["kernel_name"] == "scan_transpose"
    rows = rk.scan(ones, (k, L), (L, 1), 2, acc=torch.int64, out_dtype=torch.int64)
    # output (i, j) sits at i + k * j and holds j + 1
    ij = [(0, 0), (k - 1, 0), (0, L - 1), (k - 1, L - 1), (12345, 40000), (k - 1, 32767), (k - 2, L - 2)]
    idx = torch.tensor([i + k * j for i, j in ij], device=DEV)
    assert rows[idx].cpu().tolist() == [j + 1 for _, j in ij]
    assert bool((rows[k * (L - 1):] == L).all().item())
    del ones, rows
    torch.cuda.empty_cache()


# ------------------------------------------------ dims scans, dtype matrix
# The dims scan kernels of the f16, f64 and int64 units (and 32-bit integer
# and float64 accumulators), one layout per kernel, every output compared.

SCAN_DIMS_COMBOS = [  # (input, accumulator, output)
    (torch.float16, torch.float32, torch.float16),
    (torch.bfloat16, torch.float64, torch.float64),
    (torch.float64, torch.float64, torch.float64),
    (torch.int64, torch.int64, torch.int64),
    (torch.int32, torch.int32, torch.int32),          # sums wrap in the 32-bit accumulator
    (torch.float32, torch.float64, torch.float64),
]

SCAN_DIMS_LAYOUTS = [  # (shape, dim, strides or None)
    ((3 * TILE + 100, 3), 1, None),            # tile, look-back along each line
    ((3000, 40), 1, None),                     # row-wave
    ((40, 3000, 5), 2, None),                  # columns, look-back across chunks
    ((50, 300), 1, None),                      # lines, packed one element to a lane
    ((100, 301), 1, None),                     # lines, packed two elements to a lane
    ((300, 700), 2, (700, 1)),                 # transposing, scan dim contiguous in the input
    ((300, 700), 1, (700, 1)),                 # transposing, scan dim contiguous in the output
    ((40, 300, 50), 2, (300 * 50, 50, 1)),     # transposing, two kept dims
    ((8, 20_000), 2, (20_000, 1)),             # tiles along few row-major rows, strided outputs
    ((20_000, 8), 1, (8, 1)),                  # tiles along few row-major columns, strided inputs
]


@pytest.mark.parametrize("combo", SCAN_DIMS_COMBOS, ids=lambda c: "-".join(str(t).split(".")[1] for t in c))
@pytest.mark.parametrize("op", ["sum", "max"])
def test_scan_dims_dtype_matrix(combo, op):
    in_t, acc_t, out_t = combo
    for i, (shape, dim, strides) in enumerate(SCAN_DIMS_LAYOUTS):
        n = math.prod(shape)
        if in_t.is_floating_point:
            x = W.normal(n, 12300 + i, in_t) if in_t != torch.float64 else W.normal(n, 12300 + i).double()
            if out_t == torch.float16:
                x = x * 0.25            # prefix sums and their magnitudes stay below float16's 65,504
        else:
            x = W.randint(n, -2**20, 2**20, 12400 + i, in_t)
        scan_and_check(x, shape, strides or W.cm_strides(shape), dim, op=op, acc=acc_t, out_dtype=out_t,
                       inclusive=bool(i % 2), init=None if op != "sum" else 1)


# ------------------------------------------------------------ seeded sweep
# Views drawn from one seed per case (tests/layouts.py), scanned along a
# random dim.  Whatever kernel the planner takes, every output must match
# the oracle to the bar above.

SCAN_SWEEP_CASES = 64


@pytest.mark.parametrize("case", range(SCAN_SWEEP_CASES))
def test_seeded_scan_sweep(case):
    along_inner = case % 2 == 0                 # even cases: long contiguous lines (row-wave, tile)
    shape, strides, offset, numel, rng = random_view(30_000 + case, long_inner=along_inner)
    inner = innermost(strides)
    if along_inner and inner is not None:
        dim = inner + 1
    else:
        dim = int(rng.integers(1, len(shape) + 1))
    what = f"scan sweep case {case}: {shape} strides {strides} dim={dim} offset {offset}"
    x = W.normal(numel, 31_000 + case)
    scan_and_check(x, shape, strides, dim, init=0.5, offset=offset, what=what + " sum")
    scan_and_check(x, shape, strides, dim, op="max", inclusive=False, offset=offset, what=what + " max excl")
    xi = W.randint(numel, -10**6, 10**6, 32_000 + case)
    scan_and_check(xi, shape, strides, dim, acc=torch.int64, out_dtype=torch.int64, offset=offset,
                   what=what + " int32->int64")
    xb = W.normal(numel, 33_000 + case, torch.bfloat16)
    scan_and_check(xb, shape, strides, dim, out_dtype=torch.float32, offset=offset, what=what + " bf16->f32")
