"""GPU parity of reductions along dims (rk_reduce_dims) against the CPU oracle.

Shapes follow AcceleratedKernels.jl PR #176 (strided reductions along dims),
section "Timings": 768x1024x8 and 64x4096x32 over the middle dim, 3072x2048
and 8192x8192 over dims=2; plus the dims=1 rows and the selector's other
branches (section "This PR" item 1), the middle-dim runs (item 2), a single
output with a contiguous source taking the whole-array path (PR #139, "What
changes", last paragraph), and odd layouts served by the generic kernel.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from reduction_primitives_amd import workloads as W
from tests import golden_cases
from tests.layouts import random_view
from tests.parity import check, code_of, magnitude, raw_np

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _rk():
    import reduction_primitives_amd as rk
    rk.load()
    return rk


def dims_and_check(storage_cpu, shape, strides, dims, op="sum", map_="identity", acc=None,
                   out_dtype=None, mode="overwrite", init=None, offset=0, expect_kernel=None,
                   storage_dev=None, what=""):
    """Reduce the view (offset, shape, strides) of storage on the GPU and
    compare every output with the oracle."""
    rk = _rk()
    op_c, map_c, mode_c = rk.OPS[op], rk.MAPS[map_], rk.MODES[mode]
    in_c = code_of(storage_cpu.dtype)
    acc_c = rk.default_acc(in_c) if acc is None else code_of(acc)
    out_c = (acc_c if not O.is_fp(in_c) else in_c) if out_dtype is None else code_of(out_dtype)
    dims = (dims,) if isinstance(dims, int) else tuple(dims)
    mask = 0
    for d in dims:
        mask |= 1 << (d - 1)
    # the view must lie inside the storage before anything is launched
    last = sum((e - 1) * st for e, st in zip(shape, strides) if e > 0)
    assert math.prod(shape) == 0 or offset + last < storage_cpu.numel(), "view out of bounds"
    xd = storage_cpu.to(DEV) if storage_dev is None else storage_dev
    plan = rk.plan_dims(in_c, shape, strides, dims, acc=acc_c,
                        ptr=xd.data_ptr() + offset * xd.element_size())
    if expect_kernel is not None:
        assert plan["kernel_name"] == expect_kernel, plan
    n_out = math.prod(s for i, s in enumerate(shape) if not (mask >> i) & 1)
    prev = None
    out = None
    if mode == "fold":
        out = rk.reduce_dims(xd, shape, strides, dims, op=op, map=map_, acc=acc_c, out_dtype=out_c,
                             init=init, mode="overwrite", offset=offset)
        torch.cuda.synchronize()
        prev = raw_np(out)[:n_out]
    res = rk.reduce_dims(xd, shape, strides, dims, op=op, map=map_, acc=acc_c, out_dtype=out_c,
                         init=init, mode=mode, out=out, offset=offset)
    torch.cuda.synchronize()
    if mode == "host":
        gpu_raw = O.cast(out_c, [res])
    else:
        gpu_raw = raw_np(res)[:n_out]
    xr = raw_np(storage_cpu)[offset:]
    R, _ = O.expected_dims(op_c, map_c, in_c, acc_c, out_c, xr, shape, strides, mask, mode_c,
                           init, prev)
    start = O.start_value(op_c, acc_c, out_c, mode_c, init, prev)
    S = magnitude(map_c, in_c, acc_c, xr, start if op_c == O.SUM else 0.0,
                  reduce=(xr, shape, strides, mask)) if O.is_fp(in_c) else None
    check(op_c, out_c, gpu_raw, R, S,
          what or f"{plan['kernel_name']} {op}/{map_}/{mode} {shape} dims={dims}")
    return plan


CM = W.cm_strides


# ------------------------------------------------------------ configurations

def test_matrix_3072x2048_config():
    bf, f32 = W.matrix_3072x2048()
    shape, st = bf.shape, bf.strides
    dims_and_check(bf.data, shape, st, 2, out_dtype=torch.bfloat16, expect_kernel="tiled")
    dims_and_check(f32.data, shape, st, 2)
    dims_and_check(f32.data, shape, st, 1, expect_kernel="row")
    dims_and_check(bf.data, shape, st, 1, out_dtype=torch.bfloat16)


def test_middle_dim_config():
    for arr in W.middle_dim_3d():
        out_dt = torch.bfloat16 if arr.data.dtype == torch.bfloat16 else torch.float32
        dims_and_check(arr.data, arr.shape, arr.strides, 2, out_dtype=out_dt)


def test_matrix_8192_config():
    f32, i32 = W.matrix_8192()
    shape, st = f32.shape, f32.strides
    xd = f32.data.to(DEV)
    dims_and_check(f32.data, shape, st, 2, storage_dev=xd)
    dims_and_check(f32.data, shape, st, 1, storage_dev=xd, expect_kernel="row")
    dims_and_check(f32.data, shape, st, 2, op="max", storage_dev=xd)
    # sum of squares of the whole array into a device scalar (single output)
    dims_and_check(f32.data, shape, st, (1, 2), map_="square", init=0.0, storage_dev=xd,
                   expect_kernel="all")
    del xd
    dims_and_check(i32.data, shape, st, 1, acc=torch.int64, out_dtype=torch.int64,
                   expect_kernel="row")


def test_int32_dims_totals_beyond_int32():
    """8192x8192 of 2^20 summed over dims=1 into int64: 2^33 per output."""
    rk = _rk()
    x = torch.full((8192 * 8192,), 2**20, dtype=torch.int32, device=DEV)
    out = rk.reduce_dims(x, (8192, 8192), (1, 8192), 1, acc=torch.int64, out_dtype=torch.int64)
    assert bool((out == 2**33).all().item())
    out2 = rk.reduce_dims(x, (8192, 8192), (1, 8192), 2, acc=torch.int64, out_dtype=torch.int64)
    assert bool((out2 == 2**33).all().item())


def test_bf16_dims_partials_stay_fp32():
    """bf16 integers over dims=2 of 3072x2048: each output equals its exact
    integer sum rounded once to bf16."""
    rk = _rk()
    x = W.small_ints(3072 * 2048, -8, 8, 8100, torch.bfloat16)
    out = rk.reduce_dims(x.to(DEV), (3072, 2048), (1, 3072), 2, out_dtype=torch.bfloat16)
    exact = x.double().view(2048, 3072).sum(dim=0).numpy()
    assert np.array_equal(raw_np(out), O.cast(O.BF16, exact))


# ----------------------------------------------------------------- selector

SELECTOR_CASES = [
    # (shape, dims, dtype, expected kernel, why)
    ((65536, 16), 2, torch.float32, "thread", "reduction shorter than 32"),
    ((1 << 20, 40), 2, torch.float32, "thread", "a row of outputs of 4 MiB"),
    ((3072, 2048), 2, torch.float32, "tiled", "more outputs than elements, few wide tiles"),
    ((2048, 3072), 2, torch.float32, "columns", "fewer outputs than elements"),
    ((8192, 8192), 2, torch.float32, "columns", "wide tiles fill the device"),
    ((100, 37, 3), 2, torch.float32, "tiled", "ragged middle dim"),
    ((96, 4000, 3), 2, torch.bfloat16, "columns", "middle dim, columns split"),
    ((3000, 777), 1, torch.float32, "row", "contiguous reduced dim"),
    ((100003, 7), 1, torch.float32, "row", "few long rows (split row)"),
    ((5, 6, 7), (1, 3), torch.float32, "generic", "two non-adjacent reduced dims"),
    ((33, 5, 9, 4), (2, 4), torch.float32, "thread", "4-d, two short reduced dims"),
    ((1000, 1), (1, 2), torch.float32, "all", "single output, contiguous"),
    ((1000, 3000), 2, torch.float32, "columns", "ragged last tile, split units of uneven row counts"),
]


@pytest.mark.parametrize("case", SELECTOR_CASES, ids=lambda c: c[4].replace(" ", "_"))
def test_selector_kernels(case):
    shape, dims, dt, kern, _ = case
    n = math.prod(shape)
    x = W.normal(n, 8200 + n % 101, dt) if dt != torch.int32 else W.randint(n, -99, 99, 8200)
    dims_and_check(x, shape, CM(shape), dims, out_dtype=dt, expect_kernel=kern)


def test_selector_rules_from_tuning():
    """The selector's three rules on the device's own CU count, with the
    thresholds of the tuning table (no launch)."""
    from tests import tuning
    rk = _rk()
    t = tuning.values()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    row = t["kThreadRowBytes"] // 4
    assert rk.plan_dims(torch.float32, (row, 100), (1, row), 2)["kernel_name"] == "thread"
    n = cus * t["kTiledOutputs"] - t["kTiledOutputs"]
    assert rk.plan_dims(torch.float32, (n, 100), (1, n), 2)["kernel_name"] == "tiled"
    assert rk.plan_dims(torch.float32, (512, 31), (1, 512), 2)["kernel_name"] == "thread"
    assert rk.plan_dims(torch.float32, (512, 32), (1, 512), 2)["kernel_name"] == "tiled"


@pytest.mark.parametrize("case", SELECTOR_CASES[:7], ids=lambda c: c[4].replace(" ", "_"))
def test_selector_kernels_max_fold_int(case):
    shape, dims, _, kern, _ = case
    n = math.prod(shape)
    xi = W.randint(n, -10**6, 10**6, 8300 + n % 89)
    dims_and_check(xi, shape, CM(shape), dims, acc=torch.int64, out_dtype=torch.int64,
                   mode="fold")
    dims_and_check(xi, shape, CM(shape), dims, op="max", acc=torch.int32, out_dtype=torch.int32)
    xf = W.uniform(n, -1.0, 1.0, 8400 + n % 83)
    dims_and_check(xf, shape, CM(shape), dims, op="min", map_="abs")
    dims_and_check(xf, shape, CM(shape), dims, map_="square", init=2.0)


@pytest.mark.parametrize("case", SELECTOR_CASES, ids=lambda c: c[4].replace(" ", "_"))
def test_selector_kernels_wide_accumulators(case):
    """Each kernel with float64 accumulators over bf16 and f32 inputs: a bf16
    lane's 16-byte load widens into 8 doubles, the widest accumulator state a
    kernel holds; ragged row groups take the last, partial group."""
    shape, dims, _, _, _ = case
    n = math.prod(shape)
    for dt in (torch.bfloat16, torch.float32):
        x = W.normal(n, 8500 + n % 79, dt)
        dims_and_check(x, shape, CM(shape), dims, acc=torch.float64, out_dtype=torch.float64)
    x = W.normal(n, 8600 + n % 73, torch.bfloat16)
    dims_and_check(x, shape, CM(shape), dims, op="max", acc=torch.float64, out_dtype=torch.bfloat16)


# ------------------------------------------------------------------ layouts

@pytest.mark.parametrize("offset", [1, 2, 3, 5])
def test_offset_views(offset):
    for shape, dims in [((3072, 64), 2), ((64, 3000), 2), ((100, 37, 3), 2), ((777, 45), 1)]:
        n = math.prod(shape)
        x = W.normal(n + offset, 8500 + offset)
        dims_and_check(x, shape, CM(shape), dims, offset=offset)
        xb = W.normal(n + offset, 8600 + offset, torch.bfloat16)
        dims_and_check(xb, shape, CM(shape), dims, offset=offset, out_dtype=torch.float32)


def test_non_contiguous_views():
    rk = _rk()
    x = W.normal(64 * 50 * 6, 8700)
    # every other column of a 64x100... : shape (64, 25, 6) with strides (1, 128, 3200)
    dims_and_check(x, (64, 25, 6), (1, 128, 3200), 2)
    # transposed storage: reduce the slow storage dim of a row-major-like view
    dims_and_check(x, (50, 64), (64, 1), 1, expect_kernel="tiled")
    dims_and_check(x, (50, 64), (64, 1), 2, expect_kernel="row")
    # single output over a strided view (whole-array passes, strided addressing)
    dims_and_check(x, (800,), (2,), 1, expect_kernel="all_strided")
    dims_and_check(x, (40, 30), (3, 200), (1, 2), expect_kernel="all_strided")
    p = rk.plan_dims(torch.float32, (40, 30), (3, 200), (1, 2))
    assert p["launches"] in (1, 2)
    # broadcast (stride 0) dims
    dims_and_check(x, (64, 10), (1, 0), 2)


# --------------------------------------------------------- general layouts
# Several reduced dims that do not merge, 4-d arrays, outputs that are not
# contiguous in the input.  Contiguous runs of outputs take the tile kernels
# with the extra reduced dims as segments of rows; everything else takes the
# generic kernel, split over blocks when there are few outputs.

GENERAL_CASES = [
    # (storage numel, shape, strides, dims, expected kernel, why)
    (128 * 100 * 2 * 64, (128, 100, 2, 64), CM((128, 100, 2, 64)), (2, 4), "columns",
     "4-d, dims 2 and 4: whole segments per split"),
    (128 * 3 * 3000, (128, 3000, 3), (1, 384, 128), (2, 3), "columns",
     "permuted view, dims 2 and 3: splits inside segments"),
    (3072 * 8 * 20, (3072, 20, 8), (1, 3072 * 8, 3072), (2, 3), "tiled",
     "permuted view, more outputs than elements"),
    (64 * 500 * 16 * 6, (64, 500, 16, 6), CM((64, 500, 16, 6)), (2, 4), "columns",
     "middle-dim runs with a second reduced dim"),
    (64 * 50 * 16 * 6, (64, 50, 16, 6), CM((64, 50, 16, 6)), (2, 4), "tiled",
     "middle-dim runs, more outputs than elements"),
    (33 * 5 * 9 * 4, (33, 5, 9, 4), CM((33, 5, 9, 4)), (2, 4), "thread", "short reductions"),
    (31000, (130, 7, 11, 3), (1, 130 * 11 * 3, 131, 130 * 11), (2, 3, 4), "columns",
     "three reduced dims, strides not 16-byte multiples"),
    (5 * 6 * 7, (5, 6, 7), CM((5, 6, 7)), (1, 3), "generic", "non-adjacent dims, kept dim strided"),
    (49 * 64 * 256, (49, 64, 256), CM((49, 64, 256)), (1, 3), "generic",
     "per-channel statistics of 7x7 maps"),
    (3136 * 16 * 24, (3136, 16, 24), CM((3136, 16, 24)), (1, 3), "row",
     "per-channel statistics of 56x56 maps: rows of 12.5 KB as segments"),
    (100000 * 3 * 2, (100000, 3, 2), CM((100000, 3, 2)), (1, 3), "row",
     "few outputs: pieces of one segment's row"),
    (2000 * 3 * 5 * 7, (2000, 3, 5, 7), CM((2000, 3, 5, 7)), (1, 3, 4), "row",
     "three reduced dims, rows of 8 KB"),
    (1025 * 9 * 5, (1025, 9, 5), CM((1025, 9, 5)), (1, 3), "row",
     "rows of 4100 bytes: every row at its own 16-byte phase"),
    (2 * 300 * 40, (300, 40), (2, 600), 1, "generic", "strided gather along the reduced dim"),
    # permuted views: the kept dims run contiguously only in storage order, so
    # the tile kernels number outputs in that order and store each one at its
    # place in the output
    (7680000, (64, 3000, 40), (40, 2560, 1), 2, "columns", "permuted view, kept dims transposed in storage"),
    (69300, (33, 700, 3), (3, 99, 1), 2, "columns", "permuted view, element loads"),
    (102400, (64, 50, 32), (32, 2048, 1), 2, "tiled", "permuted view, short reduced dim"),
    (1536000, (16, 300, 8, 40), (8, 5120, 1, 128), 2, "tiled", "permuted 4-d view, three kept dims in storage order"),
    (60000, (100, 20, 30), (600, 1, 20), 1, "tiled", "permuted view, reduced dim outermost"),
    (3465, (7, 5, 9, 11), (5, 1, 385, 35), 3, "thread", "permuted 4-d view, thread per output"),
]


@pytest.mark.parametrize("case", GENERAL_CASES, ids=lambda c: c[5].replace(" ", "_"))
def test_general_layouts(case):
    numel, shape, strides, dims, kern, _ = case
    x = W.normal(numel, 9600 + numel % 97)
    dims_and_check(x, shape, strides, dims, expect_kernel=kern, init=0.5)
    dims_and_check(x, shape, strides, dims, op="max", expect_kernel=kern)
    xb = W.normal(numel, 9700 + numel % 89, torch.bfloat16)
    dims_and_check(xb, shape, strides, dims, out_dtype=torch.float32, map_="square")
    xi = W.randint(numel, -10**6, 10**6, 9800 + numel % 83)
    dims_and_check(xi, shape, strides, dims, acc=torch.int64, out_dtype=torch.int64, mode="fold")
    dims_and_check(xi, shape, strides, dims, op="min", acc=torch.int32, out_dtype=torch.int32)


@pytest.mark.parametrize("case", [c for c in GENERAL_CASES if c[4] in ("columns", "generic")],
                         ids=lambda c: c[5].replace(" ", "_"))
def test_general_layouts_both_finishes(case):
    """Split general layouts: the one-launch and the two-launch finish agree
    bit for bit (same partials, same fold order)."""
    rk = _rk()
    numel, shape, strides, dims, kern, _ = case
    x = W.normal(numel, 9900 + numel % 79).to(DEV)
    res = {}
    for on in (1, 0):
        prev = rk.rk_debug_set_fused_finish(on)
        try:
            res[on] = raw_np(rk.reduce_dims(x, shape, strides, dims, init=0.25))
            torch.cuda.synchronize()
        finally:
            rk.rk_debug_set_fused_finish(prev)
    assert np.array_equal(res[0], res[1])


# More than 32 blocks (or waves) per output: the one-launch finish counts
# their arrivals in groups of 32, the last group possibly partial, then the
# groups on the output's top counter.
MANY_SPLIT_CASES = [
    ((3, 1_000_000), 2, "columns"),          # 256 splits: 8 full groups
    ((1_000_003, 3), 1, "row"),              # 488 splits: the last group holds 8
    ((2, 50_000, 3), 2, "columns"),          # 86 splits: 32, 32, 22
    ((999, 3, 1001), (1, 3), "generic"),     # 244 splits, element loads
]


@pytest.mark.parametrize("case", MANY_SPLIT_CASES, ids=lambda c: f"{c[2]}_{'x'.join(map(str, c[0]))}")
def test_many_splits_grouped_arrivals(case):
    rk = _rk()
    shape, dims, kern = case
    numel = math.prod(shape)
    plan = rk.plan_dims(torch.float32, shape, CM(shape), dims)
    assert plan["kernel_name"] == kern and plan["split"] > 32 and plan["launches"] == 1, plan
    xi = W.randint(numel, -1000, 1000, 9970 + numel % 71)
    dims_and_check(xi, shape, CM(shape), dims, acc=torch.int64, out_dtype=torch.int64, expect_kernel=kern)
    xf = W.normal(numel, 9980 + numel % 73)
    xd = xf.to(DEV)
    res = {}
    for on in (1, 0):
        prev = rk.rk_debug_set_fused_finish(on)
        try:
            dims_and_check(xf, shape, CM(shape), dims, init=0.5, expect_kernel=kern, storage_dev=xd)
            dims_and_check(xf, shape, CM(shape), dims, op="max", expect_kernel=kern, storage_dev=xd)
            res[on] = raw_np(rk.reduce_dims(xd, shape, CM(shape), dims, init=0.5))
            torch.cuda.synchronize()
        finally:
            rk.rk_debug_set_fused_finish(prev)
    # the tile and generic kernels' last block folds the partials in split
    # order, as the second launch does: the same bits.  The row kernel's last
    # wave folds them across its lanes (one memory round trip for hundreds of
    # partials), so only the oracle checks above bind it.
    if kern != "row":
        assert np.array_equal(res[0], res[1])


@pytest.mark.parametrize("offset", [1, 3, 4])
def test_general_layout_offsets(offset):
    """The generic kernel takes 16-byte loads only when every reduced row
    starts 16-byte aligned; an offset view falls back to element loads."""
    shape = (1000, 8, 12)
    x = W.normal(math.prod(shape) + offset, 9950 + offset)
    plan = dims_and_check(x, shape, CM(shape), (1, 3), offset=offset, expect_kernel="generic")
    assert plan["vec"] == (4 if offset % 4 == 0 else 1)
    xb = W.normal(math.prod(shape) + offset, 9960 + offset, torch.bfloat16)
    dims_and_check(xb, shape, CM(shape), (1, 3), offset=offset, out_dtype=torch.float32)


@pytest.mark.parametrize("offset", [1, 2, 3])
def test_row_segments_offsets(offset):
    """The row kernel over segments peels a scalar head and tail off every
    row piece, so views at any element offset keep 16-byte loads."""
    shape = (3136, 16, 24)
    x = W.normal(math.prod(shape) + offset, 9990 + offset)
    plan = dims_and_check(x, shape, CM(shape), (1, 3), offset=offset, expect_kernel="row")
    assert plan["vec"] == 4
    xi = W.randint(math.prod(shape) + offset, -10**6, 10**6, 9995 + offset)
    dims_and_check(xi, shape, CM(shape), (1, 3), offset=offset, acc=torch.int64, out_dtype=torch.int64,
                   expect_kernel="row")


def test_general_layout_plans():
    rk = _rk()
    p = rk.plan_dims(torch.float32, (128, 3000, 3), (1, 384, 128), (2, 3))
    assert p["kernel_name"] == "columns" and p["split"] > 3
    p = rk.plan_dims(torch.float32, (3136, 16, 24), CM((3136, 16, 24)), (1, 3))
    assert p["kernel_name"] == "row" and p["split"] > 1
    assert p["workspace_bytes"] >= p["split"] * 16 * 4
    p = rk.plan_dims(torch.float32, (1000, 16, 24), CM((1000, 16, 24)), (1, 3))
    assert p["kernel_name"] == "generic" and p["split"] > 1


def test_dims_all_masked_equals_whole_array():
    rk = _rk()
    x = W.normal(300 * 70, 8800).to(DEV)
    a = rk.reduce_dims(x, (300, 70), (1, 300), (1, 2), init=0.5)
    b = rk.reduce_all(x, init=0.5)
    torch.cuda.synchronize()
    assert raw_np(a)[0] == raw_np(b)[0]


def test_empty_and_degenerate():
    rk = _rk()
    x = W.normal(1000, 8900)
    # a zero-length reduced dim: every output is the starting value
    out = rk.reduce_dims(x.to(DEV), (10, 0), (1, 10), 2, init=1.25)
    torch.cuda.synchronize()
    assert np.all(raw_np(out)[:10] == np.float32(1.25))
    out = rk.reduce_dims(x.to(DEV), (10, 0), (1, 10), 2, op="max")
    assert np.all(np.isneginf(raw_np(out)[:10]))
    # no outputs: nothing is written
    guard = torch.full((4,), 3.0, device=DEV)
    rk.reduce_dims(x.to(DEV), (0, 10), (1, 1), 2, out=guard)
    torch.cuda.synchronize()
    assert np.all(raw_np(guard) == 3.0)
    # a single element, host mode
    v = rk.reduce_dims(x.to(DEV), (1, 1), (1, 1), (1, 2), mode="host", init=1.0)
    assert v == pytest.approx(1.0 + float(x[0]), rel=1e-6)
    # no reduced dims: each output is f(x) (+) init
    dims_and_check(x, (10, 100), (1, 10), (), map_="square", init=1.0)
    dims_and_check(x, (1000,), (1,), (), op="max")
    # host mode with one output of a dims reduction
    dims_and_check(x, (1, 1000), (1, 1), 2, mode="host", init=-2.0)


@pytest.mark.parametrize("case", [c for c in golden_cases.load() if "shape" in c],
                         ids=lambda c: c["id"])
def test_golden_dims(case):
    rk = _rk()
    c = case
    x = torch.from_numpy(np.ascontiguousarray(c["x_raw"]).copy()).to(DEV)
    shape = c["shape"]
    dims = tuple(d + 1 for d in range(len(shape)) if (c["mask"] >> d) & 1)
    out = None
    if c["mode"] == "fold":
        out = torch.from_numpy(np.ascontiguousarray(c["prev_raw"]).copy()).to(DEV)
    res = rk.reduce_dims(x, shape, CM(shape), dims, op=c["op"], map=c["map"], acc=c["acc_code"],
                         out_dtype=c["out_code"], init=c.get("init"), mode=c["mode"], out=out)
    torch.cuda.synchronize()
    assert list(res.cpu().numpy()) == list(c["expected"]), c["id"]


def test_workspace_reuse_for_split_dims():
    rk = _rk()
    ws = torch.full((1 << 22,), 0xFF, dtype=torch.uint8, device=DEV)
    for shape, dims, dt in [((64, 4096, 32), 2, torch.float32), ((2048, 3072), 2, torch.bfloat16),
                            ((100003, 7), 1, torch.float32)]:
        n = math.prod(shape)
        x = W.normal(n, 9000 + n % 7, dt)
        in_c = rk.dtype_code(dt)
        mask = 1 << (dims - 1)
        p = rk.plan_dims(dt, shape, CM(shape), dims)
        assert p["split"] > 1, p
        need = rk.rk_workspace_size(in_c, rk.RK_F32, len(shape), shape, CM(shape), mask)
        assert 0 < need <= ws.numel()
        out = rk.reduce_dims(x.to(DEV), shape, CM(shape), dims, out_dtype=torch.float32, workspace=ws)
        torch.cuda.synchronize()
        xr = raw_np(x)
        R = O.reduce_dims(O.SUM, O.IDENTITY, in_c, O.F32, xr, shape, CM(shape), mask, 0.0)
        S = magnitude(O.IDENTITY, in_c, O.F32, xr, 0.0, reduce=(xr, shape, CM(shape), mask))
        check(O.SUM, O.F32, raw_np(out), R, S, f"reuse {shape}")


# ------------------------------------------------------------ dtype matrix
# The dims kernels of every input dtype's translation unit: each accumulator
# and output the dtype table allows for f16, f64 and int64 inputs (f32, bf16
# and int32 inputs run through the cases above), on one layout per kernel.

DIMS_COMBOS = [  # (input, accumulator, output)
    (torch.float16, torch.float32, torch.float16),
    (torch.float16, torch.float64, torch.float32),
    (torch.float64, torch.float64, torch.float64),
    (torch.float64, torch.float64, torch.float32),
    (torch.int64, torch.int64, torch.int64),
    (torch.int32, torch.int32, torch.int32),          # sums wrap in the 32-bit accumulator
    (torch.float32, torch.float64, torch.float64),
]

DIMS_LAYOUTS = [  # (shape, reduced dims)
    ((1000, 3000), 2),        # columns, plain
    ((96, 1000, 3), 2),       # columns, middle dim
    ((3000, 777), 1),         # row
    ((2100, 300, 21), (1, 3)),  # row over 21 segments (4 KB rows and longer), several per split unit
    ((3072, 256), 2),         # tiled
    ((65536, 16), 2),         # thread per output
    ((500, 9, 7), (1, 3)),    # generic
]


def _draw_dims(dtype, n, seed, out_dtype):
    if dtype.is_floating_point:
        x = W.normal(n, seed, dtype) if dtype != torch.float64 else W.normal(n, seed).double()
        if out_dtype == torch.float16:
            x = x * 0.25        # sums of up to 44,100 values of N(0, 1/16): a few hundred at most
        return x
    return W.randint(n, -2**20, 2**20, seed, dtype)


@pytest.mark.parametrize("combo", DIMS_COMBOS, ids=lambda c: "-".join(str(t).split(".")[1] for t in c))
@pytest.mark.parametrize("op", ["sum", "max"])
def test_dims_dtype_matrix(combo, op):
    in_dt, acc_dt, out_dt = combo
    for i, (shape, dims) in enumerate(DIMS_LAYOUTS):
        x = _draw_dims(in_dt, math.prod(shape), 9800 + 10 * i, out_dt)
        dims_and_check(x, shape, CM(shape), dims, op=op, acc=acc_dt, out_dtype=out_dt)


# ------------------------------------------------------------ seeded sweep
# Views drawn from one seed per case (tests/layouts.py) with a random
# non-empty set of reduced dims, mostly leaving some dims kept.  Whatever
# kernel the planner takes, every output must match the oracle.

SWEEP_CASES = 96


def _random_view(seed):
    shape, strides, offset, numel, rng = random_view(seed)
    nd = len(shape)
    k = nd if nd == 1 or rng.random() < 0.15 else int(rng.integers(1, nd))   # mostly some dims kept
    dims = tuple(sorted(int(d) + 1 for d in rng.choice(nd, k, replace=False)))
    return shape, strides, dims, offset, numel


@pytest.mark.parametrize("case", range(SWEEP_CASES))
def test_seeded_layout_sweep(case):
    shape, strides, dims, offset, numel = _random_view(20_000 + case)
    what = f"sweep case {case}: {shape} strides {strides} dims={dims} offset {offset}"
    x = W.normal(numel, 21_000 + case)
    dims_and_check(x, shape, strides, dims, init=0.5, offset=offset, what=what + " sum")
    dims_and_check(x, shape, strides, dims, op="max", offset=offset, what=what + " max")
    xi = W.randint(numel, -10**6, 10**6, 22_000 + case)
    dims_and_check(xi, shape, strides, dims, acc=torch.int64, out_dtype=torch.int64, mode="fold",
                   offset=offset, what=what + " int32->int64 fold")
    xb = W.normal(numel, 23_000 + case, torch.bfloat16)
    dims_and_check(xb, shape, strides, dims, map_="square", out_dtype=torch.float32, offset=offset,
                   what=what + " bf16 square")
