"""Host-side checks of librk.so that need no GPU: exports, plans, validation.

Nothing here launches a kernel: plans are computed for an explicit CU count,
and every rk_reduce_* call made here is rejected by validation before any
launch.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _rk():
    import reduction_primitives_amd as rk
    rk.load()
    return rk


def test_library_exports_every_declared_function():
    rk = _rk()
    with open(os.path.join(ROOT, "include", "rk.h")) as f:
        header = f.read()
    declared = set(re.findall(r"\b(rk_[a-z0-9_]+)\s*\(", header))
    assert declared == set(rk.EXPORTS)
    lib = ctypes.CDLL(rk.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings():
    rk = _rk()
    assert rk.status_string(0) == "ok"
    assert "invalid" in rk.status_string(1)
    assert "unsupported" in rk.status_string(2)
    assert "HIP" in rk.status_string(3)
    assert rk.status_string(99) == "unknown status"


# ------------------------------------------------------------------- plans

def plan(dtype, shape, dims, strides=None, cus=256, ptr=0):
    import reduction_primitives_amd as rk
    from reduction_primitives_amd.workloads import cm_strides
    return rk.plan_dims(dtype, shape, strides or cm_strides(shape), dims, ptr=ptr, num_cus=cus)


def test_whole_array_plan():
    rk = _rk()
    assert rk.rk_debug_set_fused_finish(1) in (0, 1)
    info = rk.rk_plan_all(rk.RK_F32, rk.RK_F32, 0, 10**8, 256)
    # one launch: the last first-pass block to arrive folds the partials
    assert info.kernel == rk.RK_KERNEL_ALL and info.launches == 1
    assert info.grid == 1024 and info.block == 256 and info.vec == 4
    assert info.workspace_bytes == 4352          # (1024 + 1) * 4 rounded to 256
    small = rk.rk_plan_all(rk.RK_F32, rk.RK_F32, 0, 10**4, 256)
    assert small.grid == 1 and small.launches == 1
    # the grid cap follows the CU count
    assert rk.rk_plan_all(rk.RK_F32, rk.RK_F32, 0, 10**8, 80).grid == 320
    # workspace: one accumulator per first-pass block plus the final slot
    d = rk.rk_plan_all(rk.RK_I32, rk.RK_I64, 0, 10**8, 256)
    assert d.workspace_bytes == ((1024 + 1) * 8 + 255) // 256 * 256


def test_two_input_plan_matches_one_input_plan():
    """Same grid and workspace as the one-input pass; 16-byte loads of x
    whenever there is a body of at least one vector beyond y's first chunk
    (y in 16-byte loads too, shifted into place when the two inputs sit at
    different offsets from a 16-byte boundary); element loads otherwise."""
    rk = _rk()
    for n in (0, 1, 10**4, 10**6 + 3, 10**8):
        one = rk.rk_plan_all(rk.RK_F32, rk.RK_F32, 0, n, 256)
        two = rk.rk_plan_all2(rk.RK_F32, rk.RK_F32, 0, 0, n, 256)
        assert (two.grid, two.workspace_bytes, two.vec) == (one.grid, one.workspace_bytes, 4)
        assert two.kernel == rk.RK_KERNEL_ALL2
        shifted = n >= 16
        assert rk.rk_plan_all2(rk.RK_F32, rk.RK_F32, 16, 4, n, 256).vec == (4 if shifted else 1)
        assert rk.rk_plan_all2(rk.RK_F32, rk.RK_F32, 20, 36, n, 256).vec == 4
        assert rk.rk_plan_all2(rk.RK_BF16, rk.RK_F32, 2, 4, n, 256).vec == (8 if shifted else 1)
        assert rk.rk_plan_all2(rk.RK_F64, rk.RK_F64, 8, 16, n, 256).vec == (2 if shifted else 1)


def test_config_shapes_take_the_expected_kernels():
    import torch
    assert plan(torch.bfloat16, (3072, 2048), 2)["kernel_name"] == "tiled"
    assert plan(torch.float32, (3072, 2048), 2)["kernel_name"] == "tiled"
    assert plan(torch.float32, (3072, 2048), 1)["kernel_name"] == "row"
    assert plan(torch.bfloat16, (768, 1024, 8), 2)["kernel_name"] == "tiled"
    assert plan(torch.float32, (768, 1024, 8), 2)["kernel_name"] == "tiled"
    p = plan(torch.float32, (64, 4096, 32), 2)
    assert p["kernel_name"] == "columns" and p["split"] > 1 and p["launches"] == 1
    p = plan(torch.float32, (8192, 8192), 2)
    assert p["kernel_name"] == "columns"
    assert plan(torch.float32, (8192, 8192), 1)["kernel_name"] == "row"
    assert plan(torch.int32, (8192, 8192), 1)["kernel_name"] == "row"
    p = plan(torch.float32, (8192, 8192), (1, 2))
    assert p["kernel_name"] == "all" and p["n_out"] == 1 and p["reduce_len"] == 8192 * 8192


def test_selector_rules():
    """The three rules of the selector, with thresholds read from the tuning
    table (so the test follows the table, not hard-coded numbers)."""
    import torch
    from tests import tuning
    t = tuning.values()
    cus = 256
    row_f32 = t["kThreadRowBytes"] // 4           # outputs in a threshold-wide f32 row
    # rule 1: a row of outputs at least kThreadRowBytes wide, or a short reduction
    assert plan(torch.float32, (row_f32, 100), 2)["kernel_name"] == "thread"
    assert plan(torch.float32, (row_f32 - 4, 100), 2)["kernel_name"] != "thread"
    assert plan(torch.bfloat16, (2 * row_f32, 100), 2)["kernel_name"] == "thread"
    m_short = t["kMinReduceLen"]
    assert plan(torch.float32, (1000, m_short - 1), 2)["kernel_name"] == "thread"
    assert plan(torch.float32, (1000, m_short), 2)["kernel_name"] == "tiled"
    # rule 2: outputs >= elements per output and fewer narrow tiles than CUs -> tiled
    w = t["kTiledOutputs"]
    n_fill = cus * t["kFillTilesPerCu"] * w       # outputs whose narrow tiles fill the device
    assert plan(torch.float32, (n_fill - w, 1000), 2)["kernel_name"] == "tiled"
    assert plan(torch.float32, (n_fill, 1000), 2)["kernel_name"] == "columns"
    assert plan(torch.float32, (999, 1000), 2)["kernel_name"] == "columns"   # outputs < elements
    # "fill the device" scales with the CU count
    assert plan(torch.float32, (8192, 8192), 2, cus=cus)["kernel_name"] == "columns"
    assert plan(torch.float32, (8192, 8192), 2, cus=2 * cus)["kernel_name"] == "tiled"
    # rule 3 splits along the reduced dim to reach the block target
    p = plan(torch.float32, (64, 100000), 2)
    assert p["kernel_name"] == "columns" and p["split"] > 1
    assert p["grid"] <= cus * t["kColumnsBlocksPerCu"] * 2
    p = plan(torch.float32, (8192, 8192), 2)
    assert p["tile_outputs"] == t["kColumnsRowBytes"] // 4
    assert p["grid"] == cus * t["kColumnsBlocksPerCu"]
    # short runs narrow the columns tile (but never below kColumnsMinRowBytes)
    assert plan(torch.float32, (64, 4096, 32), 2)["tile_outputs"] == 64
    assert plan(torch.float32, (16, 4096, 32), 2)["tile_outputs"] == t["kColumnsMinRowBytes"] // 4
    # tile shapes: tiled tiles are kTiledOutputs wide, thread tiles one block of vectors
    assert plan(torch.bfloat16, (3072, 2048), 2)["tile_outputs"] == w
    assert plan(torch.float32, (row_f32, 100), 2)["tile_outputs"] == t["kThreadBlock"] * 4


def test_general_layouts_route():
    """Reduced dims that do not merge: contiguous runs of outputs take the
    tile kernels (the other reduced dims index segments of rows); a
    contiguous reduced dim of at least 4 KB rows takes the row kernel (the
    other reduced dims index segments of those rows); anything else the
    generic kernel, split over blocks when outputs are few."""
    import torch
    f32 = torch.float32
    p = plan(f32, (128, 3000, 3), (2, 3), strides=(1, 384, 128))
    assert p["kernel_name"] == "columns" and p["split"] == 69 and p["vec"] == 4
    p = plan(f32, (128, 100, 2, 64), (2, 4))
    assert p["kernel_name"] == "columns" and p["split"] == 32
    p = plan(f32, (3072, 20, 8), (2, 3), strides=(1, 3072 * 8, 3072))
    assert p["kernel_name"] == "tiled" and p["split"] == 1
    p = plan(f32, (130, 7, 11, 3), (2, 3, 4), strides=(1, 4290, 131, 1430))
    assert p["kernel_name"] == "columns" and p["vec"] == 1      # 131 * 4 bytes: no 16-byte rows
    p = plan(f32, (49, 64, 256), (1, 3))
    assert p["kernel_name"] == "generic" and p["split"] == 3 and p["launches"] == 1
    assert p["vec"] == 1                                             # 49-element rows
    p = plan(f32, (3136, 16, 24), (1, 3))                           # 12.5 KB rows, 24 segments
    assert p["kernel_name"] == "row" and p["split"] == 24 and p["grid"] == 16 * 24 // 4
    assert p["vec"] == 4                                             # 16-byte loads after each row's head
    assert plan(f32, (3136, 16, 24), (1, 3), ptr=4)["vec"] == 4
    assert plan(torch.bfloat16, (3136, 16, 24), (1, 3))["vec"] == 8
    assert p["workspace_bytes"] == 1536                              # 24 * 16 * 4 rounded to 256
    p = plan(f32, (3136, 256, 84), (1, 3))                          # per-channel statistics
    assert p["kernel_name"] == "row" and p["split"] == 8 and p["launches"] == 1   # 11 segments each
    p = plan(f32, (100_000, 3, 2), (1, 3))                          # pieces of one segment's row
    assert p["kernel_name"] == "row" and p["split"] > 2 and p["split"] % 2 == 0
    p = plan(f32, (1000, 8, 12), (1, 3))                            # 4000-byte rows: generic
    assert p["kernel_name"] == "generic"
    p = plan(f32, (5000, 3000), (1,), strides=(3, 15000))            # no stride-1 dim
    assert p["kernel_name"] == "generic" and p["split"] == 1


def test_normalisation_drops_unit_dims_and_merges():
    import torch
    # (768, 1024, 8) reduced over dims 1 and 2 merges into one contiguous run per batch
    p = plan(torch.float32, (768, 1024, 8), (1, 2))
    assert p["kernel_name"] == "row" and p["n_out"] == 8 and p["reduce_len"] == 768 * 1024
    # unit dims vanish
    assert plan(torch.float32, (1, 3072, 1, 2048), 4, strides=(1, 1, 3072, 3072))["kernel_name"] == "tiled"
    # every dim reduced, contiguous: the whole-array path
    assert plan(torch.float32, (100, 7, 3), (1, 2, 3))["kernel_name"] == "all"
    # kept dims split by a reduced dim: runs of outputs (middle dim)
    p = plan(torch.float32, (768, 1024, 8), 2)
    assert p["n_out"] == 768 * 8 and p["reduce_len"] == 1024


def test_vector_loads_need_alignment():
    import torch
    assert plan(torch.float32, (3072, 2048), 2)["vec"] == 4
    assert plan(torch.float32, (3072, 2048), 2, ptr=4)["vec"] == 1          # misaligned base
    assert plan(torch.float32, (3070, 2048), 2)["vec"] == 1                 # odd run / stride
    assert plan(torch.bfloat16, (3072, 2048), 2)["vec"] == 8


def test_workspace_sizes():
    rk = _rk()
    from reduction_primitives_amd.workloads import cm_strides
    assert rk.rk_workspace_size(rk.RK_F32, rk.RK_F32, 2, (3072, 2048), cm_strides((3072, 2048)), 2) == 0
    ws = rk.rk_workspace_size(rk.RK_F32, rk.RK_F32, 3, (64, 4096, 32), cm_strides((64, 4096, 32)), 2)
    p = plan(__import__("torch").float32, (64, 4096, 32), 2)
    assert ws == (p["split"] * 2048 * 4 + 255) // 256 * 256
    assert rk.rk_workspace_size(rk.RK_F32, rk.RK_F32, 1, (10**8,), (1,), 1) > 0
    # invalid layouts give 0
    assert rk.rk_workspace_size(rk.RK_F32, rk.RK_F32, 5, (1,) * 5, (1,) * 5, 1) == 0
    assert rk.rk_workspace_size(rk.RK_F32, rk.RK_F32, 2, (3, 4), (1, 3), 4) == 0


def test_plan_rejects_bad_layouts():
    rk = _rk()
    with pytest.raises(rk.RkError):
        rk.rk_plan_dims(rk.RK_F32, rk.RK_F32, 0, 0, (), (), 0)
    with pytest.raises(rk.RkError):
        rk.rk_plan_dims(rk.RK_F32, rk.RK_F32, 0, 2, (3, -1), (1, 3), 1)
    with pytest.raises(rk.RkError):
        rk.rk_plan_dims(rk.RK_F32, rk.RK_F32, 0, 2, (3, 4), (1, -3), 1)
    with pytest.raises(rk.RkError):
        rk.rk_plan_dims(rk.RK_F32, rk.RK_F32, 0, 2, (3, 4), (1, 3), 0b100)


def test_plan_rejects_views_beyond_62_bit_counts():
    """Extents, strides, element counts and byte spans at or above 2^62 are
    rejected before any product could overflow (the planner's 64-bit
    arithmetic, exercised at random under the sanitizers in
    tests/test_sanitizers.py); the largest views below the limit plan."""
    rk = _rk()
    big = 2**62
    bad = [((big,), (1,), 1), ((2**31, 2**31), (1, 2**31), 1), ((4, 5), (1, big // 2), 1),
           ((2**32, 2**30), (1, 2**32), 2), ((3, 4), (1, big), 1), ((2**60,), (1,), 1)]
    for shape, strides, mask in bad:
        with pytest.raises(rk.RkError):
            rk.rk_plan_dims(rk.RK_F32, rk.RK_F32, 0, len(shape), shape, strides, mask, 256)
        assert rk.rk_workspace_size(rk.RK_F32, rk.RK_F32, len(shape), shape, strides, mask) == 0
    with pytest.raises(rk.RkError):
        rk.rk_plan_all(rk.RK_F32, rk.RK_F32, 0, 2**60, 256)
    with pytest.raises(rk.RkError):
        rk.rk_plan_scan(rk.RK_F32, rk.RK_F32, rk.RK_F32, 0, 0, 2, (2**31, 2**31), (1, 2**31), 0, 256)
    # just below: 2^59 f32 elements (2^61 bytes) in one dim, and a broadcast dim
    assert rk.rk_plan_all(rk.RK_F32, rk.RK_F32, 0, 2**59, 256).grid == 1024
    assert rk.rk_plan_dims(rk.RK_F32, rk.RK_F32, 0, 2, (2**20, 2**30), (1, 0), 2, 256).n_out == 2**20


# -------------------------------------------------------------- validation

FAKE = 0x10000          # never dereferenced: every call below fails validation


@pytest.mark.parametrize("args,code", [
    (dict(op=3), 1), (dict(map_=3), 1), (dict(mode=3), 1), (dict(in_dtype=9), 1),
    (dict(acc=1), 2),                       # bf16 accumulator
    (dict(acc=4), 2),                       # integer accumulator for float input
    (dict(in_dtype=3, acc=0), 2),           # accumulator narrower than the input
    (dict(out=4), 2),                       # int output of a float reduction
    (dict(n=-1), 1), (dict(ptr=None), 1), (dict(ptr=FAKE + 2), 1), (dict(out_ptr=None), 1),
    (dict(ws=None), 1), (dict(ws=FAKE + 4), 1), (dict(out_ptr=FAKE), 1),
])
def test_reduce_all_validation(args, code):
    rk = _rk()
    rc = rk.rk_reduce_all(args.get("op", 0), args.get("map_", 0), args.get("in_dtype", 0),
                          args.get("acc", 0), args.get("out", 0), args.get("ptr", FAKE),
                          args.get("n", 100), None, args.get("mode", 0),
                          args.get("out_ptr", FAKE + 4096), args.get("ws", FAKE + 8192), None)
    assert rc == code


@pytest.mark.parametrize("args,code", [
    (dict(op=3), 1), (dict(map2=3), 1), (dict(mode=3), 1), (dict(in_dtype=9), 1),
    (dict(acc=4), 2), (dict(in_dtype=4, acc=0), 2),
    (dict(n=-1), 1), (dict(a=None), 1), (dict(b=None), 1), (dict(b=FAKE + 2), 1),
    (dict(out_ptr=None), 1), (dict(ws=None), 1), (dict(ws=FAKE + 4), 1),
    (dict(out_ptr=FAKE), 1), (dict(out_ptr=FAKE + 1024), 1),        # out aliases a or b
])
def test_reduce_all2_validation(args, code):
    rk = _rk()
    rc = rk.rk_reduce_all2(args.get("op", 0), args.get("map2", 0), args.get("in_dtype", 0),
                           args.get("acc", 0), args.get("out", 0), args.get("a", FAKE),
                           args.get("b", FAKE + 1024), args.get("n", 100), None, args.get("mode", 0),
                           args.get("out_ptr", FAKE + 4096), args.get("ws", FAKE + 8192), None)
    assert rc == code


@pytest.mark.parametrize("args,code", [
    (dict(ndim=0), 1), (dict(ndim=5), 1), (dict(mask=0b100), 1), (dict(shape=(3, -4)), 1),
    (dict(strides=(1, -3)), 1), (dict(mode=2), 1),          # host mode with 4 outputs
    (dict(ptr=FAKE + 1), 1), (dict(out_ptr=FAKE), 1), (dict(acc=5), 2),
])
def test_reduce_dims_validation(args, code):
    rk = _rk()
    ndim = args.get("ndim", 2)
    shape = args.get("shape", (3, 4))[:max(ndim, 0)] if ndim <= 2 else (1,) * ndim
    strides = args.get("strides", (1, 3))[:max(ndim, 0)] if ndim <= 2 else (1,) * ndim
    rc = rk.rk_reduce_dims(0, 0, 0, args.get("acc", 0), 0, args.get("ptr", FAKE), ndim, shape,
                           strides, args.get("mask", 0b10), None, args.get("mode", 0),
                           args.get("out_ptr", FAKE + 4096), FAKE + 8192, None)
    assert rc == code


def test_fused_finish_switch_changes_launch_count():
    rk = _rk()
    prev = rk.rk_debug_set_fused_finish(0)
    try:
        assert rk.rk_plan_all(rk.RK_F32, rk.RK_F32, 0, 10**8, 256).launches == 2
        assert plan(__import__("torch").float32, (64, 4096, 32), 2)["launches"] == 2
    finally:
        rk.rk_debug_set_fused_finish(prev)
    assert rk.rk_plan_all(rk.RK_F32, rk.RK_F32, 0, 10**8, 256).launches == (1 if prev else 2)


def test_launch_event_hook_pairs():
    rk = _rk()
    assert rk.rk_debug_set_launch_events(FAKE, None) == rk.RK_ERR_INVALID_ARGUMENT
    assert rk.rk_debug_set_launch_events(None, None) == rk.RK_OK


def test_stream_read_validation():
    rk = _rk()
    lib = rk.load()
    ok, bad = rk.RK_OK, rk.RK_ERR_INVALID_ARGUMENT
    assert lib.rk_debug_stream_read(FAKE, 0, 0, FAKE, None) == ok          # nothing to read: no launch
    assert lib.rk_debug_stream_read(FAKE, 8, 0, FAKE, None) == bad         # not whole vectors
    assert lib.rk_debug_stream_read(FAKE, -16, 0, FAKE, None) == bad
    assert lib.rk_debug_stream_read(FAKE, 16, -1, FAKE, None) == bad
    assert lib.rk_debug_stream_read(FAKE + 4, 16, 0, FAKE, None) == bad    # unaligned
    assert lib.rk_debug_stream_read(None, 16, 0, FAKE, None) == bad
    assert lib.rk_debug_stream_read(FAKE, 16, 0, None, None) == bad
    assert lib.rk_debug_device_info(None, None, None) == bad
    assert lib.rk_debug_set_finish_tag(None, 0xFFFFFFFF) == bad            # above the last tag


# ------------------------------------------------------------------- scans

def test_scan_plans():
    import reduction_primitives_amd as rk
    f32 = rk.RK_F32
    tile = 16 * 16 * 64 * 4                     # waves * chunks * lanes * floats per 16 bytes
    small = 4 * 8 * 64 * 4                      # 256-thread tiles: 4 waves of 8 chunks
    p = rk.rk_plan_scan(f32, f32, f32, 0, 0, 1, [10**8], [1], 0, 256)
    assert p.kernel == rk.RK_KERNEL_SCAN_TILE and p.tile_outputs == tile and p.vec == 4
    assert p.split == (10**8 + tile - 1) // tile and p.grid == p.split
    assert p.launches == 1                      # tile state in a library slot: no clearing launch
    prev = rk.rk_debug_set_fused_finish(0)
    try:
        assert rk.rk_plan_scan(f32, f32, f32, 0, 0, 1, [10**8], [1], 0, 256).launches == 2
    finally:
        rk.rk_debug_set_fused_finish(prev)
    assert rk.rk_plan_scan(f32, f32, f32, 0, 0, 1, [4096 * tile], [1], 0, 256).launches == 1
    big = rk.rk_plan_scan(f32, f32, f32, 0, 0, 1, [4097 * tile], [1], 0, 256)
    assert big.split == 4097 and big.launches == 2      # more tiles than a slot holds
    # workspace: 256-byte header, then 32-byte records, four to a line
    tiles = p.split
    assert p.workspace_bytes == -(-(256 + -(-tiles // 4) * 128) // 256) * 256
    p = rk.rk_plan_scan(f32, f32, f32, 4, 0, 1, [10**8], [1], 0, 256)                # unaligned input
    assert p.vec == 1 and p.block == 256
    # outputs wider than the inputs: lanes take as many elements as make 16 bytes of output
    i32, i64, f64, bf16 = rk.RK_I32, rk.RK_I64, rk.RK_F64, rk.RK_BF16
    assert rk.rk_plan_scan(i32, i64, i64, 0, 0, 1, [10**6], [1], 0, 256).vec == 2
    assert rk.rk_plan_scan(i32, i64, i64, 8, 0, 1, [10**6], [1], 0, 256).vec == 2      # 8-byte loads
    assert rk.rk_plan_scan(i32, i64, i64, 4, 0, 1, [10**6], [1], 0, 256).vec == 1
    assert rk.rk_plan_scan(i32, i64, i32, 0, 0, 1, [10**6], [1], 0, 256).vec == 4      # narrow output
    assert rk.rk_plan_scan(f32, f64, f64, 0, 0, 1, [10**6], [1], 0, 256).vec == 2
    assert rk.rk_plan_scan(bf16, f32, f32, 0, 0, 1, [10**6], [1], 0, 256).vec == 4
    assert rk.rk_plan_scan(bf16, f32, bf16, 0, 0, 1, [10**6], [1], 0, 256).vec == 8
    assert rk.rk_plan_scan(f32, f32, rk.RK_BF16, 0, 2, 1, [10**6], [1], 0, 256).vec == 1   # 2-byte aligned out
    assert rk.rk_plan_scan(f32, f32, rk.RK_BF16, 0, 8, 1, [10**6], [1], 0, 256).vec == 4
    # large tiles: 16 chunks of the input's 16-byte vector per lane, counted in
    # loads of `vec` elements and at most 32 of them (64 had gone to scratch)
    n = 4 * 10**7
    for tin, tacc, vec, lane_elems in ((bf16, f32, 4, 128), (bf16, f64, 2, 64), (i32, i64, 2, 64), (f32, f32, 4, 64)):
        p = rk.rk_plan_scan(tin, tacc, tacc, 0, 0, 1, [n], [1], 0, 256)
        assert p.block == 1024 and p.vec == vec and p.tile_outputs == 1024 * lane_elems, (tin, tacc)
    p = rk.rk_plan_scan(f32, f32, f32, 0, 0, 1, [4000], [1], 0, 256)
    assert p.kernel == rk.RK_KERNEL_SCAN_ROWWAVE and p.workspace_bytes == 0 and p.block == 256
    p = rk.rk_plan_scan(f32, f32, f32, 0, 0, 1, [5000], [1], 0, 256)       # one short line: tiles
    assert p.kernel == rk.RK_KERNEL_SCAN_TILE and p.block == 256 and p.split == 1
    # fewer large tiles than CUs: quarter-size tiles of 256-thread blocks
    p = rk.rk_plan_scan(f32, f32, f32, 0, 0, 1, [10**6], [1], 0, 256)
    assert p.block == 256 and p.tile_outputs == small and p.split == -(-10**6 // small)
    assert rk.rk_plan_scan(f32, f32, f32, 0, 0, 1, [10**8], [1], 0, 256).block == 1024
    # 8192 x 8192 along dims=1 (8192 contiguous lines: a wave each) and dims=2 (strided)
    p = rk.rk_plan_scan(f32, f32, f32, 0, 0, 2, [8192, 8192], [1, 8192], 0, 256)
    assert p.kernel == rk.RK_KERNEL_SCAN_ROWWAVE and p.n_out == 8192 * 8192
    p = rk.rk_plan_scan(f32, f32, f32, 0, 0, 2, [tile, 8], [1, tile], 0, 256)
    assert p.kernel == rk.RK_KERNEL_SCAN_TILE and p.split == tile // small and p.grid == 8 * (tile // small)
    p = rk.rk_plan_scan(f32, f32, f32, 0, 0, 2, [tile, 300], [1, tile], 0, 256)
    assert p.kernel == rk.RK_KERNEL_SCAN_TILE and p.split == 1 and p.grid == 300 and p.block == 1024
    p = rk.rk_plan_scan(f32, f32, f32, 0, 0, 2, [8192, 8192], [1, 8192], 1, 256)
    assert p.kernel == rk.RK_KERNEL_SCAN_COLUMNS and p.vec == 4 and p.launches == 1
    assert p.tile_outputs == 128 * 256 and p.split == 32 and p.grid == 64 * 32 and p.block == 512
    # the workspace covers both tile geometries: 16-byte loads (128 lines x 256
    # positions) and element loads (64 lines x 128 positions)
    # (256-byte header, flags 32 to a line, then 16 bytes per line of a tile)
    scalar_tiles = 128 * 64
    assert p.workspace_bytes == -(-(256 + -(-scalar_tiles // 32) * 128 + scalar_tiles * 64 * 16) // 256) * 256
    assert rk.rk_plan_scan(f32, f32, f32, 4, 0, 2, [8192, 8192], [1, 8192], 1, 256).vec == 1
    p = rk.rk_plan_scan(f32, f32, f32, 0, 0, 2, [10, 100], [1, 10], 1, 256)
    assert p.kernel == rk.RK_KERNEL_SCAN_LINES and p.workspace_bytes == 0        # runs of 10 lines
    p = rk.rk_plan_scan(f32, f32, f32, 0, 0, 2, [50, 300], [1, 50], 0, 256)
    assert p.kernel == rk.RK_KERNEL_SCAN_LINES                      # lines shorter than a wave's chunk
    p = rk.rk_plan_scan(f32, f32, f32, 0, 0, 2, [255, 300], [1, 255], 0, 256)
    assert p.kernel == rk.RK_KERNEL_SCAN_LINES                      # packed, four elements to a lane
    p = rk.rk_plan_scan(f32, f32, f32, 0, 0, 2, [256, 300], [1, 256], 0, 256)
    assert p.kernel == rk.RK_KERNEL_SCAN_ROWWAVE                    # four wave chunks and longer
    # input and output contiguous along different axes: the transposing tiles.
    # A row-major 512 x 3000 matrix along its rows (tiles of 256 lines x 64
    # positions), along its columns (256 lines x 32), and a permuted view
    # whose kept dims are contiguous in input and output apart (32 x 32 lines
    # x 16 positions); 8-byte accumulators halve the positions.  The state
    # holds 16 bytes per line of a tile, as the columns kernel's.
    p = rk.rk_plan_scan(f32, f32, f32, 0, 0, 2, [512, 3000], [3000, 1], 1, 256)
    assert p.kernel == rk.RK_KERNEL_SCAN_TRANSPOSE and p.block == 256 and p.vec == 1
    assert p.split == -(-3000 // 64) and p.grid == 2 * p.split and p.tile_outputs == 256 * 64
    assert p.workspace_bytes == -(-(256 + -(-p.grid // 32) * 128 + p.grid * 256 * 16) // 256) * 256
    p = rk.rk_plan_scan(i32, i64, i64, 0, 0, 2, [512, 3000], [3000, 1], 1, 256)
    assert p.kernel == rk.RK_KERNEL_SCAN_TRANSPOSE and p.split == -(-3000 // 32) and p.tile_outputs == 256 * 32
    p = rk.rk_plan_scan(f32, f32, f32, 0, 0, 2, [512, 3000], [3000, 1], 0, 256)
    assert p.kernel == rk.RK_KERNEL_SCAN_TRANSPOSE and p.split == 16 and p.grid == 16 * -(-3000 // 256)
    p = rk.rk_plan_scan(f32, f32, f32, 0, 0, 3, [64, 3000, 40], [40, 2560, 1], 1, 256)
    assert p.kernel == rk.RK_KERNEL_SCAN_TRANSPOSE and p.split == -(-3000 // 16) and p.grid == 4 * p.split
    assert p.tile_outputs == 32 * 32 * 16 and p.launches == 1
    # too few lines for such tiles, the scan dim contiguous in the input: the
    # tile kernel along each line (outputs stored one by one), 256-thread
    # tiles while the large ones number fewer than the CUs
    p = rk.rk_plan_scan(f32, f32, f32, 0, 0, 2, [8, 10**6], [10**6, 1], 1, 256)
    assert p.kernel == rk.RK_KERNEL_SCAN_TILE and p.block == 256 and p.vec == 4 and p.split == -(-10**6 // small)
    assert rk.rk_plan_scan(f32, f32, f32, 0, 0, 2, [5, 10001], [10001, 1], 1, 256).vec == 1
    assert rk.rk_plan_scan(f32, f32, f32, 0, 0, 2, [40, 500000], [500000, 1], 1, 256).block == 1024
    # bf16 into f64: 256-thread tiles (eight f64 a lane in the large ones went to scratch memory)
    assert rk.rk_plan_scan(bf16, f64, f64, 0, 0, 2, [40, 500000], [500000, 1], 1, 256).block == 256
    assert rk.rk_plan_scan(f32, f32, f32, 0, 0, 2, [63, 500000], [500000, 1], 1, 256).kernel == rk.RK_KERNEL_SCAN_TILE
    assert rk.rk_plan_scan(f32, f32, f32, 0, 0, 2, [64, 500000], [500000, 1], 1, 256).kernel == rk.RK_KERNEL_SCAN_TRANSPOSE
    # the mirror, the scan dim contiguous in the output only: element loads
    # s_in apart, 256-thread tiles; the transposing tiles from 64 lines
    p = rk.rk_plan_scan(f32, f32, f32, 0, 0, 2, [10**6, 8], [8, 1], 0, 256)
    assert p.kernel == rk.RK_KERNEL_SCAN_TILE and p.block == 256 and p.vec == 1 and p.split == -(-10**6 // small)
    assert rk.rk_plan_scan(f32, f32, f32, 0, 0, 2, [500000, 63], [63, 1], 0, 256).kernel == rk.RK_KERNEL_SCAN_TILE
    assert rk.rk_plan_scan(f32, f32, f32, 0, 0, 2, [500000, 64], [64, 1], 0, 256).kernel == rk.RK_KERNEL_SCAN_TRANSPOSE
    # shorter than a wave's chunk, or too short a contiguous run: a thread per line
    assert rk.rk_plan_scan(f32, f32, f32, 0, 0, 2, [10, 200], [200, 1], 1, 256).kernel == rk.RK_KERNEL_SCAN_LINES
    assert rk.rk_plan_scan(f32, f32, f32, 0, 0, 2, [300, 10], [10, 1], 1, 256).kernel == rk.RK_KERNEL_SCAN_LINES
    p = rk.rk_plan_scan(f32, f32, f32, 0, 0, 3, [0, 5, 5], [1, 1, 5], 1, 256)
    assert p.kernel == rk.RK_KERNEL_NONE and p.launches == 0
    with pytest.raises(rk.RkError):
        rk.rk_plan_scan(f32, f32, f32, 0, 0, 2, [3, 4], [1, 3], 2, 256)


@pytest.mark.parametrize("args,code", [
    (dict(op=3), 1), (dict(in_dtype=9), 1), (dict(acc=4), 2), (dict(out=4), 2),
    (dict(dim=1), 1), (dict(dim=-1), 1), (dict(ndim=0), 1), (dict(inclusive=2), 1),
    (dict(ptr=None), 1), (dict(ptr=FAKE + 2), 1), (dict(out_ptr=None), 1), (dict(out_ptr=FAKE + 2), 1),
    (dict(out_ptr=FAKE + 4), 1),                # overlaps the input without being it
    (dict(ws=None), 1), (dict(ws=FAKE + 4), 1),
])
def test_scan_validation(args, code):
    rk = _rk()
    n = 10**6                                   # takes the tile kernel, so it needs a workspace
    rc = rk.rk_scan_dims(args.get("op", 0), args.get("in_dtype", 0), args.get("acc", 0), args.get("out", 0),
                         args.get("ptr", FAKE), args.get("ndim", 1), [n], [1], args.get("dim", 0), None,
                         args.get("inclusive", 1), args.get("out_ptr", FAKE + 8 * n),
                         args.get("ws", FAKE + 16 * n), None)
    assert rc == code
