"""GPU parity of the two-input whole-array path (rk_reduce_all2) against the
CPU oracle.

The source is f(a_i, b_i) for two arrays of one dtype -- the broadcast that
AcceleratedKernels.jl PR #139 ("What changes", and the fused sources of its
test list under "Compatibility") lets the whole-array path take.  Covered:
one tile, one pass and two passes; both 16-byte and element loads (inputs at
the same or at different offsets from a 16-byte boundary); every op, map and
dtype combination; init, fold, overwrite and host; exact closed forms; both
finishing paths.

Bar: as for one input (tests/parity.py).  One reading differs: the oracle
evaluates a floating map in double, the kernel in the accumulator type.  For
mul and absdiff of f32, bf16 or f16 inputs with an f32 accumulator both give
the same rounded value (the exact product or difference fits a double), so
max/min stay bit-exact; for sqdiff the kernel rounds a - b before squaring,
so max/min of sqdiff with an f32 accumulator are held to 3 * 2^-24 relative.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
from reduction_primitives_amd import workloads as W
from tests.parity import check, code_of, raw_np, tolerance

pytestmark = pytest.mark.gpu

DEV = "cuda"
MAP2 = {"mul": O.MUL, "sqdiff": O.SQDIFF, "absdiff": O.ABSDIFF}
OPS = {"sum": O.SUM, "max": O.MAX, "min": O.MIN}


def _rk():
    import reduction_primitives_amd as rk
    rk.load()
    return rk


def magnitude2(map2, in_c, a_raw, b_raw, start):
    """S = |s| + sum |f(a, b)| in float64 (a scale for the tolerance only)."""
    a = O.widen(in_c, a_raw) if O.is_fp(in_c) else a_raw.astype(np.float64)
    b = O.widen(in_c, b_raw) if O.is_fp(in_c) else b_raw.astype(np.float64)
    f = {O.MUL: a * b, O.SQDIFF: (a - b) ** 2, O.ABSDIFF: np.abs(a - b)}[map2]
    return abs(float(start)) + float(np.abs(f).sum())


def run2(a_cpu, b_cpu, map2="mul", op="sum", acc=None, out_dtype=None, mode="overwrite", init=None,
         off_a=0, off_b=0, n=None, what=""):
    """Reduce f(a[off_a:off_a+n], b[off_b:off_b+n]) on the GPU and check it."""
    rk = _rk()
    op_c, map_c, mode_c = OPS[op], MAP2[map2], rk.MODES[mode]
    in_c = code_of(a_cpu.dtype)
    acc_c = rk.default_acc(in_c) if acc is None else code_of(acc)
    out_c = (acc_c if not O.is_fp(in_c) else in_c) if out_dtype is None else code_of(out_dtype)
    if n is None:
        n = min(a_cpu.numel() - off_a, b_cpu.numel() - off_b)
    ad, bd = a_cpu.to(DEV), b_cpu.to(DEV)
    av, bv = ad[off_a:off_a + n], bd[off_b:off_b + n]
    ar, br = raw_np(a_cpu)[off_a:off_a + n], raw_np(b_cpu)[off_b:off_b + n]
    prev, out = None, None
    if mode == "fold":
        out = rk.reduce_all2(av, bv, map2, op=op, acc=acc_c, out_dtype=out_c, init=init)
        torch.cuda.synchronize()
        prev = raw_np(out)
    res = rk.reduce_all2(av, bv, map2, op=op, acc=acc_c, out_dtype=out_c, init=init, mode=mode, out=out)
    torch.cuda.synchronize()
    gpu_raw = O.cast(out_c, [res]) if mode == "host" else raw_np(res)
    R, _ = O.expected_all2(op_c, map_c, in_c, acc_c, out_c, ar, br, mode_c, init, prev)
    start = O.start_value(op_c, acc_c, out_c, mode_c, init, prev)
    if mode == "fold":
        start = start[0]
    what = what or f"{op}/{map2}/{mode} n={n} offs=({off_a},{off_b})"
    if O.is_fp(in_c):
        S = magnitude2(map_c, in_c, ar, br, start if op_c == O.SUM else 0.0)
    else:
        S = None
    if op_c != O.SUM and map_c == O.SQDIFF and acc_c == O.F32:
        # the kernel's f32 value, then the output's own rounding
        g = float(O.widen(out_c, np.asarray(gpu_raw).reshape(-1))[0])
        tol = 3 * 2.0**-24 * abs(R) + float(tolerance(out_c, [R], [0.0])[0])
        assert abs(g - R) <= tol or g == R, f"{what}: gpu {g!r} oracle {R!r}"
    else:
        check(op_c, out_c, gpu_raw, [R], S, what)
    return res


# ------------------------------------------------------------ configurations

@pytest.mark.parametrize("n", [10**6, 10**8])
def test_vector_pair_config(n):
    """Dot product, squared and absolute distance of two N(0,1) float32
    vectors, on the device with init and fold, and to the host."""
    a, b = W.vector_pair(n)
    for m in ("mul", "sqdiff", "absdiff"):
        run2(a.data, b.data, m, init=0.5)
    run2(a.data, b.data, "mul", mode="host")
    run2(a.data, b.data, "mul", mode="fold", init=-2.0)
    run2(a.data, b.data, "absdiff", op="max")


# ----------------------------------------------------------------- geometry

def _boundary_sizes():
    tile = 256 * 8 * 4
    g = 4 * 256
    return [0, 1, 3, 4, 5, 63, 64, 65, tile - 1, tile, tile + 1, 2 * tile, 2 * tile + 1,
            3 * tile + 7, g * tile - 1, g * tile, g * tile + 1]


@pytest.mark.parametrize("n", _boundary_sizes())
def test_one_tile_one_pass_two_passes(n):
    a = W.uniform(n + 3, -1.0, 1.0, 7500 + n % 997)
    b = W.uniform(n + 3, -1.0, 1.0, 7600 + n % 991)
    run2(a, b, "mul", init=0.25, n=n)
    run2(a, b, "sqdiff", mode="host", n=n)
    run2(a, b, "mul", off_a=1, off_b=2, n=n)            # element loads
    ai = W.randint(n, -1000, 1000, 7700 + n % 983)
    bi = W.randint(n, -1000, 1000, 7800 + n % 977)
    run2(ai, bi, "mul", acc=torch.int64, out_dtype=torch.int64)
    run2(ai, bi, "absdiff", op="max", acc=torch.int32, out_dtype=torch.int32)


@pytest.mark.parametrize("offs", [(0, 0), (1, 1), (3, 3), (0, 1), (1, 0), (2, 3), (3, 1), (5, 1)])
def test_offsets(offs):
    """Equal offsets take 16-byte loads after a common head; unequal ones
    16-byte loads of x and of y's aligned chunks, shifted into place (element
    loads only when too short).  Checked against the plan and the oracle."""
    rk = _rk()
    oa, ob = offs
    for n in (5, 1000, 123457, 3 * 10**6 + 1):
        a = W.uniform(n + 8, -1.0, 1.0, 7900 + oa)
        b = W.uniform(n + 8, -1.0, 1.0, 7910 + ob)
        ad, bd = a.to(DEV), b.to(DEV)
        plan = rk.rk_plan_all2(rk.RK_F32, rk.RK_F32, ad[oa:].data_ptr(), bd[ob:].data_ptr(), n)
        assert plan.vec == (4 if (oa - ob) % 4 == 0 or n > 5 else 1)
        run2(a, b, "mul", init=0.5, off_a=oa, off_b=ob, n=n)
        run2(a, b, "absdiff", op="min", off_a=oa, off_b=ob, n=n)
        hb = W.normal(n + 8, 7920 + oa, torch.bfloat16)
        run2(hb, hb, "sqdiff", out_dtype=torch.float32, off_a=oa, off_b=ob, n=n)


@pytest.mark.parametrize("dt", [torch.float64, torch.float16, torch.bfloat16, torch.int32, torch.int64],
                         ids=lambda t: str(t).split(".")[1])
@pytest.mark.parametrize("offs", [(0, 1), (1, 0), (1, 2), (0, 3), (3, 0), (2, 7)])
def test_shifted_pairs_every_dtype(dt, offs):
    """Inputs at different 16-byte phases for every input width: y's chunks
    shifted by whole words (4- and 8-byte types) or by half words (2-byte
    types); around tile boundaries and the grid's last tile."""
    oa, ob = offs
    tile = 256 * 8 * (16 // torch.empty(0, dtype=dt).element_size())
    for n in (17, tile - 1, 3 * tile + 7, 123457):
        if dt.is_floating_point:
            a, b = W.normal(n + 8, 8100 + oa, dt), W.normal(n + 8, 8110 + ob, dt)
            acc = torch.float64 if dt == torch.float64 else torch.float32
            run2(a, b, "mul", acc=acc, out_dtype=acc, init=0.5, off_a=oa, off_b=ob, n=n)
            run2(a, b, "absdiff", op="max", acc=acc, out_dtype=acc, off_a=oa, off_b=ob, n=n)
        else:
            a, b = W.randint(n + 8, -1000, 1000, 8120 + oa, dt), W.randint(n + 8, -1000, 1000, 8130 + ob, dt)
            run2(a, b, "mul", acc=torch.int64, out_dtype=torch.int64, off_a=oa, off_b=ob, n=n)
            run2(a, b, "sqdiff", op="min", acc=torch.int64, out_dtype=torch.int64, off_a=oa, off_b=ob, n=n)


# ------------------------------------------------------------- dtype matrix

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
def test_dtype_op_map_matrix(combo, op):
    in_t, acc_t, out_t = combo
    n = 123457
    if in_t.is_floating_point:
        a = W.normal(n, 8000, in_t)
        b = W.normal(n, 8001, in_t)
        if out_t == torch.float16:
            # N(0, 1/16) inputs: sum (a-b)^2 ~ 1.5e4 and sum |a-b| ~ 3.5e4 over
            # 123,457 pairs stay below float16's 65,504, so the sums compare
            # finite values (scaling by 1/4 is exact)
            a, b = a * 0.25, b * 0.25
    else:
        a = W.randint(n, -50000, 50000, 8002, in_t)     # products overflow int32
        b = W.randint(n, -50000, 50000, 8003, in_t)
    for m in ("mul", "sqdiff", "absdiff"):
        run2(a, b, m, op=op, acc=acc_t, out_dtype=out_t, init=None if op != "sum" else 1)
        run2(a, b, m, op=op, acc=acc_t, out_dtype=out_t, mode="host")


# ------------------------------------------------------------ exact results

def test_closed_forms_on_gpu():
    rk = _rk()
    n = 10**6
    i = torch.arange(1, n + 1, dtype=torch.int32, device=DEV)
    j = torch.arange(2, n + 2, dtype=torch.int32, device=DEV)
    dot = rk.reduce_all2(i, i, "mul", acc=torch.int64, out_dtype=torch.int64)
    assert int(dot.item()) == n * (n + 1) * (2 * n + 1) // 6
    assert int(rk.reduce_all2(i, j, "sqdiff", acc=torch.int64, out_dtype=torch.int64).item()) == n
    assert rk.reduce_all2(j, i, "absdiff", acc=torch.int64, out_dtype=torch.int64, mode="host",
                          init=7) == n + 7
    p = W.randperm(n, 8100).to(DEV)
    ones = torch.ones(n, dtype=torch.int32, device=DEV)
    assert int(rk.reduce_all2(p, ones, "mul", op="max", acc=torch.int32, out_dtype=torch.int32).item()) == n - 1
    assert int(rk.reduce_all2(p, ones, "mul", op="min", acc=torch.int32, out_dtype=torch.int32).item()) == 0
    # the same array as both inputs: sum of squares, equal to the one-input map
    x = W.small_ints(n, -100, 100, 8101).to(DEV)
    assert float(rk.reduce_all2(x, x, "mul").item()) == float(rk.reduce_all(x, map="square").item())
    # int32 accumulator wraps: 65536 * 65536 = 2^32 -> 0
    w = torch.tensor([65536, 3], dtype=torch.int32, device=DEV)
    assert int(rk.reduce_all2(w, w, "mul", acc=torch.int32, out_dtype=torch.int32).item()) == 9


def test_one_launch_and_two_launch_finish_agree():
    rk = _rk()
    a, b = W.vector_pair(10**6)
    ad, bd = a.data.to(DEV), b.data.to(DEV)
    res = {}
    for on in (1, 0):
        prev = rk.rk_debug_set_fused_finish(on)
        try:
            res[on] = [raw_np(rk.reduce_all2(ad, bd, m)) for m in ("mul", "sqdiff", "absdiff")]
            res[on].append(raw_np(rk.reduce_all2(ad[1:-1], bd[2:], "mul")))
            torch.cuda.synchronize()
        finally:
            rk.rk_debug_set_fused_finish(prev)
    for x, y in zip(res[1], res[0]):
        assert np.array_equal(x, y)


def test_repeated_calls_are_deterministic():
    rk = _rk()
    a, b = W.vector_pair(10**6)
    ad, bd = a.data.to(DEV), b.data.to(DEV)
    outs = torch.empty(50, device=DEV)
    for k in range(50):
        rk.reduce_all2(ad, bd, "mul", out=outs[k:k + 1])
    torch.cuda.synchronize()
    assert torch.unique(outs).numel() == 1


def test_invalid_arguments_are_rejected():
    rk = _rk()
    a = torch.ones(100, device=DEV)
    b = torch.ones(100, device=DEV)
    out = torch.zeros(1, device=DEV)
    ws = rk.workspace_for(rk.rk_workspace_size(rk.RK_F32, rk.RK_F32, 1, [100], [1], 1), DEV)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    call = lambda **kw: rk.rk_reduce_all2(  # noqa: E731
        kw.get("op", 0), kw.get("map2", 0), kw.get("in_", rk.RK_F32), kw.get("acc", rk.RK_F32),
        kw.get("outd", rk.RK_F32), kw.get("a", a.data_ptr()), kw.get("b", b.data_ptr()), kw.get("n", 100),
        None, kw.get("mode", 0), kw.get("out", out.data_ptr()), ws.data_ptr(), st)
    assert call() == rk.RK_OK
    assert call(map2=3) == rk.RK_ERR_INVALID_ARGUMENT
    assert call(op=5) == rk.RK_ERR_INVALID_ARGUMENT
    assert call(n=-1) == rk.RK_ERR_INVALID_ARGUMENT
    assert call(b=0) == rk.RK_ERR_INVALID_ARGUMENT
    assert call(b=b.data_ptr() + 2) == rk.RK_ERR_INVALID_ARGUMENT      # not element aligned
    assert call(out=a.data_ptr()) == rk.RK_ERR_INVALID_ARGUMENT        # out aliases an input
    assert call(out=b.data_ptr()) == rk.RK_ERR_INVALID_ARGUMENT
    assert call(acc=rk.RK_I32) == rk.RK_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert float(out.item()) == 100.0


def test_beyond_2_31_elements():
    """Two inputs of more than 2^31 elements (2 x 8.6 GB of int32 ones):
    64-bit indexing on both load paths; the totals are closed forms."""
    rk = _rk()
    n = 2**31 + 5
    ones = torch.ones(n + 1, dtype=torch.int32, device=DEV)
    assert int(rk.reduce_all2(ones[:n], ones[1:], "mul", acc=torch.int64, out_dtype=torch.int64).item()) == n
    twos = torch.full((n,), 2, dtype=torch.int32, device=DEV)
    assert int(rk.reduce_all2(ones[:n], twos, "absdiff", acc=torch.int64, out_dtype=torch.int64).item()) == n
    del ones, twos
    torch.cuda.empty_cache()


# ------------------------------------------------------------ seeded sweep
# Pairs drawn from one seed per case: an input type, each input at its own
# offset of 0-7 elements (so every pair of 16-byte phases occurs), a length
# log-uniform up to 2 million, a map, an op and a finishing mode.

SWEEP2_TYPES = [  # (input, accumulator and output)
    (torch.float32, torch.float32), (torch.bfloat16, torch.float32), (torch.float16, torch.float32),
    (torch.float64, torch.float64), (torch.int32, torch.int64), (torch.int64, torch.int64),
]


@pytest.mark.parametrize("case", range(64))
def test_seeded_pair_sweep(case):
    rng = np.random.default_rng(40_000 + case)
    in_t, acc_t = SWEEP2_TYPES[int(rng.integers(0, len(SWEEP2_TYPES)))]
    oa, ob = int(rng.integers(0, 8)), int(rng.integers(0, 8))
    n = int(round(np.exp(rng.uniform(0, np.log(2e6)))))
    m = ["mul", "sqdiff", "absdiff"][int(rng.integers(0, 3))]
    op = ["sum", "max", "min"][int(rng.integers(0, 3))]
    mode = ["overwrite", "fold", "host"][int(rng.integers(0, 3))]
    if in_t.is_floating_point:
        a, b = W.normal(n + 8, 41_000 + case, in_t), W.normal(n + 8, 42_000 + case, in_t)
    else:
        a = W.randint(n + 8, -1000, 1000, 41_000 + case, in_t)
        b = W.randint(n + 8, -1000, 1000, 42_000 + case, in_t)
    run2(a, b, m, op=op, acc=acc_t, out_dtype=acc_t, mode=mode, init=0.5 if op == "sum" and in_t.is_floating_point
         else None, off_a=oa, off_b=ob, n=n,
         what=f"pair sweep case {case}: {in_t} {op}/{m}/{mode} n={n} offs=({oa},{ob})")
