"""GPU parity of the whole-array path (rk_reduce_all) against the CPU oracle.

Covers the categories AcceleratedKernels.jl PR #139 lists for single-output
reductions (section "Compatibility", last paragraph): one tile, one pass and
two passes; init, fold and overwrite; an accumulator wider than the output
whose partials do not fit it; workspace reuse; offset views; mapped sources.
Inputs are the seeded workloads of the pages' benchmark table ("Numbers":
Float32 sums of 10^4, 10^6 and 10^8 elements).
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
from reduction_primitives_amd import workloads as W
from tests import assoc, golden_cases
from tests.parity import check, code_of, magnitude, raw_np

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _rk():
    import reduction_primitives_amd as rk
    rk.load()
    return rk


def run_and_check(x_cpu, op="sum", map_="identity", acc=None, out_dtype=None, mode="overwrite",
                  init=None, offset=0, what="", allow_inf=False):
    """Reduce x_cpu[offset:] on the GPU and compare with the oracle."""
    rk = _rk()
    op_c, map_c, mode_c = rk.OPS[op], rk.MAPS[map_], rk.MODES[mode]
    in_c = code_of(x_cpu.dtype)
    acc_c = rk.default_acc(in_c) if acc is None else code_of(acc)
    out_c = (acc_c if not O.is_fp(in_c) else in_c) if out_dtype is None else code_of(out_dtype)
    xd = x_cpu.to(DEV)
    view = xd[offset:]
    xr = raw_np(x_cpu)[offset:]
    prev = None
    out = None
    if mode == "fold":
        # the output's previous value: an overwrite with init first
        out = rk.reduce_all(view, op=op, map=map_, acc=acc_c, out_dtype=out_c, init=init,
                            mode="overwrite")
        torch.cuda.synchronize()
        prev = raw_np(out)
    res = rk.reduce_all(view, op=op, map=map_, acc=acc_c, out_dtype=out_c, init=init, mode=mode,
                        out=out)
    torch.cuda.synchronize()
    if mode == "host":
        gpu_raw = O.cast(out_c, [res]) if not O.is_fp(out_c) else None
        if O.is_fp(out_c):
            gpu_raw = O.cast(out_c, [res])      # host value is exactly representable
    else:
        gpu_raw = raw_np(res)
    R, _ = O.expected_all(op_c, map_c, in_c, acc_c, out_c, xr, mode_c, init, prev)
    start = O.start_value(op_c, acc_c, out_c, mode_c, init, prev)
    if mode == "fold":
        start = start[0]
    S = magnitude(map_c, in_c, acc_c, xr, start if op_c == O.SUM else 0.0)
    check(op_c, out_c, gpu_raw, [R], S, what or f"{op}/{map_}/{mode} n={view.numel()}", allow_inf=allow_inf)
    return res


# ------------------------------------------------------------ configurations

def test_whole_small_config():
    """10^4 float32 U[-1,1) to the host; the same draw as int32 summed into int64."""
    xf, xi = W.whole_small()
    run_and_check(xf.data, mode="host", init=0.0)
    run_and_check(xi.data, acc=torch.int64, out_dtype=torch.int64, mode="host")


@pytest.mark.parametrize("n", [10**6, 10**8])
def test_whole_large_config(n):
    """10^6 / 10^8 float32 U[0,1): host; device with init 1.5, overwrite then
    fold; max and min of a permutation of 0..n-1 (int32, bit-exact)."""
    xf, perm = W.whole_large(n)
    run_and_check(xf.data, mode="host")
    run_and_check(xf.data, mode="overwrite", init=1.5)
    run_and_check(xf.data, mode="fold", init=1.5)
    rk = _rk()
    pd = perm.data.to(DEV)
    mx = rk.reduce_all(pd, op="max", acc=torch.int32, out_dtype=torch.int32)
    mn = rk.reduce_all(pd, op="min", acc=torch.int32, out_dtype=torch.int32)
    assert int(mx.item()) == n - 1 and int(mn.item()) == 0
    run_and_check(perm.data, op="max", acc=torch.int32, out_dtype=torch.int32)
    run_and_check(perm.data, op="min", acc=torch.int32, out_dtype=torch.int32, mode="host")


# ----------------------------------------------------------------- geometry

def _plan(n, dtype=torch.float32, ptr=0):
    rk = _rk()
    return rk.rk_plan_all(rk.dtype_code(dtype), rk.default_acc(rk.dtype_code(dtype)), ptr, n)


def _boundary_sizes():
    tile = 256 * 8 * 4           # block * unroll * float32 per 16 bytes (checked below)
    g = 4 * 256
    return [0, 1, 3, 4, 5, 63, 64, 65, tile - 1, tile, tile + 1, 2 * tile, 2 * tile + 1,
            3 * tile + 7, g * tile - 1, g * tile, g * tile + 1, 10**4 + 3]


def test_tile_constant_matches_plan():
    tile = 256 * 8 * 4
    assert _plan(2 * tile).grid == 1 and _plan(2 * tile).launches == 1
    assert _plan(2 * tile + 4).grid > 1


@pytest.mark.parametrize("n", _boundary_sizes())
def test_one_tile_one_pass_two_passes(n):
    x = W.uniform(n, -1.0, 1.0, 7000 + n % 997)
    for mode in ("overwrite", "host"):
        run_and_check(x, mode=mode, init=0.25)
    xi = W.randint(n, -1000, 1000, 7100 + n % 991)
    run_and_check(xi, acc=torch.int64, out_dtype=torch.int64)
    run_and_check(xi, op="max", acc=torch.int32, out_dtype=torch.int32)


@pytest.mark.parametrize("offset", range(1, 8))
def test_offset_views(offset):
    for n in (5, 1000, 123457):
        x = W.uniform(n + offset, -1.0, 1.0, 7200 + offset)
        run_and_check(x, offset=offset, init=0.5)
        xb = W.normal(n + offset, 7300 + offset, torch.bfloat16)
        run_and_check(xb, offset=offset, out_dtype=torch.float32)
        xi = W.randint(n + offset, -10**6, 10**6, 7400 + offset)
        run_and_check(xi, offset=offset, acc=torch.int64, out_dtype=torch.int64, mode="host")


# ------------------------------------------------------------- dtype matrix

COMBOS = [  # (input, accumulator, output)
    (torch.float32, torch.float32, torch.float32),
    (torch.float32, torch.float64, torch.float64),
    (torch.float32, torch.float32, torch.bfloat16),
    (torch.bfloat16, torch.float32, torch.bfloat16),
    (torch.bfloat16, torch.float32, torch.float32),
    (torch.float16, torch.float32, torch.float16),
    (torch.float16, torch.float64, torch.float32),
    (torch.float64, torch.float64, torch.float64),
    (torch.float64, torch.float64, torch.float32),
    (torch.int32, torch.int32, torch.int32),
    (torch.int32, torch.int64, torch.int64),
    (torch.int32, torch.int64, torch.int32),
    (torch.int64, torch.int64, torch.int64),
]


def _draw(dtype, n, seed, out_dtype=None):
    if dtype.is_floating_point:
        x = W.normal(n, seed, dtype) if dtype != torch.float64 else W.normal(n, seed).double()
        if out_dtype == torch.float16:
            # N(0, 1/16): sum |x| ~ 2.0e4 and sum x^2 ~ 6.3e3 over 100,003
            # values, twice that after a fold, all below float16's 65,504, so
            # every mode compares finite values (scaling by 1/4 is exact)
            x = x * 0.25
        return x
    return W.randint(n, -2**20, 2**20, seed, dtype)


@pytest.mark.parametrize("combo", COMBOS, ids=lambda c: "-".join(str(t).split(".")[1] for t in c))
@pytest.mark.parametrize("op", ["sum", "max", "min"])
@pytest.mark.parametrize("map_", ["identity", "square", "abs"])
def test_dtype_op_map_matrix(combo, op, map_):
    in_dt, acc_dt, out_dt = combo
    x = _draw(in_dt, 100_003, 7500, out_dt)
    run_and_check(x, op=op, map_=map_, acc=acc_dt, out_dtype=out_dt, init=None)
    run_and_check(x, op=op, map_=map_, acc=acc_dt, out_dtype=out_dt, mode="fold")


def test_f16_output_overflows_to_inf():
    """A float32 accumulator holds a sum that float16 cannot: the sum of
    squares of 100,003 N(0,1) values (~1.0e5) stays finite in the
    accumulator, and only the single final conversion to float16 gives +inf
    (partials keep the accumulator's type: PR #139, "Compatibility").  The
    same call into float32 is checked by value."""
    x = W.normal(100_003, 7500, torch.float16)
    for map_ in ("square", "abs"):
        R = run_and_check(x, map_=map_, acc=torch.float32, out_dtype=torch.float32)
        assert 6.6e4 < float(R.item()) < 1.2e5
        res = run_and_check(x, map_=map_, acc=torch.float32, out_dtype=torch.float16, allow_inf=True)
        assert float(res.float().item()) == float("inf")
        res = run_and_check(x, map_=map_, acc=torch.float32, out_dtype=torch.float16, mode="host",
                            allow_inf=True)
        assert res == float("inf")


# ---------------------------------------------------------- exactness pins

def test_integer_valued_float_sums_are_exact():
    """Integers in [-8, 8]: every partial sum is exact in float32, so the GPU
    must equal the oracle bit for bit whatever its reduction tree."""
    rk = _rk()
    x = W.small_ints(10**6, -8, 8, 7600)
    out = rk.reduce_all(x.to(DEV), init=3.0)
    want = O.cast(O.F32, [O.reduce_all(O.SUM, O.IDENTITY, O.F32, O.F32, raw_np(x), 3.0)])
    assert raw_np(out)[0] == want[0]


def test_bf16_partials_stay_fp32():
    """bf16 integers summed with an f32 accumulator into bf16: equals the
    exact sum rounded once to bf16; bf16 partials would break this."""
    rk = _rk()
    x = W.small_ints(3 * 10**5 + 17, -8, 8, 7700, torch.bfloat16)
    out = rk.reduce_all(x.to(DEV), out_dtype=torch.bfloat16)
    exact = int(x.double().sum().item())
    assert raw_np(out)[0] == O.cast(O.BF16, [float(exact)])[0]


def test_int64_accumulator_beyond_int32():
    rk = _rk()
    x = torch.full((10**6,), 2**30, dtype=torch.int32)
    out = rk.reduce_all(x.to(DEV), acc=torch.int64, out_dtype=torch.int64)
    assert int(out.item()) == 10**6 * 2**30
    # int64 accumulator, int32 output: partials overflow int32, the total does not
    x = torch.tensor([2**30, 2**30, -2**30, -2**30, 5] * 1000, dtype=torch.int32)
    out = rk.reduce_all(x.to(DEV), acc=torch.int64, out_dtype=torch.int32)
    assert int(out.item()) == 5000


def _golden_tensor(raw, dtype_name):
    if dtype_name in ("bf16", "f16"):
        t = torch.from_numpy(np.ascontiguousarray(raw).view(np.int16).copy())
        return t.view(torch.bfloat16 if dtype_name == "bf16" else torch.float16)
    return torch.from_numpy(np.ascontiguousarray(raw).copy())


@pytest.mark.parametrize("case", [c for c in golden_cases.load() if "shape" not in c],
                         ids=lambda c: c["id"])
def test_golden_whole(case):
    rk = _rk()
    c = case
    xd = _golden_tensor(c["x_raw"], c["in"]).to(DEV)
    out = None
    if c["mode"] == "fold":
        out = _golden_tensor(c["prev_raw"], c["out"]).to(DEV)
    res = rk.reduce_all(xd, op=c["op"], map=c["map"], acc=c["acc_code"], out_dtype=c["out_code"],
                        init=c.get("init"), mode=c["mode"], out=out)
    torch.cuda.synchronize()
    got = res if c["mode"] == "host" else O.widen(c["out_code"], raw_np(res))[0]
    assert got == c["expected"], c["id"]
    if "expected_bits" in c:
        assert int(raw_np(res).view(np.uint16)[0]) == c["expected_bits"]


@pytest.mark.parametrize("seed", range(8))
def test_result_is_one_association_order(seed):
    """Tiny float32 sums: the GPU's value is one of the values some
    association order of the operands (init included) yields."""
    rk = _rk()
    rng = np.random.default_rng(900 + seed)
    n = 2 + seed % 5
    x = rng.uniform(-1, 1, n).astype(np.float32)
    init = float(np.float32(rng.uniform(-1, 1)))
    got = rk.reduce_all(torch.from_numpy(x).to(DEV), init=init).item()
    results = assoc.f32_results([np.float32(init)] + list(x), "sum")
    assert np.float32(got) in results


# ------------------------------------------------- workspace and buffers

def test_workspace_reuse_with_garbage():
    rk = _rk()
    ws = torch.full((1 << 16,), 0xFF, dtype=torch.uint8, device=DEV)
    for n, dt, op in [(10**6, torch.float32, "sum"), (12345, torch.int32, "max"),
                      (3 * 10**5, torch.bfloat16, "sum"), (10**6 + 1, torch.float64, "min")]:
        x = _draw(dt, n, 7800 + n % 13)
        in_c = rk.dtype_code(dt)
        need = rk.rk_workspace_size(in_c, rk.default_acc(in_c), 1, [n], [1], 1)
        assert need <= ws.numel()
        res = rk.reduce_all(x.to(DEV), op=op, workspace=ws, mode="host")
        xr = raw_np(x)
        acc_c = rk.default_acc(in_c)
        out_c = in_c if O.is_fp(in_c) else acc_c
        R, _ = O.expected_all(rk.OPS[op], O.IDENTITY, in_c, acc_c, out_c, xr, O.HOST)
        S = magnitude(O.IDENTITY, in_c, acc_c, xr, 0.0)
        check(rk.OPS[op], out_c, O.cast(out_c, [res]), [R], S, f"reuse {dt} {op}")


def test_output_neighbours_untouched():
    rk = _rk()
    guard = torch.full((8,), -12345.0, device=DEV)
    x = W.uniform(10**6, 0.0, 1.0, 7900).to(DEV)
    rk.reduce_all(x, out=guard[3:4], init=1.0)
    torch.cuda.synchronize()
    g = guard.cpu()
    assert all(g[i].item() == -12345.0 for i in (0, 1, 2, 4, 5, 6, 7))


def test_repeated_runs_identical():
    rk = _rk()
    x = W.normal(5 * 10**6 + 3, 7950).to(DEV)
    vals = {rk.reduce_all(x).item() for _ in range(10)}
    assert len(vals) == 1


def test_runs_on_a_side_stream():
    rk = _rk()
    x = W.uniform(10**6, 0.0, 1.0, 7960)
    s = torch.cuda.Stream()
    xd = x.to(DEV)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        out = rk.reduce_all(xd, init=2.0)
    s.synchronize()
    R = O.reduce_all(O.SUM, O.IDENTITY, O.F32, O.F32, raw_np(x), 2.0)
    assert abs(out.item() - R) <= 1e-5 * (2.0 + R)


def test_stream_argument_allocates_on_that_stream(monkeypatch):
    """stream= names a stream other than the current one: the workspace the
    binding allocates belongs to that stream, so once the call returns (and
    frees it) the current stream cannot be handed its bytes while the call's
    kernels -- queued behind other work -- still write and read them.  Two
    launches, so the partials really pass through the workspace."""
    rk = _rk()
    seen = []
    real = rk.workspace_for

    def spy(nbytes, device):
        t = real(nbytes, device)
        seen.append((t.data_ptr(), t.numel()))
        return t
    monkeypatch.setattr(rk, "workspace_for", spy)
    x = W.uniform(10**6 + 3, 0.0, 1.0, 7965)
    a, b = W.vector_pair(10**5 + 1)
    m = W.uniform(512 * 8192, -1.0, 1.0, 7966)
    xd, ad, bd, md = x.to(DEV), a.data.to(DEV), b.data.to(DEV), m.to(DEV)
    assert rk.plan_dims(torch.float32, (512, 8192), (1, 512), 2)["workspace_bytes"] > 0
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    prev = rk.rk_debug_set_fused_finish(0)
    try:
        with torch.cuda.stream(side):
            torch.cuda._sleep(50_000_000)       # the calls below queue behind this
        r_all = rk.reduce_all(xd, init=2.0, stream=side)
        r_all2 = rk.reduce_all2(ad, bd, "mul", stream=side)
        r_dims = rk.reduce_dims(md, (512, 8192), (1, 512), 2, stream=side)
        r_scan = rk.scan(xd, stream=side)
        assert len(seen) == 4
        # the current stream allocates and scribbles while the side stream waits
        junk = [torch.empty(nb, dtype=torch.uint8, device=DEV) for _, nb in seen]
        for (p, nb), j in zip(seen, junk):
            q = j.data_ptr()
            assert q + j.numel() <= p or p + nb <= q, "a freed workspace went to the current stream"
            j.fill_(0xFF)
        side.synchronize()
    finally:
        rk.rk_debug_set_fused_finish(prev)
    torch.cuda.synchronize()
    xr = raw_np(x)
    R = O.reduce_all(O.SUM, O.IDENTITY, O.F32, O.F32, xr, 2.0)
    check(O.SUM, O.F32, raw_np(r_all), [R], 2.0 + float(np.abs(xr.astype(np.float64)).sum()), "all")
    R2 = O.reduce_all2(O.SUM, O.MUL, O.F32, O.F32, raw_np(a.data), raw_np(b.data), 0.0)
    S2 = float((a.data.double() * b.data.double()).abs().sum())
    check(O.SUM, O.F32, raw_np(r_all2), [R2], S2, "all2")
    mr = raw_np(m)
    Rd = O.reduce_dims(O.SUM, O.IDENTITY, O.F32, O.F32, mr, (512, 8192), (1, 512), 0b10, 0.0)
    Sd = O.reduce_dims(O.SUM, O.ABS, O.F32, O.F32, mr, (512, 8192), (1, 512), 0b10, 0.0)
    check(O.SUM, O.F32, raw_np(r_dims), Rd, Sd, "dims")
    # inclusive prefix sums of values in [0, 1): S_k = R_k, and the tile
    # scan's longest rounding chain here is below 160 additions
    Rs = O.scan_dims(O.SUM, O.F32, O.F32, xr, (xr.size,), (1,), 0, 0.0, True)
    c = raw_np(r_scan).astype(np.float64)
    assert np.all(np.abs(c - Rs) <= 1e-5 * Rs)


def test_launch_event_hook_times_first_pass():
    rk = _rk()
    x = W.uniform(10**7, 0.0, 1.0, 7970).to(DEV)
    b, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b.record(); e.record()               # creates the underlying HIP events
    torch.cuda.synchronize()
    assert rk.rk_debug_set_launch_events(ctypes.c_void_p(b.cuda_event),
                                         ctypes.c_void_p(e.cuda_event)) == 0
    try:
        rk.reduce_all(x)
    finally:
        rk.rk_debug_set_launch_events(None, None)
    torch.cuda.synchronize()
    assert b.elapsed_time(e) > 0.0


def test_invalid_arguments_rejected_without_writing():
    rk = _rk()
    x = torch.ones(100, device=DEV)
    out = torch.full((1,), 7.0, device=DEV)
    ws = torch.empty(4096, dtype=torch.uint8, device=DEV)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    bad = [
        dict(op=3), dict(map_=5), dict(mode=9), dict(n=-1), dict(acc=rk.RK_BF16),
        dict(acc=rk.RK_I32), dict(out_dtype=rk.RK_I32), dict(ptr=x.data_ptr() + 2),
        dict(ws=0), dict(out_ptr=0), dict(out_ptr=x.data_ptr()),
    ]
    for b in bad:
        rc = rk.rk_reduce_all(b.get("op", 0), b.get("map_", 0), rk.RK_F32, b.get("acc", rk.RK_F32),
                              b.get("out_dtype", rk.RK_F32), b.get("ptr", x.data_ptr()),
                              b.get("n", 100), None, b.get("mode", 0),
                              b.get("out_ptr", out.data_ptr()), b.get("ws", ws.data_ptr()), st)
        assert rc in (rk.RK_ERR_INVALID_ARGUMENT, rk.RK_ERR_UNSUPPORTED), b
    torch.cuda.synchronize()
    assert out.item() == 7.0


def test_beyond_2_31_elements():
    """Inputs of more than 2^31 elements (8.6 GB of int32 ones): 64-bit
    indexing in the whole-array, row and columns kernels.  Totals are closed
    forms, so every result is exact."""
    rk = _rk()
    n = 2**31 + 5
    ones = torch.ones(n, dtype=torch.int32, device=DEV)
    total = rk.reduce_all(ones, acc=torch.int64, out_dtype=torch.int64)
    assert int(total.item()) == n
    v = rk.reduce_all(ones[3:], acc=torch.int64, out_dtype=torch.int64, mode="host")
    assert v == n - 3
    # dims=1 over three long rows (row kernel, offsets beyond 2^31 elements)
    m = (n - 2) // 3
    rows = rk.reduce_dims(ones, (m, 3), (1, m), 1, acc=torch.int64, out_dtype=torch.int64)
    assert rows.cpu().tolist() == [m, m, m]
    # dims=2 over a strided dim whose last rows sit past 2^31 elements (columns kernel)
    L, k = 1 << 16, (n // (1 << 16))
    cols = rk.reduce_dims(ones, (L, k), (1, L), 2, acc=torch.int64, out_dtype=torch.int64)
    assert bool((cols == k).all().item())
    del ones
    torch.cuda.empty_cache()


# ------------------------------------------------------------ seeded sweep
# Calls drawn from one seed per case: a row of the dtype table, an op, a map,
# a finishing mode, a start offset of 0-7 elements and a length log-uniform
# up to 3 million (100,003 at most into float16, whose sums must stay finite).

@pytest.mark.parametrize("case", range(64))
def test_seeded_whole_sweep(case):
    rng = np.random.default_rng(50_000 + case)
    in_dt, acc_dt, out_dt = COMBOS[int(rng.integers(0, len(COMBOS)))]
    op = ["sum", "max", "min"][int(rng.integers(0, 3))]
    map_ = ["identity", "square", "abs"][int(rng.integers(0, 3))]
    mode = ["overwrite", "fold", "host"][int(rng.integers(0, 3))]
    offset = int(rng.integers(0, 8))
    n = int(round(np.exp(rng.uniform(0, np.log(3e6)))))
    if out_dt == torch.float16:
        n = min(n, 100_003)
    x = _draw(in_dt, n + offset, 51_000 + case, out_dt)
    init = None if op != "sum" else (0.5 if in_dt.is_floating_point else 3)
    run_and_check(x, op=op, map_=map_, acc=acc_dt, out_dtype=out_dt, mode=mode, init=init, offset=offset,
                  what=f"whole sweep case {case}: {in_dt}->{acc_dt}->{out_dt} {op}/{map_}/{mode} n={n} offset {offset}")
