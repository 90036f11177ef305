"""GPU tests of the two ways a split reduction finishes.

A whole-array reduction, a split columns reduction and a split row reduction
either finish in the last block to arrive (one launch, arrival counters in
library memory) or in a second launch.  Both must meet the oracle bar; the
whole-array and columns variants fold the partials in the same order, so they
must agree bit for bit.  Also covered: counters returning to zero across many
calls, calls on several streams at once, and more streams than counter slots
(the overflow takes the second-launch path).
"""
import ctypes
import math

import numpy as np
import pytest
import torch

import oracle as O
from reduction_primitives_amd import workloads as W
from tests.parity import check, magnitude, raw_np

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _rk():
    import reduction_primitives_amd as rk
    rk.load()
    return rk


class fused:
    """Context manager switching the one-launch finish on or off."""

    def __init__(self, on):
        self.on = on

    def __enter__(self):
        self.prev = _rk().rk_debug_set_fused_finish(1 if self.on else 0)

    def __exit__(self, *exc):
        _rk().rk_debug_set_fused_finish(self.prev)


SPLIT_CASES = [
    # (shape, dims, dtype, kernel)
    ((10**7 + 3,), 1, torch.float32, "all"),
    ((64, 4096, 32), 2, torch.float32, "columns"),
    ((8192, 8192), 2, torch.float32, "columns"),
    ((96, 4000, 3), 2, torch.bfloat16, "columns"),
    ((100003, 7), 1, torch.float32, "row"),
    ((50001, 3), 1, torch.int32, "row"),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: f"{c[3]}-{'x'.join(map(str, c[0]))}")
def test_one_launch_and_two_launch_finish_agree(case):
    rk = _rk()
    shape, dims, dt, kern = case
    n = math.prod(shape)
    x = (W.randint(n, -10**6, 10**6, 9100) if dt == torch.int32
         else W.normal(n, 9100, dt))
    st = W.cm_strides(shape)
    xd = x.to(DEV)
    plan = rk.plan_dims(dt, shape, st, dims)
    assert plan["kernel_name"] == kern
    assert kern == "all" or plan["split"] > 1
    results = {}
    for on in (True, False):
        with fused(on):
            out = rk.reduce_dims(xd, shape, st, dims, out_dtype=torch.float32 if dt.is_floating_point
                                 else torch.int64, acc=torch.int64 if dt == torch.int32 else None,
                                 init=0.5 if dt.is_floating_point else 3)
            torch.cuda.synchronize()
            results[on] = raw_np(out)
    in_c = O.F32 if dt == torch.float32 else O.BF16 if dt == torch.bfloat16 else O.I32
    acc_c = O.I64 if dt == torch.int32 else O.F32
    out_c = O.F32 if dt.is_floating_point else O.I64
    mask = 0
    for d in ((dims,) if isinstance(dims, int) else dims):
        mask |= 1 << (d - 1)
    xr = raw_np(x)
    start = 0.5 if dt.is_floating_point else 3
    R = O.reduce_dims(O.SUM, O.IDENTITY, in_c, acc_c, xr, shape, st, mask, start)
    S = magnitude(O.IDENTITY, in_c, acc_c, xr, start, reduce=(xr, shape, st, mask)) \
        if dt.is_floating_point else None
    for on in (True, False):
        check(O.SUM, out_c, results[on][:R.size], R, S, f"{kern} fused={on}")
    if kern in ("all", "columns") or not dt.is_floating_point:
        assert np.array_equal(results[True], results[False])


def test_counters_return_to_zero_over_many_calls():
    """200 one-launch calls in a row on one stream all give the same value,
    which needs every arrival counter back at zero after each call."""
    rk = _rk()
    x = W.normal(3 * 10**6 + 5, 9200).to(DEV)
    xi = W.randint(64 * 4096 * 32, -1000, 1000, 9201).to(DEV)
    with fused(True):
        outs = torch.empty(200, device=DEV)
        for i in range(200):
            rk.reduce_all(x, out=outs[i:i + 1])
        outs_i = torch.empty((50, 2048), dtype=torch.int64, device=DEV)
        for i in range(50):
            rk.reduce_dims(xi, (64, 4096, 32), (1, 64, 64 * 4096), 2, acc=torch.int64,
                           out_dtype=torch.int64, out=outs_i[i])
        torch.cuda.synchronize()
    assert torch.unique(outs).numel() == 1
    assert bool((outs_i == outs_i[0]).all().item())
    want = O.reduce_all(O.SUM, O.IDENTITY, O.F32, O.F32, raw_np(x.cpu()), 0.0)
    S = O.reduce_all(O.SUM, O.ABS, O.F32, O.F32, raw_np(x.cpu()), 0.0)
    assert abs(float(outs[0]) - want) <= 1e-5 * S


def test_concurrent_streams_and_slot_overflow():
    """Reductions queued on 40 streams at once (more streams than counter
    slots): every result matches the oracle."""
    rk = _rk()
    n = 2 * 10**6 + 17
    xs = [W.uniform(n, -1.0, 1.0, 9300 + i) for i in range(8)]
    xds = [x.to(DEV) for x in xs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(40)]
    outs = []
    with fused(True):
        for i, s in enumerate(streams):
            with torch.cuda.stream(s):
                outs.append(rk.reduce_all(xds[i % 8], init=float(i)))
        for s in streams:
            s.synchronize()
    for i, out in enumerate(outs):
        xr = raw_np(xs[i % 8])
        R = O.reduce_all(O.SUM, O.IDENTITY, O.F32, O.F32, xr, float(i))
        S = i + O.reduce_all(O.SUM, O.ABS, O.F32, O.F32, xr, 0.0)
        assert abs(float(out.item()) - R) <= 1e-5 * S, i


def test_host_mode_and_fold_with_one_launch():
    rk = _rk()
    x = W.uniform(10**7, 0.0, 1.0, 9400)
    xd = x.to(DEV)
    xr = raw_np(x)
    R = O.reduce_all(O.SUM, O.IDENTITY, O.F32, O.F32, xr, 0.25)
    with fused(True):
        v = rk.reduce_all(xd, init=0.25, mode="host")
        out = rk.reduce_all(xd, init=0.25)
        rk.reduce_all(xd, mode="fold", out=out)
        torch.cuda.synchronize()
    assert abs(v - R) <= 1e-5 * R
    assert abs(float(out.item()) - (2 * R - 0.25)) <= 2e-5 * R


def test_host_mode_copy_back_path():
    """With RK_HOST_COPY set the bare partial is copied back from the
    workspace instead of written to pinned host memory; same results."""
    import os
    import subprocess
    import sys
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "import torch, reduction_primitives_amd as rk\n"
        "from reduction_primitives_amd import workloads as W\n"
        "x = W.uniform(5 * 10**6 + 3, -1.0, 1.0, 9500).cuda()\n"
        "xi = W.randint(1000, -50, 50, 9501).cuda()\n"
        "print(repr(rk.reduce_all(x, mode='host', init=0.5)))\n"
        "print(repr(rk.reduce_all(xi, mode='host', acc=torch.int64, out_dtype=torch.int64)))\n"
    ) % os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = {}
    for copy in (True, False):
        env = dict(os.environ)
        env.pop("RK_HOST_COPY", None)
        if copy:
            env["RK_HOST_COPY"] = "1"
        proc = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                              timeout=240)
        assert proc.returncode == 0, proc.stderr[-2000:]
        res[copy] = proc.stdout.split()
    assert res[True] == res[False]
    x = W.uniform(5 * 10**6 + 3, -1.0, 1.0, 9500)
    R = O.reduce_all(O.SUM, O.IDENTITY, O.F32, O.F32, raw_np(x), 0.5)
    S = 0.5 + O.reduce_all(O.SUM, O.ABS, O.F32, O.F32, raw_np(x), 0.0)
    assert abs(float(res[True][0]) - R) <= 1e-5 * S
    xi = W.randint(1000, -50, 50, 9501)
    assert int(res[True][1]) == int(xi.long().sum())


def test_collection_tags_across_the_wrap():
    """Whole-array passes collect their blocks' partials by the call's tag;
    the call that reaches the last tag (2^32 - 1) clears the slot's words
    and the next starts again at 1.  Calls on one stream across that wrap,
    with 4-byte (f32) and 8-byte (int32 -> int64) partials, give exact
    results; so do calls after it."""
    import reduction_primitives_amd as rk
    rk.load()
    s = torch.cuda.Stream()
    st = ctypes.c_void_p(s.cuda_stream)
    n = 3 * 10**6 + 11
    assert rk.rk_plan_all(rk.RK_F32, rk.RK_F32, 0, n, 256).grid > 1
    xs = [W.small_ints(n, -8, 8, 15000 + i) for i in range(6)]          # exact in f32 in any order
    xis = [W.randint(n, -10**6, 10**6, 15100 + i) for i in range(6)]
    xds = [x.to("cuda") for x in xs]
    xids = [x.to("cuda") for x in xis]
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        assert rk.rk_debug_set_finish_tag(st, 0xFFFFFFFD) == rk.RK_OK    # next tags: ..FE, ..FF (wrap), 1, 2
        outs = []
        for i in range(6):
            outs.append(rk.reduce_all(xds[i], init=0.0))
            outs.append(rk.reduce_all(xids[i], acc=torch.int64, out_dtype=torch.int64))
    s.synchronize()
    for i in range(6):
        assert float(outs[2 * i].item()) == float(xs[i].double().sum()), i
        assert int(outs[2 * i + 1].item()) == int(xis[i].long().sum()), i
    assert rk.rk_debug_set_finish_tag(st, 0xFFFFFFFF) == rk.RK_ERR_INVALID_ARGUMENT
