"""GPU tests of the error paths: a wait inside a launch that gives up, and a
launch that fails.

PR #139 ("Finish whole-array reductions on the device", section
"Compatibility") applies init once and keeps intermediate values out of the
output; so a call that cannot finish must leave `out` as it was and say so,
never store a fold of the partials it happened to see.  The
waits are forced to give up from the host (a test hook makes them wait for a
tag or flag no block sets, for a few polls), so every kernel still ends
normally; the failed launches are refused before anything is enqueued.
"""
import ctypes
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle as O
from reduction_primitives_amd import workloads as W
from tests.parity import check, raw_np

pytestmark = pytest.mark.gpu

DEV = "cuda"
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _rk():
    import reduction_primitives_amd as rk
    rk.load()
    return rk


class forced_give_up:
    """Every collection / look-back wait gives up after `polls` polls."""

    def __init__(self, polls=8):
        self.polls = polls

    def __enter__(self):
        assert _rk().rk_debug_force_wait_timeout(self.polls) == 0

    def __exit__(self, *exc):
        _rk().rk_debug_force_wait_timeout(-1)


def test_collection_that_gives_up_stores_nothing_and_is_reported():
    rk = _rk()
    n = 10**7 + 3
    x = W.uniform(n, 0.0, 1.0, 9600)
    xi = W.randint(3 * 10**6 + 1, -10**6, 10**6, 9601)
    xd, xid = x.to(DEV), xi.to(DEV)
    p = rk.rk_plan_all(rk.RK_F32, rk.RK_F32, xd.data_ptr(), n)
    assert p.grid > 1 and p.launches == 1                  # finishes by collection
    ns = 3 * 65536 + 5                                     # a scan of several look-back tiles
    assert rk.plan_scan(torch.float32, (ns,), (1,), 1)["kernel_name"] == "scan_tile"
    s = torch.cuda.Stream()
    st = ctypes.c_void_p(s.cuda_stream)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        rk.rk_stream_timeouts(st)                          # start from a cleared count
        out = torch.full((1,), 7.0, device=DEV)
        outi = torch.full((1,), -5, dtype=torch.int64, device=DEV)
        with forced_give_up():
            rk.reduce_all(xd, init=1.0, out=out)           # 4-byte partials
            rk.reduce_all(xid, acc=torch.int64, out_dtype=torch.int64, out=outi)   # 8-byte partials
            assert rk.rk_stream_timeouts(st) == 2
            assert float(out.item()) == 7.0 and int(outi.item()) == -5          # nothing stored
            with pytest.raises(rk.RkError) as e:
                rk.reduce_all(xd, mode="host")
            assert e.value.status == rk.RK_ERR_HIP
            assert rk.rk_stream_timeouts(st) == 1
            rk.scan(xd[:ns])
            assert rk.rk_stream_timeouts(st) >= 1
        assert rk.rk_stream_timeouts(st) == 0
        # the next calls on the stream are exact again
        out = rk.reduce_all(xd, init=1.0)
        outi = rk.reduce_all(xid, acc=torch.int64, out_dtype=torch.int64)
        v = rk.reduce_all(xd, mode="host")
        c = rk.scan(xd[:ns])
    s.synchronize()
    xr = raw_np(x)
    R = O.reduce_all(O.SUM, O.IDENTITY, O.F32, O.F32, xr, 1.0)
    check(O.SUM, O.F32, raw_np(out), [R], R, "overwrite after a give-up")
    R0 = O.reduce_all(O.SUM, O.IDENTITY, O.F32, O.F32, xr, 0.0)
    check(O.SUM, O.F32, O.cast(O.F32, [v]), [R0], R0, "host after a give-up")
    assert int(outi.item()) == int(xi.long().sum())
    Rs = O.scan_dims(O.SUM, O.F32, O.F32, xr[:ns], (ns,), (1,), 0, 0.0, True)
    assert np.all(np.abs(raw_np(c).astype(np.float64) - Rs) <= 1e-5 * Rs)
    assert rk.rk_stream_timeouts(st) == 0


def test_transposing_scan_give_up_is_reported():
    """A transposing scan (a row-major matrix along its rows) whose
    look-back waits all give up: the stream's count records it, and the next
    call on the stream is exact."""
    rk = _rk()
    shape, strides = (300, 2000), (2000, 1)
    x = W.randint(600_000, -1000, 1000, 9620)
    xd = x.to(DEV)
    plan = rk.plan_scan(torch.int32, shape, strides, 2, acc=torch.int64)
    assert plan["kernel_name"] == "scan_transpose" and plan["split"] > 1
    s = torch.cuda.Stream()
    st = ctypes.c_void_p(s.cuda_stream)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        rk.rk_stream_timeouts(st)
        with forced_give_up():
            rk.scan(xd, shape, strides, 2, acc=torch.int64, out_dtype=torch.int64)
            assert rk.rk_stream_timeouts(st) >= 1
        assert rk.rk_stream_timeouts(st) == 0
        c = rk.scan(xd, shape, strides, 2, acc=torch.int64, out_dtype=torch.int64)
    s.synchronize()
    R = O.scan_dims(O.SUM, O.I32, O.I64, raw_np(x), shape, strides, 1, 0, True)
    assert np.array_equal(raw_np(c), R)
    assert rk.rk_stream_timeouts(st) == 0


def test_host_copy_back_reports_a_give_up():
    """Host mode without the pinned result buffer (RK_HOST_COPY): the result
    is copied back from the workspace with the call's sequence word, so a
    call whose collection gave up is told apart from stale bytes."""
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "import torch, reduction_primitives_amd as rk\n"
        "from reduction_primitives_amd import workloads as W\n"
        "x = W.uniform(10**7 + 3, 0.0, 1.0, 9600).cuda()\n"
        "print(repr(rk.reduce_all(x, mode='host', init=1.0)))\n"
        "rk.rk_debug_force_wait_timeout(8)\n"
        "try:\n"
        "    rk.reduce_all(x, mode='host', init=1.0)\n"
        "    print('no-error')\n"
        "except rk.RkError as e:\n"
        "    print('status', e.status)\n"
        "rk.rk_debug_force_wait_timeout(-1)\n"
        "print(repr(rk.reduce_all(x, mode='host', init=1.0)))\n"
    ) % ROOT
    env = dict(os.environ, RK_HOST_COPY="1")
    proc = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=240)
    assert proc.returncode == 0, proc.stderr[-2000:]
    lines = proc.stdout.split("\n")
    assert lines[1] == "status 3", proc.stdout
    x = W.uniform(10**7 + 3, 0.0, 1.0, 9600)
    R = O.reduce_all(O.SUM, O.IDENTITY, O.F32, O.F32, raw_np(x), 1.0)
    for v in (float(lines[0]), float(lines[2])):
        assert abs(v - R) <= 1e-5 * R


def test_failed_launch_returns_hip_error_and_writes_nothing():
    """A launch the runtime refuses (forced by the test hook before anything
    is enqueued) returns RK_ERR_HIP and leaves out and the workspace as they
    were; the next call is exact."""
    rk = _rk()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    x = W.uniform(10**6 + 5, -1.0, 1.0, 9700)
    m = W.uniform(512 * 8192, -1.0, 1.0, 9701)
    xd, md = x.to(DEV), m.to(DEV)
    wsz = max(rk.rk_workspace_size(rk.RK_F32, rk.RK_F32, 1, [x.numel()], [1], 1),
              rk.rk_workspace_size(rk.RK_F32, rk.RK_F32, 2, (512, 8192), (1, 512), 2),
              rk.rk_scan_workspace_size(rk.RK_F32, rk.RK_F32, 1, [x.numel()], [1], 0))
    ws = torch.full((wsz,), 0xAB, dtype=torch.uint8, device=DEV)
    out1 = torch.full((1,), 7.0, device=DEV)
    outd = torch.full((512,), 7.0, device=DEV)
    outs = torch.full((x.numel(),), 7.0, device=DEV)
    host = ctypes.c_float(7.0)
    torch.cuda.synchronize()
    calls = [
        lambda: rk.rk_reduce_all(0, 0, rk.RK_F32, rk.RK_F32, rk.RK_F32, xd.data_ptr(), x.numel(), None,
                                 rk.RK_MODE_OVERWRITE, out1.data_ptr(), ws.data_ptr(), st),
        lambda: rk.rk_reduce_all(0, 0, rk.RK_F32, rk.RK_F32, rk.RK_F32, xd.data_ptr(), x.numel(), None,
                                 rk.RK_MODE_HOST, ctypes.addressof(host), ws.data_ptr(), st),
        lambda: rk.rk_reduce_all2(0, 0, rk.RK_F32, rk.RK_F32, rk.RK_F32, xd.data_ptr(), xd.data_ptr(),
                                  x.numel(), None, rk.RK_MODE_OVERWRITE, out1.data_ptr(), ws.data_ptr(), st),
        lambda: rk.rk_reduce_dims(0, 0, rk.RK_F32, rk.RK_F32, rk.RK_F32, md.data_ptr(), 2, (512, 8192),
                                  (1, 512), 2, None, rk.RK_MODE_OVERWRITE, outd.data_ptr(), ws.data_ptr(), st),
        lambda: rk.rk_scan(0, rk.RK_F32, rk.RK_F32, rk.RK_F32, xd.data_ptr(), x.numel(), None, 1,
                           outs.data_ptr(), ws.data_ptr(), st),
    ]
    prev = rk.rk_debug_set_fused_finish(0)      # two-launch paths too
    try:
        for fused in (0, 1):
            rk.rk_debug_set_fused_finish(fused)
            for i, call in enumerate(calls):
                assert rk.rk_debug_fail_launches(1) == 0
                assert call() == rk.RK_ERR_HIP, (fused, i)
                torch.cuda.synchronize()
                assert bool((ws == 0xAB).all()), (fused, i)
                assert float(out1.item()) == 7.0 and bool((outd == 7.0).all()) and bool((outs == 7.0).all())
                assert host.value == 7.0
    finally:
        rk.rk_debug_fail_launches(0)
        rk.rk_debug_set_fused_finish(prev)
    # the hook is used up: the same calls now run
    for call in calls:
        assert call() == rk.RK_OK
    torch.cuda.synchronize()
    xr, mr = raw_np(x), raw_np(m)
    S = float(np.abs(xr.astype(np.float64)).sum())
    R = O.reduce_all(O.SUM, O.IDENTITY, O.F32, O.F32, xr, 0.0)
    check(O.SUM, O.F32, O.cast(O.F32, [host.value]), [R], S, "host")
    R2 = O.reduce_all2(O.SUM, O.MUL, O.F32, O.F32, xr, xr, 0.0)
    check(O.SUM, O.F32, raw_np(out1), [R2], R2, "all2")
    Rd = O.reduce_dims(O.SUM, O.IDENTITY, O.F32, O.F32, mr, (512, 8192), (1, 512), 0b10, 0.0)
    Sd = O.reduce_dims(O.SUM, O.ABS, O.F32, O.F32, mr, (512, 8192), (1, 512), 0b10, 0.0)
    check(O.SUM, O.F32, raw_np(outd), Rd, Sd, "dims")
