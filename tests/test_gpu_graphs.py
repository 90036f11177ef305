"""Reductions and scans captured in a HIP graph and replayed.

With the fused finish on, every kernel here finishes through state that
resets itself (the arrival counters of a split reduction, the look-back slot
of a scan); with it off, reductions take a second launch and the scan clears
its workspace state with a fill kernel.  Either way the calls launch no
memset and allocate nothing, so a captured sequence of calls must give
correct results on every replay.  Between replays the test does its own
eager work (new inputs copied in, eager library calls, synchronisations) and
checks each replay against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle as O
from reduction_primitives_amd import workloads as W
from tests.parity import raw_np

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _rk():
    import reduction_primitives_amd as rk
    rk.load()
    return rk


@pytest.mark.parametrize("fused", [True, False])
def test_graph_replays(fused):
    rk = _rk()
    prev = rk.rk_debug_set_fused_finish(int(fused))
    try:
        _replays(rk, fused)
    finally:
        rk.rk_debug_set_fused_finish(prev)


def _replays(rk, fused):
    n = 3 * 10**6 + 7
    shape, strides = (8192, 512), (1, 8192)               # split columns reduction over dims=2
    m = 4 * 10**6 + 3
    x = torch.empty(n, dtype=torch.int32, device=DEV)
    y = torch.empty(n, dtype=torch.int32, device=DEV)
    mat = torch.empty(8192 * 512, dtype=torch.int32, device=DEV)
    s = torch.empty(m, dtype=torch.int32, device=DEV)
    out_all = torch.empty(1, dtype=torch.int64, device=DEV)
    out_dot = torch.empty(1, dtype=torch.int64, device=DEV)
    out_dims = torch.empty(8192, dtype=torch.int64, device=DEV)
    out_scan = torch.empty(m, dtype=torch.int64, device=DEV)
    out_tr = torch.empty(8192 * 512, dtype=torch.int64, device=DEV)
    tr_shape, tr_strides = (512, 8192), (8192, 1)          # the matrix read row-major, scanned along its rows
    ws_all = rk.workspace_for(rk.rk_workspace_size(rk.RK_I32, rk.RK_I64, 1, [n], [1], 1), DEV)
    ws_dims = rk.workspace_for(rk.rk_workspace_size(rk.RK_I32, rk.RK_I64, 2, shape, strides, 0b10), DEV)
    ws_scan = rk.workspace_for(rk.rk_scan_workspace_size(rk.RK_I32, rk.RK_I64, 1, [m], [1], 0), DEV)
    ws_tr = rk.workspace_for(rk.rk_scan_workspace_size(rk.RK_I32, rk.RK_I64, 2, tr_shape, tr_strides, 1), DEV)
    plan_tr = rk.plan_scan(torch.int32, tr_shape, tr_strides, 2, acc=torch.int64)
    assert plan_tr["kernel_name"] == "scan_transpose" and plan_tr["launches"] == (1 if fused else 2)
    assert rk.plan_dims(torch.int32, shape, strides, 2, acc=torch.int64)["split"] > 1
    plan = rk.plan_scan(torch.int32, (m,), (1,), 1, acc=torch.int64)
    assert plan["kernel_name"] == "scan_tile"
    assert plan["launches"] == (1 if fused else 2)        # state in the library slot, or cleared workspace

    def calls():
        rk.reduce_all(x, acc=torch.int64, out_dtype=torch.int64, init=5, out=out_all, workspace=ws_all)
        rk.reduce_all2(x, y, "mul", acc=torch.int64, out_dtype=torch.int64, out=out_dot, workspace=ws_all)
        rk.reduce_dims(mat, shape, strides, 2, acc=torch.int64, out_dtype=torch.int64, out=out_dims,
                       workspace=ws_dims)
        rk.scan(s, acc=torch.int64, out_dtype=torch.int64, out=out_scan, workspace=ws_scan)
        rk.scan(mat, tr_shape, tr_strides, 2, acc=torch.int64, out_dtype=torch.int64, out=out_tr, workspace=ws_tr)

    def fill(seed):
        xs = W.randint(n, -1000, 1000, seed)
        ys = W.randint(n, -1000, 1000, seed + 1)
        ms = W.randint(8192 * 512, -1000, 1000, seed + 2)
        ss = W.randint(m, -1000, 1000, seed + 3)
        x.copy_(xs.to(DEV)); y.copy_(ys.to(DEV)); mat.copy_(ms.to(DEV)); s.copy_(ss.to(DEV))
        return xs, ys, ms, ss

    def check(data):
        xs, ys, ms, ss = data
        assert int(out_all.item()) == int(xs.long().sum()) + 5
        assert int(out_dot.item()) == int((xs.long() * ys.long()).sum())
        want = ms.long().view(512, 8192).sum(dim=0).numpy()
        assert np.array_equal(raw_np(out_dims), want)
        assert np.array_equal(raw_np(out_scan), np.cumsum(ss.numpy().astype(np.int64)))
        rows = np.cumsum(ms.numpy().astype(np.int64).reshape(512, 8192), axis=1)
        assert np.array_equal(raw_np(out_tr), rows.T.reshape(-1))      # column-major (512, 8192) output

    data = fill(14000)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                      # warm-up outside the capture
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    check(data)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for rep in range(5):
        data = fill(14100 + 10 * rep)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check(data)
        # eager work between replays: the same calls outside the graph
        calls()
        torch.cuda.synchronize()
        check(data)
