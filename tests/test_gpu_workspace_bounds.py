"""GPU checks that every call stays inside the workspace size the library
reports, and writes nothing around its output.

Each call gets a buffer holding exactly the reported workspace bytes between
two guard regions filled with a byte pattern, and an output with guards on
both sides; after the call (and a second one reusing the same buffers) the
guards must be intact and the results must still meet the oracle bar.
Covers the whole-array passes (one launch and two), the split dims kernels,
two-input sources, and both look-back scans.
"""
import numpy as np
import pytest
import torch

import oracle as O
from reduction_primitives_amd import workloads as W
from tests.parity import raw_np

pytestmark = pytest.mark.gpu

DEV = "cuda"
GUARD = 4096
PATTERN = 0xA5


def _rk():
    import reduction_primitives_amd as rk
    rk.load()
    return rk


def guarded(nbytes):
    """(whole buffer, view of the nbytes in the middle, 256-byte aligned)."""
    buf = torch.full((GUARD + max(nbytes, 0) + GUARD,), PATTERN, dtype=torch.uint8, device=DEV)
    return buf, buf[GUARD:GUARD + nbytes]


def guards_intact(buf, nbytes):
    b = raw_np(buf)
    return bool(np.all(b[:GUARD] == PATTERN) and np.all(b[GUARD + nbytes:] == PATTERN))


def guarded_out(n, dtype):
    esz = torch.empty((), dtype=dtype).element_size()
    buf = torch.full((2 * GUARD + n * esz,), PATTERN, dtype=torch.uint8, device=DEV)
    return buf, buf[GUARD:GUARD + n * esz].view(dtype)


@pytest.mark.parametrize("fused", [1, 0])
def test_whole_array_workspace(fused):
    rk = _rk()
    prev = rk.rk_debug_set_fused_finish(fused)
    try:
        for n in (5, 10**4, 10**6 + 3, 10**8):
            x = W.uniform(n, -1.0, 1.0, 13000 + n % 7)
            xd = x.to(DEV)
            nb = rk.rk_workspace_size(rk.RK_F32, rk.RK_F32, 1, [n], [1], 1)
            wbuf, ws = guarded(nb)
            obuf, out = guarded_out(1, torch.float32)
            for _ in range(2):
                rk.reduce_all(xd, init=0.5, out=out, workspace=ws)
                v = rk.reduce_all(xd, mode="host", workspace=ws)
            torch.cuda.synchronize()
            assert guards_intact(wbuf, nb) and guards_intact(obuf, 4), n
            R = O.reduce_all(O.SUM, O.IDENTITY, O.F32, O.F32, raw_np(x), 0.5)
            S = 0.5 + O.reduce_all(O.SUM, O.ABS, O.F32, O.F32, raw_np(x), 0.0)
            assert abs(float(out.item()) - R) <= 1e-5 * S
            assert abs(v - (R - 0.5)) <= 1e-5 * S
    finally:
        rk.rk_debug_set_fused_finish(prev)


@pytest.mark.parametrize("fused", [1, 0])
def test_split_dims_workspace(fused):
    rk = _rk()
    prev = rk.rk_debug_set_fused_finish(fused)
    try:
        cases = [((8192, 8192), (1, 8192), 2), ((100003, 7), (1, 100003), 1),
                 ((3136, 16, 24), W.cm_strides((3136, 16, 24)), (1, 3)),
                 ((128, 3000, 3), (1, 384, 128), (2, 3))]
        for shape, strides, dims in cases:
            numel = max(int(np.prod(shape)), sum((e - 1) * s for e, s in zip(shape, strides)) + 1)
            x = W.normal(numel, 13100 + numel % 11).to(DEV)
            mask = 0
            for d in ((dims,) if isinstance(dims, int) else dims):
                mask |= 1 << (d - 1)
            nb = rk.rk_workspace_size(rk.RK_F32, rk.RK_F32, len(shape), shape, strides, mask)
            plan = rk.plan_dims(torch.float32, shape, strides, dims)
            assert nb == plan["workspace_bytes"] and (plan["split"] > 1) == (nb > 0)
            wbuf, ws = guarded(nb)
            obuf, out = guarded_out(plan["n_out"], torch.float32)
            for _ in range(2):
                rk.reduce_dims(x, shape, strides, dims, out=out, workspace=ws if nb else None)
            torch.cuda.synchronize()
            assert guards_intact(wbuf, nb) and guards_intact(obuf, 4 * plan["n_out"]), (shape, dims)
            ref = rk.reduce_dims(x, shape, strides, dims)
            torch.cuda.synchronize()
            assert np.allclose(raw_np(out), raw_np(ref)[:plan["n_out"]], rtol=1e-5, atol=1e-3)
    finally:
        rk.rk_debug_set_fused_finish(prev)


def test_two_input_workspace():
    rk = _rk()
    for n, offs in ((10**6, (0, 0)), (10**7 + 1, (1, 2))):
        a = W.normal(n + 4, 13200).to(DEV)[offs[0]:offs[0] + n]
        b = W.normal(n + 4, 13201).to(DEV)[offs[1]:offs[1] + n]
        nb = rk.rk_workspace_size(rk.RK_F32, rk.RK_F32, 1, [n], [1], 1)
        wbuf, ws = guarded(nb)
        obuf, out = guarded_out(1, torch.float32)
        for _ in range(2):
            rk.reduce_all2(a, b, "mul", out=out, workspace=ws)
        torch.cuda.synchronize()
        assert guards_intact(wbuf, nb) and guards_intact(obuf, 4)


@pytest.mark.parametrize("shape,strides,dim", [
    ((10**8,), (1,), 1),                    # tile kernel, 1,526 tiles
    ((100003, 3), (1, 100003), 1),          # tile kernel, look-back per line
    ((8192, 8192), (1, 8192), 2),           # columns kernel, 16-byte loads
    ((130, 2000), (1, 131), 2),             # columns kernel, element loads
])
def test_scan_workspace(shape, strides, dim):
    rk = _rk()
    numel = max(int(np.prod(shape)), sum((e - 1) * s for e, s in zip(shape, strides)) + 1)
    x = W.small_ints(numel, -4, 4, 13300 + numel % 13).to(DEV)
    nb = rk.rk_scan_workspace_size(rk.RK_F32, rk.RK_F32, len(shape), shape, strides, dim - 1)
    assert nb > 0
    wbuf, ws = guarded(nb)
    total = int(np.prod(shape))
    obuf, out = guarded_out(total, torch.float32)
    for inclusive in (True, False):
        rk.scan(x, shape, strides, dim, out=out, workspace=ws, inclusive=inclusive)
    torch.cuda.synchronize()
    assert guards_intact(wbuf, nb) and guards_intact(obuf, 4 * total)
    # integer-valued data: every prefix is exact in f32 (|prefix| < 2^24)
    R = O.scan_dims(O.SUM, O.F32, O.F32, raw_np(x.cpu()), shape, strides, dim - 1, 0.0, False)
    assert np.array_equal(raw_np(out).astype(np.float64), R)
