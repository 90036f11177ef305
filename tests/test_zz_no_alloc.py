"""GPU test of rk_reduce_dims_no_workspace, the entry point for callers that
cannot allocate: the library's static scratch stands in for the workspace.

Each case runs the no-workspace call and the workspace call (rk_reduce_dims)
on the same input through the C ABI: the results must be the same bits (the
same kernels fold in the same order) and meet the oracle bar.  Two calls in a
row on the shared scratch, the second with a smaller input, show that a call
reads nothing the previous one left there.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
from reduction_primitives_amd import workloads as W
from tests.parity import check, raw_np

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _rk():
    import reduction_primitives_amd as rk
    rk.load()
    return rk


def _both(x_cpu, shape, dims, op="sum", acc=torch.float32, out_dtype=torch.float32, mode="overwrite", init=None):
    """(no-workspace result, workspace result) of one reduction, raw outputs."""
    rk = _rk()
    strides = [1]
    for e in shape[:-1]:
        strides.append(strides[-1] * e)
    mask = 0
    for d in dims:
        mask |= 1 << (d - 1)
    in_c, acc_c, out_c = rk.dtype_code(x_cpu.dtype), rk.dtype_code(acc), rk.dtype_code(out_dtype)
    op_c, mode_c = rk.OPS[op], rk.MODES[mode]
    xd = x_cpu.to(DEV)
    n_out = int(np.prod([e for i, e in enumerate(shape) if not (mask >> i) & 1])) if len(dims) < len(shape) else 1
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    init_p = rk.init_arg(acc_c, init)
    ws = torch.empty(max(rk.rk_workspace_size(in_c, acc_c, len(shape), shape, strides, mask), 256),
                     dtype=torch.uint8, device=DEV)
    if mode == "host":
        a, b = rk._CTYPE[out_c](), rk._CTYPE[out_c]()
        assert rk.rk_reduce_dims_no_workspace(op_c, 0, in_c, acc_c, out_c, xd.data_ptr(), len(shape), shape,
                                              strides, mask, init_p, mode_c, ctypes.addressof(a), st) == 0
        assert rk.rk_reduce_dims(op_c, 0, in_c, acc_c, out_c, xd.data_ptr(), len(shape), shape, strides, mask,
                                 init_p, mode_c, ctypes.addressof(b), ws.data_ptr(), st) == 0
        ga = O.cast(out_c, [rk.decode_host_out(a, out_c)])
        gb = O.cast(out_c, [rk.decode_host_out(b, out_c)])
    else:
        oa = torch.full((n_out,), 3, dtype=out_dtype, device=DEV)
        ob = torch.full((n_out,), 3, dtype=out_dtype, device=DEV)
        assert rk.rk_reduce_dims_no_workspace(op_c, 0, in_c, acc_c, out_c, xd.data_ptr(), len(shape), shape,
                                              strides, mask, init_p, mode_c, oa.data_ptr(), st) == 0
        assert rk.rk_reduce_dims(op_c, 0, in_c, acc_c, out_c, xd.data_ptr(), len(shape), shape, strides, mask,
                                 init_p, mode_c, ob.data_ptr(), ws.data_ptr(), st) == 0
        torch.cuda.synchronize()
        ga, gb = raw_np(oa), raw_np(ob)
    assert np.array_equal(np.asarray(ga).view(np.uint8), np.asarray(gb).view(np.uint8)), (shape, dims, op, mode)
    # the oracle bar
    xr = raw_np(x_cpu)
    s = init if init is not None else O.identity(O.SUM if op == "sum" else (O.MAX if op == "max" else O.MIN), acc_c)
    R = O.reduce_dims(op_c, O.IDENTITY, in_c, acc_c, xr, shape, strides, mask, s)
    S = None
    if O.is_fp(in_c):
        S = O.reduce_dims(O.SUM, O.ABS, in_c, acc_c, xr, shape, strides, mask, 0.0) + abs(s if op == "sum" else 0.0)
    check(op_c, out_c, ga, R, S, f"{shape} dims={dims} {op} {mode}")
    return ga


CASES = [
    # (larger call, then a smaller one): the columns kernel split over blocks,
    # the row kernel split over waves, and a whole array in many blocks
    (((8192, 8192), (2,)), ((64, 4096, 32), (2,))),
    (((100003, 7), (1,)), ((5003, 7), (1,))),
    (((10**7 + 3,), (1,)), ((100003,), (1,))),
]


@pytest.mark.parametrize("case", CASES, ids=["columns", "row", "whole"])
def test_no_workspace_matches_workspace_call(case):
    for i, (shape, dims) in enumerate(case):
        x = W.uniform(int(np.prod(shape)), -1.0, 1.0, 16000 + i)
        _both(x, shape, dims, init=0.5)
        _both(x, shape, dims, op="max")


def test_no_workspace_host_mode_and_int64():
    """Host mode copies its result back from the scratch (no pinned buffer);
    int32 sums into int64 are exact."""
    for n in (10**7 + 3, 1000):
        x = W.uniform(n, -1.0, 1.0, 16100 + n % 7)
        _both(x, (n,), (1,), mode="host", init=0.25)
        xi = W.randint(n, -10**6, 10**6, 16200 + n % 7)
        _both(xi, (n,), (1,), acc=torch.int64, out_dtype=torch.int64, mode="host")
    xi = W.randint(8192 * 4096, -2**20, 2**20, 16300)
    _both(xi, (8192, 4096), (2,), acc=torch.int64, out_dtype=torch.int64)


def test_no_workspace_rejects_bad_arguments_like_the_workspace_call():
    rk = _rk()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = torch.full((1,), 7.0, device=DEV)
    x = torch.ones(100, device=DEV)
    assert rk.rk_reduce_dims_no_workspace(0, 0, rk.RK_F32, rk.RK_F32, rk.RK_F32, x.data_ptr(), 1, (100,), (1,), 1,
                                          None, 9, out.data_ptr(), st) == rk.RK_ERR_INVALID_ARGUMENT
    assert rk.rk_reduce_dims_no_workspace(0, 0, rk.RK_F32, rk.RK_BF16, rk.RK_F32, x.data_ptr(), 1, (100,), (1,), 1,
                                          None, 0, out.data_ptr(), st) == rk.RK_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert float(out.item()) == 7.0
    assert "scratch" in rk.status_string(rk.RK_ERR_TOO_LARGE)
