"""NaN and infinity inputs (reading s4 of the design: NaN propagates through
sum, max and min, as Julia's and PyTorch's reductions do; the pages print
no result for them, so beyond "the output is NaN" these cases are checked
against what IEEE arithmetic fixes: +inf wins a max, -inf a min, inf + x is
inf, inf - inf is NaN).  Positions cover the scalar head, the vector body,
the last block and the scalar tail of each kernel's split of the input."""
import math

import numpy as np
import pytest
import torch

from reduction_primitives_amd import workloads as W
from tests.parity import raw_np

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _rk():
    import reduction_primitives_amd as rk
    rk.load()
    return rk


def _positions(n):
    return sorted({0, 1, 5, n // 2, n - 2, n - 1})


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16, torch.float64], ids=lambda t: str(t).split(".")[1])
def test_whole_array_nan_propagates(dt):
    rk = _rk()
    n = 3 * 10**6 + 5
    base = W.uniform(n, -1.0, 1.0, 16000).to(dt)
    for i in _positions(n):
        x = base.clone()
        x[i] = float("nan")
        xd = x.to(DEV)[1:] if i > 0 else x.to(DEV)          # also an unaligned view
        for op in ("sum", "max", "min"):
            r = rk.reduce_all(xd, op=op, acc=torch.float64 if dt == torch.float64 else torch.float32,
                              out_dtype=torch.float64 if dt == torch.float64 else torch.float32)
            assert math.isnan(float(r.item())), (i, op)
        assert math.isnan(rk.reduce_all(xd, mode="host"))


def test_whole_array_infinities():
    rk = _rk()
    n = 2 * 10**6 + 3
    x = W.uniform(n, -1.0, 1.0, 16010)
    x[n // 3] = float("inf")
    x[2 * n // 3] = float("-inf")
    xd = x.to(DEV)
    assert float(rk.reduce_all(xd, op="max").item()) == math.inf
    assert float(rk.reduce_all(xd, op="min").item()) == -math.inf
    assert math.isnan(float(rk.reduce_all(xd).item()))              # inf + (-inf)
    y = x.clone()
    y[2 * n // 3] = 0.5
    assert float(rk.reduce_all(y.to(DEV)).item()) == math.inf


@pytest.mark.parametrize("shape,dims", [((1000, 300), 2), ((300, 1000), 1), ((8192, 64), 2), ((64, 50, 7), 2),
                                        ((3136, 16, 24), (1, 3))], ids=str)
def test_dims_nan_stays_in_its_output(shape, dims):
    rk = _rk()
    st = W.cm_strides(shape)
    n = math.prod(shape)
    x = W.uniform(n, -1.0, 1.0, 16020 + n % 97)
    dims_t = (dims,) if isinstance(dims, int) else dims
    kept = [i for i in range(len(shape)) if i + 1 not in dims_t]
    idx = [0] * len(shape)
    for i in range(len(shape)):
        idx[i] = shape[i] // 2
    flat = sum(ix * s for ix, s in zip(idx, st))
    x[flat] = float("nan")
    for op in ("sum", "max", "min"):
        r = raw_np(rk.reduce_dims(x.to(DEV), shape, st, dims, op=op))
        out_shape = [shape[i] for i in kept]
        o = 0
        mul = 1
        for k, i in enumerate(kept):
            o += idx[i] * mul
            mul *= shape[i]
        assert np.isnan(r[o]), (op, o)
        assert np.isnan(r).sum() == 1, (op, int(np.isnan(r).sum()))


def test_two_input_nan_and_scan_nan():
    rk = _rk()
    n = 10**6 + 7
    a = W.uniform(n, -1.0, 1.0, 16030)
    b = W.uniform(n, -1.0, 1.0, 16031)
    a[n - 1] = float("nan")
    for m in ("mul", "sqdiff", "absdiff"):
        assert math.isnan(float(rk.reduce_all2(a.to(DEV), b.to(DEV), m).item()))
    assert math.isnan(float(rk.reduce_all2(a.to(DEV)[1:], b.to(DEV)[:-1], "mul").item()))   # shifted loads
    # scans: NaN from its position on (inclusive), one later (exclusive)
    k = 123457
    x = W.uniform(n, -1.0, 1.0, 16032)
    x[k] = float("nan")
    for op in ("sum", "max", "min"):
        inc = raw_np(rk.scan(x.to(DEV), op=op))
        exc = raw_np(rk.scan(x.to(DEV), op=op, inclusive=False))
        assert not np.isnan(inc[:k]).any() and np.isnan(inc[k:]).all(), op
        assert not np.isnan(exc[:k + 1]).any() and np.isnan(exc[k + 1:]).all(), op
