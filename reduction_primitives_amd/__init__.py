"""Device-wide mapreduce for AMD Instinct MI355X (gfx950).

Python face of librk.so.  ``rk_reduce_all``, ``rk_reduce_all2``, ``rk_reduce_dims``,
``rk_workspace_size`` and the plan/diagnostic calls keep the C ABI's names
(see include/rk.h); ``reduce_all`` and ``reduce_dims`` below only marshal torch
tensors into those calls (``reduce_all2`` for a two-input source) -- pick dtype codes, allocate the output and the
workspace with torch, pass the current HIP stream.  All arithmetic happens
in the library's kernels; there is no fallback path.
"""
from __future__ import annotations

import contextlib
import ctypes
import math

from ._native import (  # noqa: F401
    EXPORTS, KERNEL_NAMES, LIB_PATH, RK_BF16, RK_ERR_HIP, RK_ERR_INVALID_ARGUMENT, RK_ERR_TOO_LARGE,
    RK_ERR_UNSUPPORTED, RK_F16, RK_F32, RK_F64, RK_I32, RK_I64, RK_KERNEL_ALL,
    RK_KERNEL_ALL2, RK_KERNEL_ALL_STRIDED, RK_KERNEL_COLUMNS, RK_KERNEL_GENERIC, RK_KERNEL_NONE,
    RK_KERNEL_ROW, RK_KERNEL_SCAN_COLUMNS, RK_KERNEL_SCAN_LINES, RK_KERNEL_SCAN_ROWWAVE, RK_KERNEL_SCAN_TILE,
    RK_KERNEL_SCAN_TRANSPOSE, RK_KERNEL_THREAD,
    RK_KERNEL_TILED, RK_MAP2_ABSDIFF, RK_MAP2_MUL, RK_MAP2_SQDIFF,
    RK_MAP_ABS, RK_MAP_IDENTITY, RK_MAP_SQUARE,
    RK_MODE_FOLD, RK_MODE_HOST, RK_MODE_OVERWRITE, RK_OK, RK_OP_MAX, RK_OP_MIN, RK_OP_SUM,
    RkError, load, rk_debug_device_info, rk_debug_fail_launches, rk_debug_force_wait_timeout,
    rk_debug_set_finish_tag, rk_debug_set_fused_finish, rk_debug_set_launch_events, rk_stream_timeouts,
    rk_debug_stream_read, rk_plan_all, rk_plan_all2, rk_plan_dims,
    rk_plan_info, rk_plan_scan, rk_reduce_all, rk_reduce_all2, rk_reduce_dims, rk_reduce_dims_no_workspace,
    rk_scan, rk_scan_dims,
    rk_scan_workspace_size, rk_workspace_size, status_string)

OPS = {"sum": RK_OP_SUM, "max": RK_OP_MAX, "min": RK_OP_MIN}
MAPS = {"identity": RK_MAP_IDENTITY, "square": RK_MAP_SQUARE, "abs": RK_MAP_ABS}
MAPS2 = {"mul": RK_MAP2_MUL, "sqdiff": RK_MAP2_SQDIFF, "absdiff": RK_MAP2_ABSDIFF}
MODES = {"overwrite": RK_MODE_OVERWRITE, "fold": RK_MODE_FOLD, "host": RK_MODE_HOST}
DTYPE_SIZE = {RK_F32: 4, RK_BF16: 2, RK_F16: 2, RK_F64: 8, RK_I32: 4, RK_I64: 8}
_CTYPE = {RK_F32: ctypes.c_float, RK_F64: ctypes.c_double, RK_I32: ctypes.c_int32,
          RK_I64: ctypes.c_int64, RK_BF16: ctypes.c_uint16, RK_F16: ctypes.c_uint16}


def _torch():
    import torch
    return torch


_DTYPE_CODES = None


def dtype_code(dt) -> int:
    """rk dtype code of a torch dtype (or pass an int code through)."""
    global _DTYPE_CODES
    if isinstance(dt, int):
        return dt
    if _DTYPE_CODES is None:
        torch = _torch()
        _DTYPE_CODES = {torch.float32: RK_F32, torch.bfloat16: RK_BF16, torch.float16: RK_F16,
                        torch.float64: RK_F64, torch.int32: RK_I32, torch.int64: RK_I64}
    return _DTYPE_CODES[dt]


def torch_dtype(code: int):
    torch = _torch()
    return {RK_F32: torch.float32, RK_BF16: torch.bfloat16, RK_F16: torch.float16,
            RK_F64: torch.float64, RK_I32: torch.int32, RK_I64: torch.int64}[code]


def default_acc(in_code: int) -> int:
    """f32 for floating inputs up to 4 bytes, f64 for f64, i64 for integers."""
    if in_code in (RK_F32, RK_BF16, RK_F16):
        return RK_F32
    if in_code == RK_F64:
        return RK_F64
    return RK_I64


def _code(table, v):
    return table[v] if isinstance(v, str) else int(v)


def init_arg(acc_code: int, init):
    """Host buffer holding `init` in the accumulator type (None -> NULL)."""
    if init is None:
        return None
    ct = _CTYPE[acc_code]
    return ctypes.byref(ct(init if acc_code in (RK_F32, RK_F64) else int(init)))


def decode_host_out(buf, out_code: int):
    """Python value of a host-mode output buffer."""
    v = buf.value
    if out_code == RK_BF16:
        return ctypes.c_float.from_buffer_copy(ctypes.c_uint32(v << 16)).value
    if out_code == RK_F16:
        import numpy as np
        return float(np.array([v], np.uint16).view(np.float16)[0])
    return v


def _stream_handle(stream, device_index=None):
    """hipStream_t of `stream`, or of the current stream of the device (read
    without building a Stream object: host-mode calls are latency-bound)."""
    torch = _torch()
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream)
    if device_index is None:
        device_index = torch.cuda.current_device()
    return ctypes.c_void_p(torch._C._cuda_getCurrentRawStream(device_index))


def _on(stream):
    """Allocate on `stream` when one is given: a buffer the call allocates
    (workspace, output) then belongs to the stream its kernels run on, so
    the caching allocator hands its bytes to no other stream's work before
    those kernels are done (it is freed, or returned, while they may still
    run)."""
    if stream is None:
        return contextlib.nullcontext()
    return _torch().cuda.stream(stream)


def workspace_for(nbytes: int, device):
    torch = _torch()
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _check(rc, what):
    if rc != RK_OK:
        raise RkError(rc, what)


def reduce_all(x, op="sum", map="identity", acc=None, out_dtype=None, init=None,
               mode="overwrite", out=None, workspace=None, stream=None):
    """Whole-array reduction of a contiguous device tensor (views with a
    storage offset are fine).  Returns `out` (device modes) or a Python value
    (host mode)."""
    torch = _torch()
    if not x.is_contiguous():
        raise ValueError("reduce_all takes a contiguous tensor; use reduce_dims for views")
    in_code = dtype_code(x.dtype)
    acc_code = default_acc(in_code) if acc is None else dtype_code(acc)
    out_code = in_code if out_dtype is None else dtype_code(out_dtype)
    if out_code in (RK_I32, RK_I64) and in_code in (RK_I32, RK_I64) and out_dtype is None:
        out_code = acc_code
    op_c, map_c, mode_c = _code(OPS, op), _code(MAPS, map), _code(MODES, mode)
    n = x.numel()
    with _on(stream):
        if workspace is None:
            workspace = workspace_for(rk_workspace_size(in_code, acc_code, 1, [n], [1], 1), x.device)
        if out is None and mode_c != RK_MODE_HOST:
            out = torch.empty(1, dtype=torch_dtype(out_code), device=x.device)
    st = _stream_handle(stream, x.get_device())
    if mode_c == RK_MODE_HOST:
        buf = _CTYPE[out_code]()
        rc = rk_reduce_all(op_c, map_c, in_code, acc_code, out_code, x.data_ptr(), n,
                           init_arg(acc_code, init), mode_c, ctypes.addressof(buf),
                           workspace.data_ptr(), st)
        _check(rc, "rk_reduce_all")
        return decode_host_out(buf, out_code)
    rc = rk_reduce_all(op_c, map_c, in_code, acc_code, out_code, x.data_ptr(), n,
                       init_arg(acc_code, init), mode_c, out.data_ptr(), workspace.data_ptr(), st)
    _check(rc, "rk_reduce_all")
    return out


def reduce_all2(a, b, map2="mul", op="sum", acc=None, out_dtype=None, init=None,
                mode="overwrite", out=None, workspace=None, stream=None):
    """Whole-array reduction of f(a_i, b_i) over two contiguous device
    tensors of one dtype and size (map2: "mul", "sqdiff" or "absdiff").
    Returns `out` (device modes) or a Python value (host mode)."""
    torch = _torch()
    if not (a.is_contiguous() and b.is_contiguous()):
        raise ValueError("reduce_all2 takes contiguous tensors")
    if a.dtype != b.dtype or a.numel() != b.numel():
        raise ValueError("reduce_all2 takes two tensors of one dtype and size")
    in_code = dtype_code(a.dtype)
    acc_code = default_acc(in_code) if acc is None else dtype_code(acc)
    out_code = in_code if out_dtype is None else dtype_code(out_dtype)
    if out_code in (RK_I32, RK_I64) and in_code in (RK_I32, RK_I64) and out_dtype is None:
        out_code = acc_code
    op_c, map_c, mode_c = _code(OPS, op), _code(MAPS2, map2), _code(MODES, mode)
    n = a.numel()
    with _on(stream):
        if workspace is None:
            workspace = workspace_for(rk_workspace_size(in_code, acc_code, 1, [n], [1], 1), a.device)
        if out is None and mode_c != RK_MODE_HOST:
            out = torch.empty(1, dtype=torch_dtype(out_code), device=a.device)
    st = _stream_handle(stream, a.get_device())
    if mode_c == RK_MODE_HOST:
        buf = _CTYPE[out_code]()
        rc = rk_reduce_all2(op_c, map_c, in_code, acc_code, out_code, a.data_ptr(), b.data_ptr(), n,
                            init_arg(acc_code, init), mode_c, ctypes.addressof(buf),
                            workspace.data_ptr(), st)
        _check(rc, "rk_reduce_all2")
        return decode_host_out(buf, out_code)
    rc = rk_reduce_all2(op_c, map_c, in_code, acc_code, out_code, a.data_ptr(), b.data_ptr(), n,
                        init_arg(acc_code, init), mode_c, out.data_ptr(), workspace.data_ptr(), st)
    _check(rc, "rk_reduce_all2")
    return out


def reduce_dims(x, shape, strides, dims, op="sum", map="identity", acc=None, out_dtype=None,
                init=None, mode="overwrite", out=None, workspace=None, stream=None, offset=0):
    """Reduction along `dims` (1-based, Julia style) of the column-major view
    (shape, strides in elements) of device tensor x's storage, starting
    `offset` elements into x.  Returns `out` (flat, column-major over the
    kept dims) or, in host mode, a Python value."""
    torch = _torch()
    in_code = dtype_code(x.dtype)
    acc_code = default_acc(in_code) if acc is None else dtype_code(acc)
    out_code = in_code if out_dtype is None else dtype_code(out_dtype)
    if out_code in (RK_I32, RK_I64) and in_code in (RK_I32, RK_I64) and out_dtype is None:
        out_code = acc_code
    if isinstance(dims, int):
        dims = (dims,)
    mask = 0
    for d in dims:
        mask |= 1 << (int(d) - 1)
    op_c, map_c, mode_c = _code(OPS, op), _code(MAPS, map), _code(MODES, mode)
    ndim = len(shape)
    n_out = math.prod(int(s) for i, s in enumerate(shape) if not (mask >> i) & 1)
    ptr = x.data_ptr() + int(offset) * x.element_size()
    with _on(stream):
        if workspace is None:
            workspace = workspace_for(rk_workspace_size(in_code, acc_code, ndim, shape, strides, mask),
                                      x.device)
        if out is None and mode_c != RK_MODE_HOST:
            out = torch.empty(max(n_out, 1), dtype=torch_dtype(out_code), device=x.device)
    st = _stream_handle(stream, x.get_device())
    if mode_c == RK_MODE_HOST:
        buf = _CTYPE[out_code]()
        rc = rk_reduce_dims(op_c, map_c, in_code, acc_code, out_code, ptr, ndim, shape, strides,
                            mask, init_arg(acc_code, init), mode_c, ctypes.addressof(buf),
                            workspace.data_ptr(), st)
        _check(rc, "rk_reduce_dims")
        return decode_host_out(buf, out_code)
    rc = rk_reduce_dims(op_c, map_c, in_code, acc_code, out_code, ptr, ndim, shape, strides, mask,
                        init_arg(acc_code, init), mode_c, out.data_ptr(), workspace.data_ptr(), st)
    _check(rc, "rk_reduce_dims")
    return out


def scan(x, shape=None, strides=None, dim=1, op="sum", acc=None, out_dtype=None, init=None,
         inclusive=True, out=None, workspace=None, stream=None, offset=0):
    """Scan along `dim` (1-based, Julia style) of the column-major view
    (shape, strides in elements) of device tensor x's storage, starting
    `offset` elements into x; shape/strides default to x as a flat 1-d
    array.  Returns `out`: the view's shape, flat, column-major.  `out` may
    be x itself for an in-place scan of a contiguous view."""
    torch = _torch()
    in_code = dtype_code(x.dtype)
    acc_code = default_acc(in_code) if acc is None else dtype_code(acc)
    out_code = in_code if out_dtype is None else dtype_code(out_dtype)
    if out_code in (RK_I32, RK_I64) and in_code in (RK_I32, RK_I64) and out_dtype is None:
        out_code = acc_code
    if shape is None:
        shape, strides = (x.numel() - int(offset),), (1,)
    d0 = int(dim) - 1
    total = math.prod(int(s) for s in shape)
    ptr = x.data_ptr() + int(offset) * x.element_size()
    with _on(stream):
        if workspace is None:
            workspace = workspace_for(rk_scan_workspace_size(in_code, acc_code, len(shape), shape, strides, d0),
                                      x.device)
        if out is None:
            out = torch.empty(max(total, 1), dtype=torch_dtype(out_code), device=x.device)
    rc = rk_scan_dims(_code(OPS, op), in_code, acc_code, out_code, ptr, len(shape), shape, strides, d0,
                      init_arg(acc_code, init), int(bool(inclusive)), out.data_ptr(), workspace.data_ptr(),
                      _stream_handle(stream, x.get_device()))
    _check(rc, "rk_scan_dims")
    return out


def plan_scan(dtype, shape, strides, dim, acc=None, out_dtype=None, ptr=0, out=0, num_cus=0) -> dict:
    """The plan rk_scan_dims would use, as a dict (no launch)."""
    in_code = dtype_code(dtype)
    acc_code = default_acc(in_code) if acc is None else dtype_code(acc)
    out_code = acc_code if out_dtype is None else dtype_code(out_dtype)
    info = rk_plan_scan(in_code, acc_code, out_code, ptr, out, len(shape), shape, strides, int(dim) - 1, num_cus)
    d = {f: getattr(info, f) for f, _ in rk_plan_info._fields_}
    d["kernel_name"] = KERNEL_NAMES[info.kernel]
    return d


def plan_dims(dtype, shape, strides, dims, acc=None, ptr=0, num_cus=0) -> dict:
    """The plan rk_reduce_dims would use, as a dict (no launch)."""
    in_code = dtype_code(dtype)
    acc_code = default_acc(in_code) if acc is None else dtype_code(acc)
    if isinstance(dims, int):
        dims = (dims,)
    mask = 0
    for d in dims:
        mask |= 1 << (int(d) - 1)
    info = rk_plan_dims(in_code, acc_code, ptr, len(shape), shape, strides, mask, num_cus)
    d = {f: getattr(info, f) for f, _ in rk_plan_info._fields_}
    d["kernel_name"] = KERNEL_NAMES[info.kernel]
    return d
