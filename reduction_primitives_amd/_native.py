"""ctypes binding of librk.so (include/rk.h), argument marshalling only.

The functions here carry the C ABI's names and arguments.  Every step of a
reduction runs in the library's HIP kernels; nothing here computes.  Loading
fails loudly when the library has not been built: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librk.so")

# enums of include/rk.h
RK_OK, RK_ERR_INVALID_ARGUMENT, RK_ERR_UNSUPPORTED, RK_ERR_HIP, RK_ERR_TOO_LARGE = 0, 1, 2, 3, 4
RK_OP_SUM, RK_OP_MAX, RK_OP_MIN = 0, 1, 2
RK_MAP_IDENTITY, RK_MAP_SQUARE, RK_MAP_ABS = 0, 1, 2
RK_MAP2_MUL, RK_MAP2_SQDIFF, RK_MAP2_ABSDIFF = 0, 1, 2
RK_F32, RK_BF16, RK_F16, RK_F64, RK_I32, RK_I64 = 0, 1, 2, 3, 4, 5
RK_MODE_OVERWRITE, RK_MODE_FOLD, RK_MODE_HOST = 0, 1, 2
(RK_KERNEL_NONE, RK_KERNEL_ALL, RK_KERNEL_ALL_STRIDED, RK_KERNEL_THREAD, RK_KERNEL_TILED,
 RK_KERNEL_COLUMNS, RK_KERNEL_ROW, RK_KERNEL_GENERIC, RK_KERNEL_ALL2, RK_KERNEL_SCAN_TILE,
 RK_KERNEL_SCAN_ROWWAVE, RK_KERNEL_SCAN_LINES, RK_KERNEL_SCAN_COLUMNS, RK_KERNEL_SCAN_TRANSPOSE) = range(14)
KERNEL_NAMES = {0: "none", 1: "all", 2: "all_strided", 3: "thread", 4: "tiled", 5: "columns",
                6: "row", 7: "generic", 8: "all2", 9: "scan_tile", 10: "scan_rowwave",
                11: "scan_lines", 12: "scan_columns", 13: "scan_transpose"}

# every function include/rk.h declares
EXPORTS = ("rk_workspace_size", "rk_reduce_all", "rk_reduce_all2", "rk_reduce_dims", "rk_status_string",
           "rk_plan_all", "rk_plan_all2", "rk_plan_dims", "rk_debug_set_fused_finish",
           "rk_debug_set_launch_events", "rk_scan_workspace_size", "rk_scan", "rk_scan_dims",
           "rk_plan_scan", "rk_debug_stream_read", "rk_debug_device_info", "rk_debug_set_finish_tag",
           "rk_stream_timeouts", "rk_debug_force_wait_timeout", "rk_debug_fail_launches",
           "rk_reduce_dims_no_workspace")


class rk_plan_info(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int), ("launches", ctypes.c_int), ("grid", ctypes.c_int64),
                ("block", ctypes.c_int), ("split", ctypes.c_int), ("vec", ctypes.c_int),
                ("tile_outputs", ctypes.c_int), ("n_out", ctypes.c_int64),
                ("reduce_len", ctypes.c_int64), ("workspace_bytes", ctypes.c_size_t)]


class RkError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})" if what
                         else f"{status_string(status)} (status {status})")


_lib = None


def load() -> ctypes.CDLL:
    """Load librk.so; raises when it is missing (build it first)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"librk.so not found at {LIB_PATH}; build it with "
            "`python -m reduction_primitives_amd.build` (there is no fallback path)")
    # torch's HIP runtime must be the one the library binds to (same SONAME)
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, u32, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint32,
                             ctypes.c_size_t)
    p64 = ctypes.POINTER(ctypes.c_int64)
    lib.rk_workspace_size.argtypes = [i32, i32, i32, p64, p64, u32]
    lib.rk_workspace_size.restype = sz
    lib.rk_reduce_all.argtypes = [i32, i32, i32, i32, i32, vp, i64, vp, i32, vp, vp, vp]
    lib.rk_reduce_all.restype = i32
    lib.rk_reduce_all2.argtypes = [i32, i32, i32, i32, i32, vp, vp, i64, vp, i32, vp, vp, vp]
    lib.rk_reduce_all2.restype = i32
    lib.rk_reduce_dims.argtypes = [i32, i32, i32, i32, i32, vp, i32, p64, p64, u32, vp, i32, vp, vp, vp]
    lib.rk_reduce_dims.restype = i32
    lib.rk_reduce_dims_no_workspace.argtypes = [i32, i32, i32, i32, i32, vp, i32, p64, p64, u32, vp, i32, vp, vp]
    lib.rk_reduce_dims_no_workspace.restype = i32
    lib.rk_scan_workspace_size.argtypes = [i32, i32, i32, p64, p64, i32]
    lib.rk_scan_workspace_size.restype = sz
    lib.rk_scan.argtypes = [i32, i32, i32, i32, vp, i64, vp, i32, vp, vp, vp]
    lib.rk_scan.restype = i32
    lib.rk_scan_dims.argtypes = [i32, i32, i32, i32, vp, i32, p64, p64, i32, vp, i32, vp, vp, vp]
    lib.rk_scan_dims.restype = i32
    lib.rk_plan_scan.argtypes = [i32, i32, i32, vp, vp, i32, p64, p64, i32, i32, ctypes.POINTER(rk_plan_info)]
    lib.rk_plan_scan.restype = i32
    lib.rk_status_string.argtypes = [i32]
    lib.rk_status_string.restype = ctypes.c_char_p
    lib.rk_plan_all.argtypes = [i32, i32, vp, i64, i32, ctypes.POINTER(rk_plan_info)]
    lib.rk_plan_all.restype = i32
    lib.rk_plan_all2.argtypes = [i32, i32, vp, vp, i64, i32, ctypes.POINTER(rk_plan_info)]
    lib.rk_plan_all2.restype = i32
    lib.rk_plan_dims.argtypes = [i32, i32, vp, i32, p64, p64, u32, i32, ctypes.POINTER(rk_plan_info)]
    lib.rk_plan_dims.restype = i32
    lib.rk_debug_set_fused_finish.argtypes = [i32]
    lib.rk_debug_set_fused_finish.restype = i32
    lib.rk_debug_set_launch_events.argtypes = [vp, vp]
    lib.rk_debug_set_launch_events.restype = i32
    lib.rk_debug_stream_read.argtypes = [vp, i64, i32, vp, vp]
    lib.rk_debug_stream_read.restype = i32
    lib.rk_debug_device_info.argtypes = [p64, p64, p64]
    lib.rk_debug_device_info.restype = i32
    lib.rk_debug_set_finish_tag.argtypes = [vp, u32]
    lib.rk_debug_set_finish_tag.restype = i32
    lib.rk_stream_timeouts.argtypes = [vp, ctypes.POINTER(ctypes.c_uint64)]
    lib.rk_stream_timeouts.restype = i32
    lib.rk_debug_force_wait_timeout.argtypes = [i64]
    lib.rk_debug_force_wait_timeout.restype = i32
    lib.rk_debug_fail_launches.argtypes = [i32]
    lib.rk_debug_fail_launches.restype = i32
    _lib = lib
    return lib


def _i64_array(vals):
    vals = [int(v) for v in vals]
    return (ctypes.c_int64 * max(1, len(vals)))(*vals)


def status_string(status: int) -> str:
    return load().rk_status_string(int(status)).decode()


def rk_workspace_size(in_dtype, acc_dtype, ndim, shape, strides, reduce_mask) -> int:
    return int(load().rk_workspace_size(in_dtype, acc_dtype, ndim, _i64_array(shape),
                                        _i64_array(strides), reduce_mask))


def rk_reduce_all(op, map_, in_dtype, acc_dtype, out_dtype, ptr, n, init, mode, out, workspace,
                  stream) -> int:
    """Raw call; `init` and host-mode `out` are ctypes objects or None/addresses."""
    return int(load().rk_reduce_all(op, map_, in_dtype, acc_dtype, out_dtype, ptr, n, init, mode,
                                    out, workspace, stream))


def rk_reduce_all2(op, map2, in_dtype, acc_dtype, out_dtype, a, b, n, init, mode, out, workspace,
                   stream) -> int:
    return int(load().rk_reduce_all2(op, map2, in_dtype, acc_dtype, out_dtype, a, b, n, init, mode,
                                     out, workspace, stream))


def rk_reduce_dims(op, map_, in_dtype, acc_dtype, out_dtype, ptr, ndim, shape, strides,
                   reduce_mask, init, mode, out, workspace, stream) -> int:
    return int(load().rk_reduce_dims(op, map_, in_dtype, acc_dtype, out_dtype, ptr, ndim,
                                     _i64_array(shape), _i64_array(strides), reduce_mask, init,
                                     mode, out, workspace, stream))


def rk_reduce_dims_no_workspace(op, map_, in_dtype, acc_dtype, out_dtype, ptr, ndim, shape, strides,
                                reduce_mask, init, mode, out, stream) -> int:
    """rk_reduce_dims with the library's scratch in place of a workspace."""
    return int(load().rk_reduce_dims_no_workspace(op, map_, in_dtype, acc_dtype, out_dtype, ptr, ndim,
                                                  _i64_array(shape), _i64_array(strides), reduce_mask, init,
                                                  mode, out, stream))


def rk_plan_all(in_dtype, acc_dtype, ptr, n, num_cus=0) -> rk_plan_info:
    info = rk_plan_info()
    rc = load().rk_plan_all(in_dtype, acc_dtype, ptr, n, num_cus, ctypes.byref(info))
    if rc:
        raise RkError(rc, "rk_plan_all")
    return info


def rk_plan_all2(in_dtype, acc_dtype, a, b, n, num_cus=0) -> rk_plan_info:
    info = rk_plan_info()
    rc = load().rk_plan_all2(in_dtype, acc_dtype, a, b, n, num_cus, ctypes.byref(info))
    if rc:
        raise RkError(rc, "rk_plan_all2")
    return info


def rk_plan_dims(in_dtype, acc_dtype, ptr, ndim, shape, strides, reduce_mask, num_cus=0) -> rk_plan_info:
    info = rk_plan_info()
    rc = load().rk_plan_dims(in_dtype, acc_dtype, ptr, ndim, _i64_array(shape), _i64_array(strides),
                             reduce_mask, num_cus, ctypes.byref(info))
    if rc:
        raise RkError(rc, "rk_plan_dims")
    return info


def rk_scan_workspace_size(in_dtype, acc_dtype, ndim, shape, strides, dim) -> int:
    return int(load().rk_scan_workspace_size(in_dtype, acc_dtype, ndim, _i64_array(shape),
                                             _i64_array(strides), dim))


def rk_scan(op, in_dtype, acc_dtype, out_dtype, ptr, n, init, inclusive, out, workspace, stream) -> int:
    return int(load().rk_scan(op, in_dtype, acc_dtype, out_dtype, ptr, n, init, inclusive, out, workspace,
                              stream))


def rk_scan_dims(op, in_dtype, acc_dtype, out_dtype, ptr, ndim, shape, strides, dim, init, inclusive, out,
                 workspace, stream) -> int:
    return int(load().rk_scan_dims(op, in_dtype, acc_dtype, out_dtype, ptr, ndim, _i64_array(shape),
                                   _i64_array(strides), dim, init, inclusive, out, workspace, stream))


def rk_plan_scan(in_dtype, acc_dtype, out_dtype, ptr, out, ndim, shape, strides, dim, num_cus=0) -> rk_plan_info:
    info = rk_plan_info()
    rc = load().rk_plan_scan(in_dtype, acc_dtype, out_dtype, ptr, out, ndim, _i64_array(shape),
                             _i64_array(strides), dim, num_cus, ctypes.byref(info))
    if rc:
        raise RkError(rc, "rk_plan_scan")
    return info


def rk_debug_set_fused_finish(enable: int) -> int:
    return int(load().rk_debug_set_fused_finish(int(enable)))


def rk_debug_set_launch_events(begin, end) -> int:
    return int(load().rk_debug_set_launch_events(begin, end))


def rk_debug_set_finish_tag(stream, e: int) -> int:
    return int(load().rk_debug_set_finish_tag(stream, int(e)))


def rk_debug_stream_read(ptr, nbytes, grid, sink, stream) -> None:
    rc = load().rk_debug_stream_read(ptr, nbytes, grid, sink, stream)
    if rc:
        raise RkError(rc, "rk_debug_stream_read")


def rk_debug_device_info() -> dict:
    """The current device's compute units, memory clock (kHz) and memory bus
    width (bits)."""
    vals = [ctypes.c_int64() for _ in range(3)]
    rc = load().rk_debug_device_info(*(ctypes.byref(v) for v in vals))
    if rc:
        raise RkError(rc, "rk_debug_device_info")
    return dict(num_cus=vals[0].value, mem_clock_khz=vals[1].value, mem_bus_bits=vals[2].value)


def rk_stream_timeouts(stream) -> int:
    """Waits that gave up in calls on `stream` (a hipStream_t handle) since
    the last query; waits for the stream and clears the count."""
    n = ctypes.c_uint64()
    rc = load().rk_stream_timeouts(stream, ctypes.byref(n))
    if rc:
        raise RkError(rc, "rk_stream_timeouts")
    return int(n.value)


def rk_debug_force_wait_timeout(polls: int) -> int:
    return int(load().rk_debug_force_wait_timeout(int(polls)))


def rk_debug_fail_launches(count: int) -> int:
    return int(load().rk_debug_fail_launches(int(count)))
