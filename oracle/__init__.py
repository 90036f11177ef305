"""CPU oracle for the device-wide mapreduce -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product library never does, and this package never
imports the product: the two share no code.

The arithmetic lives in ``oracle.c`` (a sequential left-to-right fold with a
double or int64 accumulator, see the header there).  This module only loads
the compiled library, marshals numpy arrays, and picks the fold's starting
value from the finishing mode, following AcceleratedKernels.jl PR #139
("Finish whole-array reductions on the device"), section "What changes": the
last pass either applies ``init`` or continues from the output's previous
value, or hands back a bare partial that the host finishes with ``init``.
Section "Compatibility" of the same page fixes that ``init`` enters once.

Dtype, op, map and mode codes here are this package's own constants; their
integer values equal those of the library's public header so that a test can
hand the same numbers to both sides.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

SUM, MAX, MIN = 0, 1, 2
IDENTITY, SQUARE, ABS = 0, 1, 2
MUL, SQDIFF, ABSDIFF = 0, 1, 2          # two-input maps f(a, b)
F32, BF16, F16, F64, I32, I64 = 0, 1, 2, 3, 4, 5
OVERWRITE, FOLD, HOST = 0, 1, 2

FP_DTYPES = (F32, BF16, F16, F64)
INT_DTYPES = (I32, I64)
# numpy storage used for the raw bits of each dtype (bf16 and f16 as uint16)
STORAGE = {F32: np.float32, BF16: np.uint16, F16: np.uint16, F64: np.float64,
           I32: np.int32, I64: np.int64}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# RKO_LIB points the loader at another build of oracle.c (the mutation tests
# load deliberately broken copies this way); it is never built from here.
_LIB_OVERRIDE = os.environ.get("RKO_LIB")
GCC_CMD = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
           "-fPIC", "-shared", "-o", _LIB_PATH, _SRC, "-lm"]

_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so next to it (gcc, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        subprocess.run(GCC_CMD, check=True)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
    i32, i64, u32, dbl = ctypes.c_int, ctypes.c_int64, ctypes.c_uint32, ctypes.c_double
    vp = ctypes.c_void_p
    lib.rko_identity_fp.argtypes, lib.rko_identity_fp.restype = [i32], dbl
    lib.rko_identity_int.argtypes, lib.rko_identity_int.restype = [i32, i32], i64
    lib.rko_all_fp.argtypes = [i32, i32, i32, vp, i64, dbl, vp]
    lib.rko_all_int.argtypes = [i32, i32, i32, i32, vp, i64, i64, vp]
    lib.rko_all2_fp.argtypes = [i32, i32, i32, vp, vp, i64, dbl, vp]
    lib.rko_all2_int.argtypes = [i32, i32, i32, i32, vp, vp, i64, i64, vp]
    lib.rko_dims_fp.argtypes = [i32, i32, i32, vp, i32, vp, vp, u32, vp, vp]
    lib.rko_dims_int.argtypes = [i32, i32, i32, i32, vp, i32, vp, vp, u32, vp, vp]
    lib.rko_cast_fp.argtypes = [i32, vp, i64, vp]
    lib.rko_cast_int.argtypes = [i32, vp, i64, vp]
    lib.rko_widen_fp.argtypes = [i32, vp, i64, vp]
    lib.rko_widen_int.argtypes = [i32, vp, i64, vp]
    lib.rko_scan_fp.argtypes = [i32, i32, vp, i64, dbl, i32, vp]
    lib.rko_scan_int.argtypes = [i32, i32, i32, vp, i64, i64, i32, vp]
    lib.rko_scan_dims_fp.argtypes = [i32, i32, vp, i32, vp, vp, i32, dbl, i32, vp]
    lib.rko_scan_dims_int.argtypes = [i32, i32, i32, vp, i32, vp, vp, i32, i64, i32, vp]
    for name in ("rko_all_fp", "rko_all_int", "rko_all2_fp", "rko_all2_int", "rko_dims_fp", "rko_dims_int",
                 "rko_cast_fp", "rko_cast_int", "rko_widen_fp", "rko_widen_int", "rko_scan_fp",
                 "rko_scan_int", "rko_scan_dims_fp", "rko_scan_dims_int"):
        getattr(lib, name).restype = i32
    _lib = lib
    return lib


def is_fp(dtype: int) -> bool:
    return dtype in FP_DTYPES


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _raw(x: np.ndarray, dtype: int) -> np.ndarray:
    """The raw storage of x as the numpy type that holds `dtype`'s bits."""
    want = STORAGE[dtype]
    x = np.asarray(x)
    if x.dtype != want:
        if x.dtype.itemsize != np.dtype(want).itemsize:
            raise TypeError(f"array of {x.dtype} cannot hold dtype code {dtype}")
        x = x.view(want)
    return x


def identity(op: int, acc_dtype: int):
    """The op's neutral element in the accumulator type."""
    lib = _load()
    if is_fp(acc_dtype):
        return float(lib.rko_identity_fp(op))
    return int(lib.rko_identity_int(op, acc_dtype))


def wrap_int(value: int, dtype: int) -> int:
    """Two's-complement wrap of a Python int to an integer dtype's width."""
    bits = 32 if dtype == I32 else 64
    v = value & ((1 << bits) - 1)
    return v - (1 << bits) if v >> (bits - 1) else v


def reduce_all(op: int, map_: int, in_dtype: int, acc_dtype: int,
               x: np.ndarray, start):
    """Sequential fold of a contiguous 1-d array; returns the wide result."""
    lib = _load()
    x = np.ascontiguousarray(_raw(x, in_dtype)).reshape(-1)
    n = x.size
    if is_fp(in_dtype):
        out = np.zeros(1, np.float64)
        rc = lib.rko_all_fp(op, map_, in_dtype, _ptr(x), n, float(start), _ptr(out))
        if rc:
            raise ValueError("oracle rejected arguments")
        return float(out[0])
    out = np.zeros(1, np.int64)
    rc = lib.rko_all_int(op, map_, in_dtype, acc_dtype, _ptr(x), n,
                         wrap_int(int(start), I64), _ptr(out))
    if rc:
        raise ValueError("oracle rejected arguments")
    return int(out[0])


def reduce_all2(op: int, map2: int, in_dtype: int, acc_dtype: int, a: np.ndarray,
                b: np.ndarray, start):
    """Sequential fold of f(a_i, b_i) over two contiguous 1-d arrays."""
    lib = _load()
    a = np.ascontiguousarray(_raw(a, in_dtype)).reshape(-1)
    b = np.ascontiguousarray(_raw(b, in_dtype)).reshape(-1)
    if a.size != b.size:
        raise ValueError("inputs differ in length")
    if is_fp(in_dtype):
        out = np.zeros(1, np.float64)
        rc = lib.rko_all2_fp(op, map2, in_dtype, _ptr(a), _ptr(b), a.size, float(start), _ptr(out))
        if rc:
            raise ValueError("oracle rejected arguments")
        return float(out[0])
    out = np.zeros(1, np.int64)
    rc = lib.rko_all2_int(op, map2, in_dtype, acc_dtype, _ptr(a), _ptr(b), a.size,
                          wrap_int(int(start), I64), _ptr(out))
    if rc:
        raise ValueError("oracle rejected arguments")
    return int(out[0])


def expected_all2(op, map2, in_dtype, acc_dtype, out_dtype, a, b, mode, init=None, prev=None):
    """(wide result, raw stored output) of a two-input whole-array reduction."""
    s = start_value(op, acc_dtype, out_dtype, mode, init, prev)
    if mode == FOLD:
        s = s[0]
    r = reduce_all2(op, map2, in_dtype, acc_dtype, a, b, s)
    if not is_fp(acc_dtype):
        r = wrap_int(r, acc_dtype)
    return r, cast(out_dtype, [r])


def reduce_dims(op: int, map_: int, in_dtype: int, acc_dtype: int,
                storage: np.ndarray, shape, strides, mask: int, start):
    """Per-output sequential fold of a strided column-major view.

    `storage` is the flat buffer, `shape`/`strides` (elements) describe the
    view starting at storage[0], `mask` has bit d set when dim d is reduced.
    `start` is a scalar or one wide value per output.  Returns an array of
    wide results (float64 or int64), one per output in column-major order of
    the kept dims.
    """
    lib = _load()
    storage = np.ascontiguousarray(_raw(storage, in_dtype)).reshape(-1)
    shape_a = np.asarray(shape, np.int64)
    strides_a = np.asarray(strides, np.int64)
    ndim = shape_a.size
    if ndim:
        last = int(sum((s - 1) * st for s, st in zip(shape_a, strides_a) if s > 0))
        if int(np.prod(shape_a)) > 0 and last >= storage.size:
            raise ValueError("view reaches past the end of storage")
    n_out = int(np.prod([s for d, s in enumerate(shape_a) if not (mask >> d) & 1]))
    if is_fp(in_dtype):
        st = np.broadcast_to(np.asarray(start, np.float64), (n_out,)).copy()
        res = np.zeros(n_out, np.float64)
        rc = lib.rko_dims_fp(op, map_, in_dtype, _ptr(storage), ndim, _ptr(shape_a),
                             _ptr(strides_a), mask, _ptr(st), _ptr(res))
    else:
        st = np.array([wrap_int(int(v), I64) for v in
                       np.broadcast_to(np.asarray(start, dtype=object), (n_out,))],
                      np.int64)
        res = np.zeros(n_out, np.int64)
        rc = lib.rko_dims_int(op, map_, in_dtype, acc_dtype, _ptr(storage), ndim,
                              _ptr(shape_a), _ptr(strides_a), mask, _ptr(st), _ptr(res))
    if rc:
        raise ValueError("oracle rejected arguments")
    return res


def cast(out_dtype: int, wide) -> np.ndarray:
    """Store wide results in out_dtype (RNE for fp, wrap for int) as raw storage."""
    lib = _load()
    if is_fp(out_dtype):
        v = np.ascontiguousarray(np.asarray(wide, np.float64).reshape(-1))
        dst = np.zeros(v.size, STORAGE[out_dtype])
        rc = lib.rko_cast_fp(out_dtype, _ptr(v), v.size, _ptr(dst))
    else:
        v = np.ascontiguousarray(np.asarray(wide, np.int64).reshape(-1))
        dst = np.zeros(v.size, STORAGE[out_dtype])
        rc = lib.rko_cast_int(out_dtype, _ptr(v), v.size, _ptr(dst))
    if rc:
        raise ValueError("bad output dtype")
    return dst


def widen(dtype: int, raw: np.ndarray) -> np.ndarray:
    """Decode stored values of a dtype to float64 (fp) or int64 (int)."""
    lib = _load()
    raw = np.ascontiguousarray(_raw(raw, dtype)).reshape(-1)
    if is_fp(dtype):
        dst = np.zeros(raw.size, np.float64)
        rc = lib.rko_widen_fp(dtype, _ptr(raw), raw.size, _ptr(dst))
    else:
        dst = np.zeros(raw.size, np.int64)
        rc = lib.rko_widen_int(dtype, _ptr(raw), raw.size, _ptr(dst))
    if rc:
        raise ValueError("bad dtype")
    return dst


def start_value(op: int, acc_dtype: int, out_dtype: int, mode: int, init=None, prev=None):
    """The value the fold starts from, per finishing mode.

    overwrite and host: `init` (the op's identity when None), applied once;
    fold: the output's previous value `prev` (raw out storage) read back into
    the accumulator type; `init` is not applied again.
    """
    if mode == FOLD:
        w = widen(out_dtype, np.asarray(prev).reshape(-1))
        if is_fp(acc_dtype):
            return w
        return np.array([wrap_int(int(v), acc_dtype) for v in w], dtype=object)
    if init is None:
        return identity(op, acc_dtype)
    return init if is_fp(acc_dtype) else wrap_int(int(init), acc_dtype)


def expected_all(op, map_, in_dtype, acc_dtype, out_dtype, x, mode, init=None, prev=None):
    """(wide result, raw stored output) of a whole-array reduction."""
    s = start_value(op, acc_dtype, out_dtype, mode, init, prev)
    if mode == FOLD:
        s = s[0]
    r = reduce_all(op, map_, in_dtype, acc_dtype, x, s)
    if not is_fp(acc_dtype):
        r = wrap_int(r, acc_dtype)
    return r, cast(out_dtype, [r])


def expected_dims(op, map_, in_dtype, acc_dtype, out_dtype, storage, shape, strides,
                  mask, mode, init=None, prev=None):
    """(wide results, raw stored outputs) of a reduction along dims."""
    s = start_value(op, acc_dtype, out_dtype, mode, init, prev)
    r = reduce_dims(op, map_, in_dtype, acc_dtype, storage, shape, strides, mask, s)
    return r, cast(out_dtype, r)


def scan(op: int, in_dtype: int, acc_dtype: int, x: np.ndarray, start, inclusive: bool) -> np.ndarray:
    """Prefix fold of a contiguous 1-d array: one wide value per element
    (float64 or int64 wrapped to the accumulator width)."""
    lib = _load()
    x = np.ascontiguousarray(_raw(x, in_dtype)).reshape(-1)
    if is_fp(in_dtype):
        out = np.zeros(x.size, np.float64)
        rc = lib.rko_scan_fp(op, in_dtype, _ptr(x), x.size, float(start), int(bool(inclusive)), _ptr(out))
    else:
        out = np.zeros(x.size, np.int64)
        rc = lib.rko_scan_int(op, in_dtype, acc_dtype, _ptr(x), x.size, wrap_int(int(start), I64),
                              int(bool(inclusive)), _ptr(out))
    if rc:
        raise ValueError("oracle rejected arguments")
    return out


def scan_dims(op: int, in_dtype: int, acc_dtype: int, storage: np.ndarray, shape, strides, dim: int,
              start, inclusive: bool) -> np.ndarray:
    """Prefix fold along `dim` (0-based) of a strided column-major view of
    `storage`; returns the wide results for the view's shape, flat in
    column-major order."""
    lib = _load()
    storage = np.ascontiguousarray(_raw(storage, in_dtype)).reshape(-1)
    shape_a = np.asarray(shape, np.int64)
    strides_a = np.asarray(strides, np.int64)
    total = int(np.prod(shape_a))
    if total > 0:
        last = int(sum((s - 1) * st for s, st in zip(shape_a, strides_a)))
        if last >= storage.size:
            raise ValueError("view reaches past the end of storage")
    if is_fp(in_dtype):
        out = np.zeros(total, np.float64)
        rc = lib.rko_scan_dims_fp(op, in_dtype, _ptr(storage), shape_a.size, _ptr(shape_a), _ptr(strides_a),
                                  int(dim), float(start), int(bool(inclusive)), _ptr(out))
    else:
        out = np.zeros(total, np.int64)
        rc = lib.rko_scan_dims_int(op, in_dtype, acc_dtype, _ptr(storage), shape_a.size, _ptr(shape_a),
                                   _ptr(strides_a), int(dim), wrap_int(int(start), I64),
                                   int(bool(inclusive)), _ptr(out))
    if rc:
        raise ValueError("oracle rejected arguments")
    return out
