"""Parity helpers: run the HIP path and the CPU oracle on the same bytes and
compare them to the stated bar.

Bar (per output, in float64):
  * integer results, and max/min of any type: bit-exact;
  * f32 / f64 outputs:  |gpu - R| <= 1e-5 * S
  * bf16 outputs:       |gpu - R| <= 8e-3 * |R| + 1e-5 * S
  * f16 outputs:        |gpu - R| <= 1e-3 * |R| + 1e-5 * S
where R is the oracle's wide result and S = |s| + sum |f(x_i)| (s the
starting value).  The f32 bound holds for a fold whose longest chain of
rounded float32 operations is below about 160 (1e-5 / 2^-24); the kernels
keep every chain far shorter (independent accumulators per thread, then
trees).  bf16 output adds one final rounding (relative 2^-9 = 2e-3 < 8e-3).

A sum whose exact value overflows the output type has no finite value to
compare, so it passes only where a test asks for that case by name
(allow_inf=True); everywhere else an infinite expected value fails, so no
draw can hide a kernel's value behind an overflow on both sides.
"""
from __future__ import annotations

import numpy as np

import oracle as O


def raw_np(t) -> np.ndarray:
    """Raw host bytes of a torch tensor as the oracle's storage type."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def code_of(dt) -> int:
    import torch
    return {torch.float32: O.F32, torch.bfloat16: O.BF16, torch.float16: O.F16,
            torch.float64: O.F64, torch.int32: O.I32, torch.int64: O.I64}[dt]


def magnitude(map_, in_code, acc_code, x_raw, start, reduce=None):
    """S = |s| + sum |f(x)| via the oracle (wide, per output when `reduce`)."""
    if not O.is_fp(in_code):
        return None
    m = O.SQUARE if map_ == O.SQUARE else O.ABS
    if reduce is None:
        return abs(float(start)) + O.reduce_all(O.SUM, m, in_code, acc_code, x_raw, 0.0)
    storage, shape, strides, mask = reduce
    s = O.reduce_dims(O.SUM, m, in_code, acc_code, storage, shape, strides, mask, 0.0)
    return np.abs(np.broadcast_to(np.asarray(start, np.float64), s.shape)) + s


def tolerance(out_code, R, S):
    R = np.abs(np.asarray(R, np.float64))
    S = np.asarray(S, np.float64)
    if out_code == O.BF16:
        return 8e-3 * R + 1e-5 * S
    if out_code == O.F16:
        return 1e-3 * R + 1e-5 * S
    return 1e-5 * S


def check(op, out_code, gpu_raw, R, S, what="", allow_inf=False):
    """Assert the GPU's stored outputs meet the bar against oracle results R.
    allow_inf: a sum whose oracle value rounds to +-inf in the output type
    may match that infinity (an overflow test); otherwise it fails."""
    gpu_raw = np.asarray(gpu_raw).reshape(-1)
    if not O.is_fp(out_code):
        want = O.cast(out_code, np.asarray(R, np.int64).reshape(-1))
        bad = np.nonzero(gpu_raw.astype(np.int64) != want.astype(np.int64))[0]
        assert bad.size == 0, f"{what}: {bad.size} integer mismatches, first at {bad[0]}: " \
                              f"gpu {gpu_raw[bad[0]]} oracle {want[bad[0]]}"
        return
    g = O.widen(out_code, gpu_raw)
    R = np.asarray(R, np.float64).reshape(-1)
    both_nan = np.isnan(g) & np.isnan(R)
    if op != O.SUM:
        # max/min: the stored value is the input element itself, so the result
        # is exact in any order: compare the stored bits of the oracle's value
        want = O.widen(out_code, O.cast(out_code, R))
        same = (g == want) | both_nan
        bad = np.nonzero(~same)[0]
        assert bad.size == 0, f"{what}: {bad.size} max/min mismatches, first at {bad[0]}: " \
                              f"gpu {g[bad[0]]!r} oracle {want[bad[0]]!r}"
        return
    tol = tolerance(out_code, R, S).reshape(-1)
    err = np.abs(g - R)
    stored = O.widen(out_code, O.cast(out_code, R))      # R rounded to the output type
    overflow = np.isinf(stored) & ~np.isinf(R)
    assert allow_inf or not overflow.any(), \
        f"{what}: {int(overflow.sum())} expected sums overflow the output type (first at " \
        f"{np.nonzero(overflow)[0][0]}: oracle {R[np.nonzero(overflow)[0][0]]!r}); draw smaller values"
    with np.errstate(invalid="ignore"):
        ok = (err <= tol) | both_nan | (allow_inf & overflow & (g == stored))
    bad = np.nonzero(~ok)[0]
    assert bad.size == 0, f"{what}: {bad.size} outputs out of tolerance, first at {bad[0]}: " \
                          f"gpu {g[bad[0]]!r} oracle {R[bad[0]]!r} err {err[bad[0]]:.3e} tol {tol[bad[0]]:.3e}"
