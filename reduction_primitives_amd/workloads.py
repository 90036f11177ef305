"""Seeded synthetic inputs for the reductions.

This module only draws numbers: it holds none of the reduction arithmetic, so
both the GPU tests and the CPU oracle may take their inputs from it.  Every
array is drawn on the host with ``torch.Generator("cpu").manual_seed(seed)``,
so the oracle and the GPU see identical bytes.

Arrays are column-major, as on the AcceleratedKernels.jl pages (Julia
semantics): a column-major (d1, d2, d3) array is held as a flat buffer with
element strides (1, d1, d1*d2).  ``cm_strides`` gives those strides.

The shapes follow the pages' own benchmark rows: PR #139 ("Finish whole-array
reductions on the device", section "Numbers") times Float32 sums of 10^4,
10^6 and 10^8 elements; PR #176 (strided reductions along dims, section
"Timings") times sum(x; dims=2) of 768x1024x8, 64x4096x32, 3072x2048 and
8192x8192 arrays in BFloat16 and Float32.  The pages give no value
distributions; the ones used here are listed with each workload.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch


def _gen(seed: int) -> torch.Generator:
    return torch.Generator("cpu").manual_seed(int(seed))


def uniform(n: int, lo: float, hi: float, seed: int) -> torch.Tensor:
    """n float32 values lo + (hi - lo) * U[0, 1)."""
    u = torch.rand(int(n), generator=_gen(seed), dtype=torch.float32)
    if lo == 0.0 and hi == 1.0:
        return u
    return u.mul_(hi - lo).add_(lo)


def normal(n: int, seed: int, dtype=torch.float32) -> torch.Tensor:
    """n standard normal values, drawn in float32 and rounded to dtype."""
    z = torch.randn(int(n), generator=_gen(seed), dtype=torch.float32)
    return z if dtype == torch.float32 else z.to(dtype)


def randint(n: int, lo: int, hi: int, seed: int, dtype=torch.int32) -> torch.Tensor:
    """n integers drawn uniformly from the inclusive range [lo, hi]."""
    return torch.randint(int(lo), int(hi) + 1, (int(n),), generator=_gen(seed), dtype=dtype)


def small_ints(n: int, lo: int, hi: int, seed: int, dtype=torch.float32) -> torch.Tensor:
    """Integer values in [lo, hi] stored as a floating dtype (exact sums)."""
    return randint(n, lo, hi, seed, torch.int64).to(dtype)


def randperm(n: int, seed: int) -> torch.Tensor:
    """A random permutation of 0..n-1 as int32."""
    return torch.randperm(int(n), generator=_gen(seed)).to(torch.int32)


def cm_strides(shape) -> tuple:
    """Element strides of a contiguous column-major array of `shape`."""
    st, acc = [], 1
    for s in shape:
        st.append(acc)
        acc *= int(s)
    return tuple(st)


@dataclass
class Array:
    """A flat host buffer viewed as a column-major array."""
    name: str
    data: torch.Tensor          # flat, contiguous
    shape: tuple                # column-major extents
    recipe: str

    @property
    def strides(self) -> tuple:
        return cm_strides(self.shape)

    @property
    def numel(self) -> int:
        return int(math.prod(self.shape))


# ----------------------------------------------------------------- workloads
# Each function returns the arrays of one workload, drawn from seeds
# 1000 * k + j (k = workload number, j = array number).

def whole_small(n: int = 10_000) -> list:
    """10^4 float32 U[-1,1); the same draw scaled to int32 in [-1000, 1000]."""
    x = uniform(n, -1.0, 1.0, 1000)
    xi = torch.round(x * 1000.0).to(torch.int32)
    return [Array("f32_u[-1,1)", x, (n,), "U[-1,1) seed 1000"),
            Array("i32_[-1000,1000]", xi, (n,), "round(1000*U[-1,1)) seed 1000")]


def whole_large(n: int) -> list:
    """n float32 U[0,1) and a random permutation of 0..n-1 as int32."""
    j = 0 if n <= 10**6 else 2
    x = uniform(n, 0.0, 1.0, 2000 + j)
    p = randperm(n, 2001 + j)
    return [Array("f32_u[0,1)", x, (n,), f"U[0,1) seed {2000 + j}"),
            Array("i32_perm", p, (n,), f"randperm seed {2001 + j}")]


def matrix_3072x2048() -> list:
    """3072x2048 column-major N(0,1) in bfloat16 and float32."""
    shape = (3072, 2048)
    n = math.prod(shape)
    return [Array("bf16_n01", normal(n, 3000, torch.bfloat16), shape, "N(0,1)->bf16 seed 3000"),
            Array("f32_n01", normal(n, 3001), shape, "N(0,1) seed 3001")]


def middle_dim_3d() -> list:
    """(features, sequence, batch) arrays reduced over the middle dim."""
    s1, s2 = (768, 1024, 8), (64, 4096, 32)
    return [Array("bf16_768x1024x8", normal(math.prod(s1), 4000, torch.bfloat16), s1,
                  "N(0,1)->bf16 seed 4000"),
            Array("f32_768x1024x8", normal(math.prod(s1), 4001), s1, "N(0,1) seed 4001"),
            Array("f32_64x4096x32", uniform(math.prod(s2), 0.0, 1.0, 4002), s2,
                  "U[0,1) seed 4002")]


def matrix_8192() -> list:
    """8192x8192 float32 U[-1,1) and int32 in [-2^20, 2^20]."""
    shape = (8192, 8192)
    n = math.prod(shape)
    return [Array("f32_u[-1,1)", uniform(n, -1.0, 1.0, 5000), shape, "U[-1,1) seed 5000"),
            Array("i32_pm2^20", randint(n, -2**20, 2**20, 5001), shape,
                  "U{-2^20..2^20} seed 5001")]


def vector_pair(n: int) -> list:
    """Two float32 N(0,1) vectors of n elements, the two inputs of a fused
    source (dot product, squared and absolute distance).  PR #139 names fused
    sources without sizes; the whole-array sizes of its "Numbers" table are
    used (10^6, 10^8)."""
    j = 0 if n <= 10**6 else 2
    return [Array("f32_n01_a", normal(n, 6000 + j), (n,), f"N(0,1) seed {6000 + j}"),
            Array("f32_n01_b", normal(n, 6001 + j), (n,), f"N(0,1) seed {6001 + j}")]


@dataclass
class View:
    """A flat buffer read through an arbitrary column-major view."""
    name: str
    data: torch.Tensor
    shape: tuple
    view_strides: tuple
    dims: tuple
    recipe: str


def general_layouts() -> list:
    """Reductions over several reduced dims that do not merge into one, each
    67,108,864 float32 U[-1,1) elements (268 MB, the size of the 8192x8192
    rows).  PR #176's opening paragraphs speed up two common layouts of
    strided reductions; other layouts keep the one-thread or one-block per
    output kernels.  These are three of the others: per-channel statistics of a
    (3136, 256, 84) array over dims 1 and 3 (a contiguous reduced dim plus a
    strided one), a permuted (8192, 1024, 8) view over dims 2 and 3, and a
    4-d (1024, 2048, 8, 4) array over dims 2 and 4."""
    out = []
    shape = (3136, 256, 84)
    out.append(View("3136x256x84 f32 dims=(1,3)", uniform(math.prod(shape), -1.0, 1.0, 7000),
                    shape, cm_strides(shape), (1, 3), "U[-1,1) seed 7000"))
    shape = (8192, 1024, 8)           # storage (8192, 8, 1024), dims 2 and 3 swapped
    out.append(View("8192x1024x8 f32 permuted dims=(2,3)", uniform(math.prod(shape), -1.0, 1.0, 7001),
                    shape, (1, 8192 * 8, 8192), (2, 3), "U[-1,1) seed 7001"))
    shape = (1024, 2048, 8, 4)
    out.append(View("1024x2048x8x4 f32 dims=(2,4)", uniform(math.prod(shape), -1.0, 1.0, 7002),
                    shape, cm_strides(shape), (2, 4), "U[-1,1) seed 7002"))
    return out


def permuted_kept() -> View:
    """A view whose two kept dims are swapped against storage: (256, 1024,
    256) with strides (256, 65536, 1), i.e. storage (256, 256, 1024) read with
    dims 1 and 3 exchanged, reduced or scanned along dim 2 -- 67,108,864 float32 U[-1,1)
    elements.  The outputs are contiguous only in storage order, a layout
    PR #176's opening paragraphs leave to the one-thread or one-block per
    output kernels."""
    shape = (256, 1024, 256)
    return View("256x1024x256 f32 permuted dims=2", uniform(math.prod(shape), -1.0, 1.0, 7003),
                shape, (256, 65536, 1), (2,), "U[-1,1) seed 7003")


def short_lines() -> list:
    """Scans along dim 1 of contiguous lines shorter than 256 elements (PR
    #202's table of time ratios has scans along dims=1 beside whole ones):
    5,000,000 float32 U[-1,1) elements as lines of 50, 100 and 200."""
    out = []
    for m, seed in ((50, 7004), (100, 7005), (200, 7006)):
        shape = (m, 5_000_000 // m)
        out.append(View(f"{m}x{shape[1]} f32 cumsum dims=1", uniform(math.prod(shape), -1.0, 1.0, seed),
                        shape, cm_strides(shape), (1,), f"U[-1,1) seed {seed}"))
    return out
