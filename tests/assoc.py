"""Every float32 result a reduction tree can produce on a tiny input.

A parallel reduction may combine its operands in any order and any tree shape
(AcceleratedKernels.jl PR #139, section "Compatibility": rounding may change
because the reduction tree changed).  For a handful of operands this module
enumerates, by dynamic programming over subsets, the set of every float32
value that some binary tree over some permutation of the operands yields when
each combination is one correctly rounded float32 operation.  A GPU result
computed with float32 operations and no fused multiply-add must lie in it.
"""
from __future__ import annotations

import itertools

import numpy as np


def f32_results(values, op: str = "sum") -> set:
    vals = [np.float32(v) for v in values]
    k = len(vals)
    if k == 0:
        return set()
    memo = {}
    for i, v in enumerate(vals):
        memo[1 << i] = {v}
    full = (1 << k) - 1
    for mask in range(1, full + 1):
        if mask in memo:
            continue
        out = set()
        # split mask into sub and rest; visit each unordered pair once
        sub = (mask - 1) & mask
        low = mask & -mask
        while sub:
            if sub & low:           # sub holds the lowest bit: each split once
                rest = mask ^ sub
                if rest:
                    for a, b in itertools.product(memo[sub], memo[rest]):
                        with np.errstate(over="ignore", invalid="ignore"):
                            if op == "sum":
                                out.add(np.float32(a + b))
                            elif op == "max":
                                out.add(max(a, b))
                            else:
                                out.add(min(a, b))
            sub = (sub - 1) & mask
        memo[mask] = out
    return memo[full]
