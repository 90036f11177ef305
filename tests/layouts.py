"""Seeded random array views for the parity sweeps (no GPU, no oracle).

A view is drawn from one seed: 1-4 dims of log-uniform extents (product at
most `max_elems`), the dims laid out in storage in a random order, some of
them sliced to every second element or broadcast (stride 0), and a start
offset of 0-3 elements.  Strides and offset are in elements; `numel` is the
storage the view needs.
"""
import math

import numpy as np


def random_view(seed, max_elems=1 << 21, long_inner=False):
    """With `long_inner`, the dim stored innermost is 256-20,000 long and
    neither sliced nor broadcast (lines that the contiguous kernels take)."""
    rng = np.random.default_rng(seed)
    nd = 1 if rng.random() < 0.1 else int(rng.integers(2, 5))
    order = rng.permutation(nd)                 # storage position of each dim
    while True:
        shape = [int(round(np.exp(rng.uniform(0, np.log(400))))) for _ in range(nd)]
        if long_inner:
            shape[order[0]] = int(round(np.exp(rng.uniform(np.log(256), np.log(20000)))))
        if math.prod(shape) <= max_elems:
            break
    step = [2 if rng.random() < 0.2 else 1 for _ in range(nd)]
    if long_inner:
        step[order[0]] = 1
    strides = [0] * nd
    s = 1
    for d in order:
        strides[d] = s * step[d]
        s *= shape[d] * step[d]
    for d in range(nd):
        if shape[d] > 1 and rng.random() < 0.1 and not (long_inner and d == order[0]):
            strides[d] = 0                      # broadcast
    offset = int(rng.integers(0, 4))
    numel = offset + sum((e - 1) * st for e, st in zip(shape, strides)) + 1
    return tuple(shape), tuple(strides), offset, numel, rng


def innermost(strides):
    """Index of the dim with the smallest nonzero stride (None if all are 0)."""
    inner = [d for d, st in enumerate(strides) if st > 0]
    return min(inner, key=lambda d: strides[d]) if inner else None
