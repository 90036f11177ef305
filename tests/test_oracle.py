"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test checks the oracle against mathematics or an independent library
routine: closed forms, exact rational sums (fractions.Fraction), Shewchuk's
correctly rounded sum (math.fsum), numpy's integer and axis sums, exhaustive
enumeration of the bf16/f16 codes, hand-derived golden cases, and brute force
over every association order on tiny inputs.  A plausible slip anywhere in
the oracle (a dropped term, a wrong sign, a swapped index, a wrong rounding)
fails at least one of them; tests/test_oracle_mutants.py plants such slips in
a copy of the oracle and checks exactly that.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from tests import assoc, golden_cases

U53 = 2.0 ** -53


def _o():
    import oracle
    return oracle


def _rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------ integer sums

@pytest.mark.parametrize("n", [0, 1, 2, 1000, 10**6])
def test_int_sum_closed_form(n):
    o = _o()
    x = np.arange(1, n + 1, dtype=np.int32)
    assert o.reduce_all(o.SUM, o.IDENTITY, o.I32, o.I64, x, 0) == n * (n + 1) // 2
    x64 = np.arange(1, n + 1, dtype=np.int64)
    assert o.reduce_all(o.SUM, o.IDENTITY, o.I64, o.I64, x64, 0) == n * (n + 1) // 2


def test_int_sum_matches_numpy():
    o = _o()
    x = _rng(1).integers(-2**31, 2**31, size=200_001, dtype=np.int64).astype(np.int32)
    assert o.reduce_all(o.SUM, o.IDENTITY, o.I32, o.I64, x, 0) == int(x.astype(np.int64).sum())
    # int32 accumulator: same total modulo 2^32
    want = o.wrap_int(int(x.astype(np.int64).sum()), o.I32)
    assert o.reduce_all(o.SUM, o.IDENTITY, o.I32, o.I32, x, 0) == want


def test_sum_of_squares_closed_form():
    o = _o()
    n = 3000
    x = np.arange(1, n + 1, dtype=np.int32)
    assert o.reduce_all(o.SUM, o.SQUARE, o.I32, o.I64, x, 0) == n * (n + 1) * (2 * n + 1) // 6
    xf = np.arange(1, n + 1, dtype=np.float32)   # squares and partial sums exact in double
    assert o.reduce_all(o.SUM, o.SQUARE, o.F32, o.F32, xf, 0.0) == float(n * (n + 1) * (2 * n + 1) // 6)


def test_abs_map():
    o = _o()
    x = _rng(2).integers(-1000, 1001, size=5000).astype(np.int32)
    assert o.reduce_all(o.SUM, o.ABS, o.I32, o.I64, x, 0) == int(np.abs(x.astype(np.int64)).sum())
    assert o.reduce_all(o.MAX, o.ABS, o.I32, o.I32, x, o.identity(o.MAX, o.I32)) == int(np.abs(x).max())
    xf = x.astype(np.float32)
    assert o.reduce_all(o.SUM, o.ABS, o.F32, o.F32, xf, 0.0) == float(np.abs(x.astype(np.int64)).sum())


def test_int_map_evaluated_in_accumulator_type():
    o = _o()
    x = np.array([65536, 3], dtype=np.int32)          # 65536^2 = 2^32
    assert o.reduce_all(o.MAX, o.SQUARE, o.I32, o.I32, x, o.identity(o.MAX, o.I32)) == 9
    assert o.reduce_all(o.MAX, o.SQUARE, o.I32, o.I64, x, o.identity(o.MAX, o.I64)) == 2**32
    x = np.array([-2**31], dtype=np.int32)             # |INT32_MIN| wraps in int32
    assert o.reduce_all(o.SUM, o.ABS, o.I32, o.I32, x, 0) == -2**31
    assert o.reduce_all(o.SUM, o.ABS, o.I32, o.I64, x, 0) == 2**31


def test_int32_accumulator_wraps():
    o = _o()
    x = np.full(4, 2**30, np.int32)
    assert o.reduce_all(o.SUM, o.IDENTITY, o.I32, o.I32, x, 0) == 0
    assert o.reduce_all(o.SUM, o.IDENTITY, o.I32, o.I64, x, 0) == 2**32
    x = np.full(3, 2**62, np.int64)
    assert o.reduce_all(o.SUM, o.IDENTITY, o.I64, o.I64, x, 0) == 3 * 2**62 - 2**64
    # the same along dims: column-major (2, 4) of 2^30, summed over dims=2
    x = np.full(8, 2**30, np.int32)
    g = o.reduce_dims(o.SUM, o.IDENTITY, o.I32, o.I32, x, (2, 4), (1, 2), 0b10, 0)
    assert list(g) == [0, 0]
    g = o.reduce_dims(o.SUM, o.IDENTITY, o.I32, o.I64, x, (2, 4), (1, 2), 0b10, 0)
    assert list(g) == [2**32, 2**32]


# ------------------------------------------------------------- float sums

@pytest.mark.parametrize("seed,n", [(3, 17), (4, 1000), (5, 100_000)])
def test_fp_sum_within_bound_of_fsum(seed, n):
    o = _o()
    x = _rng(seed).uniform(-1, 1, n).astype(np.float32)
    r = o.reduce_all(o.SUM, o.IDENTITY, o.F32, o.F32, x, 0.0)
    exact = math.fsum(float(v) for v in x)
    S = float(np.abs(x.astype(np.float64)).sum())
    assert abs(r - exact) <= (n - 1) * U53 * S + 1e-300


def test_fp_sum_rational_exact_small():
    o = _o()
    x = _rng(6).uniform(0, 1, 700).astype(np.float32)
    exact = sum((Fraction(float(v)) for v in x), Fraction(0))
    r = o.reduce_all(o.SUM, o.IDENTITY, o.F32, o.F32, x, 0.0)
    S = float(np.abs(x.astype(np.float64)).sum())
    assert abs(Fraction(r) - exact) <= Fraction((len(x) - 1) * U53 * S)
    # a sequential fold in order is exactly reproduced by Python floats
    acc = 0.0
    for v in x:
        acc += float(v)
    assert r == acc


def test_fp_sum_exact_for_dyadic_data():
    o = _o()
    x = _rng(7).integers(-8, 9, 100_000).astype(np.float32) * np.float32(0.25)
    assert o.reduce_all(o.SUM, o.IDENTITY, o.F32, o.F32, x, 0.5) == float(np.sum(x.astype(np.float64))) + 0.5


def test_bf16_and_f16_inputs_decoded():
    o = _o()
    vals = np.array([1.0, -2.5, 0.1, 3.0e4, -7.0e-3], dtype=np.float32)
    bf = (vals.view(np.uint32) >> 16).astype(np.uint16)   # truncated, exact bf16 values
    dec = (bf.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert o.reduce_all(o.SUM, o.IDENTITY, o.BF16, o.F32, bf, 0.0) == math.fsum(dec)
    h = vals.astype(np.float16)
    assert o.reduce_all(o.SUM, o.IDENTITY, o.F16, o.F32, h.view(np.uint16), 0.0) == \
        math.fsum(h.astype(np.float64))


# ----------------------------------------------------------------- max/min

@pytest.mark.parametrize("n", [1, 2, 31, 100_000])
def test_max_min_of_permutation(n):
    o = _o()
    p = _rng(8).permutation(n).astype(np.int32)
    assert o.reduce_all(o.MAX, o.IDENTITY, o.I32, o.I32, p, o.identity(o.MAX, o.I32)) == n - 1
    assert o.reduce_all(o.MIN, o.IDENTITY, o.I32, o.I32, p, o.identity(o.MIN, o.I32)) == 0
    pf = p.astype(np.float32)
    assert o.reduce_all(o.MAX, o.IDENTITY, o.F32, o.F32, pf, o.identity(o.MAX, o.F32)) == n - 1
    assert o.reduce_all(o.MIN, o.IDENTITY, o.F32, o.F32, pf, o.identity(o.MIN, o.F32)) == 0


def test_max_min_match_numpy():
    o = _o()
    x = _rng(9).standard_normal(50_001).astype(np.float32)
    assert o.reduce_all(o.MAX, o.IDENTITY, o.F32, o.F32, x, -math.inf) == float(x.max())
    assert o.reduce_all(o.MIN, o.IDENTITY, o.F32, o.F32, x, math.inf) == float(x.min())
    assert o.reduce_all(o.MAX, o.SQUARE, o.F32, o.F32, x, -math.inf) == float(np.max(x.astype(np.float64) ** 2))


def test_identities_and_nan():
    o = _o()
    assert o.identity(o.SUM, o.F32) == 0.0
    assert o.identity(o.MAX, o.F32) == -math.inf and o.identity(o.MIN, o.F32) == math.inf
    assert o.identity(o.MAX, o.I32) == -2**31 and o.identity(o.MIN, o.I32) == 2**31 - 1
    assert o.identity(o.MAX, o.I64) == -2**63 and o.identity(o.MIN, o.I64) == 2**63 - 1
    x = np.array([1.0, np.nan, 3.0], np.float32)
    for op in (o.SUM, o.MAX, o.MIN):
        assert math.isnan(o.reduce_all(op, o.IDENTITY, o.F32, o.F32, x, o.identity(op, o.F32)))


# ------------------------------------------------------- init, fold, empty

def test_constant_arrays_and_init():
    o = _o()
    for n, k, c in [(0, 3.0, 1.5), (1, 3.0, 1.5), (12345, 0.75, -7.0)]:
        x = np.full(n, k, np.float32)
        assert o.reduce_all(o.SUM, o.IDENTITY, o.F32, o.F32, x, c) == c + n * k
        if n:
            assert o.reduce_all(o.MAX, o.IDENTITY, o.F32, o.F32, x, -math.inf) == k
            assert o.reduce_all(o.MIN, o.IDENTITY, o.F32, o.F32, x, math.inf) == k


def test_init_applied_exactly_once():
    o = _o()
    x = np.zeros(1000, np.float32)
    for mode in (o.OVERWRITE, o.HOST):
        r, raw = o.expected_all(o.SUM, o.IDENTITY, o.F32, o.F32, o.F32, x, mode, init=1.5)
        assert r == 1.5 and raw[0] == np.float32(1.5)
    r, _ = o.expected_all(o.SUM, o.IDENTITY, o.F32, o.F32, o.F32, x[:0], o.OVERWRITE, init=-7.0)
    assert r == -7.0
    r, _ = o.expected_all(o.MAX, o.IDENTITY, o.I32, o.I32, o.I32, np.zeros(0, np.int32), o.HOST)
    assert r == -2**31


def test_fold_continues_from_previous_value():
    o = _o()
    x = np.arange(10, dtype=np.float32)
    r1, raw1 = o.expected_all(o.SUM, o.IDENTITY, o.F32, o.F32, o.F32, x, o.OVERWRITE, init=1.5)
    assert r1 == 46.5
    r2, raw2 = o.expected_all(o.SUM, o.IDENTITY, o.F32, o.F32, o.F32, x, o.FOLD, init=1.5, prev=raw1)
    assert r2 == 46.5 + 45.0          # init is not applied a second time
    r3, _ = o.expected_all(o.MAX, o.IDENTITY, o.F32, o.F32, o.F32, x, o.FOLD,
                           prev=np.array([100.0], np.float32))
    assert r3 == 100.0
    r4, _ = o.expected_all(o.MIN, o.IDENTITY, o.I32, o.I64, o.I32, x.astype(np.int32), o.FOLD,
                           prev=np.array([-5], np.int32))
    assert r4 == -5


# ------------------------------------------------------------ final stores

def _all_bf16_values():
    codes = np.arange(0, 1 << 16, dtype=np.uint32)
    with np.errstate(invalid="ignore"):         # the NaN codes are part of the sweep
        vals = (codes << 16).view(np.float32).astype(np.float64)
    return codes.astype(np.uint16), vals


def test_bf16_cast_ties_to_even():
    o = _o()
    got = o.cast(o.BF16, [256.0, 257.0, 258.0, 259.0, 260.0, -257.0, 0.0, -0.0])
    assert list(got) == [0x4380, 0x4380, 0x4381, 0x4382, 0x4382, 0xC380, 0x0000, 0x8000]


def test_bf16_cast_is_nearest_brute_force():
    """Every double maps to the nearest finite bf16 value, ties to even code."""
    o = _o()
    codes, vals = _all_bf16_values()
    finite = np.isfinite(vals) & (codes < 0x8000)            # non-negative finite values
    pos_vals = vals[finite]
    pos_codes = codes[finite]
    order = np.argsort(pos_vals, kind="stable")
    pos_vals, pos_codes = pos_vals[order], pos_codes[order]
    # drop -0 duplicates (none among non-negative codes) and check monotone
    assert np.all(np.diff(pos_vals) > 0)
    rng = _rng(10)
    samples = np.concatenate([
        rng.uniform(0, 1e3, 4000),
        np.exp(rng.uniform(-90, 88, 4000)),
        (pos_vals[:-1] + pos_vals[1:]) / 2,                   # exact midpoints (ties)
        pos_vals,
        np.exp(rng.uniform(-103, -87, 2000)),                 # subnormal range
    ])
    got = o.cast(o.BF16, samples)
    k = np.searchsorted(pos_vals, samples)
    for v, g, kk in zip(samples, got, k):
        lo = pos_codes[max(kk - 1, 0)]
        hi = pos_codes[min(kk, len(pos_codes) - 1)]
        lo_v = pos_vals[max(kk - 1, 0)]
        hi_v = pos_vals[min(kk, len(pos_vals) - 1)]
        if v == hi_v:
            want = hi
        elif v > pos_vals[-1]:
            half = pos_vals[-1] + (pos_vals[-1] - pos_vals[-2]) / 2
            want = 0x7F80 if v >= half else pos_codes[-1]
        else:
            dlo, dhi = v - lo_v, hi_v - v
            want = lo if dlo < dhi else hi if dhi < dlo else (lo if lo % 2 == 0 else hi)
        assert int(g) == int(want), (v, hex(g), hex(want))
    assert list(o.cast(o.BF16, [1e39, -1e39, math.inf])) == [0x7F80, 0xFF80, 0x7F80]
    assert int(o.cast(o.BF16, [math.nan])[0]) & 0x7FC0 == 0x7FC0


def test_f16_cast_matches_numpy():
    o = _o()
    rng = _rng(11)
    samples = np.concatenate([rng.uniform(-7e4, 7e4, 5000),
                              np.exp(rng.uniform(-20, 11, 5000)) * rng.choice([-1, 1], 5000),
                              np.arange(-2048.5, 2048.5, 0.5)])
    got = o.cast(o.F16, samples)
    with np.errstate(over="ignore"):            # samples beyond float16's range round to infinity
        want = samples.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


def test_widen_decodes_every_code():
    o = _o()
    codes = np.arange(0, 1 << 16, dtype=np.uint16)
    f16 = o.widen(o.F16, codes)
    ref = codes.view(np.float16).astype(np.float64)
    same = (f16 == ref) | (np.isnan(f16) & np.isnan(ref))
    assert same.all()
    bf = o.widen(o.BF16, codes)
    with np.errstate(invalid="ignore"):         # the NaN codes are part of the sweep
        ref = (codes.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    same = (bf == ref) | (np.isnan(bf) & np.isnan(ref))
    assert same.all()


def test_f32_and_int_casts():
    o = _o()
    v = _rng(12).standard_normal(1000) * 1e3
    assert np.array_equal(o.cast(o.F32, v), v.astype(np.float32))
    assert list(o.cast(o.I32, [2**31, -2**31 - 1, 5])) == [-2**31, 2**31 - 1, 5]


# ------------------------------------------------------- association brute force

@pytest.mark.parametrize("seed", range(6))
def test_association_orders(seed):
    """Oracle lies within the double rounding bound of the exact sum, and for
    integers and max/min every association order gives one value, the oracle's."""
    o = _o()
    rng = _rng(100 + seed)
    n = 4 + seed % 3
    x = rng.uniform(-1, 1, n).astype(np.float32)
    init = np.float32(rng.uniform(-1, 1))
    operands = [init] + list(x)
    results = assoc.f32_results(operands, "sum")
    exact = sum((Fraction(float(v)) for v in operands), Fraction(0))
    S = sum(abs(float(v)) for v in operands)
    r = o.reduce_all(o.SUM, o.IDENTITY, o.F32, o.F32, x, float(init))
    assert abs(Fraction(r) - exact) <= Fraction(n * U53 * S)
    for v in results:                       # every tree's float32 value is near the truth
        assert abs(Fraction(float(v)) - exact) <= Fraction(n * 2.0**-24 * S)
    for op_name, op in (("max", o.MAX), ("min", o.MIN)):
        res = assoc.f32_results(operands, op_name)
        assert len(res) == 1
        assert o.reduce_all(op, o.IDENTITY, o.F32, o.F32, x, float(init)) == float(next(iter(res)))
    xi = rng.integers(-50, 50, n).astype(np.int32)
    ri = assoc.f32_results([0] + [np.float32(v) for v in xi], "sum")
    assert len(ri) == 1 and float(next(iter(ri))) == o.reduce_all(o.SUM, o.IDENTITY, o.I32, o.I64, xi, 0)


# -------------------------------------------------------------------- dims

def _cm(arr_shape_cm, rng, kind="f32"):
    n = int(np.prod(arr_shape_cm))
    if kind == "f32":
        return rng.standard_normal(n).astype(np.float32)
    return rng.integers(-1000, 1000, n).astype(np.int32)


@pytest.mark.parametrize("shape", [(5,), (4, 7), (3, 5, 6), (2, 3, 4, 5), (1, 9, 1)])
def test_dims_match_numpy(shape):
    o = _o()
    rng = _rng(20 + len(shape))
    nd = len(shape)
    strides = np.cumprod((1,) + shape[:-1]).tolist()
    xf, xi = _cm(shape, rng), _cm(shape, rng, "i32")
    # numpy view of the column-major buffer: a C array of reversed shape
    npf = xf.reshape(shape[::-1]).transpose(range(nd - 1, -1, -1))
    npi = xi.reshape(shape[::-1]).transpose(range(nd - 1, -1, -1))
    for mask in range(1, 1 << nd):
        axes = tuple(d for d in range(nd) if mask >> d & 1)
        kept = [d for d in range(nd) if not mask >> d & 1]
        def flat(a):   # kept dims in column-major order -> flat output order
            return np.transpose(a, range(len(kept) - 1, -1, -1)).reshape(-1) if kept else np.asarray(a).reshape(-1)
        wi = flat(npi.astype(np.int64).sum(axis=axes))
        gi = o.reduce_dims(o.SUM, o.IDENTITY, o.I32, o.I64, xi, shape, strides, mask, 0)
        assert np.array_equal(gi, wi)
        for op, fn in ((o.MAX, np.max), (o.MIN, np.min)):
            gf = o.reduce_dims(op, o.IDENTITY, o.F32, o.F32, xf, shape, strides, mask,
                               o.identity(op, o.F32))
            assert np.array_equal(gf, flat(fn(npf.astype(np.float64), axis=axes)))
        gs = o.reduce_dims(o.SUM, o.IDENTITY, o.F32, o.F32, xf, shape, strides, mask, 0.0)
        ws = flat(npf.astype(np.float64).sum(axis=axes))
        m = int(np.prod([shape[d] for d in axes]))
        S = flat(np.abs(npf.astype(np.float64)).sum(axis=axes))
        assert np.all(np.abs(gs - ws) <= 2 * m * U53 * S + 1e-300)


def test_dims_all_masked_equals_whole_array():
    o = _o()
    shape = (6, 5, 4)
    x = _cm(shape, _rng(30))
    g = o.reduce_dims(o.SUM, o.SQUARE, o.F32, o.F32, x, shape, (1, 6, 30), 0b111, 0.25)
    assert g.shape == (1,)
    assert g[0] == o.reduce_all(o.SUM, o.SQUARE, o.F32, o.F32, x, 0.25)


def test_dims_per_output_order_is_column_major():
    """Each output folds its reduced elements in increasing column-major order:
    it equals the whole-array fold of that output's slice gathered in order."""
    o = _o()
    shape = (4, 6, 3, 5)
    x = _cm(shape, _rng(31))
    strides = (1, 4, 24, 72)
    arr = x.reshape(shape[::-1])             # arr[l, k, j, i] = element (i, j, k, l)
    mask = 0b1010                             # reduce dims 2 and 4 (1-based)
    got = o.reduce_dims(o.SUM, o.IDENTITY, o.F32, o.F32, x, shape, strides, mask, 0.0)
    out = 0
    for k in range(shape[2]):
        for i in range(shape[0]):
            sl = np.ascontiguousarray(arr[:, k, :, i]).reshape(-1)   # (l, j): j fastest
            assert got[out] == o.reduce_all(o.SUM, o.IDENTITY, o.F32, o.F32, sl, 0.0)
            out += 1


def test_dims_strided_view():
    """A non-contiguous view (transposed strides, with an offset gap)."""
    o = _o()
    rng = _rng(32)
    base = rng.integers(-100, 100, 7 * 9).astype(np.int32)
    m = base.reshape(7, 9)                     # C order: m[r, c] at r*9 + c
    # column-major view (9, 7) with strides (1, 9) is m itself read transposed;
    # view (7, 9) with strides (9, 1) reads m[r, c] as element (r, c)
    g = o.reduce_dims(o.SUM, o.IDENTITY, o.I32, o.I64, base, (7, 9), (9, 1), 0b01, 0)
    assert np.array_equal(g, m.astype(np.int64).sum(axis=0))
    g = o.reduce_dims(o.SUM, o.IDENTITY, o.I32, o.I64, base, (7, 4), (9, 2), 0b10, 0)
    assert np.array_equal(g, m[:, 0:8:2].astype(np.int64).sum(axis=1))


# ------------------------------------------------------------------ golden

@pytest.mark.parametrize("case", golden_cases.load(), ids=lambda c: c["id"])
def test_golden(case):
    o = _o()
    c = case
    if "shape" in c:
        shape = c["shape"]
        strides = np.cumprod([1] + shape[:-1]).tolist()
        r, raw = o.expected_dims(c["op_code"], c["map_code"], c["in_code"], c["acc_code"],
                                 c["out_code"], c["x_raw"], shape, strides, c["mask"],
                                 c["mode_code"], c.get("init"), c["prev_raw"])
        assert list(o.widen(c["out_code"], raw)) == list(np.asarray(c["expected"], dtype=float)) \
            if o.is_fp(c["out_code"]) else list(raw.astype(np.int64)) == list(c["expected"])
    else:
        r, raw = o.expected_all(c["op_code"], c["map_code"], c["in_code"], c["acc_code"],
                                c["out_code"], c["x_raw"], c["mode_code"], c.get("init"),
                                c["prev_raw"])
        got = o.widen(c["out_code"], raw)[0]
        assert got == c["expected"]
        if "expected_bits" in c:
            assert int(raw.view(np.uint16)[0]) == c["expected_bits"]


# ------------------------------------------------- two-input fused sources

def test_two_input_closed_forms():
    o = _o()
    n = 2000
    a = np.arange(1, n + 1, dtype=np.int32)
    b = np.arange(2, n + 2, dtype=np.int32)
    assert o.reduce_all2(o.SUM, o.MUL, o.I32, o.I64, a, a, 0) == n * (n + 1) * (2 * n + 1) // 6
    assert o.reduce_all2(o.SUM, o.SQDIFF, o.I32, o.I64, a, b, 0) == n
    assert o.reduce_all2(o.SUM, o.ABSDIFF, o.I32, o.I64, b, a, 7) == n + 7
    c = (n - a).astype(np.int32)                      # sum i (n - i) = n * n(n+1)/2 - n(n+1)(2n+1)/6
    assert o.reduce_all2(o.SUM, o.MUL, o.I32, o.I64, a, c, 0) == \
        n * n * (n + 1) // 2 - n * (n + 1) * (2 * n + 1) // 6
    af = a.astype(np.float32)
    assert o.reduce_all2(o.SUM, o.MUL, o.F32, o.F32, af, af, 0.0) == float(n * (n + 1) * (2 * n + 1) // 6)
    p = _rng(40).permutation(n).astype(np.int32)
    ones = np.ones(n, np.int32)
    assert o.reduce_all2(o.MAX, o.MUL, o.I32, o.I32, p, ones, o.identity(o.MAX, o.I32)) == n - 1
    assert o.reduce_all2(o.MIN, o.MUL, o.I32, o.I32, p, ones, o.identity(o.MIN, o.I32)) == 0


def test_two_input_dot_against_numpy():
    o = _o()
    rng = _rng(41)
    a = rng.standard_normal(50_000).astype(np.float32)
    b = rng.standard_normal(50_000).astype(np.float32)
    a64, b64 = a.astype(np.float64), b.astype(np.float64)
    r = o.reduce_all2(o.SUM, o.MUL, o.F32, o.F32, a, b, 0.0)
    S = float(np.abs(a64 * b64).sum())
    assert abs(r - float(np.dot(a64, b64))) <= 2 * a.size * U53 * S
    ai = rng.integers(-2**20, 2**20, 50_000).astype(np.int32)
    bi = rng.integers(-2**20, 2**20, 50_000).astype(np.int32)
    assert o.reduce_all2(o.SUM, o.MUL, o.I32, o.I64, ai, bi, 0) == int(np.dot(ai.astype(np.int64), bi.astype(np.int64)))


def test_two_input_identities_exact():
    """(a-b)^2 = a^2 - 2ab + b^2 and, for a >= b, |a-b| = a - b, checked
    against exact rational sums of other oracle paths and of the data."""
    o = _o()
    rng = _rng(42)
    a = rng.uniform(-1, 1, 500).astype(np.float32)
    b = rng.uniform(-1, 1, 500).astype(np.float32)
    fa = [Fraction(float(v)) for v in a]
    fb = [Fraction(float(v)) for v in b]
    exact_sq = sum(x * x for x in fa) - 2 * sum(x * y for x, y in zip(fa, fb)) + sum(y * y for y in fb)
    r = o.reduce_all2(o.SUM, o.SQDIFF, o.F32, o.F32, a, b, 0.0)
    S = float(sum((x - y) * (x - y) for x, y in zip(fa, fb)))
    assert abs(Fraction(r) - exact_sq) <= Fraction(4 * a.size * U53 * S)
    hi, lo = np.maximum(a, b), np.minimum(a, b)
    r = o.reduce_all2(o.SUM, o.ABSDIFF, o.F32, o.F32, hi, lo, 0.0)
    exact = sum(Fraction(float(v)) for v in hi) - sum(Fraction(float(v)) for v in lo)
    assert abs(Fraction(r) - exact) <= Fraction(4 * a.size * U53 * float(exact))
    # |a - 0| folds like the one-input abs map
    z = np.zeros_like(a)
    assert o.reduce_all2(o.SUM, o.ABSDIFF, o.F32, o.F32, a, z, 0.0) == \
        o.reduce_all(o.SUM, o.ABS, o.F32, o.F32, a, 0.0)


def test_two_input_maps_wrap_in_int32():
    o = _o()
    a = np.array([65536, 3], np.int32)
    assert o.reduce_all2(o.SUM, o.MUL, o.I32, o.I32, a, a, 0) == 9          # 2^32 wraps to 0
    assert o.reduce_all2(o.SUM, o.MUL, o.I32, o.I64, a, a, 0) == 2**32 + 9
    a = np.array([2**31 - 1], np.int32)
    b = np.array([-1], np.int32)
    assert o.reduce_all2(o.SUM, o.ABSDIFF, o.I32, o.I32, a, b, 0) == -2**31   # 2^31 wraps
    assert o.reduce_all2(o.SUM, o.ABSDIFF, o.I32, o.I64, a, b, 0) == 2**31


# ------------------------------------------------------------------- scans

def test_scan_closed_forms():
    o = _o()
    n = 5000
    x = np.arange(1, n + 1, dtype=np.int32)
    k = np.arange(1, n + 1, dtype=np.int64)
    assert np.array_equal(o.scan(o.SUM, o.I32, o.I64, x, 0, True), k * (k + 1) // 2)
    assert np.array_equal(o.scan(o.SUM, o.I32, o.I64, x, 7, False), 7 + (k - 1) * k // 2)
    xf = x.astype(np.float32)                 # every prefix is an exact double
    assert np.array_equal(o.scan(o.SUM, o.F32, o.F32, xf, 0.5, True), 0.5 + (k * (k + 1) // 2))
    assert o.scan(o.SUM, o.F32, o.F32, xf[:0], 1.0, True).size == 0
    # max/min of a permutation: the running max/min
    p = _rng(50).permutation(n).astype(np.int32)
    assert np.array_equal(o.scan(o.MAX, o.I32, o.I32, p, o.identity(o.MAX, o.I32), True),
                          np.maximum.accumulate(p.astype(np.int64)))
    assert np.array_equal(o.scan(o.MIN, o.I32, o.I32, p, o.identity(o.MIN, o.I32), True),
                          np.minimum.accumulate(p.astype(np.int64)))
    ex = o.scan(o.MAX, o.I32, o.I32, p, -1, False)
    assert ex[0] == -1 and np.array_equal(ex[1:], np.maximum.accumulate(p.astype(np.int64))[:-1])


def test_scan_matches_numpy_integer_cumsum():
    o = _o()
    x = _rng(51).integers(-2**31, 2**31, 100_001).astype(np.int32)
    c = np.cumsum(x.astype(np.int64))
    assert np.array_equal(o.scan(o.SUM, o.I32, o.I64, x, 0, True), c)
    wrapped = ((c + 2**31) % 2**32) - 2**31
    assert np.array_equal(o.scan(o.SUM, o.I32, o.I32, x, 0, True), wrapped)
    y = _rng(52).integers(-2**62, 2**62, 1000).astype(np.int64)
    c = np.cumsum(y.astype(object))
    got = o.scan(o.SUM, o.I64, o.I64, y, 0, True)
    assert all(int(g) == ((int(v) + 2**63) % 2**64) - 2**63 for g, v in zip(got, c))


def test_scan_prefixes_equal_whole_array_folds():
    """Every output of the scan is the whole-array fold of its prefix, with
    the same start, bit for bit (both are the same left-to-right fold)."""
    o = _o()
    rng = _rng(53)
    for dt in (o.F32, o.BF16, o.F16, o.F64):
        v = rng.standard_normal(300).astype(np.float32)
        x = {o.F32: v, o.F64: v.astype(np.float64), o.F16: v.astype(np.float16).view(np.uint16),
             o.BF16: (v.view(np.uint32) >> 16).astype(np.uint16)}[dt]
        for op in (o.SUM, o.MAX, o.MIN):
            s = 0.25 if op == o.SUM else o.identity(op, o.F32)
            inc = o.scan(op, dt, o.F32, x, s, True)
            exc = o.scan(op, dt, o.F32, x, s, False)
            for i in (0, 1, 2, 57, 299):
                assert inc[i] == o.reduce_all(op, o.IDENTITY, dt, o.F32, x[:i + 1], s)
                assert exc[i] == o.reduce_all(op, o.IDENTITY, dt, o.F32, x[:i], s)


def test_scan_fp_exact_rational_small():
    o = _o()
    x = _rng(54).uniform(-1, 1, 400).astype(np.float32)
    r = o.scan(o.SUM, o.F32, o.F32, x, 0.0, True)
    exact = Fraction(0)
    for i, v in enumerate(x):
        exact += Fraction(float(v))
        S = float(np.abs(x[:i + 1].astype(np.float64)).sum())
        assert abs(Fraction(r[i]) - exact) <= Fraction((i + 1) * U53 * S)


def test_scan_dims_equals_line_scans():
    """Along each dim of a strided 3-d view, every line of the output is the
    1-d scan of that line of the input (lines extracted by numpy indexing)."""
    o = _o()
    shape = (5, 7, 3)
    storage = _rng(55).integers(-50, 50, 400).astype(np.int32)
    strides = (1, 6, 50)                      # a padded view: 6 > 5, 50 > 6 * 7
    idx = np.zeros(shape, np.int64)
    for i in range(shape[0]):
        for j in range(shape[1]):
            for k in range(shape[2]):
                idx[i, j, k] = i * strides[0] + j * strides[1] + k * strides[2]
    view = storage[idx]                       # view[i, j, k]
    for dim in range(3):
        for inclusive in (True, False):
            got = o.scan_dims(o.SUM, o.I32, o.I64, storage, shape, strides, dim, 3, inclusive)
            got = got.reshape(shape, order="F")
            want = np.moveaxis(view, dim, -1).astype(np.int64)
            c = np.cumsum(want, axis=-1) + 3
            if not inclusive:
                c = np.concatenate([np.full(c.shape[:-1] + (1,), 3), c[..., :-1]], axis=-1)
            assert np.array_equal(np.moveaxis(got, dim, -1), c), (dim, inclusive)
    # floating input along dim 1 agrees with the 1-d oracle line by line
    xf = _rng(56).standard_normal(400).astype(np.float32)
    got = o.scan_dims(o.MAX, o.F32, o.F32, xf, shape, strides, 1, -math.inf, True).reshape(shape, order="F")
    for i in range(shape[0]):
        for k in range(shape[2]):
            line = xf[[i * strides[0] + j * strides[1] + k * strides[2] for j in range(shape[1])]]
            assert np.array_equal(got[i, :, k], o.scan(o.MAX, o.F32, o.F32, line, -math.inf, True))
