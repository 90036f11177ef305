"""Benchmark of the device-wide mapreduce on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step runs every call of the hot path once over resident synthetic input:
  whole array, 10^8 elements (AcceleratedKernels.jl PR #139, "Numbers"):
    max and min of a permutation of 0..10^8-1 (int32), then float32 U[0,1)
    sums: into a device scalar with init = 1.5 (overwrite), folded into that
    scalar, and to a host value (finished on the host, which waits for it)
  8192x8192 column-major (PR #176, "Timings", last row):
    float32 sum over dims=2, sum over dims=1, max over dims=2, sum of
    squares of the whole array; int32 sum over dims=1 into int64
Each call reads its own copy of the input, so no call finds its data in the
256 MB Infinity Cache left behind by the previous one.

Printed: one JSON line with the aggregate algorithmic bandwidth (bytes the
method must move / time), the roofline of the dominant kernel (the float32
sum first pass, timed per launch with HIP events on its stream) with the
read ceiling beside it (a read-only kernel over the same inputs, timed the
same way), and the CPU oracle timed on the host over the same step as a
baseline.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (% of peak) for 1e8 fp32 sum and strided dims reductions"
PEAK_GBPS = 8000.0          # MI355X HBM3E, vendor figure
N_WHOLE = 10**8
SIDE = 8192
DOMINANT = "k_all_pass1<float, float, OpSum, MapIdentity>"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=30.0,
                    help="seconds of oracle work allowed for the CPU baseline")
    ap.add_argument("--cpu-min", type=float, default=10.0,
                    help="the CPU baseline repeats whole passes over the step's calls until this many "
                         "seconds of oracle work have run (within --cpu-budget)")
    ap.add_argument("--per-call-reps", type=int, default=50,
                    help="reps per round of the per-call table (0 skips it)")
    ap.add_argument("--per-call-rounds", type=int, default=3,
                    help="rounds of the per-call table (the round with the lowest median is reported)")
    ap.add_argument("--all-configs", action="store_true",
                    help="also time every configuration's calls one by one (cold and warm)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="first run one plain elementwise copy (torch.neg) of 10^8 float32, "
                         "400 MB read + 400 MB written, to scale HBM byte counters against")
    return ap.parse_args()


class Call:
    """One rk_* call of the step with its marshalled arguments."""

    def __init__(self, name, kind, bytes_alg, fn, timed=False, kernel=""):
        self.name, self.kind, self.bytes_alg, self.fn = name, kind, bytes_alg, fn
        self.timed, self.kernel = timed, kernel

    def __call__(self, k=0):
        rc = self.fn(k)
        if rc != 0:
            raise RuntimeError(f"{self.name}: rk status {rc}")


def build_step(rk, torch, dev):
    from reduction_primitives_amd import workloads as W

    log("generating inputs ...")
    t0 = time.time()
    xf, perm = W.whole_large(N_WHOLE)
    mf, mi = W.matrix_8192()
    log(f"  inputs drawn in {time.time() - t0:.1f} s")

    x = [xf.data.to(dev) for _ in range(3)]
    p = [perm.data.to(dev) for _ in range(2)]
    y = [mf.data.to(dev) for _ in range(4)]
    z = [mi.data.to(dev) for _ in range(3)]
    torch.cuda.synchronize()

    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    shape, strides = (SIDE, SIDE), (1, SIDE)
    ws_bytes = max(rk.rk_workspace_size(rk.RK_F32, rk.RK_F32, 1, [N_WHOLE], [1], 1),
                   rk.rk_workspace_size(rk.RK_I32, rk.RK_I64, 1, [N_WHOLE], [1], 1),
                   rk.rk_workspace_size(rk.RK_F32, rk.RK_F32, 2, shape, strides, 2),
                   rk.rk_workspace_size(rk.RK_F32, rk.RK_F32, 2, shape, strides, 1),
                   rk.rk_workspace_size(rk.RK_F32, rk.RK_F32, 2, shape, strides, 3),
                   rk.rk_workspace_size(rk.RK_I32, rk.RK_I64, 2, shape, strides, 1))
    ws_t = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    ws = ws_t.data_ptr()
    init15 = ctypes.c_float(1.5)
    host_out = ctypes.c_float()
    o_scalar = torch.empty(1, dtype=torch.float32, device=dev)
    o_max = torch.empty(1, dtype=torch.int32, device=dev)
    o_min = torch.empty(1, dtype=torch.int32, device=dev)
    o_d2 = torch.empty(SIDE, dtype=torch.float32, device=dev)
    o_d1 = torch.empty(SIDE, dtype=torch.float32, device=dev)
    o_mx = torch.empty(SIDE, dtype=torch.float32, device=dev)
    o_sq = torch.empty(1, dtype=torch.float32, device=dev)
    o_i = torch.empty(SIDE, dtype=torch.int64, device=dev)
    F32, I32, I64 = rk.RK_F32, rk.RK_I32, rk.RK_I64
    SUM, MAX, MIN = rk.RK_OP_SUM, rk.RK_OP_MAX, rk.RK_OP_MIN
    ID, SQ = rk.RK_MAP_IDENTITY, rk.RK_MAP_SQUARE
    OW, FO, HO = rk.RK_MODE_OVERWRITE, rk.RK_MODE_FOLD, rk.RK_MODE_HOST
    nb = N_WHOLE * 4
    mb = SIDE * SIDE * 4
    init_p = ctypes.byref(init15)
    # The three timed float32 sums come last, behind seven queued calls, so
    # their launch events never wait on an idle GPU; the host call, which
    # drains the stream, closes the step.  A call's argument k rotates it over
    # the copies of its input (k = 0 in the step), so that calls issued back
    # to back each read an input that two or more calls have not touched.
    calls = [
        Call("max_1e8_i32_perm", "all", nb + 4,
             lambda k=0: rk.rk_reduce_all(MAX, ID, I32, I32, I32, p[k % 2].data_ptr(), N_WHOLE, None, OW,
                                      o_max.data_ptr(), ws, st)),
        Call("min_1e8_i32_perm", "all", nb + 4,
             lambda k=0: rk.rk_reduce_all(MIN, ID, I32, I32, I32, p[(k + 1) % 2].data_ptr(), N_WHOLE, None, OW,
                                      o_min.data_ptr(), ws, st)),
        Call("sum_8192sq_f32_dims2", "dims", mb + SIDE * 4,
             lambda k=0: rk.rk_reduce_dims(SUM, ID, F32, F32, F32, y[k % 4].data_ptr(), 2, shape, strides, 2,
                                       None, OW, o_d2.data_ptr(), ws, st)),
        Call("sum_8192sq_f32_dims1", "dims", mb + SIDE * 4,
             lambda k=0: rk.rk_reduce_dims(SUM, ID, F32, F32, F32, y[(k + 1) % 4].data_ptr(), 2, shape, strides, 1,
                                       None, OW, o_d1.data_ptr(), ws, st)),
        Call("max_8192sq_f32_dims2", "dims", mb + SIDE * 4,
             lambda k=0: rk.rk_reduce_dims(MAX, ID, F32, F32, F32, y[(k + 2) % 4].data_ptr(), 2, shape, strides, 2,
                                       None, OW, o_mx.data_ptr(), ws, st)),
        Call("sumsq_8192sq_f32_all", "dims", mb + 4,
             lambda k=0: rk.rk_reduce_dims(SUM, SQ, F32, F32, F32, y[(k + 3) % 4].data_ptr(), 2, shape, strides, 3,
                                       None, OW, o_sq.data_ptr(), ws, st)),
        Call("sum_8192sq_i32_dims1_i64", "dims", mb + SIDE * 8,
             lambda k=0: rk.rk_reduce_dims(SUM, ID, I32, I64, I64, z[k % 3].data_ptr(), 2, shape, strides, 1,
                                       None, OW, o_i.data_ptr(), ws, st)),
        Call("sum_1e8_f32_init1.5", "all", nb + 4,
             lambda k=0: rk.rk_reduce_all(SUM, ID, F32, F32, F32, x[(k + 1) % 3].data_ptr(), N_WHOLE, init_p, OW,
                                      o_scalar.data_ptr(), ws, st), True, DOMINANT),
        Call("sum_1e8_f32_fold", "all", nb + 8,
             lambda k=0: rk.rk_reduce_all(SUM, ID, F32, F32, F32, x[(k + 2) % 3].data_ptr(), N_WHOLE, None, FO,
                                      o_scalar.data_ptr(), ws, st), True, DOMINANT),
        Call("sum_1e8_f32_host", "all", nb + 4,
             lambda k=0: rk.rk_reduce_all(SUM, ID, F32, F32, F32, x[k % 3].data_ptr(), N_WHOLE, None, HO,
                                      ctypes.addressof(host_out), ws, st), True, DOMINANT),
    ]
    outs = dict(host=host_out, scalar=o_scalar, max=o_max, min=o_min, d2=o_d2, d1=o_d1, mx=o_mx,
                sq=o_sq, i64=o_i)
    inputs = dict(xf=xf, perm=perm, mf=mf, mi=mi)
    keep = (x, p, y, z, ws_t)
    return calls, outs, inputs, keep


def plan_names(rk, torch):
    """Kernel each call takes, from the library's planner."""
    names = {}
    for dims, key in ((2, "d2"), (1, "d1"), ((1, 2), "all")):
        names[key] = rk.plan_dims(torch.float32, (SIDE, SIDE), (1, SIDE), dims)["kernel_name"]
    names["i64"] = rk.plan_dims(torch.int32, (SIDE, SIDE), (1, SIDE), 1)["kernel_name"]
    return names


def cpu_leg(inputs, outs, budget_s, host_value, min_s=10.0):
    import numpy as np

    import oracle as O

    xf = inputs["xf"].data.numpy()
    perm = inputs["perm"].data.numpy()
    mf = inputs["mf"].data.numpy()
    mi = inputs["mi"].data.numpy()
    shape, strides = (SIDE, SIDE), (1, SIDE)
    plan = [
        ("sum_1e8_f32_host", N_WHOLE * 4, lambda: O.reduce_all(O.SUM, O.IDENTITY, O.F32, O.F32, xf, 0.0)),
        ("sum_1e8_f32_init1.5", N_WHOLE * 4, lambda: O.reduce_all(O.SUM, O.IDENTITY, O.F32, O.F32, xf, 1.5)),
        ("max_1e8_i32_perm", N_WHOLE * 4, lambda: O.reduce_all(O.MAX, O.IDENTITY, O.I32, O.I32, perm, -2**31)),
        ("min_1e8_i32_perm", N_WHOLE * 4, lambda: O.reduce_all(O.MIN, O.IDENTITY, O.I32, O.I32, perm, 2**31 - 1)),
        ("sum_8192sq_f32_dims2", SIDE * SIDE * 4,
         lambda: O.reduce_dims(O.SUM, O.IDENTITY, O.F32, O.F32, mf, shape, strides, 0b10, 0.0)),
        ("sum_8192sq_f32_dims1", SIDE * SIDE * 4,
         lambda: O.reduce_dims(O.SUM, O.IDENTITY, O.F32, O.F32, mf, shape, strides, 0b01, 0.0)),
        ("max_8192sq_f32_dims2", SIDE * SIDE * 4,
         lambda: O.reduce_dims(O.MAX, O.IDENTITY, O.F32, O.F32, mf, shape, strides, 0b10, -math.inf)),
        ("sumsq_8192sq_f32_all", SIDE * SIDE * 4,
         lambda: O.reduce_all(O.SUM, O.SQUARE, O.F32, O.F32, mf, 0.0)),
        ("sum_8192sq_i32_dims1_i64", SIDE * SIDE * 4,
         lambda: O.reduce_dims(O.SUM, O.IDENTITY, O.I32, O.I64, mi, shape, strides, 0b01, 0)),
    ]
    cores_available = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    try:
        saved_affinity = os.sched_getaffinity(0)
        os.sched_setaffinity(0, {sorted(saved_affinity)[0]})
        pinned = True
    except (AttributeError, OSError):
        saved_affinity, pinned = None, False
    # Whole passes over the calls until min_s of oracle work have run (the
    # first pass's results are the ones checked), never beyond budget_s.
    results, t_total, b_total, passes = {}, 0.0, 0, 0
    while t_total <= budget_s:
        for name, nbytes, fn in plan:
            if t_total > budget_s:
                break
            t0 = time.perf_counter()
            r = fn()
            dt = time.perf_counter() - t0
            if passes == 0:
                results[name] = r
                log(f"  oracle {name}: {dt * 1e3:.1f} ms ({nbytes / dt / 1e9:.2f} GB/s)")
            t_total += dt
            b_total += nbytes
        passes += 1
        if t_total >= min_s or len(results) < len(plan):
            break
    if saved_affinity is not None:
        os.sched_setaffinity(0, saved_affinity)
    # parity of the last GPU step against these oracle results
    ok = True
    notes = []

    def near(g, r, s):
        return abs(g - r) <= 1e-5 * s

    S_x = float(np.abs(xf.astype(np.float64)).sum()) if "sum_1e8_f32_host" in results else None
    if "sum_1e8_f32_host" in results:
        ok &= near(host_value, results["sum_1e8_f32_host"], S_x)
    if "sum_1e8_f32_init1.5" in results:
        # after the fold the scalar holds (1.5 + sum) + sum
        want = results["sum_1e8_f32_init1.5"] + results["sum_1e8_f32_host"]
        ok &= near(float(outs["scalar"].item()), want, 1.5 + 2 * S_x)
    if "max_1e8_i32_perm" in results:
        ok &= int(outs["max"].item()) == results["max_1e8_i32_perm"] == N_WHOLE - 1
    if "min_1e8_i32_perm" in results:
        ok &= int(outs["min"].item()) == results["min_1e8_i32_perm"] == 0
    absm = None
    if "sum_8192sq_f32_dims2" in results:
        absm = O.reduce_dims(O.SUM, O.ABS, O.F32, O.F32, mf, shape, strides, 0b10, 0.0)
        ok &= bool(np.all(np.abs(outs["d2"].numpy() - results["sum_8192sq_f32_dims2"]) <= 1e-5 * absm))
    if "sum_8192sq_f32_dims1" in results:
        absm1 = O.reduce_dims(O.SUM, O.ABS, O.F32, O.F32, mf, shape, strides, 0b01, 0.0)
        ok &= bool(np.all(np.abs(outs["d1"].numpy() - results["sum_8192sq_f32_dims1"]) <= 1e-5 * absm1))
    if "max_8192sq_f32_dims2" in results:
        ok &= bool(np.array_equal(outs["mx"].numpy().astype(np.float64), results["max_8192sq_f32_dims2"]))
    if "sumsq_8192sq_f32_all" in results:
        r = results["sumsq_8192sq_f32_all"]
        ok &= near(float(outs["sq"].item()), r, r)
    if "sum_8192sq_i32_dims1_i64" in results:
        ok &= bool(np.array_equal(outs["i64"].numpy(), results["sum_8192sq_i32_dims1_i64"]))
    sample = (", ".join(results) if len(results) < len(plan)
              else "every call of one step except the fold, whose arithmetic is the overwrite's")
    return dict(value=round(b_total / t_total / 1e9, 3), unit="GB/s", cores=1 if pinned else None,
                kind="oracle", sample=f"{sample}, {passes} pass{'es' if passes > 1 else ''} "
                                      f"(same inputs; {b_total / 1e9:.2f} GB in {t_total:.1f} s)",
                host_cores_available=cores_available), \
        bool(ok)


def traffic_from_profile():
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, if it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_all_pass1_f32_1e8.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f)
        from reduction_primitives_amd.build import kernel_source_digest
        if rec.get("kernel_source_digest") != kernel_source_digest():
            return None
        return rec.get("hbm_bytes_per_launch")
    except Exception:
        return None


PIPE_CALLS, PIPE_ROUNDS = 20, 5


def pipelined(c, torch):
    """A device-mode call issued PIPE_CALLS times back to back on one stream,
    each on an input no call of the last two or more has read (the call's
    rotation index), all queued behind GPU work; one event pair around the
    sequence.  Per call: the sequence's time over PIPE_CALLS, launch gaps
    between calls included.  Median and min over PIPE_ROUNDS sequences."""
    ts = []
    for _ in range(PIPE_ROUNDS):
        torch.cuda.synchronize()
        torch.cuda._sleep(5_000_000)
        b, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b.record()
        for k in range(PIPE_CALLS):
            c(k)
        e.record()
        e.synchronize()
        ts.append(b.elapsed_time(e) * 1e3 / PIPE_CALLS)
    return ts


def per_call_table(calls, torch, reps, rounds, dev):
    """Per call, the whole rk call timed cold (the Infinity Cache first filled
    with other, clean lines by reading a 1 GiB buffer) and warm (the same call
    again right after, back to back): `reps` samples of each in each of
    `rounds` rounds, the calls interleaved within a round.  Reported per call
    and mode: the min and the median of the round with the lowest median.
    Device-mode calls also get a pipelined figure (see pipelined())."""
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    ts = {c.name: {m: [[] for _ in range(rounds)] for m in ("cold", "warm")} for c in calls}

    def one(c):
        # queue work ahead of a device-mode call, so its start event does not
        # wait on the host's launch latency; a host-mode call drains the
        # stream itself and is timed by the wall clock of the call
        if c.name.endswith("_host"):
            t0 = time.perf_counter()
            c()
            return (time.perf_counter() - t0) * 1e6
        torch.cuda._sleep(200_000)
        b, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b.record()
        c()
        e.record()
        e.synchronize()
        return b.elapsed_time(e) * 1e3

    for r in range(rounds):
        for _ in range(reps):
            for c in calls:
                flush.sum()
                torch.cuda.synchronize()
                ts[c.name]["cold"][r].append(one(c))
                torch.cuda.synchronize()
                ts[c.name]["warm"][r].append(one(c))
    table = {}
    for c in calls:
        rows = {}
        for mode in ("warm", "cold"):
            best = min(ts[c.name][mode], key=statistics.median)
            rows[mode] = dict(us_min=round(min(best), 2), us_median=round(statistics.median(best), 2),
                              GBps=round(c.bytes_alg / (min(best) * 1e-6) / 1e9, 1),
                              GBps_median=round(c.bytes_alg / (statistics.median(best) * 1e-6) / 1e9, 1))
        pipe = ""
        if not c.name.endswith("_host"):
            pt = pipelined(c, torch)
            med = statistics.median(pt)
            rows["pipelined"] = dict(us_median=round(med, 2), us_min=round(min(pt), 2),
                                     GBps_median=round(c.bytes_alg / (med * 1e-6) / 1e9, 1),
                                     calls=PIPE_CALLS, rounds=PIPE_ROUNDS)
            pipe = f"  pipelined {med:8.1f} us"
        table[c.name] = rows
        log(f"  {c.name:28s} warm {rows['warm']['us_min']:8.1f} / {rows['warm']['us_median']:8.1f} us"
            f"  cold {rows['cold']['us_min']:8.1f} / {rows['cold']['us_median']:8.1f} us (min / median){pipe}")
    del flush
    return table


def configs_table(rk, torch, dev, reps):
    """Every configuration's calls timed one by one: warm (input just read)
    and cold (Infinity Cache refilled with other clean lines first), each
    queued behind GPU work so the events measure the GPU alone."""
    from reduction_primitives_amd import workloads as W

    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    rows = []

    def timed(name, fn, nbytes, kernel, is_host=False):
        res = {}
        for mode in ("warm", "cold"):
            ts = []
            for _ in range(reps):
                if mode == "cold":
                    flush.sum()
                torch.cuda.synchronize()
                if is_host:
                    # the call returns once its value is on the host: time the call alone
                    t0 = time.perf_counter()
                    fn()
                    ts.append((time.perf_counter() - t0) * 1e6)
                    continue
                torch.cuda._sleep(1_000_000)
                b, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                b.record()
                fn()
                e.record()
                e.synchronize()
                ts.append(b.elapsed_time(e) * 1e3)
            res[mode] = dict(us_min=round(min(ts), 2), us_median=round(statistics.median(ts), 2),
                             GBps=round(nbytes / (min(ts) * 1e-6) / 1e9, 1))
        rows.append(dict(call=name, kernel=kernel, bytes=nbytes, **res))
        log(f"  {name:40s} {kernel:8s} warm {res['warm']['us_min']:8.2f} us ({res['warm']['GBps']:7.1f} GB/s)"
            f"  cold {res['cold']['us_min']:8.2f} us ({res['cold']['GBps']:7.1f} GB/s)")

    def whole(name, x, **kw):
        host = kw.get("mode") == "host"
        in_c = rk.dtype_code(x.dtype)
        acc_c = rk.dtype_code(kw["acc"]) if "acc" in kw else rk.default_acc(in_c)
        ws = rk.workspace_for(rk.rk_workspace_size(in_c, acc_c, 1, [x.numel()], [1], 1), dev)
        out = None if host else torch.zeros(1, dtype=kw.get("out_dtype", x.dtype), device=dev)

        def fn():
            rk.reduce_all(x, workspace=ws, out=out, **kw)
            return host
        timed(name, fn, x.numel() * x.element_size(), "all", is_host=host)

    def dims(name, arr, xd, d, **kw):
        plan = rk.plan_dims(xd.dtype, arr.shape, arr.strides, d)
        ws = rk.workspace_for(plan["workspace_bytes"], dev)
        out_dt = kw.get("out_dtype", xd.dtype)
        out = torch.zeros(max(1, plan["n_out"]), dtype=out_dt, device=dev)

        def fn():
            rk.reduce_dims(xd, arr.shape, arr.strides, d, workspace=ws, out=out, **kw)
            return False
        timed(name, fn, xd.numel() * xd.element_size(), plan["kernel_name"])

    def pair(name, a, b, map2, **kw):
        ws = rk.workspace_for(rk.rk_workspace_size(rk.dtype_code(a.dtype), rk.default_acc(rk.dtype_code(a.dtype)),
                                                   1, [a.numel()], [1], 1), dev)
        out = torch.zeros(1, dtype=a.dtype, device=dev)
        plan = rk.rk_plan_all2(rk.dtype_code(a.dtype), rk.default_acc(rk.dtype_code(a.dtype)),
                               a.data_ptr(), b.data_ptr(), a.numel())

        def fn():
            rk.reduce_all2(a, b, map2, workspace=ws, out=out, **kw)
            return False
        timed(name, fn, 2 * a.numel() * a.element_size(), "all2" if plan.vec > 1 else "all2/elt")

    xf, xi = W.whole_small()
    whole("1e4 f32 sum -> host", xf.data.to(dev), mode="host")
    whole("1e4 i32 sum -> int64 host", xi.data.to(dev), acc=torch.int64, out_dtype=torch.int64, mode="host")
    for n in (10**6, 10**8):
        xf, perm = W.whole_large(n)
        xd, pd = xf.data.to(dev), perm.data.to(dev)
        whole(f"{n:.0e} f32 sum -> host", xd, mode="host")
        whole(f"{n:.0e} f32 sum init 1.5 -> device", xd, init=1.5)
        whole(f"{n:.0e} f32 sum fold -> device", xd, mode="fold")
        whole(f"{n:.0e} i32 perm max", pd, op="max", acc=torch.int32, out_dtype=torch.int32)
        whole(f"{n:.0e} i32 perm min", pd, op="min", acc=torch.int32, out_dtype=torch.int32)
        del xd, pd
    for n in (10**6, 10**8):
        a, b = W.vector_pair(n)
        ad, bd = a.data.to(dev), b.data.to(dev)
        pair(f"{n:.0e} f32 dot (a*b)", ad, bd, "mul")
        pair(f"{n:.0e} f32 squared distance", ad, bd, "sqdiff")
        pair(f"{n:.0e} f32 dot, offsets 1 and 2", ad[1:n - 1], bd[2:], "mul")
        del ad, bd
    bf, f32 = W.matrix_3072x2048()
    bd, fd = bf.data.to(dev), f32.data.to(dev)
    dims("3072x2048 bf16 dims=2 -> bf16", bf, bd, 2)
    dims("3072x2048 f32 dims=2", f32, fd, 2)
    dims("3072x2048 f32 dims=1", f32, fd, 1)
    dims("3072x2048 bf16 dims=1 -> bf16", bf, bd, 1)
    for arr in W.middle_dim_3d():
        dims(f"{'x'.join(map(str, arr.shape))} {arr.name.split('_')[0]} dims=2", arr, arr.data.to(dev), 2)
    def view(name, xd, shape, strides, d):
        plan = rk.plan_dims(xd.dtype, shape, strides, d)
        ws = rk.workspace_for(plan["workspace_bytes"], dev)
        out = torch.zeros(max(1, plan["n_out"]), dtype=xd.dtype, device=dev)

        def fn():
            rk.reduce_dims(xd, shape, strides, d, workspace=ws, out=out)
            return False
        timed(name, fn, math.prod(shape) * xd.element_size(), plan["kernel_name"])

    def scan(name, xd, shape, strides, d, **kw):
        in_c = rk.dtype_code(xd.dtype)
        acc_c = rk.dtype_code(kw["acc"]) if "acc" in kw else rk.default_acc(in_c)
        out_t = kw.get("out_dtype", xd.dtype)
        ws = rk.workspace_for(rk.rk_scan_workspace_size(in_c, acc_c, len(shape), shape, strides, d - 1), dev)
        out = torch.empty(math.prod(shape), dtype=out_t, device=dev)
        plan = rk.plan_scan(xd.dtype, shape, strides, d, acc=acc_c, out_dtype=out_t, ptr=xd.data_ptr(),
                            out=out.data_ptr())

        def fn():
            rk.scan(xd, shape, strides, d, workspace=ws, out=out, **kw)
            return False
        nbytes = math.prod(shape) * (xd.element_size() + out.element_size())
        timed(name, fn, nbytes, plan["kernel_name"])

    xf, perm = W.whole_large(10**8)
    xd, pd = xf.data.to(dev), perm.data.to(dev)
    # one GPU's shard of the 1e8 sum split over eight GPUs (50 MB: fits the
    # Infinity Cache, so the cold figure is the one that counts)
    shard = xd[: 10**8 // 8]
    whole("1.25e7 f32 sum (1e8 over 8 GPUs, one shard)", shard, init=1.5)
    # reference, not a library call: torch's plain copy moves a scan's bytes
    dst = torch.empty_like(xd)

    def copy_fn():
        dst.copy_(xd)
        return False
    timed("1e+08 f32 copy (torch, read + write reference)", copy_fn, 8 * 10**8, "torch")
    del dst
    scan("1e+08 f32 cumsum (read + write)", xd, (10**8,), (1,), 1)
    scan("1e+08 f32 running max, exclusive", xd, (10**8,), (1,), 1, op="max", inclusive=False)
    scan("1e+08 i32 cumsum -> int64", pd, (10**8,), (1,), 1, acc=torch.int64, out_dtype=torch.int64)
    del xd, pd
    xf, _ = W.whole_large(10**6)
    scan("1e+06 f32 cumsum", xf.data.to(dev), (10**6,), (1,), 1)
    mf, _ = W.matrix_8192()
    md = mf.data.to(dev)
    scan("8192x8192 f32 cumsum dims=1", md, mf.shape, mf.strides, 1)
    scan("8192x8192 f32 cumsum dims=2", md, mf.shape, mf.strides, 2)
    # the same storage read as its transpose (a row-major matrix): input and
    # output contiguous along different axes
    rm = (mf.shape[1], 1)
    scan("8192x8192 f32 row-major cumsum dims=2", md, mf.shape, rm, 2)
    scan("8192x8192 f32 row-major cumsum dims=1", md, mf.shape, rm, 1)
    # few lines contiguous on one side only: 8 row-major rows along their rows, and the mirror
    scan("8x1000000 f32 row-major cumsum dims=2", md, (8, 10**6), (10**6, 1), 2)
    scan("1000000x8 f32 row-major cumsum dims=1", md, (10**6, 8), (8, 1), 1)
    del md
    pv = W.permuted_kept()
    scan("256x1024x256 f32 permuted cumsum dims=2", pv.data.to(dev), pv.shape, pv.view_strides, 2)
    for arr in W.general_layouts() + [W.permuted_kept()]:
        xd = arr.data.to(dev)
        view(arr.name, xd, arr.shape, arr.view_strides, arr.dims)
        del xd
    for arr in W.short_lines():
        scan(arr.name, arr.data.to(dev), arr.shape, arr.view_strides, arr.dims[0])
    mf, mi = W.matrix_8192()
    md, mid = mf.data.to(dev), mi.data.to(dev)
    dims("8192x8192 f32 sum dims=2", mf, md, 2)
    dims("8192x8192 f32 sum dims=1", mf, md, 1)
    dims("8192x8192 f32 max dims=2", mf, md, 2, op="max")
    dims("8192x8192 f32 sum of squares (all)", mf, md, (1, 2), map="square", init=0.0)
    dims("8192x8192 i32 sum dims=1 -> int64", mi, mid, 1, acc=torch.int64, out_dtype=torch.int64)
    del flush
    return rows


def read_ceiling(rk, torch, bufs, launches=30):
    """The device's streaming-read ceiling: the library's read-only kernel
    (16-byte non-temporal loads, one integer operation per word, no stores)
    over buffers of the size a set of calls reads (the 400 MB whole-array
    inputs, the 268 MB matrices), at a few grid sizes, each launch timed by
    events around it as the calls' kernels are.
    Consecutive launches read different buffers, so none finds the previous
    one's lines in the Infinity Cache.  Returns the best grid's figures."""
    sink = torch.zeros(1, dtype=torch.int32, device=bufs[0].device)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    nbytes = bufs[0].numel() * bufs[0].element_size()
    best = None
    for grid in (512, 1024, 2048, 4096):
        for i in range(3):
            rk.rk_debug_stream_read(bufs[i % len(bufs)].data_ptr(), nbytes, grid, sink.data_ptr(), st)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(launches)]
        for b, e in ev:
            b.record(); e.record()      # creates the HIP events
        torch.cuda.synchronize()
        for i, (b, e) in enumerate(ev):
            # the events on the kernel's own dispatch packet, as the calls' are
            rk.rk_debug_set_launch_events(ctypes.c_void_p(b.cuda_event), ctypes.c_void_p(e.cuda_event))
            try:
                rk.rk_debug_stream_read(bufs[i % len(bufs)].data_ptr(), nbytes, grid, sink.data_ptr(), st)
            finally:
                rk.rk_debug_set_launch_events(None, None)
        torch.cuda.synchronize()
        us = [b.elapsed_time(e) * 1e3 for b, e in ev]
        row = dict(grid=grid, avg_launch_us=round(statistics.mean(us), 2), min_us=round(min(us), 2))
        row["GBps"] = round(nbytes / (row["avg_launch_us"] * 1e-6) / 1e9, 1)
        log(f"  read ceiling, grid {grid:5d}: {row['avg_launch_us']:.2f} us avg, {row['min_us']:.2f} us min,"
            f" {row['GBps']:.1f} GB/s")
        if best is None or row["avg_launch_us"] < best["avg_launch_us"]:
            best = row
    return best


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              "(this library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch

    import reduction_primitives_amd as rk
    rk.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    log(f"device: {props.name}, {props.multi_processor_count} CUs")

    calls, outs, inputs, keep = build_step(rk, torch, dev)
    if args.calibration_copy:
        src = keep[0][0]
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del dst
    kernels = plan_names(rk, torch)
    bytes_step = sum(c.bytes_alg for c in calls)

    def step(events=None, every=False):
        for c in calls:
            if events is not None and (c.timed or every):
                b, e = events.pop()
                rk.rk_debug_set_launch_events(ctypes.c_void_p(b.cuda_event), ctypes.c_void_p(e.cuda_event))
                try:
                    c()
                finally:
                    rk.rk_debug_set_launch_events(None, None)
            else:
                c()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    n_timed = sum(1 for c in calls if c.timed) * args.steps
    pairs = []
    for _ in range(n_timed):
        b, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b.record(); e.record()          # creates the HIP events
        pairs.append((b, e))
    torch.cuda.synchronize()
    pending = list(reversed(pairs))

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(pending)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    ms_per_step = elapsed * 1e3 / args.steps
    value = bytes_step * args.steps / elapsed / 1e9
    launch_ms = [b.elapsed_time(e) for b, e in pairs]
    avg_launch_s = statistics.mean(launch_ms) * 1e-3
    achieved = N_WHOLE * 4 / avg_launch_s / 1e9
    log(f"step: {ms_per_step:.3f} ms, {value:.1f} GB/s aggregate ({value / PEAK_GBPS:.1%} of peak)")
    log(f"dominant kernel {DOMINANT}: {avg_launch_s * 1e6:.1f} us per launch, {achieved:.1f} GB/s")

    # every call's first kernel on its own dispatch packet's events, over as
    # many more steps (outside the timed region above)
    ev_all = []
    for _ in range(len(calls) * args.steps):
        b, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b.record(); e.record()
        ev_all.append((b, e))
    torch.cuda.synchronize()
    pending = list(reversed(ev_all))
    for _ in range(args.steps):
        step(pending, every=True)
    torch.cuda.synchronize()
    per_kernel_us = {c.name: [] for c in calls}
    for i, (b, e) in enumerate(ev_all):
        per_kernel_us[calls[i % len(calls)].name].append(b.elapsed_time(e) * 1e3)

    ceiling = read_ceiling(rk, torch, keep[0] + keep[1])
    ceiling_268 = read_ceiling(rk, torch, keep[2])
    mem = rk.rk_debug_device_info()
    log(f"read ceiling: {ceiling['GBps']:.1f} GB/s (grid {ceiling['grid']}); dominant kernel at "
        f"{achieved / ceiling['GBps']:.1%} of it")
    log(f"read ceiling over 268 MB: {ceiling_268['GBps']:.1f} GB/s (grid {ceiling_268['grid']})")
    kernels_table = {}
    for c in calls:
        us = statistics.mean(per_kernel_us[c.name])
        ceil = ceiling_268 if "8192" in c.name else ceiling
        gbps = c.bytes_alg / (us * 1e-6) / 1e9
        kernels_table[c.name] = dict(avg_us=round(us, 2), min_us=round(min(per_kernel_us[c.name]), 2),
                                     GBps=round(gbps, 1), frac_of_peak=round(gbps / PEAK_GBPS, 4),
                                     frac_of_read_ceiling=round(us and ceil["avg_launch_us"] / us, 4))
        log(f"  kernel of {c.name:28s} {us:7.2f} us avg  {gbps:7.1f} GB/s  {gbps / PEAK_GBPS:6.1%} of peak  "
            f"{ceil['avg_launch_us'] / us:6.1%} of the read ceiling at its size")

    host_value = outs["host"].value
    snap = {k: (v.detach().cpu().clone() if hasattr(v, "detach") else v) for k, v in outs.items()}
    per_call = (per_call_table(calls, torch, args.per_call_reps, args.per_call_rounds, dev)
                if args.per_call_reps > 0 else None)

    configs = configs_table(rk, torch, dev, 5) if args.all_configs else None

    cpu, parity = None, None
    if not args.no_cpu:
        log("CPU oracle baseline ...")
        cpu, parity = cpu_leg(inputs, snap, args.cpu_budget, host_value, args.cpu_min)

    traffic = traffic_from_profile()
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32,i32,i64",
        "data": "synthetic (seeded torch CPU generator, copied to HBM before timing)",
        "config": {
            "workload": "1e8 fp32 whole-array sum (host; device init=1.5; fold) + 1e8 int32 "
                        "permutation max and min + 8192x8192 fp32 column-major sum dims=2, sum "
                        "dims=1, max dims=2, whole-array sum of squares + 8192x8192 int32 sum "
                        "dims=1 into int64",
            "calls_per_step": len(calls),
            "algorithmic_bytes_per_step": bytes_step,
            "value_frac_of_peak": round(value / PEAK_GBPS, 4),
            "kernels_8192": kernels,
            "device": props.name,
            "cus": props.multi_processor_count,
            "memory": dict(clock_khz=mem["mem_clock_khz"], bus_bits=mem["mem_bus_bits"],
                           clock_x_bus_GBps=round(mem["mem_clock_khz"] * 1e3 * mem["mem_bus_bits"] / 8 / 1e9, 1)),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_GBPS, 4),
            "traffic": traffic,
            "kernel": DOMINANT,
            "algorithmic_bytes_per_launch": N_WHOLE * 4,
            "avg_launch_us": round(avg_launch_s * 1e6, 2),
            "launches_timed": len(launch_ms),
            "read_ceiling_GBps": ceiling["GBps"],
            "read_ceiling_grid": ceiling["grid"],
            "frac_of_read_ceiling": round(achieved / ceiling["GBps"], 4),
            "read_ceiling_268MB_GBps": ceiling_268["GBps"],
            "read_ceiling_268MB_us": ceiling_268["avg_launch_us"],
        },
        "kernels": kernels_table,
        "cpu_baseline": cpu,
        "parity_vs_oracle": parity,
        "per_call": per_call,
        "per_call_method": (f"{args.per_call_reps} reps x {args.per_call_rounds} rounds, calls interleaved; "
                            "min and median of the round with the lowest median; pipelined: "
                            f"{PIPE_CALLS} calls back to back on rotating inputs, one event pair, "
                            f"median of {PIPE_ROUNDS} sequences" if per_call else None),
        "configs": configs,
    }
    del keep
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
