"""Build librk.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m reduction_primitives_amd.build [--force]

Each input dtype's kernels are one translation unit; they compile in
parallel with hipcc and link into reduction_primitives_amd/librk.so.
Objects go to reduction_primitives_amd/_build/.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "librk.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")

ARCH = "gfx950"
# -ffp-contract=off: a mapped square followed by a sum stays a rounded
# multiply then a rounded add, never one fused operation.
# -packed-fp32-ops: the compiler emits no packed FP32 VALU instructions.
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-I" + INCLUDE, "-I" + CSRC]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I" + INCLUDE, "-I" + CSRC]

KERNEL_UNITS = ["kern_f32.hip", "kern_bf16.hip", "kern_f16.hip", "kern_f64.hip",
                "kern_i32.hip", "kern_i64.hip",
                "scan_f32.hip", "scan_bf16.hip", "scan_f16.hip", "scan_f64.hip",
                "scan_i32.hip", "scan_i64.hip", "diag.hip"]
HIP_HOST_UNITS = ["rk_api.cpp"]           # host code that calls the HIP runtime
PURE_UNITS = ["rk_plan.cpp"]              # plain C++


# The files the reduction kernels of kern_f32.hip are compiled from (the
# scan translation units and the host code are not among them).
REDUCTION_KERNEL_SOURCES = ["kern_f32.hip", "rk_kernels.hpp", "rk_device.hpp", "rk_launch.hpp", "rk_plan.hpp"]


def _code_only(text: str) -> str:
    """C++ source without comments and with whitespace runs collapsed (the
    kernel sources hold no string literals with comment markers)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_digest(sources=None) -> str:
    """SHA-256 over the code (comments and layout ignored) and compile flags
    of the float32 reduction kernels: identifies the kernels a stored counter
    profile was taken on.  `sources` maps file names to text (default: the
    files in csrc)."""
    import hashlib
    h = hashlib.sha256(" ".join(HIP_FLAGS[:-2]).encode())
    for name in REDUCTION_KERNEL_SOURCES:
        if sources is None:
            with open(os.path.join(CSRC, name)) as f:
                text = f.read()
        else:
            text = sources[name]
        h.update(name.encode() + b"\0" + _code_only(text).encode())
    return h.hexdigest()


def _headers():
    hs = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hpp", ".h"))]
    hs.append(os.path.join(INCLUDE, "rk.h"))
    return hs


def _stale(obj: str, src: str) -> bool:
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    return any(os.path.getmtime(p) > t for p in [src] + _headers())


def _compile(src_name: str, force: bool):
    src = os.path.join(CSRC, src_name)
    obj = os.path.join(OUT_DIR, src_name + ".o")
    if not force and not _stale(obj, src):
        return obj, None
    if src_name in PURE_UNITS:
        cmd = ["g++"] + HOST_FLAGS + ["-c", src, "-o", obj]
    elif src_name in HIP_HOST_UNITS:
        cmd = [HIPCC] + HIP_FLAGS + ["-x", "hip", "-c", src, "-o", obj]
    else:
        cmd = [HIPCC] + HIP_FLAGS + ["-c", src, "-o", obj]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{proc.stdout}\n{proc.stderr}")
    # hipcc's host pass does not know the packed-fp32 feature and says so
    noise = [l for l in proc.stderr.splitlines() if l.strip() and "packed-fp32-ops" not in l]
    return obj, "\n".join(noise) or None


def build(force: bool = False, jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every unit (only stale ones unless force) and link librk.so."""
    os.makedirs(OUT_DIR, exist_ok=True)
    units = KERNEL_UNITS + HIP_HOST_UNITS + PURE_UNITS
    jobs = jobs or min(len(units), max(1, min(os.cpu_count() or 1, 16)))
    objs = []
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for obj, msg in ex.map(lambda s: _compile(s, force), units):
            objs.append(obj)
            if msg and verbose:
                print(msg, file=sys.stderr)
    newest = max(os.path.getmtime(o) for o in objs)
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < newest:
        tmp = LIB + ".tmp"
        cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs + \
              ["-Wl,-rpath," + os.path.join(ROCM, "lib")]
        proc = subprocess.run(cmd, capture_output=True, text=True)
        if proc.returncode != 0:
            raise RuntimeError(f"link failed: {' '.join(cmd)}\n{proc.stdout}\n{proc.stderr}")
        os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--force", action="store_true", help="recompile every unit")
    ap.add_argument("-j", "--jobs", type=int, default=None)
    args = ap.parse_args(argv)
    print(build(force=args.force, jobs=args.jobs, verbose=True))


if __name__ == "__main__":
    main()
