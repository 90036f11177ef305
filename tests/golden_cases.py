"""Loader for tests/golden/closed_forms.json (hand-derived expected values)."""
from __future__ import annotations

import json
import os

import numpy as np

_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "closed_forms.json")

OPS = {"sum": 0, "max": 1, "min": 2}
MAPS = {"identity": 0, "square": 1, "abs": 2}
DTYPES = {"f32": 0, "bf16": 1, "f16": 2, "f64": 3, "i32": 4, "i64": 5}
MODES = {"overwrite": 0, "fold": 1, "host": 2}
NP_VALUE = {"f32": np.float32, "bf16": np.float32, "f16": np.float16, "f64": np.float64,
            "i32": np.int32, "i64": np.int64}


def to_raw(values, dtype: str) -> np.ndarray:
    """Exactly representable values -> raw storage of `dtype` (bf16 as uint16)."""
    a = np.asarray(values, dtype=np.float64 if dtype in ("f32", "bf16", "f16", "f64") else np.int64)
    if dtype == "bf16":
        f = a.astype(np.float32)
        assert np.all(f.view(np.uint32) & 0xFFFF == 0), "value not exact in bf16"
        return (f.view(np.uint32) >> 16).astype(np.uint16)
    if dtype == "f16":
        return a.astype(np.float16).view(np.uint16)
    return a.astype(NP_VALUE[dtype])


def _values(spec):
    if "list" in spec:
        return list(spec["list"])
    if "range" in spec:
        return list(range(*spec["range"]))
    v, count = spec["const"]
    return [v] * count


def load():
    with open(_PATH) as f:
        doc = json.load(f)
    cases = []
    for c in doc["cases"]:
        d = dict(c)
        d["op_code"] = OPS[c["op"]]
        d["map_code"] = MAPS[c["map"]]
        d["in_code"], d["acc_code"], d["out_code"] = (DTYPES[c["in"]], DTYPES[c["acc"]],
                                                      DTYPES[c["out"]])
        d["mode_code"] = MODES[c["mode"]]
        d["x_raw"] = to_raw(_values(c["x"]), c["in"])
        if c.get("prev") is not None:
            d["prev_raw"] = to_raw(np.atleast_1d(c["prev"]), c["out"])
        else:
            d["prev_raw"] = None
        cases.append(d)
    return cases
