"""The gfx950 tuning table, read from the planner's header, so that tests
derive the expected kernel choices from the same values the library uses."""
import os
import re

_HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "reduction_primitives_amd", "csrc", "rk_plan.hpp")


def values() -> dict:
    with open(_HDR) as f:
        text = f.read()
    body = text[text.index("namespace tune {"):text.index("}  // namespace tune")]
    out = {}
    for name, expr in re.findall(r"constexpr\s+\w+\s+(k\w+)\s*=\s*([^;]+);", body):
        out[name] = int(eval(expr, {}, dict(out)))
    return out
