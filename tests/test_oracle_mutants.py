"""The oracle's pins catch plausible slips (mutation testing, CPU only).

Each mutant is a copy of oracle/oracle.c with one deliberate, plausible
mistake: a dropped term, a flipped sign or comparison, a transposed index, a
wrong rounding step, a wrong bias or an init applied twice.  The copy is
compiled to a temporary library and the pin suite (tests/test_oracle.py) is
run against it in a child process; every mutant must make the suite fail.
The real oracle is untouched.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, text in oracle.c, replacement, which occurrence: 1 = first only)
MUTANTS = [
    ("drop_first_term", "for (int64_t i = 0; i < n; ++i)\n        acc = op_fp(",
     "for (int64_t i = 1; i < n; ++i)\n        acc = op_fp("),
    ("sum_sign", "case O_SUM:\n        return acc + v;", "case O_SUM:\n        return acc - v;"),
    ("max_compare", "return v > acc ? v : acc;", "return v < acc ? v : acc;"),
    ("min_compare", "return v < acc ? v : acc;", "return v < acc ? acc : v;"),
    ("init_twice_fp", "double acc = start;", "double acc = start + start;"),
    ("init_dropped_int", "int64_t acc = start;", "int64_t acc = 0;"),
    ("abs_is_identity", "case M_ABS: return fabs(v);", "case M_ABS: return v;"),
    ("square_is_double", "case M_SQUARE: u = u * u; break;", "case M_SQUARE: u = u + u; break;"),
    ("no_i32_wrap", "if (dtype == D_I32)\n        return (int64_t)(int32_t)",
     "if (dtype == D_I64)\n        return (int64_t)(int32_t)"),
    ("max_identity_zero", "if (op == O_MAX) return -INFINITY;", "if (op == O_MAX) return 0.0;"),
    ("bf16_truncates", "nearbyint(ldexp(a, -q))", "floor(ldexp(a, -q))"),
    ("bf16_decode_shift", "(uint32_t)h << 16", "(uint32_t)h << 15"),
    ("f16_decode_bias", "expo - 25", "expo - 24"),
    ("f16_encode_bias", "(e - 1 + 15) << 10", "(e + 15) << 10"),
    ("dims_transposed_stride", "off += idx[d] * strides[d];",
     "off += idx[d] * strides[ndim - 1 - d];"),
    ("dims_out_index", "out_stride[d] = no;\n            no *= shape[d];",
     "no *= shape[d];\n            out_stride[d] = no - 1;"),
    ("dims_int_no_wrap", "result[o] = wrap_to(acc_dtype, result[o]);", "(void)0;"),
    ("map2_mul_is_add", "case M2_MUL: return a * b;", "case M2_MUL: return a + b;"),
    ("map2_sqdiff_sign", "case M2_SQDIFF: return (a - b) * (a - b);", "case M2_SQDIFF: return (a + b) * (a - b);"),
    ("map2_absdiff_no_abs", "case M2_ABSDIFF: return fabs(a - b);", "case M2_ABSDIFF: return a - b;"),
    ("map2_int_mul", "case M2_MUL: r = ua * ub; break;", "case M2_MUL: r = ua * ua; break;"),
    ("all2_second_operand", "load_fp(in_dtype, b, i)));", "load_fp(in_dtype, a, i)));"),
    ("scan_inclusive_stores_before", "run = op_fp(op, run, v);\n            out[i] = run;",
     "out[i] = run;\n            run = op_fp(op, run, v);"),
    ("scan_int_start_dropped", "int64_t run = wrap_to(acc_dtype, start);", "int64_t run = 0;"),
    ("scan_int_no_wrap", "run = wrap_to(acc_dtype, op_int(op, run, v));\n            out[i] = run;",
     "run = op_int(op, run, v);\n            out[i] = run;"),
    ("scan_dims_wrong_dim", "if (d == dim) {\n            line_stride[d] = 0;",
     "if (d + 1 == dim) {\n            line_stride[d] = 0;"),
    ("scan_dims_int_exclusive_swapped", "out[t] = run[l];\n            run[l] = wrap_to(acc_dtype, op_int(op, run[l], v));",
     "run[l] = wrap_to(acc_dtype, op_int(op, run[l], v));\n            out[t] = run[l];"),
]


def _compile(src_text: str, out_dir: str) -> str:
    c_path = os.path.join(out_dir, "oracle_mutant.c")
    so_path = os.path.join(out_dir, "liboracle_mutant.so")
    with open(c_path, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-std=c11", "-fPIC", "-shared",
                    "-o", so_path, c_path, "-lm"], check=True)
    return so_path


def _run_pins(lib_path: str) -> int:
    env = dict(os.environ, RKO_LIB=lib_path, PYTHONDONTWRITEBYTECODE="1")
    proc = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", "test_oracle.py")],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return proc.returncode


def test_unmutated_copy_passes():
    with open(SRC) as f:
        text = f.read()
    with tempfile.TemporaryDirectory() as d:
        assert _run_pins(_compile(text, d)) == 0


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    with open(SRC) as f:
        text = f.read()
    assert old in text, f"mutation site of {name} not found in oracle.c"
    mutated = text.replace(old, new, 1)
    with tempfile.TemporaryDirectory() as d:
        assert _run_pins(_compile(mutated, d)) != 0, f"pins did not catch mutant {name}"
