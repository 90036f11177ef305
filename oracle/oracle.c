/*
 * oracle.c -- plain, sequential CPU reference for the device-wide mapreduce.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no header, table or helper with the GPU path.
 *
 * What it computes is the plain definition of a mapped reduction, as stated on
 * the AcceleratedKernels.jl pull-request pages:
 *   - "Finish whole-array reductions on the device" (PR #139), sections
 *     "What changes" and "Compatibility": a whole array is folded with `op`
 *     after applying `f` to every element; `init` enters exactly once;
 *     alternatively the fold continues from the output's previous value;
 *     partial results live in the accumulator type until the final store.
 *   - PR #176 (strided reductions along dims), section "This PR": the same
 *     fold for each output of a reduction along one or more dimensions of a
 *     column-major array.
 *   - PR #139, "What changes" and the test list under "Compatibility": the
 *     source may be a lazy broadcast, here of two arrays, f(a_i, b_i), folded
 *     the same way (rko_all2_*).
 *   - PR #202 (tile scans), opening paragraph: accumulate!, the same fold
 *     with every prefix stored, over a whole array or along one dim
 *     (rko_scan_*).
 * The GPU path reaches the same exact value by re-associating the fold; the
 * pages state that only rounding may differ when the reduction tree changes
 * (PR #139, "Compatibility").  So this file is the definition written out:
 * one left-to-right loop in index order, no blocking, no reordering.
 *
 * Precision: floating-point inputs are accumulated in double (exact decoding
 * of f32, bf16 and f16; f64 is kept as is), integers in int64 with explicit
 * two's-complement wrap-around to the accumulator width.  Integer maps
 * (square, abs) are evaluated in the accumulator type, because the method
 * widens an element to the accumulator before mapping it; for floating point
 * the map is evaluated in double.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared (no -ffast-math), so every
 * double operation is a single correctly rounded IEEE operation in program
 * order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Codes of this file; the integer values match the library's public enums so a
 * test can pass the same numbers to both, but nothing is shared. */
enum { O_SUM = 0, O_MAX = 1, O_MIN = 2 };
enum { M_IDENTITY = 0, M_SQUARE = 1, M_ABS = 2 };
enum { D_F32 = 0, D_BF16 = 1, D_F16 = 2, D_F64 = 3, D_I32 = 4, D_I64 = 5 };

static int is_fp_dtype(int d) { return d == D_F32 || d == D_BF16 || d == D_F16 || d == D_F64; }
static int is_int_dtype(int d) { return d == D_I32 || d == D_I64; }

/* ---------------------------------------------------------------- decoding */

static double bf16_bits_to_double(uint16_t h)
{
    /* bf16 is the upper half of an IEEE binary32 pattern. */
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static double f16_bits_to_double(uint16_t h)
{
    /* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
    int sign = h >> 15;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);                 /* subnormal: frac * 2^-24 */
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(frac + 1024), expo - 25);  /* (1 + frac/1024) * 2^(expo-15) */
    return sign ? -v : v;
}

static double load_fp(int dtype, const void *x, int64_t i)
{
    switch (dtype) {
    case D_F32: return (double)((const float *)x)[i];
    case D_BF16: return bf16_bits_to_double(((const uint16_t *)x)[i]);
    case D_F16: return f16_bits_to_double(((const uint16_t *)x)[i]);
    case D_F64: return ((const double *)x)[i];
    }
    return NAN;
}

static int64_t load_int(int dtype, const void *x, int64_t i)
{
    if (dtype == D_I32)
        return (int64_t)((const int32_t *)x)[i];
    return ((const int64_t *)x)[i];
}

/* Two's-complement wrap of v to the width of an integer dtype. */
static int64_t wrap_to(int dtype, int64_t v)
{
    if (dtype == D_I32)
        return (int64_t)(int32_t)(uint32_t)(uint64_t)v;
    return v;
}

/* --------------------------------------------------------- map and operator */

static double map_fp(int map, double v)
{
    switch (map) {
    case M_SQUARE: return v * v;
    case M_ABS: return fabs(v);
    }
    return v;
}

/* Integer maps are evaluated in the accumulator type, with wrap-around. */
static int64_t map_int(int map, int acc_dtype, int64_t v)
{
    uint64_t u = (uint64_t)v;
    switch (map) {
    case M_SQUARE: u = u * u; break;
    case M_ABS: u = v < 0 ? (uint64_t)0 - u : u; break;
    }
    return wrap_to(acc_dtype, (int64_t)u);
}

/* max/min propagate NaN: once either operand is NaN the result is NaN. */
static double op_fp(int op, double acc, double v)
{
    switch (op) {
    case O_SUM:
        return acc + v;
    case O_MAX:
        if (isnan(acc) || isnan(v))
            return NAN;
        return v > acc ? v : acc;
    case O_MIN:
        if (isnan(acc) || isnan(v))
            return NAN;
        return v < acc ? v : acc;
    }
    return NAN;
}

static int64_t op_int(int op, int64_t acc, int64_t v)
{
    switch (op) {
    case O_SUM: return (int64_t)((uint64_t)acc + (uint64_t)v);
    case O_MAX: return v > acc ? v : acc;
    case O_MIN: return v < acc ? v : acc;
    }
    return 0;
}

/* --------------------------------------------------------------- identities */

double rko_identity_fp(int op)
{
    if (op == O_MAX) return -INFINITY;
    if (op == O_MIN) return INFINITY;
    return 0.0;
}

int64_t rko_identity_int(int op, int acc_dtype)
{
    if (op == O_MAX) return acc_dtype == D_I32 ? (int64_t)INT32_MIN : INT64_MIN;
    if (op == O_MIN) return acc_dtype == D_I32 ? (int64_t)INT32_MAX : INT64_MAX;
    return 0;
}

/* ------------------------------------------------------------- whole array */

/* R = start (+) f(x[0]) (+) f(x[1]) (+) ... (+) f(x[n-1]), left to right. */
int rko_all_fp(int op, int map, int in_dtype, const void *x, int64_t n,
               double start, double *result)
{
    if (!is_fp_dtype(in_dtype) || n < 0 || (n > 0 && !x) || !result)
        return -1;
    double acc = start;
    for (int64_t i = 0; i < n; ++i)
        acc = op_fp(op, acc, map_fp(map, load_fp(in_dtype, x, i)));
    *result = acc;
    return 0;
}

int rko_all_int(int op, int map, int in_dtype, int acc_dtype, const void *x,
                int64_t n, int64_t start, int64_t *result)
{
    if (!is_int_dtype(in_dtype) || !is_int_dtype(acc_dtype) || n < 0 ||
        (n > 0 && !x) || !result)
        return -1;
    int64_t acc = start;
    for (int64_t i = 0; i < n; ++i)
        acc = op_int(op, acc, map_int(map, acc_dtype, load_int(in_dtype, x, i)));
    *result = wrap_to(acc_dtype, acc);
    return 0;
}

/* ------------------------------------------------- two-input (fused) source */

/*
 * Whole-array reduction of a fused two-input source, f(a_i, b_i): the
 * broadcast of two arrays that AcceleratedKernels.jl PR #139 ("What
 * changes", last paragraph, and its test list) routes to the whole-array
 * path.  f is a*b, (a-b)^2 or |a-b|, evaluated after widening both
 * elements: in double for floating point, in the accumulator type (with
 * wrap-around) for integers.  Same left-to-right fold as rko_all_*.
 */
enum { M2_MUL = 0, M2_SQDIFF = 1, M2_ABSDIFF = 2 };

static double map2_fp(int map2, double a, double b)
{
    switch (map2) {
    case M2_MUL: return a * b;
    case M2_SQDIFF: return (a - b) * (a - b);
    case M2_ABSDIFF: return fabs(a - b);
    }
    return NAN;
}

static int64_t map2_int(int map2, int acc_dtype, int64_t a, int64_t b)
{
    uint64_t ua = (uint64_t)wrap_to(acc_dtype, a), ub = (uint64_t)wrap_to(acc_dtype, b), r = 0;
    int64_t d;
    switch (map2) {
    case M2_MUL: r = ua * ub; break;
    case M2_SQDIFF:
        d = wrap_to(acc_dtype, (int64_t)(ua - ub));
        r = (uint64_t)d * (uint64_t)d;
        break;
    case M2_ABSDIFF:
        d = wrap_to(acc_dtype, (int64_t)(ua - ub));
        r = d < 0 ? (uint64_t)0 - (uint64_t)d : (uint64_t)d;
        break;
    }
    return wrap_to(acc_dtype, (int64_t)r);
}

int rko_all2_fp(int op, int map2, int in_dtype, const void *a, const void *b, int64_t n,
                double start, double *result)
{
    if (!is_fp_dtype(in_dtype) || n < 0 || (n > 0 && (!a || !b)) || !result)
        return -1;
    double acc = start;
    for (int64_t i = 0; i < n; ++i)
        acc = op_fp(op, acc, map2_fp(map2, load_fp(in_dtype, a, i), load_fp(in_dtype, b, i)));
    *result = acc;
    return 0;
}

int rko_all2_int(int op, int map2, int in_dtype, int acc_dtype, const void *a, const void *b,
                 int64_t n, int64_t start, int64_t *result)
{
    if (!is_int_dtype(in_dtype) || !is_int_dtype(acc_dtype) || n < 0 ||
        (n > 0 && (!a || !b)) || !result)
        return -1;
    int64_t acc = start;
    for (int64_t i = 0; i < n; ++i)
        acc = op_int(op, acc, map2_int(map2, acc_dtype, load_int(in_dtype, a, i),
                                       load_int(in_dtype, b, i)));
    *result = wrap_to(acc_dtype, acc);
    return 0;
}

/* -------------------------------------------------------------------- dims */

/*
 * Reduction along the dims whose bit is set in `mask` of a column-major
 * strided array: shape[d] elements along dim d, element stride strides[d].
 * Outputs are the kept dims, stored contiguously in column-major order.  Each
 * output's fold starts from start[o] and takes its elements in increasing
 * column-major order of their reduced indices.  This walks the input once, in
 * column-major order, so every output sees exactly that order.
 */
static int dims_setup(int ndim, const int64_t *shape, const int64_t *strides,
                      uint32_t mask, int64_t *out_stride, int64_t *n_out,
                      int64_t *total)
{
    if (ndim < 1 || ndim > 8 || !shape || !strides)
        return -1;
    if (mask >> ndim)
        return -1;
    int64_t no = 1, tot = 1;
    for (int d = 0; d < ndim; ++d) {
        if (shape[d] < 0 || strides[d] < 0)
            return -1;
        tot *= shape[d];
        if (mask & (1u << d)) {
            out_stride[d] = 0;
        } else {
            out_stride[d] = no;
            no *= shape[d];
        }
    }
    *n_out = no;
    *total = tot;
    return 0;
}

int rko_dims_fp(int op, int map, int in_dtype, const void *x, int ndim,
                const int64_t *shape, const int64_t *strides, uint32_t mask,
                const double *start, double *result)
{
    int64_t ostr[8], n_out, total;
    if (!is_fp_dtype(in_dtype) || dims_setup(ndim, shape, strides, mask, ostr, &n_out, &total))
        return -1;
    for (int64_t o = 0; o < n_out; ++o)
        result[o] = start[o];
    int64_t idx[8] = {0};
    for (int64_t t = 0; t < total; ++t) {
        int64_t off = 0, o = 0;
        for (int d = 0; d < ndim; ++d) {
            off += idx[d] * strides[d];
            o += idx[d] * ostr[d];
        }
        result[o] = op_fp(op, result[o], map_fp(map, load_fp(in_dtype, x, off)));
        for (int d = 0; d < ndim; ++d) {   /* column-major odometer: dim 0 fastest */
            if (++idx[d] < shape[d])
                break;
            idx[d] = 0;
        }
    }
    return 0;
}

int rko_dims_int(int op, int map, int in_dtype, int acc_dtype, const void *x,
                 int ndim, const int64_t *shape, const int64_t *strides,
                 uint32_t mask, const int64_t *start, int64_t *result)
{
    int64_t ostr[8], n_out, total;
    if (!is_int_dtype(in_dtype) || !is_int_dtype(acc_dtype) ||
        dims_setup(ndim, shape, strides, mask, ostr, &n_out, &total))
        return -1;
    for (int64_t o = 0; o < n_out; ++o)
        result[o] = start[o];
    int64_t idx[8] = {0};
    for (int64_t t = 0; t < total; ++t) {
        int64_t off = 0, o = 0;
        for (int d = 0; d < ndim; ++d) {
            off += idx[d] * strides[d];
            o += idx[d] * ostr[d];
        }
        result[o] = op_int(op, result[o], map_int(map, acc_dtype, load_int(in_dtype, x, off)));
        for (int d = 0; d < ndim; ++d) {
            if (++idx[d] < shape[d])
                break;
            idx[d] = 0;
        }
    }
    for (int64_t o = 0; o < n_out; ++o)
        result[o] = wrap_to(acc_dtype, result[o]);
    return 0;
}

/* ------------------------------------------------------------------- scans */

/*
 * Prefix folds (scans): AcceleratedKernels.jl PR #202 (tile scans), opening
 * paragraph -- accumulate! over a whole array, and along one dim.  Output k
 * of a line is s (+) x_0 (+) ... (+) x_k when inclusive, and
 * s (+) x_0 (+) ... (+) x_(k-1) when exclusive (so the first output is s).
 * The running value is a double (floating inputs) or an int64 wrapped to the
 * accumulator width after every step (integers), updated left to right.
 */
int rko_scan_fp(int op, int in_dtype, const void *x, int64_t n, double start, int inclusive,
                double *out)
{
    if (!is_fp_dtype(in_dtype) || n < 0 || (n > 0 && (!x || !out)))
        return -1;
    double run = start;
    for (int64_t i = 0; i < n; ++i) {
        const double v = load_fp(in_dtype, x, i);
        if (inclusive) {
            run = op_fp(op, run, v);
            out[i] = run;
        } else {
            out[i] = run;
            run = op_fp(op, run, v);
        }
    }
    return 0;
}

int rko_scan_int(int op, int in_dtype, int acc_dtype, const void *x, int64_t n, int64_t start,
                 int inclusive, int64_t *out)
{
    if (!is_int_dtype(in_dtype) || !is_int_dtype(acc_dtype) || n < 0 || (n > 0 && (!x || !out)))
        return -1;
    int64_t run = wrap_to(acc_dtype, start);
    for (int64_t i = 0; i < n; ++i) {
        const int64_t v = wrap_to(acc_dtype, load_int(in_dtype, x, i));
        if (inclusive) {
            run = wrap_to(acc_dtype, op_int(op, run, v));
            out[i] = run;
        } else {
            out[i] = run;
            run = wrap_to(acc_dtype, op_int(op, run, v));
        }
    }
    return 0;
}

/*
 * Scan along dim `dim` (0-based) of a strided column-major view: every line
 * (all indices fixed but the one along `dim`) is scanned on its own, from
 * `start`.  The output has the view's shape, stored contiguously in
 * column-major order.  The input is walked once in column-major order, which
 * visits each line's elements in increasing order along `dim`.
 */
static int scan_dims_setup(int ndim, const int64_t *shape, const int64_t *strides, int dim,
                           int64_t *line_stride, int64_t *n_lines, int64_t *total)
{
    if (ndim < 1 || ndim > 8 || !shape || !strides || dim < 0 || dim >= ndim)
        return -1;
    int64_t nl = 1, tot = 1;
    for (int d = 0; d < ndim; ++d) {
        if (shape[d] < 0 || strides[d] < 0)
            return -1;
        tot *= shape[d];
        if (d == dim) {
            line_stride[d] = 0;
        } else {
            line_stride[d] = nl;
            nl *= shape[d];
        }
    }
    *n_lines = nl;
    *total = tot;
    return 0;
}

int rko_scan_dims_fp(int op, int in_dtype, const void *x, int ndim, const int64_t *shape,
                     const int64_t *strides, int dim, double start, int inclusive, double *out)
{
    int64_t lstr[8], n_lines, total;
    if (!is_fp_dtype(in_dtype) || scan_dims_setup(ndim, shape, strides, dim, lstr, &n_lines, &total))
        return -1;
    if (total == 0)
        return 0;
    double *run = malloc(sizeof(double) * (size_t)n_lines);
    if (!run)
        return -1;
    for (int64_t l = 0; l < n_lines; ++l)
        run[l] = start;
    int64_t idx[8] = {0};
    for (int64_t t = 0; t < total; ++t) {       /* t is also the output's column-major index */
        int64_t off = 0, l = 0;
        for (int d = 0; d < ndim; ++d) {
            off += idx[d] * strides[d];
            l += idx[d] * lstr[d];
        }
        const double v = load_fp(in_dtype, x, off);
        if (inclusive) {
            run[l] = op_fp(op, run[l], v);
            out[t] = run[l];
        } else {
            out[t] = run[l];
            run[l] = op_fp(op, run[l], v);
        }
        for (int d = 0; d < ndim; ++d) {
            if (++idx[d] < shape[d])
                break;
            idx[d] = 0;
        }
    }
    free(run);
    return 0;
}

int rko_scan_dims_int(int op, int in_dtype, int acc_dtype, const void *x, int ndim,
                      const int64_t *shape, const int64_t *strides, int dim, int64_t start,
                      int inclusive, int64_t *out)
{
    int64_t lstr[8], n_lines, total;
    if (!is_int_dtype(in_dtype) || !is_int_dtype(acc_dtype) ||
        scan_dims_setup(ndim, shape, strides, dim, lstr, &n_lines, &total))
        return -1;
    if (total == 0)
        return 0;
    int64_t *run = malloc(sizeof(int64_t) * (size_t)n_lines);
    if (!run)
        return -1;
    for (int64_t l = 0; l < n_lines; ++l)
        run[l] = wrap_to(acc_dtype, start);
    int64_t idx[8] = {0};
    for (int64_t t = 0; t < total; ++t) {
        int64_t off = 0, l = 0;
        for (int d = 0; d < ndim; ++d) {
            off += idx[d] * strides[d];
            l += idx[d] * lstr[d];
        }
        const int64_t v = wrap_to(acc_dtype, load_int(in_dtype, x, off));
        if (inclusive) {
            run[l] = wrap_to(acc_dtype, op_int(op, run[l], v));
            out[t] = run[l];
        } else {
            out[t] = run[l];
            run[l] = wrap_to(acc_dtype, op_int(op, run[l], v));
        }
        for (int d = 0; d < ndim; ++d) {
            if (++idx[d] < shape[d])
                break;
            idx[d] = 0;
        }
    }
    free(run);
    return 0;
}

/* ----------------------------------------------------------- final storing */

/*
 * Round a double to the nearest value with `bits` significant bits, ties to
 * even, with the subnormal quantum 2^min_q and overflow to infinity at
 * 2^max_e (IEEE round-to-nearest-even done in one step from double).
 */
static double round_to_format(double a, int bits, int min_q, int max_e)
{
    if (a == 0.0 || isinf(a) || isnan(a))
        return a;
    int e;
    frexp(a, &e);              /* a = f * 2^e with f in [0.5, 1) */
    int q = e - bits;          /* weight of the last kept bit */
    if (q < min_q)
        q = min_q;
    double r = ldexp(nearbyint(ldexp(a, -q)), q);   /* default mode: ties to even */
    if (r >= ldexp(1.0, max_e))
        r = INFINITY;
    return r;
}

static uint16_t double_to_bf16_bits(double v)
{
    if (isnan(v))
        return signbit(v) ? 0xffc0 : 0x7fc0;
    /* bf16: 8 significant bits, exponent range of binary32. */
    double r = round_to_format(fabs(v), 8, -133, 128);
    float f = (float)r;        /* exact: r has at most 8 significant bits */
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    uint16_t h = (uint16_t)(bits >> 16);
    return signbit(v) ? (uint16_t)(h | 0x8000) : h;
}

static uint16_t double_to_f16_bits(double v)
{
    if (isnan(v))
        return signbit(v) ? 0xfe00 : 0x7e00;
    /* binary16: 11 significant bits, subnormal quantum 2^-24, max < 2^16. */
    double r = round_to_format(fabs(v), 11, -24, 16);
    uint16_t h;
    if (isinf(r)) {
        h = 0x7c00;
    } else if (r < ldexp(1.0, -14)) {
        h = (uint16_t)ldexp(r, 24);                     /* subnormal or zero */
    } else {
        int e;
        double f = frexp(r, &e);                        /* r = f * 2^e, f in [0.5, 1) */
        int frac = (int)ldexp(f, 11) - 1024;            /* 10 stored fraction bits */
        h = (uint16_t)(((e - 1 + 15) << 10) | frac);
    }
    return signbit(v) ? (uint16_t)(h | 0x8000) : h;
}

/* Store n wide floating-point results in out_dtype (round to nearest even). */
int rko_cast_fp(int out_dtype, const double *v, int64_t n, void *dst)
{
    for (int64_t i = 0; i < n; ++i) {
        switch (out_dtype) {
        case D_F32: ((float *)dst)[i] = (float)v[i]; break;
        case D_BF16: ((uint16_t *)dst)[i] = double_to_bf16_bits(v[i]); break;
        case D_F16: ((uint16_t *)dst)[i] = double_to_f16_bits(v[i]); break;
        case D_F64: ((double *)dst)[i] = v[i]; break;
        default: return -1;
        }
    }
    return 0;
}

/* Store n wide integer results in out_dtype (two's-complement wrap). */
int rko_cast_int(int out_dtype, const int64_t *v, int64_t n, void *dst)
{
    for (int64_t i = 0; i < n; ++i) {
        switch (out_dtype) {
        case D_I32: ((int32_t *)dst)[i] = (int32_t)(uint32_t)(uint64_t)v[i]; break;
        case D_I64: ((int64_t *)dst)[i] = v[i]; break;
        default: return -1;
        }
    }
    return 0;
}

/* Decode n stored values of a dtype to the wide type (used to read back an
 * output's previous value, and by the tests). */
int rko_widen_fp(int dtype, const void *src, int64_t n, double *dst)
{
    if (!is_fp_dtype(dtype))
        return -1;
    for (int64_t i = 0; i < n; ++i)
        dst[i] = load_fp(dtype, src, i);
    return 0;
}

int rko_widen_int(int dtype, const void *src, int64_t n, int64_t *dst)
{
    if (!is_int_dtype(dtype))
        return -1;
    for (int64_t i = 0; i < n; ++i)
        dst[i] = load_int(dtype, src, i);
    return 0;
}
