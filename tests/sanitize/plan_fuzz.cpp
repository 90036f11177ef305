// plan_fuzz.cpp -- randomized check of the host planner (rk_plan.cpp), built
// with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_sanitizers.py; no GPU, no HIP.
//
// The planner does every call's 64-bit shape, stride, split and workspace
// arithmetic (AcceleratedKernels.jl PR #176, "This PR": one selector
// chooses the kernel and its split).  This driver feeds it random layouts --
// empty, broadcast, permuted, ragged, misaligned, and extents and strides up
// to the 2^62 limit -- over every dtype pair and several CU counts, lets the
// sanitizers catch overflow and out-of-bounds access, and checks that each
// accepted plan is consistent: its parts cover the reduced elements, its
// grid covers its units, the normalised layouts address the same span, and
// the workspace holds what the kernels write.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>

#include "rk_plan.hpp"
#include "rk_scan_plan.hpp"

using namespace rk;

static int64_t g_cases = 0, g_accepted = 0;

#define CHECK(cond)                                                                              \
    do {                                                                                         \
        if (!(cond)) {                                                                           \
            std::fprintf(stderr, "check failed: %s (line %d, case %lld)\n", #cond, __LINE__,   \
                         (long long)g_cases);                                                    \
            std::exit(1);                                                                        \
        }                                                                                        \
    } while (0)

static int64_t span_of(const Layout &l)
{
    int64_t s = 0;
    for (int i = 0; i < l.nd; ++i)
        s += (l.ext[i] - 1) * l.str[i];
    return s;
}

static void check_all_plan(const AllPlan &a, int64_t n, int acc, int cus)
{
    CHECK(a.head >= 0 && a.tail >= 0 && a.nvec >= 0);
    CHECK(a.head + a.nvec * a.vec + a.tail == n);
    CHECK(a.grid >= 1 && a.grid <= (cus > 0 ? cus : tune::kDefaultCus) * tune::kAllBlocksPerCu);
    CHECK(a.ws_bytes % 256 == 0);
    CHECK(int64_t(a.ws_bytes) >= host_seq_offset(a.grid, dtype_size(acc)) + 4);
}

static void fuzz_all(std::mt19937_64 &rng)
{
    static const int64_t ns[] = {0, 1, 2, 3, 15, 16, 17, 2047, 2048, 2049, 4096 * 3 + 5, 10000, 1000003,
                                 100000000, int64_t(1) << 31, (int64_t(1) << 40) + 7, (int64_t(1) << 59) - 1,
                                 (int64_t(1) << 61), INT64_MAX};
    const int64_t n = ns[rng() % (sizeof ns / sizeof ns[0])];
    const int in = int(rng() % 7), acc = int(rng() % 7);
    const int cus = int(rng() % 3) == 0 ? 0 : int(1 + rng() % 320);
    const uintptr_t addr = uintptr_t(rng() % 64) * (in < 6 && dtype_size(in) ? dtype_size(in) : 1);
    AllPlan a;
    ++g_cases;
    if (plan_all(in, acc, addr, n, cus, &a) != ST_OK)
        return;
    ++g_accepted;
    check_all_plan(a, n, acc, cus);
    AllPlan b;
    const uintptr_t addr2 = uintptr_t(rng() % 64) * dtype_size(in);
    if (plan_all2(in, acc, addr, addr2, n, cus, &b) == ST_OK) {
        CHECK(b.head + b.nvec * b.vec + b.tail == n);
        CHECK(b.ws_bytes == a.ws_bytes && b.grid == a.grid);
    }
}

// The column-major stride after a dim of extent e, saturated at 2^62.
static int64_t next_stride(int64_t cm, int64_t e)
{
    const __int128 v = __int128(cm) * (e > 0 ? e : 1);
    return v > (__int128(1) << 62) ? int64_t(1) << 62 : int64_t(v);
}

static int64_t pick_extent(std::mt19937_64 &rng)
{
    static const int64_t es[] = {0, 1, 1, 2, 3, 7, 8, 31, 32, 33, 64, 100, 127, 128, 129, 768, 1000, 1024,
                                 2048, 3072, 4096, 8192, 65537};
    switch (rng() % 8) {
    case 0: return int64_t(rng() % 5000);
    case 1: return int64_t(1) << (rng() % 63);          // up to 2^62: mostly rejected
    default: return es[rng() % (sizeof es / sizeof es[0])];
    }
}

static void fuzz_dims(std::mt19937_64 &rng)
{
    const int nd = int(1 + rng() % 4);
    int64_t shape[4], strides[4];
    for (int i = 0; i < nd; ++i)
        shape[i] = pick_extent(rng);
    // strides: column-major, then maybe permuted, padded, broadcast or huge
    int64_t cm = 1;
    for (int i = 0; i < nd; ++i) {
        strides[i] = cm;
        cm = next_stride(cm, shape[i]);
    }
    switch (rng() % 6) {
    case 0: std::shuffle(strides, strides + nd, rng); break;
    case 1: strides[rng() % nd] = 0; break;
    case 2:
        for (int i = 0; i < nd; ++i)
            if (strides[i] < (int64_t(1) << 60))
                strides[i] = strides[i] * int64_t(1 + rng() % 3);
        break;
    case 3: strides[rng() % nd] = int64_t(rng() % (int64_t(1) << 62)); break;
    case 4: strides[rng() % nd] = -int64_t(1 + rng() % 5); break;    // invalid: negative
    default: break;
    }
    const uint32_t mask = uint32_t(rng() % (1u << (nd + (rng() % 8 == 0 ? 1 : 0))));   // sometimes beyond ndim
    const int in = int(rng() % 6), acc = int(rng() % 6);
    const int cus = int(rng() % 3) == 0 ? 0 : int(1 + rng() % 320);
    const uintptr_t addr = uintptr_t(rng() % 64) * dtype_size(in);
    DimsPlan d;
    ++g_cases;
    if (plan_dims(in, acc, addr, nd, shape, strides, mask, cus, &d) != ST_OK)
        return;
    ++g_accepted;
    int64_t n_out = 1, m = 1, span = 0;
    for (int i = 0; i < nd; ++i) {
        if ((mask >> i) & 1)
            m *= shape[i];
        else
            n_out *= shape[i];
        if (shape[i] > 0)
            span += (shape[i] - 1) * strides[i];
    }
    CHECK(d.n_out == n_out && d.m == m);
    CHECK(d.ws_bytes % 256 == 0);
    if (d.kernel == K_NONE)
        return;
    CHECK(d.split >= 1 && d.grid >= 1);
    if (d.split > 1)
        CHECK(int64_t(d.ws_bytes) >= int64_t(d.split) * n_out * dtype_size(acc));
    if (n_out * m > 0 && d.kernel != K_ALL) {
        int64_t s = span_of(d.kept) + span_of(d.red);
        if (d.kernel == K_GENERIC && d.vec > 1)
            s = span_of(d.kept) + (d.red.ext[0] * d.vec - 1) * 1 + (span_of(d.red) - (d.red.ext[0] - 1) * d.red.str[0]);
        CHECK(s == span);                       // normalising keeps the addressed span
    }
    switch (d.kernel) {
    case K_ALL:
        check_all_plan(d.all, m, acc, cus);
        break;
    case K_THREAD: case K_TILED: case K_COLUMNS:
        CHECK(d.run_len * d.runs == n_out);
        CHECK(d.tiles == d.runs * d.tiles_per_run && d.tiles_per_run * d.tile_outputs >= d.run_len);
        CHECK(d.grid == d.tiles * d.split);
        CHECK(d.row_len * d.segs == m);
        if (d.splits_per_seg > 1) {
            CHECK(d.split == d.segs * d.splits_per_seg);
            CHECK(d.rows_per_split * (d.splits_per_seg - 1) < d.row_len);
            CHECK(d.rows_per_split * d.splits_per_seg >= d.row_len);
        } else {
            CHECK(d.segs_per_split * (d.split - 1) < d.segs && d.segs_per_split * d.split >= d.segs);
        }
        break;
    case K_ROW:
        CHECK(d.grid * (tune::kDimsBlock / 64) >= n_out * d.split);
        CHECK(d.row_len * d.segs == m);
        if (d.splits_per_seg > 1)
            CHECK(d.rows_per_split * d.splits_per_seg >= d.row_len && d.rows_per_split % d.vec == 0);
        else
            CHECK(d.segs_per_split * d.split >= d.segs);
        break;
    case K_GENERIC:
        if (m > 0)
            CHECK(d.rows_per_split * d.split >= m / d.vec && d.rows_per_split * (d.split - 1) < m / d.vec);
        CHECK(d.grid <= n_out * d.split);
        break;
    case K_ALL_STRIDED:
        CHECK(d.all.n == m && d.all.grid >= 1);
        CHECK(int64_t(d.all.ws_bytes) >= host_seq_offset(d.all.grid, dtype_size(acc)) + 4);
        break;
    default:
        CHECK(false);
    }
}

static void fuzz_scan(std::mt19937_64 &rng)
{
    const int nd = int(1 + rng() % 4);
    int64_t shape[4], strides[4];
    int64_t cm = 1;
    for (int i = 0; i < nd; ++i) {
        shape[i] = pick_extent(rng);
        strides[i] = cm;
        cm = next_stride(cm, shape[i]);
    }
    if (rng() % 3 == 0)
        std::shuffle(strides, strides + nd, rng);
    const int dim = int(rng() % nd);
    const int in = int(rng() % 6), acc = int(rng() % 6), out = int(rng() % 6);
    const int cus = int(rng() % 3) == 0 ? 0 : int(1 + rng() % 320);
    ScanPlan d;
    ++g_cases;
    if (plan_scan(in, acc, out, uintptr_t(rng() % 64) * 2, uintptr_t(rng() % 64) * 2, nd, shape, strides, dim, cus,
                  &d) != ST_OK)
        return;
    ++g_accepted;
    int64_t total = 1;
    for (int i = 0; i < nd; ++i)
        total *= shape[i];
    CHECK(d.ws_bytes % 256 == 0);
    if (total == 0)
        return;
    CHECK(d.lines * d.m == total);
    CHECK(d.tiles <= INT32_MAX && d.grid >= 1);
    if (d.kernel == SK_TILE)
        CHECK(d.tiles == d.lines * d.tiles_per_line && d.tiles_per_line * d.tile_elems >= d.m);
}

int main(int argc, char **argv)
{
    const int64_t iters = argc > 1 ? std::atoll(argv[1]) : 200000;
    std::mt19937_64 rng(argc > 2 ? std::strtoull(argv[2], nullptr, 10) : 12345);
    for (int64_t i = 0; i < iters; ++i) {
        fuzz_all(rng);
        fuzz_dims(rng);
        fuzz_scan(rng);
    }
    std::printf("ok %lld cases, %lld accepted\n", (long long)g_cases, (long long)g_accepted);
    return 0;
}
