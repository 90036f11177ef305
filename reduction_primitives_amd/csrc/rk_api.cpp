// rk_api.cpp -- the C ABI declared in include/rk.h.
//
// Validates every argument before launching anything, plans the call
// (rk_plan.cpp), hands the plan to the kernel translation unit of the input
// dtype, and, in host mode, finishes the bare partial on the host
// (AcceleratedKernels.jl PR #139, "What changes": when a host value is wanted
// the last pass stores the bare partial, which is copied back and finished
// with init on the host).
#include "rk.h"

#include <hip/hip_runtime.h>

#include <sys/syscall.h>
#include <unistd.h>

#include <atomic>
#include <chrono>
#include <cmath>
#include <mutex>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>

#include "rk_launch.hpp"
#include "rk_plan.hpp"
#include "rk_scan_plan.hpp"

namespace rk {
int launch_stream_read(const void *x, int64_t nvec, int grid, void *sink, hipStream_t st, void *ev_begin,
                       void *ev_end);  // diag.hip
}

namespace {

using namespace rk;

thread_local void *t_ev_begin = nullptr;
thread_local void *t_ev_end = nullptr;

constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

// Compute units of the current device (0 when there is no usable device).
int device_cus()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return 0;
    if (dev < kMaxDevices) {
        const int c = g_cus[dev].load(std::memory_order_relaxed);
        if (c > 0)
            return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    if (dev < kMaxDevices)
        g_cus[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

// ---- arrival-counter slots: one per (device, stream), so calls that may
// run concurrently never share a counter.  Calls on one stream are ordered,
// so they share their slot safely.  hipStreamPerThread names a different
// stream on each host thread and never gets a slot.
std::atomic<bool> g_fused_finish{true};
std::mutex g_slot_mu;
struct SlotKey { int dev; void *stream; bool used; };
SlotKey g_slots[kArriveSlots];

int arrive_slot(hipStream_t st)
{
    if (!g_fused_finish.load(std::memory_order_relaxed) || st == hipStreamPerThread)
        return -1;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return -1;
    std::lock_guard<std::mutex> lock(g_slot_mu);
    for (int i = 0; i < kArriveSlots; ++i)
        if (g_slots[i].used && g_slots[i].dev == dev && g_slots[i].stream == (void *)st)
            return i;
    for (int i = 0; i < kArriveSlots; ++i) {
        if (!g_slots[i].used) {
            g_slots[i] = SlotKey{dev, (void *)st, true};
            return i;
        }
    }
    return -1;                                  // all slots taken: two launches
}

// The slot a stream already has, or -1 (never takes a new one).
int existing_slot(hipStream_t st)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return -1;
    std::lock_guard<std::mutex> lock(g_slot_mu);
    for (int i = 0; i < kArriveSlots; ++i)
        if (g_slots[i].used && g_slots[i].dev == dev && g_slots[i].stream == (void *)st)
            return i;
    return -1;
}

// Test hooks.  g_force_wait >= 0: every whole-array collection and scan
// look-back waits for what never comes and gives up after that many polls.
// g_fail_launches > 0: that many calls return RK_ERR_HIP where they would
// launch their first kernel, launching nothing.
std::atomic<int64_t> g_force_wait{-1};
std::atomic<int> g_fail_launches{0};

bool injected_launch_failure()
{
    int n = g_fail_launches.load(std::memory_order_relaxed);
    while (n > 0 && !g_fail_launches.compare_exchange_weak(n, n - 1, std::memory_order_relaxed)) {
    }
    return n > 0;
}

bool debug_enabled()
{
    static const bool on = std::getenv("RK_DEBUG") != nullptr;
    return on;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool op_ok(int op) { return op >= 0 && op <= 2; }
bool map_ok(int map) { return map >= 0 && map <= 2; }
bool mode_ok(int mode) { return mode >= RK_MODE_OVERWRITE && mode <= RK_MODE_HOST; }

int check_types(int op, int map, int in, int acc, int out, int mode)
{
    if (!op_ok(op) || !map_ok(map) || !mode_ok(mode))
        return RK_ERR_INVALID_ARGUMENT;
    if (!dtype_known(in) || !dtype_known(acc) || !dtype_known(out))
        return RK_ERR_INVALID_ARGUMENT;
    if (!dtype_combo_ok(in, acc, out))
        return RK_ERR_UNSUPPORTED;
    return RK_OK;
}

// ------------------------------------------------------ host-side values

template <class T> uint64_t to_bits(T v)
{
    uint64_t b = 0;
    std::memcpy(&b, &v, sizeof v);
    return b;
}

uint64_t identity_bits(int op, int acc)
{
    switch (acc) {
    case F32:
        return to_bits(op == RK_OP_SUM ? 0.0f : op == RK_OP_MAX ? -INFINITY : INFINITY);
    case F64:
        return to_bits(op == RK_OP_SUM ? 0.0 : op == RK_OP_MAX ? -(double)INFINITY : (double)INFINITY);
    case I32:
        return to_bits(op == RK_OP_SUM ? int32_t(0)
                                       : op == RK_OP_MAX ? std::numeric_limits<int32_t>::min()
                                                         : std::numeric_limits<int32_t>::max());
    case I64:
        return to_bits(op == RK_OP_SUM ? int64_t(0)
                                       : op == RK_OP_MAX ? std::numeric_limits<int64_t>::min()
                                                         : std::numeric_limits<int64_t>::max());
    }
    return 0;
}

uint64_t start_bits(int op, int acc, const void *init)
{
    if (!init)
        return identity_bits(op, acc);
    uint64_t b = 0;
    std::memcpy(&b, init, dtype_size(acc));
    return b;
}

template <class T> T host_apply(int op, T a, T b)
{
    if constexpr (std::is_integral_v<T>) {
        using U = std::make_unsigned_t<T>;
        if (op == RK_OP_SUM) return (T)((U)a + (U)b);
        if (op == RK_OP_MAX) return a > b ? a : b;
        return a < b ? a : b;
    } else {
        if (op == RK_OP_SUM) return a + b;
        if (a != a || b != b) return a + b;
        if (op == RK_OP_MAX) return a > b ? a : b;
        return a < b ? a : b;
    }
}

uint16_t host_f32_to_bf16(float f)
{
    uint32_t u;
    std::memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// double -> float rounded to odd (see the device version in rk_device.hpp)
float host_f64_to_f32_odd(double d)
{
    float f = (float)d;
    if (d != d)
        return f;
    if (std::isinf(f) && !std::isinf(d))
        return d > 0 ? std::numeric_limits<float>::max() : -std::numeric_limits<float>::max();
    const double back = (double)f;
    if (back != d) {
        uint32_t b;
        std::memcpy(&b, &f, 4);
        if (std::fabs(back) > std::fabs(d))
            b -= 1;
        b |= 1u;
        std::memcpy(&f, &b, 4);
    }
    return f;
}

template <class Acc> void host_store(void *out, int out_dtype, Acc v)
{
    if constexpr (std::is_floating_point_v<Acc>) {
        float f32v = std::is_same_v<Acc, double> ? host_f64_to_f32_odd((double)v) : (float)v;
        switch (out_dtype) {
        case F32: { float r = (float)v; std::memcpy(out, &r, 4); break; }
        case F64: { double r = (double)v; std::memcpy(out, &r, 8); break; }
        case BF16: { uint16_t r = host_f32_to_bf16(f32v); std::memcpy(out, &r, 2); break; }
        case F16: { _Float16 h = (_Float16)f32v; std::memcpy(out, &h, 2); break; }
        }
    } else {
        if (out_dtype == I32) {
            int32_t r = (int32_t)(uint32_t)(uint64_t)v;
            std::memcpy(out, &r, 4);
        } else {
            int64_t r = (int64_t)v;
            std::memcpy(out, &r, 8);
        }
    }
}

template <class Acc> void host_finish_typed(int op, uint64_t init_bits, const void *partial, int have_partial,
                                            void *out, int out_dtype)
{
    Acc s, v;
    std::memcpy(&s, &init_bits, sizeof(Acc));
    Acc r = s;
    if (have_partial) {
        std::memcpy(&v, partial, sizeof(Acc));
        r = host_apply<Acc>(op, s, v);
    }
    host_store<Acc>(out, out_dtype, r);
}

void host_finish(int op, int acc, uint64_t init_bits, const void *partial, int have_partial, void *out,
                 int out_dtype)
{
    switch (acc) {
    case F32: host_finish_typed<float>(op, init_bits, partial, have_partial, out, out_dtype); break;
    case F64: host_finish_typed<double>(op, init_bits, partial, have_partial, out, out_dtype); break;
    case I32: host_finish_typed<int32_t>(op, init_bits, partial, have_partial, out, out_dtype); break;
    case I64: host_finish_typed<int64_t>(op, init_bits, partial, have_partial, out, out_dtype); break;
    }
}

int dispatch_scan(int in_dtype, const ScanLaunch &L)
{
    switch (in_dtype) {
    case F32: return launch_scan_in_f32(L);
    case BF16: return launch_scan_in_bf16(L);
    case F16: return launch_scan_in_f16(L);
    case F64: return launch_scan_in_f64(L);
    case I32: return launch_scan_in_i32(L);
    case I64: return launch_scan_in_i64(L);
    }
    return RK_ERR_INVALID_ARGUMENT;
}

int dispatch(int in_dtype, const Launch &L)
{
    switch (in_dtype) {
    case F32: return launch_in_f32(L);
    case BF16: return launch_in_bf16(L);
    case F16: return launch_in_f16(L);
    case F64: return launch_in_f64(L);
    case I32: return launch_in_i32(L);
    case I64: return launch_in_i64(L);
    }
    return RK_ERR_INVALID_ARGUMENT;
}

const char *kernel_name(int k)
{
    static const char *names[] = {"none", "all", "all_strided", "thread", "tiled", "columns", "row", "generic",
                                  "all2"};
    return (k >= 0 && k <= 8) ? names[k] : "?";
}

// Host mode: a small pinned host buffer per host thread, which the last
// pass writes the bare result into, so no copy has to be launched.  A
// host-mode call returns only after its result arrived, so one buffer per
// thread is never shared by two calls in flight.  Allocated on the thread's
// first host-mode call and freed when the thread ends (the main thread's at
// the process's end, by the system: the HIP runtime may already be shutting
// down when the main thread's thread-local objects go); NULL (copy back from
// the workspace) if pinned memory is unavailable.
struct PinnedResult {
    void *buf = nullptr;
    bool tried = false;
    ~PinnedResult()
    {
        if (buf && long(syscall(SYS_gettid)) != long(getpid()))
            (void)hipHostFree(buf);
    }
};

void *pinned_result()
{
    thread_local PinnedResult r;
    if (!r.tried) {
        r.tried = true;
        // RK_HOST_COPY set: always copy back from the workspace (tests use it)
        if (std::getenv("RK_HOST_COPY") != nullptr ||
            hipHostMalloc(&r.buf, 64, hipHostMallocPortable) != hipSuccess)
            r.buf = nullptr;
        else
            std::memset(r.buf, 0, 64);          // sequence numbers start at 1
    }
    return r.buf;
}

// Wait for the bare partial, then finish it on the host.  With the pinned
// buffer the kernel stores the result and then this call's sequence number;
// spinning on that number returns as soon as the result has landed, without
// the wake-up latency of a blocking stream wait.  Every kQueryMicros the spin
// asks the stream for errors (a query takes microseconds, so it is kept out of
// the path that sees the result), and after kSpinMicros it gives way to a
// blocking wait.  Without the buffer the partial is copied back from ws[grid]
// with the sequence word after it.  A drained stream without this call's
// sequence number means the kernel stored no result (its collection gave
// up): RK_ERR_HIP, and *out is left as it was.
constexpr int64_t kSpinMicros = 200;
constexpr int64_t kQueryMicros = 20;

int finish_on_host(int op, int acc, uint64_t init_bits, const Finish &fin, const void *ws, int grid, void *out,
                   int out_dtype, hipStream_t st)
{
    const int asz = dtype_size(acc);
    unsigned char partial[8];
    if (fin.out) {
        const volatile uint32_t *seq = reinterpret_cast<const volatile uint32_t *>(
            static_cast<const char *>(fin.out) + 8);
        const auto t0 = std::chrono::steady_clock::now();
        auto next_query = t0 + std::chrono::microseconds(kQueryMicros);
        bool arrived = false;
        for (uint32_t i = 1;; ++i) {
            if (*seq == fin.host_seq) {
                arrived = true;
                break;
            }
            if ((i & 63) == 0) {
                const auto now = std::chrono::steady_clock::now();
                if (now >= next_query) {
                    const hipError_t q = hipStreamQuery(st);
                    if (q != hipSuccess && q != hipErrorNotReady)
                        return RK_ERR_HIP;
                    if (q == hipSuccess)
                        break;                     // drained: the result is checked below
                    next_query = now + std::chrono::microseconds(kQueryMicros);
                }
                if (now - t0 > std::chrono::microseconds(kSpinMicros))
                    break;
            }
        }
        if (!arrived) {
            if (hipStreamSynchronize(st) != hipSuccess)
                return RK_ERR_HIP;
            if (*seq != fin.host_seq)
                return RK_ERR_HIP;                 // the kernel finished without a result
        }
        std::atomic_thread_fence(std::memory_order_acquire);
        std::memcpy(partial, fin.out, asz);
    } else {
        // result and sequence word: bytes [grid * asz, host_seq_offset + 4)
        const size_t first = size_t(grid) * asz;
        const size_t bytes = size_t(host_seq_offset(grid, asz)) + 4 - first;
        unsigned char back[16];
        const unsigned char *src = static_cast<const unsigned char *>(ws) + first;
        if (hipMemcpyAsync(back, src, bytes, hipMemcpyDeviceToHost, st) != hipSuccess)
            return RK_ERR_HIP;
        if (hipStreamSynchronize(st) != hipSuccess)
            return RK_ERR_HIP;
        uint32_t seq = 0;
        std::memcpy(&seq, back + bytes - 4, 4);
        if (seq != fin.host_seq)
            return RK_ERR_HIP;                     // the kernel finished without a result
        std::memcpy(partial, back, asz);
    }
    host_finish(op, acc, init_bits, partial, 1, out, out_dtype);
    return RK_OK;
}

Finish make_finish(int op, int acc, int out_dtype, int mode, const void *init, void *out, bool pinned_ok = true)
{
    Finish f;
    f.out = mode == RK_MODE_HOST ? (pinned_ok ? pinned_result() : nullptr) : out;
    f.host_seq = 0;
    if (mode == RK_MODE_HOST) {
        // a fresh sequence number per host-mode call of this thread
        thread_local uint32_t seq = 0;
        seq = seq + 1 == 0 ? 1 : seq + 1;
        f.host_seq = seq;
    }
    f.out_dtype = out_dtype;
    f.mode = mode;
    f.init_bits = start_bits(op, acc, init);
    return f;
}

int run_whole(int op, int map, int in, int acc, int out_dtype, const void *ptr, const AllPlan &a,
              int kernel, const Layout *red, const void *init, int mode, void *out, void *ws,
              hipStream_t st, const void *ptr2 = nullptr, bool pinned_ok = true)
{
    Launch L;
    std::memset(&L, 0, sizeof L);
    L.kernel = kernel;
    L.acc = acc;
    L.op = op;
    L.map = map;
    L.vec = a.vec;
    L.lanes = 1;
    L.grid = a.grid;
    L.block = a.block;
    L.all.x = ptr;
    L.all.y = ptr2;
    L.all.n = a.n;
    L.all.head = a.head;
    L.all.nvec = a.nvec;
    L.all.tail = a.tail;
    if (red) {
        L.all.nd = red->nd;
        for (int i = 0; i < red->nd; ++i) {
            L.all.ext[i] = red->ext[i];
            L.all.str[i] = red->str[i];
        }
    }
    L.all.ws = ws;
    L.all.grid = a.grid;
    L.all.arrive_slot = a.grid > 1 && arrive_counters(a.grid) <= kArriveCapacity ? arrive_slot(st) : -1;
    const int64_t force = g_force_wait.load(std::memory_order_relaxed);
    L.all.spin_limit = force >= 0 ? uint32_t(force) : kFinalSpinLimit;
    L.all.tag_xor = force >= 0 ? 0x80000000u : 0u;
    L.all.fin = make_finish(op, acc, out_dtype, mode, init, out, pinned_ok);
    L.stream = st;
    L.ev_begin = t_ev_begin;
    L.ev_end = t_ev_end;
    if (injected_launch_failure())
        return RK_ERR_HIP;
    int rc = dispatch(in, L);
    if (rc != RK_OK)
        return rc;
    if (mode == RK_MODE_HOST)
        return finish_on_host(op, acc, L.all.fin.init_bits, L.all.fin, ws, a.grid, out, out_dtype, st);
    return RK_OK;
}

// ---- the library's scratch, for rk_reduce_dims_no_workspace: device memory
// that stands in for the caller's workspace, for callers that cannot
// allocate.  Every GPU the library runs on holds its own copy, at its own
// address, until the process ends.  The array's name is a host-side stand-in
// here, never a device address: host code only uses the address that
// hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = size_t(2) << 20;
namespace scratch_unit {
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
}
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The scratch's device address on the current device (looked up on the
// first call on each device).
int scratch_address(void **p)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return RK_ERR_HIP;
    if (dev >= kMaxDevices)
        return RK_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch_unit::scratch)) != hipSuccess || !ptr)
            return RK_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *p = g_scratch_ptr[dev];
    return RK_OK;
}

// rk_reduce_dims with the workspace given (scratch: the library's own, of
// kScratchBytes; host mode then copies its result back from it instead of
// using the pinned buffer, whose first use allocates).
int reduce_dims(int op, int map, int in_dtype, int acc_dtype, int out_dtype, const void *ptr, int ndim,
                const int64_t *shape, const int64_t *strides, uint32_t reduce_mask, const void *init, int mode,
                void *out, void *workspace, void *stream, bool scratch);

}  // namespace

extern "C" {

const char *rk_status_string(int status)
{
    switch (status) {
    case RK_OK: return "ok";
    case RK_ERR_INVALID_ARGUMENT: return "invalid argument";
    case RK_ERR_UNSUPPORTED: return "unsupported dtype combination";
    case RK_ERR_HIP: return "HIP runtime error";
    case RK_ERR_TOO_LARGE: return "the call needs more workspace than the library's scratch holds (2 MiB)";
    }
    return "unknown status";
}

int rk_debug_set_fused_finish(int enable)
{
    return g_fused_finish.exchange(enable != 0) ? 1 : 0;
}

int rk_debug_set_finish_tag(void *stream, uint32_t e)
{
    if (e > 0xfffffffeu)
        return RK_ERR_INVALID_ARGUMENT;
    const int slot = arrive_slot(static_cast<hipStream_t>(stream));
    if (slot < 0)
        return RK_ERR_UNSUPPORTED;
    const int dtypes[] = {F32, BF16, F16, F64, I32, I64};
    for (int d : dtypes) {
        Launch L;
        std::memset(&L, 0, sizeof L);
        L.kernel = K_SET_TAG;
        L.all.arrive_slot = slot;
        L.all.n = e;
        L.stream = stream;
        const int rc = dispatch(d, L);
        if (rc != RK_OK)
            return rc;
    }
    return RK_OK;
}

int rk_stream_timeouts(void *stream, uint64_t *count)
{
    if (!count)
        return RK_ERR_INVALID_ARGUMENT;
    *count = 0;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (hipStreamSynchronize(st) != hipSuccess)
        return RK_ERR_HIP;
    const int slot = existing_slot(st);
    const int dtypes[] = {F32, BF16, F16, F64, I32, I64};
    for (int d : dtypes) {
        Launch L;
        std::memset(&L, 0, sizeof L);
        L.kernel = K_TAKE_TIMEOUTS;
        L.all.arrive_slot = slot;
        L.all.ws = count;
        L.all.n = 1;                            // repair the slot's tagged words after a give-up
        int rc = dispatch(d, L);
        if (rc != RK_OK)
            return rc;
        ScanLaunch S;
        std::memset(&S, 0, sizeof S);
        S.kernel = SK_TAKE_TIMEOUTS;
        S.args.slot = slot;
        S.args.ws = count;
        rc = dispatch_scan(d, S);
        if (rc != RK_OK)
            return rc;
    }
    return RK_OK;
}

int rk_debug_force_wait_timeout(int64_t polls)
{
    if (polls > int64_t(0xffffffffu))
        return RK_ERR_INVALID_ARGUMENT;
    g_force_wait.store(polls < 0 ? -1 : polls, std::memory_order_relaxed);
    return RK_OK;
}

int rk_debug_fail_launches(int count)
{
    if (count < 0)
        return RK_ERR_INVALID_ARGUMENT;
    g_fail_launches.store(count, std::memory_order_relaxed);
    return RK_OK;
}

int rk_debug_set_launch_events(void *begin, void *end)
{
    if ((begin == nullptr) != (end == nullptr))
        return RK_ERR_INVALID_ARGUMENT;
    t_ev_begin = begin;
    t_ev_end = end;
    return RK_OK;
}

int rk_debug_stream_read(const void *ptr, int64_t nbytes, int grid, void *sink, void *stream)
{
    if (nbytes < 0 || nbytes % 16 != 0 || grid < 0 || grid > (1 << 20))
        return RK_ERR_INVALID_ARGUMENT;
    if (nbytes == 0)
        return RK_OK;
    if (!ptr || !sink || reinterpret_cast<uintptr_t>(ptr) % 16 != 0 || reinterpret_cast<uintptr_t>(sink) % 4 != 0)
        return RK_ERR_INVALID_ARGUMENT;
    return launch_stream_read(ptr, nbytes / 16, grid > 0 ? grid : 2048, sink, static_cast<hipStream_t>(stream),
                              t_ev_begin, t_ev_end)
               ? RK_ERR_HIP : RK_OK;
}

int rk_debug_device_info(int64_t *num_cus, int64_t *mem_clock_khz, int64_t *mem_bus_bits)
{
    if (!num_cus || !mem_clock_khz || !mem_bus_bits)
        return RK_ERR_INVALID_ARGUMENT;
    int dev = 0, cus = 0, clk = 0, bus = 0;
    if (hipGetDevice(&dev) != hipSuccess
        || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess
        || hipDeviceGetAttribute(&clk, hipDeviceAttributeMemoryClockRate, dev) != hipSuccess
        || hipDeviceGetAttribute(&bus, hipDeviceAttributeMemoryBusWidth, dev) != hipSuccess)
        return RK_ERR_HIP;
    *num_cus = cus;
    *mem_clock_khz = clk;
    *mem_bus_bits = bus;
    return RK_OK;
}

int rk_plan_all(int in_dtype, int acc_dtype, const void *ptr, int64_t n, int num_cus, rk_plan_info *info)
{
    if (!info || !dtype_known(in_dtype) || !dtype_known(acc_dtype) || n < 0)
        return RK_ERR_INVALID_ARGUMENT;
    if (num_cus <= 0)
        num_cus = device_cus();
    AllPlan a;
    int rc = plan_all(in_dtype, acc_dtype, reinterpret_cast<uintptr_t>(ptr), n, num_cus, &a);
    if (rc)
        return rc;
    std::memset(info, 0, sizeof *info);
    info->kernel = RK_KERNEL_ALL;
    info->launches = (a.grid > 1 && arrive_counters(a.grid) <= kArriveCapacity && g_fused_finish.load()) ? 1 : a.launches;
    info->grid = a.grid;
    info->block = a.block;
    info->split = 1;
    info->vec = a.vec;
    info->tile_outputs = 1;
    info->n_out = 1;
    info->reduce_len = n;
    info->workspace_bytes = a.ws_bytes;
    return RK_OK;
}

int rk_plan_all2(int in_dtype, int acc_dtype, const void *a, const void *b, int64_t n, int num_cus,
                 rk_plan_info *info)
{
    if (!info || !dtype_known(in_dtype) || !dtype_known(acc_dtype) || n < 0)
        return RK_ERR_INVALID_ARGUMENT;
    if (num_cus <= 0)
        num_cus = device_cus();
    AllPlan p;
    int rc = plan_all2(in_dtype, acc_dtype, reinterpret_cast<uintptr_t>(a), reinterpret_cast<uintptr_t>(b), n,
                       num_cus, &p);
    if (rc)
        return rc;
    std::memset(info, 0, sizeof *info);
    info->kernel = RK_KERNEL_ALL2;
    info->launches = (p.grid > 1 && arrive_counters(p.grid) <= kArriveCapacity && g_fused_finish.load()) ? 1 : p.launches;
    info->grid = p.grid;
    info->block = p.block;
    info->split = 1;
    info->vec = p.vec;
    info->tile_outputs = 1;
    info->n_out = 1;
    info->reduce_len = n;
    info->workspace_bytes = p.ws_bytes;
    return RK_OK;
}

int rk_plan_dims(int in_dtype, int acc_dtype, const void *ptr, int ndim, const int64_t *shape,
                 const int64_t *strides, uint32_t reduce_mask, int num_cus, rk_plan_info *info)
{
    if (!info)
        return RK_ERR_INVALID_ARGUMENT;
    if (num_cus <= 0)
        num_cus = device_cus();
    DimsPlan d;
    int rc = plan_dims(in_dtype, acc_dtype, reinterpret_cast<uintptr_t>(ptr), ndim, shape, strides,
                       reduce_mask, num_cus, &d);
    if (rc)
        return rc;
    std::memset(info, 0, sizeof *info);
    info->kernel = d.kernel;
    info->launches = (d.fused_ok && g_fused_finish.load()) ? 1 : d.launches;
    info->grid = d.grid;
    info->block = d.block;
    info->split = d.split;
    info->vec = d.vec;
    info->tile_outputs = d.tile_outputs;
    info->n_out = d.n_out;
    info->reduce_len = d.m;
    info->workspace_bytes = d.ws_bytes;
    return RK_OK;
}

size_t rk_workspace_size(int in_dtype, int acc_dtype, int ndim, const int64_t *shape, const int64_t *strides,
                         uint32_t reduce_mask)
{
    const int cus = device_cus();
    DimsPlan d;
    if (plan_dims(in_dtype, acc_dtype, 0, ndim, shape, strides, reduce_mask, cus, &d) != ST_OK)
        return 0;
    return d.ws_bytes;
}

int rk_reduce_all(int op, int map, int in_dtype, int acc_dtype, int out_dtype, const void *ptr, int64_t n,
                  const void *init, int mode, void *out, void *workspace, void *stream)
{
    int rc = check_types(op, map, in_dtype, acc_dtype, out_dtype, mode);
    if (rc)
        return rc;
    if (n < 0 || (n > 0 && !ptr) || !out || !workspace)
        return RK_ERR_INVALID_ARGUMENT;
    if (!aligned(ptr, dtype_size(in_dtype)) || !aligned(out, dtype_size(out_dtype)) ||
        !aligned(workspace, 8))
        return RK_ERR_INVALID_ARGUMENT;
    if (mode != RK_MODE_HOST && out == ptr)
        return RK_ERR_INVALID_ARGUMENT;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (mode == RK_MODE_HOST && n == 0) {          // nothing to reduce: s itself
        host_finish(op, acc_dtype, start_bits(op, acc_dtype, init), nullptr, 0, out, out_dtype);
        return RK_OK;
    }
    AllPlan a;
    rc = plan_all(in_dtype, acc_dtype, reinterpret_cast<uintptr_t>(ptr), n, device_cus(), &a);
    if (rc)
        return rc;
    if (debug_enabled())
        std::fprintf(stderr, "rk_reduce_all: n=%lld grid=%d block=%d head=%lld nvec=%lld tail=%lld launches=%d\n",
                     (long long)n, a.grid, a.block, (long long)a.head, (long long)a.nvec, (long long)a.tail,
                     a.launches);
    return run_whole(op, map, in_dtype, acc_dtype, out_dtype, ptr, a, K_ALL, nullptr, init, mode, out, workspace,
                     st);
}

int rk_reduce_all2(int op, int map2, int in_dtype, int acc_dtype, int out_dtype, const void *a, const void *b,
                   int64_t n, const void *init, int mode, void *out, void *workspace, void *stream)
{
    int rc = check_types(op, map2, in_dtype, acc_dtype, out_dtype, mode);
    if (rc)
        return rc;
    if (n < 0 || (n > 0 && (!a || !b)) || !out || !workspace)
        return RK_ERR_INVALID_ARGUMENT;
    const size_t isz = dtype_size(in_dtype);
    if (!aligned(a, isz) || !aligned(b, isz) || !aligned(out, dtype_size(out_dtype)) || !aligned(workspace, 8))
        return RK_ERR_INVALID_ARGUMENT;
    if (mode != RK_MODE_HOST && (out == a || out == b))
        return RK_ERR_INVALID_ARGUMENT;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (mode == RK_MODE_HOST && n == 0) {
        host_finish(op, acc_dtype, start_bits(op, acc_dtype, init), nullptr, 0, out, out_dtype);
        return RK_OK;
    }
    AllPlan p;
    rc = plan_all2(in_dtype, acc_dtype, reinterpret_cast<uintptr_t>(a), reinterpret_cast<uintptr_t>(b), n,
                   device_cus(), &p);
    if (rc)
        return rc;
    if (debug_enabled())
        std::fprintf(stderr, "rk_reduce_all2: n=%lld grid=%d block=%d vec=%d head=%lld nvec=%lld tail=%lld\n",
                     (long long)n, p.grid, p.block, p.vec, (long long)p.head, (long long)p.nvec, (long long)p.tail);
    return run_whole(op, map2, in_dtype, acc_dtype, out_dtype, a, p, K_ALL2, nullptr, init, mode, out, workspace,
                     st, b);
}

int rk_reduce_dims(int op, int map, int in_dtype, int acc_dtype, int out_dtype, const void *ptr, int ndim,
                   const int64_t *shape, const int64_t *strides, uint32_t reduce_mask, const void *init, int mode,
                   void *out, void *workspace, void *stream)
{
    return reduce_dims(op, map, in_dtype, acc_dtype, out_dtype, ptr, ndim, shape, strides, reduce_mask, init, mode,
                       out, workspace, stream, false);
}

int rk_reduce_dims_no_workspace(int op, int map, int in_dtype, int acc_dtype, int out_dtype, const void *ptr,
                                int ndim, const int64_t *shape, const int64_t *strides, uint32_t reduce_mask,
                                const void *init, int mode, void *out, void *stream)
{
    return reduce_dims(op, map, in_dtype, acc_dtype, out_dtype, ptr, ndim, shape, strides, reduce_mask, init, mode,
                       out, nullptr, stream, true);
}

}  // extern "C"

namespace {

int reduce_dims(int op, int map, int in_dtype, int acc_dtype, int out_dtype, const void *ptr, int ndim,
                const int64_t *shape, const int64_t *strides, uint32_t reduce_mask, const void *init, int mode,
                void *out, void *workspace, void *stream, bool scratch)
{
    int rc = check_types(op, map, in_dtype, acc_dtype, out_dtype, mode);
    if (rc)
        return rc;
    if (!shape || !strides || ndim < 1 || ndim > kMaxDims || !out)
        return RK_ERR_INVALID_ARGUMENT;
    DimsPlan d;
    rc = plan_dims(in_dtype, acc_dtype, reinterpret_cast<uintptr_t>(ptr), ndim, shape, strides, reduce_mask,
                   device_cus(), &d);
    if (rc)
        return rc;
    const int64_t total = d.n_out * d.m;
    if ((total > 0 && !ptr) || (ptr && !aligned(ptr, dtype_size(in_dtype))))
        return RK_ERR_INVALID_ARGUMENT;
    if (!aligned(out, dtype_size(out_dtype)))
        return RK_ERR_INVALID_ARGUMENT;
    if (mode == RK_MODE_HOST && d.n_out != 1)
        return RK_ERR_INVALID_ARGUMENT;
    if (mode != RK_MODE_HOST && out == ptr)
        return RK_ERR_INVALID_ARGUMENT;
    if (scratch) {
        if (d.ws_bytes > kScratchBytes)
            return RK_ERR_TOO_LARGE;
    } else if (d.ws_bytes > 0 && (!workspace || !aligned(workspace, 8))) {
        return RK_ERR_INVALID_ARGUMENT;
    }
    if (d.grid > std::numeric_limits<int32_t>::max())
        return RK_ERR_UNSUPPORTED;
    if (debug_enabled())
        std::fprintf(stderr,
                     "rk_reduce_dims: kernel=%s n_out=%lld m=%lld grid=%lld block=%d split=%d vec=%d tile=%d "
                     "ws=%zu\n",
                     kernel_name(d.kernel), (long long)d.n_out, (long long)d.m, (long long)d.grid, d.block,
                     d.split, d.vec, d.tile_outputs, d.ws_bytes);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (d.kernel == K_NONE)
        return RK_OK;
    if (mode == RK_MODE_HOST && d.m == 0) {
        host_finish(op, acc_dtype, start_bits(op, acc_dtype, init), nullptr, 0, out, out_dtype);
        return RK_OK;
    }
    if (scratch) {
        rc = scratch_address(&workspace);
        if (rc)
            return rc;
    }
    if (d.kernel == K_ALL)
        return run_whole(op, map, in_dtype, acc_dtype, out_dtype, ptr, d.all, K_ALL, nullptr, init, mode, out,
                         workspace, st, nullptr, !scratch);
    if (d.kernel == K_ALL_STRIDED)
        return run_whole(op, map, in_dtype, acc_dtype, out_dtype, ptr, d.all, K_ALL_STRIDED, &d.red, init, mode,
                         out, workspace, st, nullptr, !scratch);
    if (mode == RK_MODE_HOST)
        return RK_ERR_INVALID_ARGUMENT;   // single outputs always take a whole-array path above

    Launch L;
    std::memset(&L, 0, sizeof L);
    L.kernel = d.kernel;
    L.acc = acc_dtype;
    L.op = op;
    L.map = map;
    L.vec = d.vec;
    L.lanes = d.lanes;
    L.grid = d.grid;
    L.block = d.block;
    DimsArgs &a = L.dims;
    a.x = ptr;
    a.ws = workspace;
    a.n_out = d.n_out;
    a.m = d.m;
    a.s_red = d.s_red;
    a.row_len = d.row_len;
    a.seg_nd = d.seg.nd;
    for (int i = 0; i < d.seg.nd && i < 3; ++i) {
        a.seg_ext[i] = d.seg.ext[i];
        a.seg_str[i] = d.seg.str[i];
    }
    a.segs = d.segs;
    a.segs_per_split = d.segs_per_split;
    a.splits_per_seg = d.splits_per_seg;
    a.run_len = d.run_len;
    a.tiles_per_run = d.tiles_per_run;
    a.tiles = d.tiles;
    a.rows_per_split = d.rows_per_split;
    a.split = d.split;
    a.outer_nd = d.outer.nd;
    for (int i = 0; i < d.outer.nd && i < 3; ++i) {
        a.outer_ext[i] = d.outer.ext[i];
        a.outer_str[i] = d.outer.str[i];
    }
    a.kept_nd = d.kept.nd;
    for (int i = 0; i < d.kept.nd; ++i) {
        a.kept_ext[i] = d.kept.ext[i];
        a.kept_str[i] = d.kept.str[i];
    }
    a.red_nd = d.red.nd;
    for (int i = 0; i < d.red.nd; ++i) {
        a.red_ext[i] = d.red.ext[i];
        a.red_str[i] = d.red.str[i];
    }
    a.fin = make_finish(op, acc_dtype, out_dtype, mode, init, out);
    a.omap.nd = d.out_map.nd;
    for (int i = 0; i < 4; ++i) {
        a.omap.ext[i] = i < d.out_map.nd ? d.out_map.ext[i] : 0;
        a.omap.str[i] = i < d.out_map.nd ? d.out_map.str[i] : 0;
    }
    a.arrive_slot = d.fused_ok ? arrive_slot(st) : -1;
    L.stream = st;
    L.ev_begin = t_ev_begin;
    L.ev_end = t_ev_end;
    if (injected_launch_failure())
        return RK_ERR_HIP;
    return dispatch(in_dtype, L);
}

}  // namespace

extern "C" {

size_t rk_scan_workspace_size(int in_dtype, int acc_dtype, int ndim, const int64_t *shape, const int64_t *strides,
                              int dim)
{
    ScanPlan d;
    if (plan_scan(in_dtype, acc_dtype, acc_dtype, 0, 0, ndim, shape, strides, dim, device_cus(), &d) != ST_OK)
        return 0;
    return d.ws_bytes;
}

int rk_plan_scan(int in_dtype, int acc_dtype, int out_dtype, const void *ptr, const void *out, int ndim,
                 const int64_t *shape, const int64_t *strides, int dim, int num_cus, rk_plan_info *info)
{
    if (!info)
        return RK_ERR_INVALID_ARGUMENT;
    if (num_cus <= 0)
        num_cus = device_cus();
    ScanPlan d;
    int rc = plan_scan(in_dtype, acc_dtype, out_dtype, reinterpret_cast<uintptr_t>(ptr),
                       reinterpret_cast<uintptr_t>(out), ndim, shape, strides, dim, num_cus, &d);
    if (rc)
        return rc;
    std::memset(info, 0, sizeof *info);
    info->kernel = d.kernel == SK_TILE ? RK_KERNEL_SCAN_TILE
                   : d.kernel == SK_ROWWAVE ? RK_KERNEL_SCAN_ROWWAVE
                   : d.kernel == SK_LINES ? RK_KERNEL_SCAN_LINES
                   : d.kernel == SK_COLUMNS ? RK_KERNEL_SCAN_COLUMNS
                   : d.kernel == SK_TRANSPOSE ? RK_KERNEL_SCAN_TRANSPOSE : RK_KERNEL_NONE;
    const bool lookback = d.kernel == SK_TILE || d.kernel == SK_COLUMNS || d.kernel == SK_TRANSPOSE;
    // a look-back scan clears its state with a launch of its own unless the
    // state fits a library slot
    const int64_t cap = d.kernel == SK_TILE ? kScanRecCapacity : kScanFlagCapacity;
    info->launches = d.kernel == SK_NONE ? 0
                     : lookback && !(d.tiles <= cap && g_fused_finish.load()) ? 2 : 1;
    info->grid = d.grid;
    info->block = d.block;
    info->split = int(d.kernel == SK_COLUMNS || d.kernel == SK_TRANSPOSE ? d.chunks
                      : d.tiles_per_line > 0                            ? d.tiles_per_line
                                                                        : 1);
    info->vec = d.vec;
    info->tile_outputs = int(d.tile_elems);
    info->n_out = d.lines * d.m;
    info->reduce_len = d.m;
    info->workspace_bytes = d.ws_bytes;
    return RK_OK;
}

int rk_scan_dims(int op, int in_dtype, int acc_dtype, int out_dtype, const void *ptr, int ndim,
                 const int64_t *shape, const int64_t *strides, int dim, const void *init, int inclusive, void *out,
                 void *workspace, void *stream)
{
    int rc = check_types(op, 0, in_dtype, acc_dtype, out_dtype, RK_MODE_OVERWRITE);
    if (rc)
        return rc;
    if (!shape || !strides || ndim < 1 || ndim > kMaxDims || dim < 0 || dim >= ndim || !out)
        return RK_ERR_INVALID_ARGUMENT;
    if (inclusive != 0 && inclusive != 1)
        return RK_ERR_INVALID_ARGUMENT;
    ScanPlan d;
    rc = plan_scan(in_dtype, acc_dtype, out_dtype, reinterpret_cast<uintptr_t>(ptr), reinterpret_cast<uintptr_t>(out),
                   ndim, shape, strides, dim, device_cus(), &d);
    if (rc)
        return rc;
    const int64_t total = d.lines * d.m;
    const size_t isz = dtype_size(in_dtype), osz = dtype_size(out_dtype);
    if ((total > 0 && !ptr) || (ptr && !aligned(ptr, isz)) || !aligned(out, osz))
        return RK_ERR_INVALID_ARGUMENT;
    if (d.ws_bytes > 0 && (!workspace || !aligned(workspace, 8)))
        return RK_ERR_INVALID_ARGUMENT;
    if (total > 0) {
        // the output may be the input itself (same layout and element size), but may not overlap it otherwise
        int64_t last = 0, cm = 1;
        bool same_layout = isz == osz;
        for (int i = 0; i < ndim; ++i) {
            last += (shape[i] - 1) * strides[i];
            same_layout = same_layout && (shape[i] == 1 || strides[i] == cm);
            cm *= shape[i];
        }
        const uintptr_t a0 = reinterpret_cast<uintptr_t>(ptr), a1 = a0 + size_t(last + 1) * isz;
        const uintptr_t b0 = reinterpret_cast<uintptr_t>(out), b1 = b0 + size_t(total) * osz;
        const bool overlap = a0 < b1 && b0 < a1;
        if (overlap && !(b0 == a0 && same_layout))
            return RK_ERR_INVALID_ARGUMENT;
    }
    if (d.grid > std::numeric_limits<int32_t>::max())
        return RK_ERR_UNSUPPORTED;
    if (debug_enabled())
        std::fprintf(stderr, "rk_scan_dims: kernel=%d lines=%lld m=%lld grid=%lld vec=%d tiles=%lld ws=%zu\n",
                     d.kernel, (long long)d.lines, (long long)d.m, (long long)d.grid, d.vec, (long long)d.tiles,
                     d.ws_bytes);
    if (d.kernel == SK_NONE)
        return RK_OK;
    ScanLaunch L;
    std::memset(&L, 0, sizeof L);
    L.kernel = d.kernel;
    L.acc = acc_dtype;
    L.op = op;
    L.vec = d.vec;
    L.tmode = d.tmode;
    L.tstr = d.tstr;
    L.grid = d.grid;
    L.block = d.block;
    ScanArgs &a = L.args;
    a.x = ptr;
    a.out = out;
    a.ws = workspace;
    a.m = d.m;
    a.lines = d.lines;
    a.kept_nd = d.kept_in.nd;
    for (int i = 0; i < d.kept_in.nd; ++i) {
        a.kept_ext[i] = d.kept_in.ext[i];
        a.kept_in[i] = d.kept_in.str[i];
        a.kept_out[i] = d.kept_out[i];
    }
    a.s_in = d.s_in;
    a.s_out = d.s_out;
    a.tiles_per_line = d.tiles_per_line;
    a.tiles = d.tiles;
    a.col_tiles_per_run = d.col_tiles_per_run;
    a.col_tiles = d.col_tiles;
    a.inclusive = inclusive;
    a.out_dtype = out_dtype;
    a.init_bits = start_bits(op, acc_dtype, init);
    // look-back state in a library slot when the tiles' state fits one (no clearing launch)
    a.slot = (d.kernel == SK_TILE && d.tiles <= kScanRecCapacity) ||
                     ((d.kernel == SK_COLUMNS || d.kernel == SK_TRANSPOSE) && d.tiles <= kScanFlagCapacity)
                 ? arrive_slot(static_cast<hipStream_t>(stream))
                 : -1;
    const int64_t force = g_force_wait.load(std::memory_order_relaxed);
    a.spin_limit = force >= 0 ? uint32_t(force) : uint32_t(tune::kScanSpinLimit);
    a.force_wait = force >= 0 ? 1u : 0u;
    L.stream = stream;
    L.ev_begin = t_ev_begin;
    L.ev_end = t_ev_end;
    if (injected_launch_failure())
        return RK_ERR_HIP;
    return dispatch_scan(in_dtype, L);
}

int rk_scan(int op, int in_dtype, int acc_dtype, int out_dtype, const void *ptr, int64_t n, const void *init,
            int inclusive, void *out, void *workspace, void *stream)
{
    if (n < 0)
        return RK_ERR_INVALID_ARGUMENT;
    const int64_t shape[1] = {n}, strides[1] = {1};
    return rk_scan_dims(op, in_dtype, acc_dtype, out_dtype, ptr, 1, shape, strides, 0, init, inclusive, out,
                        workspace, stream);
}

}  // extern "C"
