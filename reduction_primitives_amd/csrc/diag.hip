// diag.hip -- a streaming-read kernel that measures the device's read
// bandwidth ceiling.  It loads every 16-byte vector of a buffer exactly once
// (non-temporal loads, eight in flight per thread, grid-stride over tiles),
// combines the words with XOR -- one integer operation per word, the least
// work any kernel can do with the bytes -- and stores nothing unless the
// combination equals a fixed magic word.  A whole-array reduction moves the
// same bytes, so its time against this kernel's is the part of the
// achievable read bandwidth it reaches.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

namespace rk {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kReadBlock = 256;
constexpr int kReadUnroll = 8;
constexpr uint32_t kReadMagic = 0x9e3779b9u;

__global__ __launch_bounds__(kReadBlock) void k_stream_read(const u32x4_t *x, int64_t nvec, uint32_t *sink)
{
    constexpr int64_t T = int64_t(kReadBlock) * kReadUnroll;
    const int64_t tiles = nvec / T;
    u32x4_t a = {0u, 0u, 0u, 0u};
    for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
        const u32x4_t *p = x + t * T + threadIdx.x;
        u32x4_t w[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u)
            w[u] = __builtin_nontemporal_load(p + u * kReadBlock);
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u)
            a ^= w[u];
    }
    // fewer than one tile of vectors remain: one per thread of the grid
    const int64_t stride = int64_t(gridDim.x) * kReadBlock;
    for (int64_t i = tiles * T + int64_t(blockIdx.x) * kReadBlock + threadIdx.x; i < nvec; i += stride)
        a ^= __builtin_nontemporal_load(x + i);
    const uint32_t v = a.x ^ a.y ^ a.z ^ a.w;
    if (v == kReadMagic)
        sink[0] = v;
}

}  // namespace

// nvec 16-byte vectors at x (16-byte aligned); grid blocks of 256 threads.
// With an event pair the events ride on the kernel's own dispatch packet, as
// the reductions' first launches do under the same timing hook.
int launch_stream_read(const void *x, int64_t nvec, int grid, void *sink, hipStream_t st, void *ev_begin,
                       void *ev_end)
{
    if (nvec <= 0)
        return 0;
    const u32x4_t *p = static_cast<const u32x4_t *>(x);
    uint32_t *s = static_cast<uint32_t *>(sink);
    if (ev_begin && ev_end)
        hipExtLaunchKernelGGL(k_stream_read, dim3(grid), dim3(kReadBlock), 0, st, static_cast<hipEvent_t>(ev_begin),
                              static_cast<hipEvent_t>(ev_end), 0, p, nvec, s);
    else
        k_stream_read<<<grid, kReadBlock, 0, st>>>(p, nvec, s);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace rk
