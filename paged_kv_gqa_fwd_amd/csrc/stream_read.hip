// Streaming-read probe (gfx950): reads a device buffer once with 16-byte
// non-temporal loads and nothing else, the on-box ceiling of a pure HBM read
// stream that the HBM-bound attention kernels are compared against.  Each
// thread keeps 4 or 8 loads in flight per step of a grid-stride loop and
// writes the XOR of what it read, so no load can be dropped.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "attn_device.h"
#include "paged_attn.h"

namespace pa {

template <int kReadUnroll>
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4 *__restrict__ p, size_t n16,
                                                               uint32_t *__restrict__ sink) {
    size_t i = (size_t)blockIdx.x * kThreads * kReadUnroll + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * kThreads * kReadUnroll;
    uint32_t acc = 0;
    for (; i < n16; i += stride) {
        u32x4 v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u)
            v[u] = (i + (size_t)u * kThreads < n16) ? __builtin_nontemporal_load(p + i + (size_t)u * kThreads)
                                                    : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

}  // namespace pa

extern "C" int attn_stream_read(const void *buf, size_t bytes, uint32_t *sink, int32_t grid, int32_t depth,
                                void *stream) {
    if (!buf || !sink) return ATTN_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0 || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0 ||
        (bytes & 15u) != 0)
        return ATTN_ERR_ALIGN;
    if (grid < 1 || grid > 65535 || (depth != 4 && depth != 8)) return ATTN_ERR_SHAPE;
    if (bytes == 0) return ATTN_OK;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const auto *p = static_cast<const pa::u32x4 *>(buf);
    if (depth == 4)
        hipLaunchKernelGGL(pa::stream_read_kernel<4>, dim3(grid), dim3(pa::kThreads), 0, st, p, bytes / 16, sink);
    else
        hipLaunchKernelGGL(pa::stream_read_kernel<8>, dim3(grid), dim3(pa::kThreads), 0, st, p, bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}
