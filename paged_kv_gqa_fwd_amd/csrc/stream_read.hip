// Streaming-read probe (gfx950): reads a device buffer once with 16-byte
// non-temporal loads and nothing else, the on-box ceiling of a pure HBM read
// stream that the HBM-bound attention kernels are compared against.  Each
// thread keeps four loads in flight per step of a grid-stride loop (with 512
// workgroups the fastest depth measured on MI355X) and writes the XOR of
// what it read, so no load can be dropped.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "attn_device.h"
#include "paged_attn.h"

namespace pa {

constexpr int kReadUnroll = 4;

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

extern "C" int attn_stream_read(const void *buf, size_t bytes, uint32_t *sink, int32_t grid, void *stream) {
    if (!buf || !sink) return ATTN_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0 || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0 ||
        (bytes & 15u) != 0)
        return ATTN_ERR_ALIGN;
    if (grid < 1 || grid > 65535) return ATTN_ERR_SHAPE;
    if (bytes == 0) return ATTN_OK;
    hipLaunchKernelGGL(pa::stream_read_kernel, dim3(grid), dim3(pa::kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const pa::u32x4 *>(buf), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}
