// Measurement kernels: a streaming read (practical HBM read ceiling) and a
// plain copy of known size (calibrates hardware byte counters).
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr unsigned kMaxGrid = 65536;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ src,
                                                               uint64_t n16, u32x4* sink) {
    u32x4 x = {0u, 0u, 0u, 0u};
    const uint64_t stride = (uint64_t)gridDim.x * kThreads;
    uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    // eight independent nontemporal loads in flight per iteration
    for (; i + 7 * stride < n16; i += 8 * stride) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(&src[i + u * stride]);
#pragma unroll
        for (int u = 0; u < 8; ++u) x ^= v[u];
    }
    for (; i < n16; i += stride) x ^= __builtin_nontemporal_load(&src[i]);
    // reduce so the loads cannot be dropped; one write per workgroup
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
        x[0] ^= __shfl_xor(x[0], s);
        x[1] ^= __shfl_xor(x[1], s);
        x[2] ^= __shfl_xor(x[2], s);
        x[3] ^= __shfl_xor(x[3], s);
    }
    if (threadIdx.x == 0) sink[blockIdx.x] = x;
}

__global__ __launch_bounds__(kThreads) void copy_kernel(u32x4* __restrict__ dst,
                                                        const u32x4* __restrict__ src,
                                                        uint64_t n16) {
    const uint64_t stride = (uint64_t)gridDim.x * kThreads;
    for (uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride)
        dst[i] = src[i];
}

unsigned grid_for(uint64_t n16) {
    uint64_t g = (n16 + kThreads - 1) / kThreads;
    if (g > kMaxGrid) g = kMaxGrid;
    if (g == 0) g = 1;
    return (unsigned)g;
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, void* sink, hipStream_t s) {
    const uint64_t n16 = bytes / 16;
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid_for(n16)), dim3(kThreads), 0, s,
                       static_cast<const u32x4*>(src), n16, static_cast<u32x4*>(sink));
    return hipGetLastError();
}

hipError_t launch_copy(void* dst, const void* src, size_t bytes, hipStream_t s) {
    const uint64_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    hipLaunchKernelGGL(copy_kernel, dim3(grid_for(n16)), dim3(kThreads), 0, s,
                       static_cast<u32x4*>(dst), static_cast<const u32x4*>(src), n16);
    return hipGetLastError();
}

}  // namespace pa
