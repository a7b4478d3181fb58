// Measurement kernels: a streaming read (practical HBM read ceiling) and a
// plain copy of known size (calibrates hardware byte counters).
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr unsigned kMaxGrid = 65536;

// Streaming read: one workgroup per compute unit, each streaming a
// contiguous region; every wavefront keeps kReadLoads 1 KB slices (64 lanes
// x 16 B, nontemporal) in flight per step.  Measured on the MI355X over 4 GiB:
// 7.3 TB/s, against 7.0 for a grid-stride form with 65536 short-lived
// workgroups and less for fewer slices in flight.  sink[blockIdx.x] gets the
// XOR of every 16-byte word the workgroup read, so the XOR over the sink is
// that of the whole buffer.
constexpr int kReadLoads = 8;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ src,
                                                               uint64_t n16, u32x4* sink) {
    __shared__ u32x4 part[kThreads / 64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    constexpr uint64_t kStep = (uint64_t)kThreads * kReadLoads;   // 16-B words per step
    const uint64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const uint64_t span = (per + kStep - 1) / kStep * kStep;
    const uint64_t beg = min(n16, (uint64_t)blockIdx.x * span);
    const uint64_t end = min(n16, beg + span);
    u32x4 x = {0u, 0u, 0u, 0u};
    uint64_t off = beg;
    for (; off + kStep <= end; off += kStep) {
        const u32x4* p = src + off + (uint64_t)wave * 64 * kReadLoads + lane;
        u32x4 v[kReadLoads];
#pragma unroll
        for (int u = 0; u < kReadLoads; ++u) v[u] = __builtin_nontemporal_load(p + u * 64);
#pragma unroll
        for (int u = 0; u < kReadLoads; ++u) x ^= v[u];
    }
    for (uint64_t i = off + threadIdx.x; i < end; i += kThreads) x ^= __builtin_nontemporal_load(&src[i]);
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
        x[0] ^= __shfl_xor(x[0], s);
        x[1] ^= __shfl_xor(x[1], s);
        x[2] ^= __shfl_xor(x[2], s);
        x[3] ^= __shfl_xor(x[3], s);
    }
    if (lane == 0) part[wave] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        u32x4 t = part[0];
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) t ^= part[w];
        sink[blockIdx.x] = t;
    }
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
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const unsigned grid = cus < 1 ? 1u : cus > (int)kMaxGrid ? kMaxGrid : (unsigned)cus;
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kThreads), 0, s,
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
