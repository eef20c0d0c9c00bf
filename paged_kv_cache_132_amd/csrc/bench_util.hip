// Streaming read and copy kernels used only for measurement: the achievable
// HBM read bandwidth on this device, and a copy of known size to calibrate
// hardware byte counters.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "pa_bench.h"

namespace {

constexpr int kThreads = 256;
constexpr int kGrid = 256 * 8;          // 8 workgroups per CU on a 256-CU part

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kUnroll = 8;

// Each workgroup streams one contiguous slice with nontemporal 16-byte loads,
// kUnroll loads per thread in flight (the fastest plain read found on this
// part).  Bytes past the last full slice are read by workgroup 0.
__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                        uint32_t* __restrict__ sink) {
    const size_t per = n16 / gridDim.x;
    const u32x4* p = src + blockIdx.x * per;
    uint32_t acc = 0;
    size_t i = threadIdx.x;
    for (; i + (kUnroll - 1) * kThreads < per; i += kUnroll * kThreads) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * kThreads);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < per; i += kThreads) {
        const u32x4 v = __builtin_nontemporal_load(p + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (blockIdx.x == 0) {
        for (size_t k = per * gridDim.x + threadIdx.x; k < n16; k += kThreads) {
            const u32x4 v = src[k];
            acc ^= v.x ^ v.y ^ v.z ^ v.w;
        }
    }
    __shared__ uint32_t red[kThreads];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int w = kThreads / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] ^= red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(kThreads) void copy_kernel(uint4* __restrict__ dst, const uint4* __restrict__ src,
                                                        size_t n16) {
    const size_t stride = (size_t)gridDim.x * kThreads;
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

}  // namespace

extern "C" {

int pa_bench_read_grid(void) { return kGrid; }

int pa_bench_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
    if (!src || !sink || (bytes & 15)) return -1;
    hipLaunchKernelGGL(read_kernel, dim3(kGrid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(src), bytes / 16, sink);
    return (int)hipGetLastError();
}

int pa_bench_copy(void* dst, const void* src, size_t bytes, void* stream) {
    if (!src || !dst || (bytes & 15)) return -1;
    hipLaunchKernelGGL(copy_kernel, dim3(kGrid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<uint4*>(dst), static_cast<const uint4*>(src), bytes / 16);
    return (int)hipGetLastError();
}

}  // extern "C"
