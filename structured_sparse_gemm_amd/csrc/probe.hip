// probe.hip -- a plain streaming read of device memory, the measured ceiling
// the bandwidth-bound products are compared against.  It reads every byte of
// a buffer once, in contiguous 16-byte pieces per lane (1 KiB per wave per
// load), with several loads in flight per lane, and does nothing with the
// data but fold it into one word per workgroup (stored only if the fold hits
// a value chosen so that it practically never does, which keeps the loads
// alive).  Same grid shape rules as the products: many more workgroups than
// CUs, and non-temporal loads, as the decode products use for their weights.
#include <algorithm>

#include "ssg_device.hpp"
#include "ssg_kernels.hpp"

namespace ssg {

namespace {

constexpr int kProbeThreads = 512;
constexpr int kProbeUnroll = 4;

__global__ void __launch_bounds__(kProbeThreads) k_stream_read(const i32x4* __restrict__ src, int64_t n16,
                                                              uint32_t* sink) {
    const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
    int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
    uint32_t x = 0;
    for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
        i32x4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) x ^= (uint32_t)(v[u].x ^ v[u].y ^ v[u].z ^ v[u].w);
    }
    for (; i < n16; i += stride) {
        const i32x4 v = __builtin_nontemporal_load(src + i);
        x ^= (uint32_t)(v.x ^ v.y ^ v.z ^ v.w);
    }
    if (x == 0x9E3779B9u) sink[blockIdx.x] = x;
}

}  // namespace

int64_t stream_read_grid(int64_t bytes) {
    const int64_t n16 = bytes / 16;
    return std::max<int64_t>(1, std::min<int64_t>((n16 + kProbeThreads * kProbeUnroll - 1) /
                                                      (kProbeThreads * kProbeUnroll), 8192));
}

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t s) {
    const int64_t grid = stream_read_grid(bytes);
    hipLaunchKernelGGL(k_stream_read, dim3((unsigned)grid), dim3(kProbeThreads), 0, s,
                       reinterpret_cast<const i32x4*>(src), bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace ssg
