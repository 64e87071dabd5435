// Streaming probes: kernels that only move bytes, the floor a launch of the
// scoring kernel is measured against on the same GPU, in the same units.
// Not part of the method; tq.h declares them under "measurement probes".
//
//  * read: every 16-byte word of a buffer is loaded once (one word per lane,
//    256-lane workgroups), folded into a value that is stored only if it
//    equals an improbable constant, so the loads cannot be dropped;
//  * write: every 16-byte word of a buffer is stored once (four words per
//    lane);
//  * read then write: workgroup k loads its slice of the source (two words per
//    lane) and then stores its slice of the destination with values that
//    depend on what it loaded, the dependency of a scoring launch (codes in,
//    scores out) without its arithmetic.
#include "tq_common.hpp"

namespace tq {
namespace {

constexpr int kProbeThreads = 256;
constexpr uint32_t kImprobable = 0x9E3779B9u;

__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const uint4* __restrict__ src, int64_t n16,
                                                                   uint32_t* __restrict__ sink) {
    const int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
    if (i >= n16) return;
    const uint4 v = src[i];
    const uint32_t x = v.x ^ v.y ^ v.z ^ v.w;
    if (x == kImprobable) sink[0] = x;
}

constexpr int kWritePer = 4;

__global__ __launch_bounds__(kProbeThreads) void probe_write_kernel(uint4* __restrict__ dst, int64_t n16,
                                                                    uint32_t value) {
    const int64_t i0 = (int64_t)blockIdx.x * kProbeThreads * kWritePer + threadIdx.x;
#pragma unroll
    for (int k = 0; k < kWritePer; ++k) {
        const int64_t i = i0 + (int64_t)k * kProbeThreads;
        if (i < n16) dst[i] = make_uint4(value, value + 1u, value + 2u, value + (uint32_t)k);
    }
}

constexpr int kReadPer = 2;

__global__ __launch_bounds__(kProbeThreads) void probe_read_write_kernel(const uint4* __restrict__ src, int64_t n_r16,
                                                                         uint4* __restrict__ dst, int64_t n_w16,
                                                                         int64_t w16_per_group) {
    const int64_t r0 = (int64_t)blockIdx.x * kProbeThreads * kReadPer + threadIdx.x;
    uint32_t acc = 0u;
    uint4 v[kReadPer];
#pragma unroll
    for (int k = 0; k < kReadPer; ++k) {
        const int64_t i = r0 + (int64_t)k * kProbeThreads;
        v[k] = i < n_r16 ? src[i] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int k = 0; k < kReadPer; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    const int64_t w0 = (int64_t)blockIdx.x * w16_per_group;
    for (int64_t k = threadIdx.x; k < w16_per_group; k += kProbeThreads) {
        const int64_t i = w0 + k;
        if (i < n_w16) dst[i] = make_uint4(acc, acc + 1u, acc + 2u, acc + 3u);
    }
}

}  // namespace

hipError_t launch_probe_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream) {
    const int64_t n16 = bytes / 16;
    const int64_t grid = (n16 + kProbeThreads - 1) / kProbeThreads;
    hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)grid), dim3(kProbeThreads), 0, stream,
                       static_cast<const uint4*>(src), n16, sink);
    return hipGetLastError();
}

hipError_t launch_probe_write(void* dst, int64_t bytes, hipStream_t stream) {
    const int64_t n16 = bytes / 16;
    const int64_t per = (int64_t)kProbeThreads * kWritePer;
    const int64_t grid = (n16 + per - 1) / per;
    hipLaunchKernelGGL(probe_write_kernel, dim3((unsigned)grid), dim3(kProbeThreads), 0, stream,
                       static_cast<uint4*>(dst), n16, 0x01020304u);
    return hipGetLastError();
}

hipError_t launch_probe_read_write(const void* src, int64_t rbytes, void* dst, int64_t wbytes, hipStream_t stream) {
    const int64_t n_r16 = rbytes / 16, n_w16 = wbytes / 16;
    const int64_t per = (int64_t)kProbeThreads * kReadPer;
    int64_t grid = (n_r16 + per - 1) / per;
    if (grid < 1) grid = 1;
    const int64_t w_per = (n_w16 + grid - 1) / grid;
    hipLaunchKernelGGL(probe_read_write_kernel, dim3((unsigned)grid), dim3(kProbeThreads), 0, stream,
                       static_cast<const uint4*>(src), n_r16, static_cast<uint4*>(dst), n_w16, w_per);
    return hipGetLastError();
}

}  // namespace tq
