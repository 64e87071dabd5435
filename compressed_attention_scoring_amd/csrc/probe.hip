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
//    scores out) without its arithmetic;
//  * tile pattern: the loads and stores of the unpacked 32 x 32 scorer, in its
//    grid, without its arithmetic: each wavefront takes 32-key tiles, lane
//    (col, g) loads half of key col's index row and half of its sign row (16
//    bytes per lane and instruction, so an instruction touches 32 rows) and
//    gamma, folds them into one word, and stores 16 words of the [B, S] output
//    in the accumulator order of the matrix cores (two 128-byte rows per
//    instruction, streaming stores through a descriptor that drops rows past B
//    and keys past S).
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

constexpr int kTileKeys = 32;
constexpr uint32_t kWord3 = 0x00020000u;     // raw 32-bit buffer
constexpr uint32_t kDrop = 0x80000000u;      // offset of a key past S: beyond every descriptor here
constexpr int kStreaming = 2;                // store cache policy of the scorer

template <int D>
__global__ __launch_bounds__(kProbeThreads) void probe_tile_kernel(const uint8_t* __restrict__ idx,
                                                                   const uint8_t* __restrict__ sign,
                                                                   const float* __restrict__ gamma,
                                                                   float* __restrict__ out, int B, int S) {
    constexpr int NW = D / 2 / 16;           // 16-byte words of a lane's half row
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 31, g = lane >> 5;
    const int ntiles = (S + kTileKeys - 1) / kTileKeys;
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(out, 0, (int)((uint32_t)min(B, 32) * (uint32_t)S * 4u), kWord3);
    for (int t = blockIdx.x * 4 + wave; t < ntiles; t += gridDim.x * 4) {
        const int key = min(t * kTileKeys + col, S - 1);
        const uint4* pi = reinterpret_cast<const uint4*>(idx + (int64_t)key * D + g * (D / 2));
        const uint4* ps = reinterpret_cast<const uint4*>(sign + (int64_t)key * D + g * (D / 2));
        uint4 wi[NW], ws[NW];
#pragma unroll
        for (int k = 0; k < NW; ++k) wi[k] = pi[k];
#pragma unroll
        for (int k = 0; k < NW; ++k) ws[k] = ps[k];
        uint32_t x = __float_as_uint(gamma[key]);
#pragma unroll
        for (int k = 0; k < NW; ++k) x ^= wi[k].x ^ wi[k].y ^ wi[k].z ^ wi[k].w ^ ws[k].x ^ ws[k].y ^ ws[k].z ^ ws[k].w;
        const int s = t * kTileKeys + col;
        const uint32_t lo = s < S ? ((uint32_t)g * 4u * (uint32_t)S + (uint32_t)s) * 4u : kDrop;
#pragma unroll
        for (int v = 0; v < 16; ++v)
            __builtin_amdgcn_raw_buffer_store_b32(x + (uint32_t)v, r,
                                                  lo + (uint32_t)(8 * (v >> 2) + (v & 3)) * (uint32_t)S * 4u, 0,
                                                  kStreaming);
    }
}

}  // namespace

bool probe_tile_supported(int B, int S, int D) {
    return B >= 1 && B <= 32 && S >= 1 && S < (1 << 24) && (D == 64 || D == 128 || D == 256);
}

hipError_t launch_probe_tile(const uint8_t* idx, const uint8_t* sign, const float* gamma, float* out, int B, int S,
                             int D, hipStream_t stream) {
    if (!probe_tile_supported(B, S, D)) return hipErrorInvalidValue;
    const int ntiles = (S + kTileKeys - 1) / kTileKeys;
    // the grid of the LDS-staged scorer at one 32-query tile: a tile per
    // wavefront up to 256 workgroups (one per compute unit), then grid-stride
    const int grid = min((ntiles + 3) / 4, 256);
    switch (D) {
        case 64:
            hipLaunchKernelGGL(probe_tile_kernel<64>, dim3(grid), dim3(kProbeThreads), 0, stream, idx, sign, gamma, out, B, S);
            break;
        case 128:
            hipLaunchKernelGGL(probe_tile_kernel<128>, dim3(grid), dim3(kProbeThreads), 0, stream, idx, sign, gamma, out, B, S);
            break;
        default:
            hipLaunchKernelGGL(probe_tile_kernel<256>, dim3(grid), dim3(kProbeThreads), 0, stream, idx, sign, gamma, out, B, S);
            break;
    }
    return hipGetLastError();
}

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
