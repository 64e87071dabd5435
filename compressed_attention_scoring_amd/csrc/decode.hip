// Debug decode: expand compressed keys of either layout into the unpacked
// layout (one byte per index, int8 +-1 per sign, float32 gamma), bit-exactly.
//
// Packed indices are LSB-first bitstreams: coordinate d of a b-bit key sits at
// bits [b*d, b*d + b) of the key's bytes as one little-endian integer, so it
// may straddle a byte boundary when b = 3 ("TurboQuant: Rotate-then-Quantize
// KV Caches at 3 Bits", section 8, on 48-byte 3-bit slots). Signs are one bit
// per coordinate, 1 meaning +1. gamma widens from fp16 exactly.
#include "tq_common.hpp"

namespace tq {
namespace {

__global__ __launch_bounds__(256) void decode_kernel(
    const uint8_t* __restrict__ idx, const uint8_t* __restrict__ sign,
    const void* __restrict__ gamma, int layout, int bits,
    uint8_t* __restrict__ idx_out, int8_t* __restrict__ sign_out,
    float* __restrict__ gamma_out, int64_t keys, int D) {
    const int64_t total = keys * D;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t idx_row = idx_row_bytes(layout, bits, D);
    const int64_t sign_row = sign_row_bytes(layout, D);
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
        const int64_t key = e / D;
        const int d = (int)(e - key * D);
        uint8_t code;
        int8_t sg;
        if (layout == 0) {
            code = idx[key * idx_row + d];
            sg = (int8_t)sign[key * sign_row + d];
        } else {
            const int bit = bits * d;
            const uint8_t* row = idx + key * idx_row;
            uint32_t w = row[bit >> 3];
            if ((bit & 7) + bits > 8) w |= (uint32_t)row[(bit >> 3) + 1] << 8;
            code = (uint8_t)((w >> (bit & 7)) & ((1u << bits) - 1u));
            sg = ((sign[key * sign_row + (d >> 3)] >> (d & 7)) & 1u) ? (int8_t)1 : (int8_t)-1;
        }
        idx_out[e] = code;
        sign_out[e] = sg;
        if (d == 0) {
            gamma_out[key] = layout == 0 ? reinterpret_cast<const float*>(gamma)[key]
                                         : (float)reinterpret_cast<const _Float16*>(gamma)[key];
        }
    }
}

}  // namespace

hipError_t launch_decode(KeyStreams keys, int layout, int bits,
                         uint8_t* idx_out, int8_t* sign_out, float* gamma_out,
                         int P, int S, int D, hipStream_t stream) {
    const int64_t nkeys = (int64_t)P * S;
    const int64_t total = nkeys * D;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(decode_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       keys.idx, keys.sign, keys.gamma, layout, bits,
                       idx_out, sign_out, gamma_out, nkeys, D);
    return hipGetLastError();
}

}  // namespace tq
