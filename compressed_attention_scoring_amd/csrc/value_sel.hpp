// Selector bytes for the value side of the attention products: packed value
// indices (BW bits per coordinate, LSB-first) of eight keys, one lane's W bits
// of each key already shifted to bit 0, turned into the v_perm selector bytes
// of tile t (coordinate t of the lane: the field at bit BW t), keys 0-3 in sel0
// and 4-7 in sel1, one key per byte.
//
// Byte-transposed: tb[gk][k] holds byte k of the bits of keys 4 gk .. 4 gk + 3
// (one key per byte), built once per eight keys with two v_perm per dword; a
// field inside one byte is then a shift and a mask for four keys at once, and a
// field that crosses into the next byte (3-bit fields at bits 6 and 15 of 24)
// is read from 16-bit windows of bytes k and k + 1.
#pragma once

#include <stdint.h>

namespace tq {

template <int BW, int W>
struct ValueSelectors {
    static_assert(BW == 2 || BW == 3, "packed value indices");
    static_assert(W <= 32, "a lane's bits of one key fit one dword");
    static constexpr int NBY = (W + 7) / 8;
    uint32_t tb[2][NBY];

    __device__ __forceinline__ explicit ValueSelectors(const uint64_t (&vb)[8]) {
#pragma unroll
        for (int gk = 0; gk < 2; ++gk) {
            const uint32_t v0 = (uint32_t)vb[4 * gk], v1 = (uint32_t)vb[4 * gk + 1];
            const uint32_t v2 = (uint32_t)vb[4 * gk + 2], v3 = (uint32_t)vb[4 * gk + 3];
#pragma unroll
            for (int k = 0; k < NBY; ++k) {
                // bytes 0, 1 <- byte k of v0, v1; bytes 2, 3 <- byte k of v2, v3 (0x0C: zero)
                const uint32_t lo_sel = (uint32_t)k | (uint32_t)(4 + k) << 8 | 0x0C0C0000u;
                const uint32_t hi_sel = 0x00000C0Cu | (uint32_t)k << 16 | (uint32_t)(4 + k) << 24;
                tb[gk][k] = __builtin_amdgcn_perm(v1, v0, lo_sel) | __builtin_amdgcn_perm(v3, v2, hi_sel);
            }
        }
    }

    __device__ __forceinline__ void tile(int t, uint32_t& sel0, uint32_t& sel1) const {
        constexpr uint32_t m8 = ((1u << BW) - 1u) * 0x01010101u;
        constexpr uint32_t m16 = ((1u << BW) - 1u) * 0x00010001u;
        const int o = BW * t, k = o >> 3, sh = o & 7;
        uint32_t sel[2];
#pragma unroll
        for (int gk = 0; gk < 2; ++gk) {
            if (sh + BW <= 8) {
                sel[gk] = (tb[gk][k] >> sh) & m8;
            } else {
                const uint32_t a = tb[gk][k], b = tb[gk][k + 1];
                const uint32_t x01 = (__builtin_amdgcn_perm(b, a, 0x05010400u) >> sh) & m16;   // keys 0, 1
                const uint32_t x23 = (__builtin_amdgcn_perm(b, a, 0x07030602u) >> sh) & m16;   // keys 2, 3
                sel[gk] = __builtin_amdgcn_perm(x23, x01, 0x06040200u);
            }
        }
        sel0 = sel[0];
        sel1 = sel[1];
    }
};

// Stand-in where the fields are bytes or span more than a dword (nothing to build).
struct NoValueSelectors {
    __device__ __forceinline__ explicit NoValueSelectors(const uint64_t (&)[8]) {}
};

}  // namespace tq
