// Device helpers shared by the matrix-core scoring kernels (gfx950).
//
// fp32 accuracy from f16 matrix cores: an fp32 operand x, scaled by a power
// of two so that its row maximum sits in [2^13, 2^14), is split into
// x_hi = f16(x) and x_lo = f16(x - x_hi); the products of f16 pairs are exact
// in the fp32 accumulator, so three products (hi.hi, lo.hi, hi.lo) carry about
// 22 significant bits. Key-side codebook values come from byte tables looked
// up with v_perm, signs are moved into the f16 sign of 1.0; nothing is
// gathered from memory.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {
namespace ops {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kOneOne = 0x3C003C00u;   // two f16 1.0
constexpr uint32_t kSignBits = 0x80008000u;

union Op8 {
    f16x8 h;
    uint32_t u[4];
};

__device__ __forceinline__ uint32_t perm(uint32_t hi_src, uint32_t lo_src, uint32_t sel) {
    return __builtin_amdgcn_perm(hi_src, lo_src, sel);
}

// Four selector bytes (each < 8) -> two dwords of f16 pairs from a byte table
// tab = {low bytes of entries 0-3, low bytes of 4-7, high bytes of 0-3, high bytes of 4-7}.
// o0 holds the entries of selector bytes 0, 1 (low, high half), o1 those of bytes 2, 3.
__device__ __forceinline__ void lut4(uint32_t x, const uint32_t (&tab)[4], uint32_t& o0, uint32_t& o1) {
    const uint32_t lo = perm(tab[1], tab[0], x);
    const uint32_t hi = perm(tab[3], tab[2], x);
    o0 = perm(hi, lo, 0x05010400u);
    o1 = perm(hi, lo, 0x07030602u);
}

// (x & sign bits) | f16 1.0 pair in one v_bitop3_b32 (truth table 0xEA is
// (S0 & S1) | S2): bits 15 and 31 of x become the signs of +-1.0 in the low
// and high f16 halves.
__device__ __forceinline__ uint32_t signs_of(uint32_t x) {
    return __builtin_amdgcn_bitop3_b32(x, kSignBits, kOneOne, 0xEA);
}

// Selector bytes of four consecutive 3-bit fields of v (fields 0-3 of v).
__device__ __forceinline__ uint32_t sel3x4(uint32_t v) {
    return (v & 7u) | ((v << 5) & 0x700u) | ((v << 10) & 0x70000u) | ((v << 15) & 0x7000000u);
}

// A power of two bringing maxabs into [2^13, 2^14); 1 if maxabs is 0 or not
// finite. The exponent is clamped so the scale stays a finite normal float
// (a maximum below 2^-113 gets 2^126 and then sits below 2^13 after scaling,
// which costs only relative precision of values that small).
__device__ __forceinline__ float pow2_scale_for(float maxabs) {
    if (!(maxabs > 0.f) || !(maxabs < 3.0e38f)) return 1.f;
    int e;
    (void)frexpf(maxabs, &e);   // maxabs = f * 2^e, f in [0.5, 1)
    return ldexpf(1.f, min(126, 14 - e));
}

__device__ __forceinline__ void split_f16(float x, uint16_t& hi, uint16_t& lo) {
    const _Float16 h = (_Float16)x;
    const _Float16 l = (_Float16)(x - (float)h);
    hi = __builtin_bit_cast(uint16_t, h);
    lo = __builtin_bit_cast(uint16_t, l);
}

__device__ __forceinline__ uint32_t pack_f16(uint16_t lo, uint16_t hi) { return (uint32_t)lo | ((uint32_t)hi << 16); }

// Score stores go through a raw buffer descriptor covering the valid rows of one
// 32-query tile of the output, so the hardware drops writes to rows past B.
// Keys past S get a lane offset of 2^31, beyond any descriptor here. Every store
// therefore issues on every path, with no branches, which keeps the compiler's
// count of outstanding memory operations exact: a wait for the next tile's codes
// does not also wait for this tile's stores to reach memory.
// Byte offsets are row * S * 4 + key * 4 with row < 32; the caller keeps
// S < 2^24, so every in-range offset is below 2^31 and an out-of-range key's
// offset (2^31 plus a row offset below 2^31) cannot wrap around.
constexpr uint32_t kBufferWord3 = 0x00020000u;   // raw 32-bit buffer, gfx9 family
constexpr uint32_t kDropKey = 0x80000000u;       // lane offset of a key past S
constexpr int kNonTemporal = 2;                  // cache policy: stream past the caches

// `rows` is uniform across the wavefront; readfirstlane keeps the descriptor in
// scalar registers (a clamp the compiler evaluated on the vector unit made
// every store a loop over the distinct descriptors of the wavefront's lanes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t score_rows(float* base, int rows, int S) {
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)((uint32_t)__builtin_amdgcn_readfirstlane(rows) * (uint32_t)S * 4u),
                                             kBufferWord3);
}

__device__ __forceinline__ void store_score(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, kNonTemporal);
}

// A raw buffer over `keys` rows of `row` bytes from `base`: loads past it
// return zero without a memory request, so a tile past the last key (or the
// keys past S in the last tile) costs no traffic while every load still
// issues. `keys` must be uniform across the wavefront.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t key_rows(const void* base, int keys, int row) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, keys * row, kBufferWord3);
}

typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x3_t __attribute__((ext_vector_type(3)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// N dwords at byte offset `off` (4-byte aligned) of buffer r, in the widest loads.
template <int N>
__device__ __forceinline__ void buffer_dwords(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t (&w)[N]) {
    int i = 0;
#pragma unroll
    for (; i + 4 <= N; i += 4) {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off + 4u * i, 0, 0);
        w[i] = v.x; w[i + 1] = v.y; w[i + 2] = v.z; w[i + 3] = v.w;
    }
    if constexpr (N % 4 == 3) {
        const u32x3_t v = __builtin_amdgcn_raw_buffer_load_b96(r, off + 4u * i, 0, 0);
        w[i] = v.x; w[i + 1] = v.y; w[i + 2] = v.z;
    } else if constexpr (N % 4 == 2) {
        const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, off + 4u * i, 0, 0);
        w[i] = v.x; w[i + 1] = v.y;
    } else if constexpr (N % 4 == 1) {
        w[i] = __builtin_amdgcn_raw_buffer_load_b32(r, off + 4u * i, 0, 0);
    }
}

// Codebook byte tables for lut4: the entries (up to 8, zero beyond C) times a
// power of two sc, split into f16 hi and lo parts.
__device__ __forceinline__ void codebook_tables(const float* __restrict__ codebook, int C, float& sc,
                                                uint32_t (&tab_hi)[4], uint32_t (&tab_lo)[4]) {
    float cbv[8];
    float mc = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        cbv[k] = k < C ? codebook[k] : 0.f;
        mc = fmaxf(mc, fabsf(cbv[k]));
    }
    sc = pow2_scale_for(mc);
#pragma unroll
    for (int w = 0; w < 4; ++w) tab_hi[w] = tab_lo[w] = 0u;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        uint16_t hb, lb;
        split_f16(cbv[k] * sc, hb, lb);
        const int w = k >> 2, sh = 8 * (k & 3);
        tab_hi[w] |= (uint32_t)(hb & 0xffu) << sh;
        tab_hi[2 + w] |= (uint32_t)(hb >> 8) << sh;
        tab_lo[w] |= (uint32_t)(lb & 0xffu) << sh;
        tab_lo[2 + w] |= (uint32_t)(lb >> 8) << sh;
    }
}

// The epilogue factor 1 / (s1 s2) for two powers of two, as a product of
// reciprocals so that it underflows towards 0 instead of overflowing.
__device__ __forceinline__ float inv_scales(float s1, float s2) { return (1.f / s1) * (1.f / s2); }

}  // namespace ops
}  // namespace tq
