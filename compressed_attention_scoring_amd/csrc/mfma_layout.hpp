// Operand layout of the 32 x 32 split-f16 scoring kernels (gfx950): the
// order in which each key layout's coordinates enter the contraction, the
// key-side operand builders (codebook lookups by v_perm byte tables, signs as
// f16 +-1), the code loads of one lane, and the LDS slots of the query-side
// operands that the workgroup builds once. Shared by the 32 x 32 families
// (score_lds.hip, score_reg.hip, score_shared.hip, score_fused.hip).
//
// v_mfma_f32_32x32x16_f16: lane l supplies row (or column) l % 32 and
// contraction elements 8 (l / 32) .. 8 (l / 32) + 7 of each 16-wide k-step;
// output element v of lane l is row 8 (v / 4) + 4 (l / 32) + (v % 4),
// column l % 32.
#pragma once

#include <utility>

#include <type_traits>

#include "mfma_ops.hpp"
#include "tq_common.hpp"

namespace tq {
namespace layout {

using namespace ops;

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kTileKeys = 32;

// ---------------------------------------------------------------------------
// Coordinate order. Element e (0..7) of k-step j of a lane half covers
// coordinate half_base + mse_dim(j, e) in the codebook contraction and
// half_base + qjl_dim(j, e) in the sign contraction.
// ---------------------------------------------------------------------------

// 3-bit fields t of a 24-bit group taken per k-step (four k-steps per 32
// coordinates): fields that sit inside one byte first, the two that straddle a
// byte boundary (t = 2, 5) last.
__host__ __device__ constexpr int t3_field(int jj, int hi) {
    return jj == 0 ? (hi ? 1 : 0) : jj == 1 ? (hi ? 4 : 3) : jj == 2 ? (hi ? 7 : 6) : (hi ? 5 : 2);
}

template <int LAYOUT, int BITS>
__host__ __device__ constexpr int mse_dim(int j, int e) {
    if (LAYOUT == 0) return 8 * j + e;
    if (BITS == 2) return 16 * (j / 2) + 4 * (e % 4) + 2 * (j % 2) + e / 4;
    // BITS == 3: 32-coordinate blocks of four 24-bit groups m = 0..3
    const int blk = j / 4, jj = j % 4, pos = e % 4;
    const int t = t3_field(jj, e >= 4);
    const int m = (jj == 3) ? (pos == 1 ? 2 : pos == 2 ? 1 : pos) : pos;
    return 32 * blk + 8 * m + t;
}

template <int LAYOUT>
__host__ __device__ constexpr int qjl_dim(int j, int e) {
    if (LAYOUT == 0) return 8 * j + ((e & 4) | ((e & 1) << 1) | ((e >> 1) & 1));
    return 32 * (j / 4) + 4 * (j % 4) + e / 2 + 16 * (e % 2);
}

// Inverses: the k-step j and element e that coordinate dd (within a lane half)
// occupies in each contraction.
template <int LAYOUT, int BITS>
__host__ __device__ constexpr void mse_slot(int dd, int& j, int& e) {
    if (LAYOUT == 0) {
        j = dd / 8;
        e = dd % 8;
    } else if (BITS == 2) {
        const int r = dd % 16;
        e = r / 4 + 4 * (r % 2);
        j = 2 * (dd / 16) + (r % 4) / 2;
    } else {
        const int blk = dd / 32, m = (dd % 32) / 8, t = dd % 8;
        const int jj = (t == 0 || t == 1) ? 0 : (t == 3 || t == 4) ? 1 : (t == 6 || t == 7) ? 2 : 3;
        const int hi = (t == 1 || t == 4 || t == 7 || t == 5) ? 1 : 0;
        const int pos = (jj == 3) ? (m == 1 ? 2 : m == 2 ? 1 : m) : m;
        e = pos + 4 * hi;
        j = 4 * blk + jj;
    }
}

template <int LAYOUT>
__host__ __device__ constexpr void qjl_slot(int dd, int& j, int& e) {
    if (LAYOUT == 0) {
        const int r = dd % 8;
        e = (r & 4) | ((r & 1) << 1) | ((r >> 1) & 1);   // the order is its own inverse
        j = dd / 8;
    } else {
        const int r = dd % 32, r2 = r % 16;
        e = 2 * (r2 % 4) + r / 16;
        j = 4 * (dd / 32) + r2 / 4;
    }
}

// The same slots for coordinate dd = 16*blk16 + k, written so that with k a
// compile-time constant only a few operations on blk16 remain at run time.
template <int LAYOUT, int BITS>
__host__ __device__ constexpr void mse_slot16(int blk16, int k, int& j, int& e) {
    if (LAYOUT == 0) {
        j = 2 * blk16 + k / 8;
        e = k % 8;
    } else if (BITS == 2) {
        e = k / 4 + 4 * (k % 2);
        j = 2 * blk16 + (k % 4) / 2;
    } else {
        const int h = blk16 & 1, t = k % 8;
        const int jj = (t == 0 || t == 1) ? 0 : (t == 3 || t == 4) ? 1 : (t == 6 || t == 7) ? 2 : 3;
        const int hi = (t == 1 || t == 4 || t == 7 || t == 5) ? 1 : 0;
        const int pos = (jj == 3) ? 2 * (k / 8) + h : 2 * h + k / 8;
        e = pos + 4 * hi;
        j = 4 * (blk16 >> 1) + jj;
    }
}

template <int LAYOUT>
__host__ __device__ constexpr void qjl_slot16(int blk16, int k, int& j, int& e) {
    if (LAYOUT == 0) {
        const int r = k % 8;
        e = (r & 4) | ((r & 1) << 1) | ((r >> 1) & 1);
        j = 2 * blk16 + k / 8;
    } else {
        e = 2 * (k % 4) + (blk16 & 1);
        j = 4 * (blk16 >> 1) + k / 4;
    }
}

template <int LAYOUT, int BITS, int HALF>
constexpr bool slot16_matches() {
    for (int dd = 0; dd < HALF; ++dd) {
        int j1 = 0, e1 = 0, j2 = 0, e2 = 0;
        mse_slot<LAYOUT, BITS>(dd, j1, e1);
        mse_slot16<LAYOUT, BITS>(dd / 16, dd % 16, j2, e2);
        if (j1 != j2 || e1 != e2) return false;
        qjl_slot<LAYOUT>(dd, j1, e1);
        qjl_slot16<LAYOUT>(dd / 16, dd % 16, j2, e2);
        if (j1 != j2 || e1 != e2) return false;
    }
    return true;
}
static_assert(slot16_matches<0, 0, 16>() && slot16_matches<0, 0, 128>() && slot16_matches<1, 2, 32>() &&
              slot16_matches<1, 2, 128>() && slot16_matches<1, 3, 32>() && slot16_matches<1, 3, 128>(),
              "block-split slots");

// Whole-slot prologue stores. For the unpacked layout (both operands) and the
// 2-bit layout's codebook operand, the 16 coordinates of prologue block blk16
// fill exactly slots 2 blk16 and 2 blk16 + 1 (all 8 elements of each), at
// elements that do not depend on blk16, so a thread writes each part as two
// 16-byte stores instead of sixteen 2-byte ones (which hit one LDS bank
// eight ways). block_src<...>(s, e) is the block coordinate at element e of
// slot 2 blk16 + s.
template <int LAYOUT, int BITS, bool MSE>
__host__ __device__ constexpr void block_slot16(int blk16, int k, int& j, int& e) {
    if constexpr (MSE) mse_slot16<LAYOUT, BITS>(blk16, k, j, e);
    else qjl_slot16<LAYOUT>(blk16, k, j, e);
}

template <int LAYOUT, int BITS, bool MSE>
constexpr int block_src(int s, int e) {
    for (int k = 0; k < 16; ++k) {
        int j = 0, ee = 0;
        block_slot16<LAYOUT, BITS, MSE>(0, k, j, ee);
        if (j == s && ee == e) return k;
    }
    return -1;
}

template <int LAYOUT, int BITS, bool MSE>
constexpr bool whole_block_slots() {
    for (int blk = 0; blk < 8; ++blk) {
        bool seen[2][8] = {};
        for (int k = 0; k < 16; ++k) {
            int j = 0, e = 0, j0 = 0, e0 = 0;
            block_slot16<LAYOUT, BITS, MSE>(blk, k, j, e);
            block_slot16<LAYOUT, BITS, MSE>(0, k, j0, e0);
            if (j0 < 0 || j0 > 1 || j != 2 * blk + j0 || e != e0 || seen[j0][e]) return false;
            seen[j0][e] = true;
        }
    }
    return true;
}
static_assert(whole_block_slots<0, 0, true>() && whole_block_slots<0, 0, false>() &&
              whole_block_slots<1, 2, true>(), "whole-slot prologue layouts");

// The packed layouts' sign operand: block blk16 fills the even (blk16 even) or
// odd elements of slots 4 (blk16 >> 1) + c, c = 0..3, with coordinate 4 c + i
// at element 2 i + (blk16 & 1); blocks blk16 and blk16 ^ 1 sit in adjacent
// lanes and complete each other's slots.
constexpr bool packed_sign_pairs() {
    for (int blk = 0; blk < 8; ++blk)
        for (int k = 0; k < 16; ++k) {
            int j = 0, e = 0;
            qjl_slot16<1>(blk, k, j, e);
            if (j != 4 * (blk >> 1) + k / 4 || e != 2 * (k % 4) + (blk & 1)) return false;
        }
    return true;
}
static_assert(packed_sign_pairs(), "packed sign slots");

template <int LAYOUT, int BITS, bool MSE>
__device__ __forceinline__ uint4 whole_slot(const uint16_t (&v)[16], int s) {
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
        w[q] = (uint32_t)v[block_src<LAYOUT, BITS, MSE>(s, 2 * q)] |
               ((uint32_t)v[block_src<LAYOUT, BITS, MSE>(s, 2 * q + 1)] << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// Compile-time proof that every coordinate of a lane half lands in exactly one
// (k-step, element) slot of each contraction and that the slot maps invert.
template <int LAYOUT, int BITS, int HALF>
constexpr bool orders_are_bijections() {
    for (int j = 0; j < HALF / 8; ++j) {
        for (int e = 0; e < 8; ++e) {
            int j2 = -1, e2 = -1;
            const int dm = mse_dim<LAYOUT, BITS>(j, e);
            if (dm < 0 || dm >= HALF) return false;
            mse_slot<LAYOUT, BITS>(dm, j2, e2);
            if (j2 != j || e2 != e) return false;
            const int dq = qjl_dim<LAYOUT>(j, e);
            if (dq < 0 || dq >= HALF) return false;
            qjl_slot<LAYOUT>(dq, j2, e2);
            if (j2 != j || e2 != e) return false;
        }
    }
    return true;
}
static_assert(orders_are_bijections<0, 0, 16>() && orders_are_bijections<0, 0, 32>() &&
              orders_are_bijections<0, 0, 64>() && orders_are_bijections<0, 0, 128>(), "unpacked orders");
static_assert(orders_are_bijections<1, 2, 32>() && orders_are_bijections<1, 2, 64>() &&
              orders_are_bijections<1, 2, 128>(), "2-bit orders");
static_assert(orders_are_bijections<1, 3, 32>() && orders_are_bijections<1, 3, 64>() &&
              orders_are_bijections<1, 3, 128>(), "3-bit orders");

// ---------------------------------------------------------------------------
// Key-side operand builders
// ---------------------------------------------------------------------------


template <int LAYOUT, int BITS>
struct Fmt;

template <>
struct Fmt<0, 0> {   // unpacked: one byte per index and per sign
    template <int D> static constexpr int idx_dw() { return D / 8; }   // per lane half
    template <int D> static constexpr int sign_dw() { return D / 8; }
    template <int D> static constexpr int idx_row() { return D; }
    template <int D> static constexpr int sign_row() { return D; }
    template <int NI>
    __device__ static __forceinline__ void selectors(const uint32_t (&w)[NI], int j, uint32_t& x0, uint32_t& x1) {
        x0 = w[2 * j];
        x1 = w[2 * j + 1];
    }
    template <int NS>
    __device__ static __forceinline__ void signs(const uint32_t (&s)[NS], int j, uint32_t (&o)[4]) {
        const uint32_t s0 = s[2 * j], s1 = s[2 * j + 1];
        o[0] = signs_of(s0 << 8);   // coordinates 0, 2
        o[1] = signs_of(s0);        // coordinates 1, 3
        o[2] = signs_of(s1 << 8);   // coordinates 4, 6
        o[3] = signs_of(s1);        // coordinates 5, 7
    }
};

// packed sign stream: bit 1 = +1; the f16 sign bit must be set for bit 0
template <int NS>
__device__ __forceinline__ void packed_signs(const uint32_t (&s)[NS], int j, uint32_t (&o)[4]) {
    const uint32_t nv = ~s[j / 4];
    const int k0 = 4 * (j % 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = signs_of(nv << (15 - (k0 + i)));
}

template <>
struct Fmt<1, 2> {   // 2-bit indices, 16 per dword
    template <int D> static constexpr int idx_dw() { return D / 32; }
    template <int D> static constexpr int sign_dw() { return D / 64; }
    template <int D> static constexpr int idx_row() { return D / 4; }
    template <int D> static constexpr int sign_row() { return D / 8; }
    template <int NI>
    __device__ static __forceinline__ void selectors(const uint32_t (&w)[NI], int j, uint32_t& x0, uint32_t& x1) {
        const uint32_t v = w[j / 2];
        const int k0 = 2 * (j % 2);
        x0 = (v >> (2 * k0)) & 0x03030303u;
        x1 = (v >> (2 * k0 + 2)) & 0x03030303u;
    }
    template <int NS>
    __device__ static __forceinline__ void signs(const uint32_t (&s)[NS], int j, uint32_t (&o)[4]) {
        packed_signs(s, j, o);
    }
};

template <>
struct Fmt<1, 3> {   // 3-bit indices, 32 per three dwords
    template <int D> static constexpr int idx_dw() { return 3 * D / 64; }
    template <int D> static constexpr int sign_dw() { return D / 64; }
    template <int D> static constexpr int idx_row() { return 3 * D / 8; }
    template <int D> static constexpr int sign_row() { return D / 8; }
    template <int NI>
    __device__ static __forceinline__ void selectors(const uint32_t (&w)[NI], int j, uint32_t& x0, uint32_t& x1) {
        const uint32_t W0 = w[3 * (j / 4)], W1 = w[3 * (j / 4) + 1], W2 = w[3 * (j / 4) + 2];
        constexpr uint32_t m = 0x07070707u, m2 = 0x00070007u;
        switch (j % 4) {
            case 0: {   // fields 0 and 1 of groups 0..3: bytes 0, 3, 6, 9 at bit offsets 0 and 3
                const uint32_t g = perm(W1, W0, 0x0C0C0300u) | perm(W2, W1, 0x05020C0Cu);
                x0 = g & m;
                x1 = (g >> 3) & m;
                break;
            }
            case 1: {   // fields 3 and 4: bytes 1, 4, 7, 10 at offsets 1 and 4
                const uint32_t g = perm(W1, W0, 0x0C0C0401u) | perm(W2, W1, 0x06030C0Cu);
                x0 = (g >> 1) & m;
                x1 = (g >> 4) & m;
                break;
            }
            case 2: {   // fields 6 and 7: bytes 2, 5, 8, 11 at offsets 2 and 5
                const uint32_t g = perm(W1, W0, 0x0C0C0502u) | perm(W2, W1, 0x07040C0Cu);
                x0 = (g >> 2) & m;
                x1 = (g >> 5) & m;
                break;
            }
            default: {  // fields 2 and 5 straddle bytes: 16-bit windows, groups in order 0, 2, 1, 3
                const uint32_t a = perm(W1, W0, 0x04030100u);   // bytes 0,1 | 3,4
                const uint32_t b = perm(W2, W1, 0x06050302u);   // bytes 6,7 | 9,10
                x0 = ((a >> 6) & m2) | (((b >> 6) & m2) << 8);
                const uint32_t c = perm(W1, W0, 0x05040201u);   // bytes 1,2 | 4,5
                const uint32_t d = perm(W2, W1, 0x07060403u);   // bytes 7,8 | 10,11
                x1 = ((c >> 7) & m2) | (((d >> 7) & m2) << 8);
                break;
            }
        }
    }
    template <int NS>
    __device__ static __forceinline__ void signs(const uint32_t (&s)[NS], int j, uint32_t (&o)[4]) {
        packed_signs(s, j, o);
    }
};

// Load N dwords from an address aligned to ALIGN bytes (4, 8 or 16), using the
// widest loads that alignment allows.
template <int N, int ALIGN>
__device__ __forceinline__ void load_dwords(const uint8_t* __restrict__ p, uint32_t (&v)[N]) {
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
    int i = 0;
    if constexpr (ALIGN % 16 == 0) {
#pragma unroll
        for (; i + 4 <= N; i += 4) {
            const uint4 t = *reinterpret_cast<const uint4*>(q + i);
            v[i] = t.x; v[i + 1] = t.y; v[i + 2] = t.z; v[i + 3] = t.w;
        }
    }
    if constexpr (ALIGN % 8 == 0) {
#pragma unroll
        for (; i + 2 <= N; i += 2) {
            const uint2 t = *reinterpret_cast<const uint2*>(q + i);
            v[i] = t.x; v[i + 1] = t.y;
        }
    }
#pragma unroll
    for (; i < N; ++i) v[i] = q[i];
}

constexpr int align_of_seg(int row_bytes, int seg_bytes) {
    // a lane's segment starts at key * row + m * seg from a 16-byte aligned base
    return (row_bytes % 16 == 0 && seg_bytes % 16 == 0) ? 16
         : (row_bytes % 8 == 0 && seg_bytes % 8 == 0) ? 8 : 4;
}

// Byte offset of this lane's key in row 4 * g of a tile (g = lane / 32), or
// kDropKey past the last key; output element v then adds row_offset(v, S).
__device__ __forceinline__ uint32_t lane_offset(int s, int S, int g) {
    return s < S ? ((uint32_t)g * 4u * (uint32_t)S + (uint32_t)s) * 4u : kDropKey;
}
// Rows 8 (v / 4) + (v % 4) of the MFMA output element v, in bytes; uniform.
__device__ __forceinline__ uint32_t row_offset(int v, int S) {
    return (uint32_t)(8 * (v >> 2) + (v & 3)) * (uint32_t)S * 4u;
}



// One 32-key tile's compressed codes for this lane: its segment of the key's
// index and sign streams, and the key's gamma.
template <int NI, int NS>
struct TileCodes {
    uint32_t iw[NI];
    uint32_t sw[NS];
    float gam;
};

// Four-query kernels (16 x 16 MFMA tiles, 16 keys per tile): lane group
// gq = lane / 16 owns coordinates [gq D/4, (gq + 1) D/4) of each key and reads
// its quarter of the key's index and sign rows.
constexpr int kTileKeys16 = 16;

template <int LAYOUT, int BITS, int D>
struct SmallFmt {
    using F = Fmt<LAYOUT, BITS>;
    static constexpr int Q = D / 4;                            // coordinates per lane
    static constexpr int NI = F::template idx_dw<D / 2>();     // code dwords per lane
    static constexpr int NS = F::template sign_dw<D / 2>();
    static constexpr int IDX_ROW = F::template idx_row<D>();
    static constexpr int SIGN_ROW = F::template sign_row<D>();
    static constexpr int NJ = Q / 8;                           // k-steps of 8 coordinates per lane
};

template <int LAYOUT, int BITS, int D, bool QJL = true>
__device__ __forceinline__ void load_quarter(TileCodes<SmallFmt<LAYOUT, BITS, D>::NI, SmallFmt<LAYOUT, BITS, D>::NS>& c,
                                             const uint8_t* __restrict__ idx, const uint8_t* __restrict__ sign,
                                             const void* __restrict__ gamma, int64_t key, int gq) {
    using SF = SmallFmt<LAYOUT, BITS, D>;
    constexpr int IQ = SF::IDX_ROW / 4, SQ = SF::SIGN_ROW / 4;
    load_dwords<SF::NI, align_of_seg(SF::IDX_ROW, IQ)>(idx + key * SF::IDX_ROW + gq * IQ, c.iw);
    if constexpr (QJL) load_dwords<SF::NS, align_of_seg(SF::SIGN_ROW, SQ)>(sign + key * SF::SIGN_ROW + gq * SQ, c.sw);
    if constexpr (LAYOUT == 0) c.gam = reinterpret_cast<const float*>(gamma)[key];
    else c.gam = (float)reinterpret_cast<const _Float16*>(gamma)[key];
}


// Key-side operands of k-step j: codebook hi and lo parts looked up by index,
// and signs as f16 +-1. LO = false (the single-pass f16 kernels) skips the lo
// part and leaves `clo` untouched.
template <int LAYOUT, int BITS, int NI, int NS, bool QJL = true, bool LO = true>
__device__ __forceinline__ void key_operands(const TileCodes<NI, NS>& c, int j, const uint32_t (&tab_hi)[4],
                                             const uint32_t (&tab_lo)[4], Op8& chi, Op8& clo, Op8& sg) {
    using F = Fmt<LAYOUT, BITS>;
    uint32_t x0, x1;
    F::template selectors<NI>(c.iw, j, x0, x1);
    lut4(x0, tab_hi, chi.u[0], chi.u[1]);
    lut4(x1, tab_hi, chi.u[2], chi.u[3]);
    if constexpr (LO) {
        lut4(x0, tab_lo, clo.u[0], clo.u[1]);
        lut4(x1, tab_lo, clo.u[2], clo.u[3]);
    }
    if constexpr (QJL) F::template signs<NS>(c.sw, j, sg.u);
}

// The tile loop every matrix-core scorer runs. A wavefront (or workgroup) walks
// tiles tile, tile + stride, ... below ntiles with N code buffers in turn:
// before tile t is scored from buffer i, the codes of tile t + (N - 1) stride
// are requested into the buffer tile t - stride used, so each tile's codes are
// in flight for N - 1 tiles of work. Buffers 0 .. N - 2 hold the first N - 1
// tiles' requests on entry, and tile < ntiles. `load(Phase<i>, t)` requests
// tile t's codes into buffer i (any t: the loaders clamp past the end, keeping
// every load unconditional) and `score(Phase<i>, t)` scores tile t from buffer
// i. The buffer index is a compile-time constant (the loop is unrolled N
// times), so a kernel's buffers stay in registers, each in its own array.
template <int PHASE>
struct Phase {
    static constexpr int value = PHASE;
};

template <int I, int N, typename Load, typename Score>
__device__ __forceinline__ bool rotate_step(int& tile, int stride, int ntiles, Load& load, Score& score) {
    load(Phase<(I + N - 1) % N>{}, tile + (N - 1) * stride);
    score(Phase<I>{}, tile);
    tile += stride;
    return tile >= ntiles;
}

template <int N, typename Load, typename Score, int... I>
__device__ __forceinline__ bool rotate_round(int& tile, int stride, int ntiles, Load& load, Score& score,
                                             std::integer_sequence<int, I...>) {
    bool done = false;
    ((done = done || rotate_step<I, N>(tile, stride, ntiles, load, score)), ...);
    return done;
}

template <int N, typename Load, typename Score>
__device__ __forceinline__ void rotate_tiles(int tile, int stride, int ntiles, Load&& load, Score&& score) {
    while (!rotate_round<N>(tile, stride, ntiles, load, score, std::make_integer_sequence<int, N>{})) {
    }
}

// The same walk over an array of N code buffers: load(codes, t), score(codes, t).
template <int N, typename Codes, typename Load, typename Score>
__device__ __forceinline__ void rotate_tiles(Codes (&buf)[N], int tile, int stride, int ntiles, Load&& load,
                                             Score&& score) {
    rotate_tiles<N>(
        tile, stride, ntiles,
        [&](auto ph, int t) __attribute__((always_inline)) { load(buf[decltype(ph)::value], t); },
        [&](auto ph, int t) __attribute__((always_inline)) { score(buf[decltype(ph)::value], t); });
}

// A step that owns its loads and alternates two phases (LDS buffers):
// step(Phase<0>, t), step(Phase<1>, t), ...
template <typename Step>
__device__ __forceinline__ void alternate_tiles(int tile, int stride, int ntiles, Step&& step) {
    rotate_tiles<2>(tile, stride, ntiles, [](auto, int) __attribute__((always_inline)) {}, step);
}

// instruction classes for __builtin_amdgcn_sched_group_barrier
constexpr int kSchedValu = 0x002;
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
constexpr int kValuPerMfma = 7;

// Segment m (0 or 1) of a key: coordinates [m*D/2, (m+1)*D/2). Without QJL
// (MSE-only keys) there is no sign stream and `gamma` is the key's norm.
template <int LAYOUT, int BITS, int D, bool QJL = true>
__device__ __forceinline__ void load_tile(TileCodes<Fmt<LAYOUT, BITS>::template idx_dw<D>(),
                                                    Fmt<LAYOUT, BITS>::template sign_dw<D>()>& c,
                                          const uint8_t* __restrict__ idx, const uint8_t* __restrict__ sign,
                                          const void* __restrict__ gamma, int64_t key, int m) {
    using F = Fmt<LAYOUT, BITS>;
    constexpr int NI = F::template idx_dw<D>();
    constexpr int NS = F::template sign_dw<D>();
    constexpr int IDX_ROW = F::template idx_row<D>();
    constexpr int SIGN_ROW = F::template sign_row<D>();
    constexpr int IDX_SEG = IDX_ROW / 2;
    constexpr int SIGN_SEG = SIGN_ROW / 2;
    load_dwords<NI, align_of_seg(IDX_ROW, IDX_SEG)>(idx + key * IDX_ROW + m * IDX_SEG, c.iw);
    if constexpr (QJL) load_dwords<NS, align_of_seg(SIGN_ROW, SIGN_SEG)>(sign + key * SIGN_ROW + m * SIGN_SEG, c.sw);
    if constexpr (LAYOUT == 0) c.gam = reinterpret_cast<const float*>(gamma)[key];
    else c.gam = (float)reinterpret_cast<const _Float16*>(gamma)[key];
}

// The same codes for tile t of a problem whose keys start at key0 (kTileKeys
// keys per tile; the lane's key is t * kTileKeys + col), through descriptors
// that cover the tile's keys below S: a tile past the end loads nothing and
// moves no bytes, keys past S read as zero. t must be uniform across the
// wavefront.
template <int LAYOUT, int BITS, int D, bool QJL = true>
__device__ __forceinline__ void load_tile_at(TileCodes<Fmt<LAYOUT, BITS>::template idx_dw<D>(),
                                                       Fmt<LAYOUT, BITS>::template sign_dw<D>()>& c,
                                             const uint8_t* __restrict__ idx, const uint8_t* __restrict__ sign,
                                             const void* __restrict__ gamma, int64_t key0, int t, int S, int col,
                                             int m) {
    using F = Fmt<LAYOUT, BITS>;
    constexpr int NI = F::template idx_dw<D>();
    constexpr int NS = F::template sign_dw<D>();
    constexpr int IDX_ROW = F::template idx_row<D>();
    constexpr int SIGN_ROW = F::template sign_row<D>();
    const int nk = __builtin_amdgcn_readfirstlane(max(0, min(kTileKeys, S - t * kTileKeys)));
    const int64_t k0 = key0 + (nk > 0 ? (int64_t)t * kTileKeys : 0);
    buffer_dwords<NI>(key_rows(idx + k0 * IDX_ROW, nk, IDX_ROW), (uint32_t)(col * IDX_ROW + m * (IDX_ROW / 2)), c.iw);
    if constexpr (QJL)
        buffer_dwords<NS>(key_rows(sign + k0 * SIGN_ROW, nk, SIGN_ROW), (uint32_t)(col * SIGN_ROW + m * (SIGN_ROW / 2)),
                          c.sw);
    if constexpr (LAYOUT == 0) {
        c.gam = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                              key_rows(static_cast<const float*>(gamma) + k0, nk, 4), (uint32_t)col * 4u, 0, 0));
    } else {
        const uint16_t h = __builtin_amdgcn_raw_buffer_load_b16(key_rows(static_cast<const _Float16*>(gamma) + k0, nk, 2),
                                                                (uint32_t)col * 2u, 0, 0);
        c.gam = (float)__builtin_bit_cast(_Float16, h);
    }
}

// Position of operand lane p's 16-byte slot in the LDS block of k-step j. The
// blocks of different k-steps sit 4 KiB apart (the same banks), so the eight
// 16-coordinate blocks of a query row, written together in the prologue, would
// all hit the same banks; XOR-ing bits 2-4 with the block (j >> 1) and bit 1
// with the lane half (bit 5) spreads them, while the 16 lanes of every quarter
// wave that read one k-step's block still cover 16 distinct slots (a bijection
// that keeps bits 4-5 of p within each group of 16).
__device__ __forceinline__ int slot_pos(int p, int j) {
    return p ^ (((j >> 1) & 7) << 2) ^ (((p >> 5) & 1) << 1);
}

// Prologue stores of one 16-coordinate block of a query row (block blk16 of
// operand lane p: segment p / 32, row p % 32) into the LDS operand blocks of a
// 32-query tile starting at tile_base: parts 0/1 the A hi/lo
// halves, 2/3 the T halves. Whole 16-byte slots where the layout allows
// (whole_block_slots, packed_sign_pairs); the 3-bit codebook operand keeps
// 2-byte stores. `live` is false for rows past the tile: such lanes still take
// part in the sign exchange with their neighbour but store nothing.
// LO = false (the single-pass f16 kernels) stores the hi parts only.
template <int LAYOUT, int BITS, bool QJL, int SEG, bool LO = true>
__device__ __forceinline__ void prologue_store(uint8_t* tile_base, int p, int blk16, const float (&a)[SEG],
                                               const float (&t)[SEG], float sA, float sT, bool live) {
    static_assert(SEG == 16, "blocks of 16 coordinates");
    constexpr int BLOCK = 64 * 16;
    constexpr bool WHOLE_MSE = LAYOUT == 0 || BITS == 2;    // whole_block_slots holds
    uint16_t ah[SEG], al[SEG];
#pragma unroll
    for (int k = 0; k < SEG; ++k) split_f16(a[k] * sA, ah[k], al[k]);
    if constexpr (WHOLE_MSE) {
        if (live) {
#pragma unroll
            for (int sl = 0; sl < 2; ++sl) {
                const int j = 2 * blk16 + sl;
                uint8_t* base = tile_base + (j * 4) * BLOCK + slot_pos(p, j) * 16;
                *reinterpret_cast<uint4*>(base + 0 * BLOCK) = whole_slot<LAYOUT, BITS, true>(ah, sl);
                if constexpr (LO) *reinterpret_cast<uint4*>(base + 1 * BLOCK) = whole_slot<LAYOUT, BITS, true>(al, sl);
            }
        }
    } else if (live) {
#pragma unroll
        for (int k = 0; k < SEG; ++k) {
            int j, e;
            mse_slot16<LAYOUT, BITS>(blk16, k, j, e);
            uint8_t* base = tile_base + (j * 4) * BLOCK + slot_pos(p, j) * 16 + e * 2;
            *reinterpret_cast<uint16_t*>(base + 0 * BLOCK) = ah[k];
            if constexpr (LO) *reinterpret_cast<uint16_t*>(base + 1 * BLOCK) = al[k];
        }
    }
    if constexpr (QJL) {
        uint16_t th[SEG], tl[SEG];
#pragma unroll
        for (int k = 0; k < SEG; ++k) split_f16(t[k] * sT, th[k], tl[k]);
        if constexpr (LAYOUT == 0) {
            if (live) {
#pragma unroll
                for (int sl = 0; sl < 2; ++sl) {
                    const int j = 2 * blk16 + sl;
                    uint8_t* base = tile_base + (j * 4) * BLOCK + slot_pos(p, j) * 16;
                    *reinterpret_cast<uint4*>(base + 2 * BLOCK) = whole_slot<LAYOUT, BITS, false>(th, sl);
                    if constexpr (LO)
                        *reinterpret_cast<uint4*>(base + 3 * BLOCK) = whole_slot<LAYOUT, BITS, false>(tl, sl);
                }
            }
        } else {
            // packed_sign_pairs: this lane (hb = blk16 & 1) and lane ^ 1 (the other
            // parity, same row and segment) share slots 4 (blk16 >> 1) + c. The
            // lane with hb writes slots c = 2 hb, 2 hb + 1 whole: it keeps its own
            // coordinates 4 c + i of those slots and receives the partner's.
            // Word w of slot c holds i = 2 w (low half) and 2 w + 1 (high half).
            const bool odd = (blk16 & 1) != 0;
            uint32_t own_h[4][2], own_l[4][2];
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int w = 0; w < 2; ++w) {
                    own_h[c][w] = (uint32_t)th[4 * c + 2 * w] | ((uint32_t)th[4 * c + 2 * w + 1] << 16);
                    own_l[c][w] = (uint32_t)tl[4 * c + 2 * w] | ((uint32_t)tl[4 * c + 2 * w + 1] << 16);
                }
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                uint32_t mine_h[2], mine_l[2], got_h[2], got_l[2];
#pragma unroll
                for (int w = 0; w < 2; ++w) {
                    // send the partner's slots (2 (1 - hb) + cc), keep this lane's (2 hb + cc)
                    const uint32_t send_h = odd ? own_h[cc][w] : own_h[2 + cc][w];
                    const uint32_t send_l = odd ? own_l[cc][w] : own_l[2 + cc][w];
                    mine_h[w] = odd ? own_h[2 + cc][w] : own_h[cc][w];
                    mine_l[w] = odd ? own_l[2 + cc][w] : own_l[cc][w];
                    got_h[w] = (uint32_t)__shfl_xor((int)send_h, 1);
                    got_l[w] = LO ? (uint32_t)__shfl_xor((int)send_l, 1) : 0u;
                }
                // element 2 i + parity: the even lane's value, then the odd lane's
                uint32_t oh[4], ol[4];
#pragma unroll
                for (int w = 0; w < 2; ++w) {
                    const uint32_t e0h = odd ? got_h[w] : mine_h[w], e1h = odd ? mine_h[w] : got_h[w];
                    const uint32_t e0l = odd ? got_l[w] : mine_l[w], e1l = odd ? mine_l[w] : got_l[w];
                    oh[2 * w] = __builtin_amdgcn_perm(e1h, e0h, 0x05040100u);
                    oh[2 * w + 1] = __builtin_amdgcn_perm(e1h, e0h, 0x07060302u);
                    ol[2 * w] = __builtin_amdgcn_perm(e1l, e0l, 0x05040100u);
                    ol[2 * w + 1] = __builtin_amdgcn_perm(e1l, e0l, 0x07060302u);
                }
                if (live) {
                    const int j = 4 * (blk16 >> 1) + 2 * (blk16 & 1) + cc;
                    uint8_t* base = tile_base + (j * 4) * BLOCK + slot_pos(p, j) * 16;
                    *reinterpret_cast<uint4*>(base + 2 * BLOCK) = make_uint4(oh[0], oh[1], oh[2], oh[3]);
                    if constexpr (LO)
                        *reinterpret_cast<uint4*>(base + 3 * BLOCK) = make_uint4(ol[0], ol[1], ol[2], ol[3]);
                }
            }
        }
    }
}

}  // namespace layout
}  // namespace tq
