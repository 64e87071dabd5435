// tq_score on the matrix cores for a few queries per problem over many keys:
// 16x16 tiles of four queries times four operand rows (CDNA4
// v_mfma_f32_16x16x32_f16); packed keys take the integer form of score_i8.hip.
// The scoring identity is that of score_lds.hip.
#include <type_traits>

#include "score_i8.hpp"
#include "score_families.hpp"

namespace tq {
namespace {

using namespace ops;
using namespace layout;

// ---------------------------------------------------------------------------
// Small-batch variant (a few queries per problem): v_mfma_f32_16x16x32_f16 with the 16 keys of a
// tile as columns and, as the 16 rows, four queries times four operand types:
// row 4 b + type holds A_hi, A_lo, T_hi or T_lo of query b. A 32-wide
// contraction chunk carries 16 codebook coordinates and 16 sign coordinates:
// in each lane's 8 elements, 0-3 are codebook coordinates (zero in the T rows)
// and 4-7 are sign coordinates (zero in the A rows). A third MFMA per k-step
// adds A_hi c_lo over 32 coordinates into the same accumulator (only the A_hi
// rows are non-zero in it). The output element (row 4 b + type, key) lands in
// lane 16 b + key, register type, so a lane combines the four types of its
// (query, key) pair by itself: 12 MFMAs of 16 cycles per 16 keys at D = 128,
// where padding four queries to the 32-row tile costs 40 of 32 cycles per 32.
// Lane group gq = lane / 16 owns coordinates [gq D/4, (gq + 1) D/4) of each key
// and unpacks them in the same orders as the other variants (mse_dim and
// qjl_dim over a D/2-coordinate half, here used on a D/4 quarter).
// Query groups of four beyond the first (B = 5..8) are further workgroup rows.
// ---------------------------------------------------------------------------
// QJL = false (MSE-only keys, gamma = the key's norm, no sign stream): row
// types 0 and 1 stay A_hi and A_lo against the codebook's hi part in elements
// 0-3, type 2 is A_hi against its lo part in elements 4-7, type 3 is zero, so
// two MFMAs per k-step cover what takes three with signs.
// F16 = true (with QJL): the codebook enters as its f16 hi part only (no lo
// lookups, no third MFMA); the query's lo rows ride in the same two
// instructions as its hi rows, so they are kept.
template <int LAYOUT, int BITS, int D, int MINW, bool QJL = true, bool F16 = false>
__global__ __launch_bounds__(kThreads, MINW) void score_mfma16_kernel(
    const float* __restrict__ A, const float* __restrict__ T,
    const uint8_t* __restrict__ idx, const uint8_t* __restrict__ sign,
    const void* __restrict__ gamma, const float* __restrict__ codebook, int C,
    float* __restrict__ scores, int B, int S, float coef) {
    using SF = SmallFmt<LAYOUT, BITS, D>;
    using F = Fmt<LAYOUT, BITS>;
    constexpr int NI = SF::NI, NS = SF::NS, NJ = SF::NJ, Q = SF::Q;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int p = blockIdx.z;
    const int b0 = blockIdx.y * 4;                 // this workgroup's four queries
    const int nb = min(4, B - b0);
    const int ntiles = (S + kTileKeys16 - 1) / kTileKeys16;
    int tile = blockIdx.x * kWaves + wave;
    const int stride = gridDim.x * kWaves;
    if (tile >= ntiles) return;                    // no barrier in this kernel
    const int gq = lane >> 4;                      // lane group: coordinate quarter / output query
    const int kc = lane & 15;                      // key column
    const int r = lane & 15;                       // operand row = 4 b + type
    const int rb = r >> 2, rtype = r & 3;
    const int64_t key0 = (int64_t)p * S;

    // this lane's quarter row: A for types 0-1, T for types 2-3 (query rb,
    // clamped: queries past B are computed but never stored)
    const float* src = (rtype < 2 || !QJL ? A : T) + ((int64_t)p * B + b0 + min(rb, nb - 1)) * D + gq * Q;
    float x[Q];
#pragma unroll
    for (int k = 0; k < Q; k += 4) {
        const float4 v = *reinterpret_cast<const float4*>(src + k);
        x[k] = v.x; x[k + 1] = v.y; x[k + 2] = v.z; x[k + 3] = v.w;
    }
    // Code buffers of the tile loop: a packed tile's codes are 3-5 registers a
    // lane, so five buffers (four tiles in flight) fit the four wavefronts per
    // SIMD the launch asks for (GQA: 104.0 -> 99.1 us against three); unpacked
    // codes (17 registers) and the six-wavefront MSE form keep three.
    constexpr int NBUF = (QJL && LAYOUT == 1) ? 5 : 3;
    TileCodes<NI, NS> codes[NBUF];
    TileCodes<NI, NS>& cur = codes[0];
    asm volatile("" ::: "memory");
    load_quarter<LAYOUT, BITS, D, QJL>(cur, idx, sign, gamma, key0 + min(tile * kTileKeys16 + kc, S - 1), gq);
    asm volatile("" ::: "memory");
    float sc;
    uint32_t tab_hi[4], tab_lo[4];
    codebook_tables(codebook, C, sc, tab_hi, tab_lo);

    // row scale: max over the row's four quarters (lanes r, r + 16, r + 32, r + 48)
    float mx = 0.f;
#pragma unroll
    for (int k = 0; k < Q; ++k) mx = fmaxf(mx, fabsf(x[k]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float s_row = pow2_scale_for(mx);
    // epilogue factors of output query gq: its A scale sits in row 4 gq (lane 4 gq),
    // its T scale in row 4 gq + 2
    const float sA_out = __shfl(s_row, 4 * gq);
    const float sT_out = __shfl(s_row, 4 * gq + 2);
    const float kx = inv_scales(sA_out, sc);
    const float ky = coef / sT_out;

    // operands: for k-step j, ops[j][0] and [1] pair codebook-hi elements 0-3
    // (coordinates mse_dim(j, 0..3) and (j, 4..7)) with sign elements 4-7
    // (coordinates qjl_dim(j, 0..3) and (j, 4..7)); ops[j][2] is A_hi over
    // mse_dim(j, 0..7) for the codebook-lo product.
    constexpr int NO = QJL && !F16 ? 3 : 2;
    Op8 ops[NJ][NO];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float xa = x[mse_dim<LAYOUT, BITS>(j, 4 * h + e)] * s_row;
                const _Float16 ha = (_Float16)xa;
                const _Float16 la = (_Float16)(xa - (float)ha);
                ops[j][h].h[e] = rtype == 0 ? ha : rtype == 1 ? la : (_Float16)0.f;
                if constexpr (QJL) {
                    const float xt = x[qjl_dim<LAYOUT>(j, 4 * h + e)] * s_row;
                    const _Float16 ht = (_Float16)xt;
                    const _Float16 lt = (_Float16)(xt - (float)ht);
                    ops[j][h].h[4 + e] = rtype == 2 ? ht : rtype == 3 ? lt : (_Float16)0.f;
                } else {
                    ops[j][h].h[4 + e] = rtype == 2 ? ha : (_Float16)0.f;
                }
            }
        }
        if constexpr (QJL && !F16) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float xa = x[mse_dim<LAYOUT, BITS>(j, e)] * s_row;
                ops[j][NO - 1].h[e] = rtype == 0 ? (_Float16)xa : (_Float16)0.f;
            }
        }
    }

    const __amdgpu_buffer_rsrc_t out_r = score_rows(scores + ((int64_t)p * B + b0) * S, nb, S);

    auto tile_scores = [&](const TileCodes<NI, NS>& c, int t) __attribute__((always_inline)) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            uint32_t x0, x1;
            F::template selectors<NI>(c.iw, j, x0, x1);
            Op8 k0, k1;
            lut4(x0, tab_hi, k0.u[0], k0.u[1]);
            lut4(x1, tab_hi, k1.u[0], k1.u[1]);
            if constexpr (QJL) {
                uint32_t sgn[4];
                F::template signs<NS>(c.sw, j, sgn);
                Op8 kl;
                k0.u[2] = sgn[0]; k0.u[3] = sgn[1];
                k1.u[2] = sgn[2]; k1.u[3] = sgn[3];
                if constexpr (!F16) {
                    lut4(x0, tab_lo, kl.u[0], kl.u[1]);
                    lut4(x1, tab_lo, kl.u[2], kl.u[3]);
                }
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ops[j][0].h, k0.h, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ops[j][1].h, k1.h, acc, 0, 0, 0);
                if constexpr (!F16)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ops[j][NO - 1].h, kl.h, acc, 0, 0, 0);
            } else {
                lut4(x0, tab_lo, k0.u[2], k0.u[3]);
                lut4(x1, tab_lo, k1.u[2], k1.u[3]);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ops[j][0].h, k0.h, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ops[j][1].h, k1.h, acc, 0, 0, 0);
            }
        }
        // lane 16 b + key holds rows 4 b .. 4 b + 3 of column key: the four types
        const int s = t * kTileKeys16 + kc;
        const uint32_t off = s < S ? ((uint32_t)gq * (uint32_t)S + (uint32_t)s) * 4u : kDropKey;
        if constexpr (QJL)
            store_score(out_r, off, fmaf(ky * c.gam, acc[2] + acc[3], kx * (acc[0] + acc[1])));
        else
            store_score(out_r, off, (kx * c.gam) * ((acc[0] + acc[1]) + acc[2]));
    };

    // NBUF code buffers in turn: each tile's codes are requested NBUF - 1 tiles ahead
    auto load = [&](TileCodes<NI, NS>& c, int t) __attribute__((always_inline)) {
        load_quarter<LAYOUT, BITS, D, QJL>(c, idx, sign, gamma, key0 + min(min(t, ntiles - 1) * kTileKeys16 + kc, S - 1),
                                           gq);
    };
#pragma unroll
    for (int k = 1; k < NBUF - 1; ++k) load(codes[k], tile + k * stride);
    rotate_tiles<NBUF>(codes, tile, stride, ntiles, load, tile_scores);
}


// Small-batch launch: workgroup rows are groups of four queries; MINW
// wavefronts per SIMD are resident (the kernel needs about 105 registers at
// D = 128 with signs), so 256 * MINW workgroups fill the chip.
template <int LAYOUT, int BITS, int D, bool QJL = true, bool F16 = false>
hipError_t launch_small_d(const float* A, const float* T, KeyStreams k, const float* codebook, int C,
                          float* scores, int P, int B, int S, hipStream_t stream) {
    // without signs the kernel needs about 72 registers at D = 128: six wavefronts per SIMD
    constexpr int MINW = D <= 128 ? (QJL ? 4 : 6) : 2;
    const int groups_y = (B + 3) / 4;
    const int ntiles = (S + kTileKeys16 - 1) / kTileKeys16;
    int64_t gx = (ntiles + kWaves - 1) / kWaves;
    int64_t cap = 256LL * MINW / ((int64_t)groups_y * P);
    if (cap < 1) cap = 1;
    if (gx > cap) gx = cap;
    const float coef = (float)(kSqrtHalfPi / (double)D);
    hipLaunchKernelGGL((score_mfma16_kernel<LAYOUT, BITS, D, MINW, QJL, F16>), dim3((unsigned)gx, groups_y, P),
                       dim3(kThreads), 0, stream, A, T, k.idx, k.sign, k.gamma, codebook, C,
                       scores, B, S, coef);
    return hipGetLastError();
}

template <int LAYOUT, int BITS, bool QJL = true, bool F16 = false>
hipError_t launch_small_layout(const float* A, const float* T, KeyStreams k, const float* codebook,
                               int C, float* scores, int P, int B, int S, int D, hipStream_t stream) {
    // packed keys: the integer form (int8 limbs of every operand)
    if constexpr (LAYOUT == 1 && !F16)
        return launch_score_i8(A, T, k, codebook, C, scores, P, B, S, D, BITS, QJL, stream);
    if (D == 128) return launch_small_d<LAYOUT, BITS, 128, QJL, F16>(A, T, k, codebook, C, scores, P, B, S, stream);
    if (D == 256) return launch_small_d<LAYOUT, BITS, 256, QJL, F16>(A, T, k, codebook, C, scores, P, B, S, stream);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_family_small(ScoreForm form, int layout, int bits, const float* A, const float* T, KeyStreams k,
                              const float* codebook, int C, float* scores, int P, int B, int S, int D,
                              hipStream_t stream) {
    auto by_layout = [&](auto qjl, auto f16) {
        constexpr bool QJL = decltype(qjl)::value, F16 = decltype(f16)::value;
        if (layout == 0) return launch_small_layout<0, 0, QJL, F16>(A, T, k, codebook, C, scores, P, B, S, D, stream);
        if (bits == 2) return launch_small_layout<1, 2, QJL, F16>(A, T, k, codebook, C, scores, P, B, S, D, stream);
        return launch_small_layout<1, 3, QJL, F16>(A, T, k, codebook, C, scores, P, B, S, D, stream);
    };
    switch (form) {
        case ScoreForm::kF16: return by_layout(std::true_type{}, std::true_type{});
        case ScoreForm::kMse: return by_layout(std::false_type{}, std::false_type{});
        default: return by_layout(std::true_type{}, std::false_type{});
    }
}

}  // namespace tq
