// tq_score on the matrix cores, query operands held in each wavefront's
// registers (CDNA4 v_mfma_f32_32x32x16_f16): the choice for 32 < B <= 96.
// The scoring identity and the split-f16 products are those of score_lds.hip.
#include "score_families.hpp"

namespace tq {
namespace {

using namespace ops;
using namespace layout;

// ---------------------------------------------------------------------------
// Query-stationary variant: each wavefront keeps one 32-query tile's operands
// (A_hi, A_lo, T_hi, T_lo: 4 x D/16 x 16 bytes per lane) in registers for its
// whole life and streams key tiles past them, so the main loop touches LDS only
// for the 32 per-row epilogue factors and needs no workgroup barrier. A lane
// builds its own operands: row lane % 32, coordinate half lane / 32, which is
// exactly the slice of A and T that the MFMA A-operand layout gives it. The
// QW wavefronts of a workgroup that hold different query tiles (B > 32) walk
// the same key tiles, so a key tile's bytes come from HBM once per workgroup and
// from the L1 cache for the others.
// ---------------------------------------------------------------------------
template <int LAYOUT, int BITS, int D, int QT, int QW, int MINW>
__global__ __launch_bounds__(kThreads, MINW) void score_qs_kernel(
    const float* __restrict__ A, const float* __restrict__ T,
    const uint8_t* __restrict__ idx, const uint8_t* __restrict__ sign,
    const void* __restrict__ gamma, const float* __restrict__ codebook, int C,
    float* __restrict__ scores, int B, int S, float coef) {
    using F = Fmt<LAYOUT, BITS>;
    constexpr int HALF = D / 2;
    constexpr int KS = D / 16;
    constexpr int NI = F::template idx_dw<D>();
    constexpr int NS = F::template sign_dw<D>();
    constexpr int KW = kWaves / QW;            // key-tile streams per workgroup
    constexpr int VPM = QT == 1 ? kValuPerMfma : (kValuPerMfma + 1) / 2;

    __shared__ float2 rowk[kWaves][QT * 32];   // per-row epilogue factors (M, R) of each wavefront

    const int lane = threadIdx.x & 63;
    // the wavefront index is uniform; saying so keeps everything derived from it
    // (query tiles, output descriptors) in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int p = blockIdx.z;
    const int b0 = (blockIdx.y * QW + wave % QW) * (QT * 32);
    if (b0 >= B) return;                       // no barrier follows: idle wavefronts just leave
    const int rows = min(QT * 32, B - b0);
    const int col = lane & 31;
    const int g = lane >> 5;
    const int ntiles = (S + kTileKeys - 1) / kTileKeys;
    const int64_t key0 = (int64_t)p * S;
    int tile = blockIdx.x * KW + wave / QW;
    const int stride = gridDim.x * KW;
    if (tile >= ntiles) return;

    // this lane's half rows of A and T (row col of each query tile, clamped:
    // rows past B are computed but never stored)
    float a[QT][HALF], t[QT][HALF];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const int64_t roff = ((int64_t)p * B + b0 + min(qt * 32 + col, rows - 1)) * D + g * HALF;
#pragma unroll
        for (int k = 0; k < HALF; k += 4) {
            const float4 va = *reinterpret_cast<const float4*>(A + roff + k);
            const float4 vt = *reinterpret_cast<const float4*>(T + roff + k);
            a[qt][k] = va.x; a[qt][k + 1] = va.y; a[qt][k + 2] = va.z; a[qt][k + 3] = va.w;
            t[qt][k] = vt.x; t[qt][k + 1] = vt.y; t[qt][k + 2] = vt.z; t[qt][k + 3] = vt.w;
        }
    }
    // first tile's codes right behind A and T (see score_mfma_kernel for why the
    // loads are unconditional and fenced)
    TileCodes<NI, NS> codes[2];               // code buffers of the tile loop
    TileCodes<NI, NS>& cur = codes[0];
    asm volatile("" ::: "memory");
    load_tile_at<LAYOUT, BITS, D>(cur, idx, sign, gamma, key0, tile, S, col, g);
    asm volatile("" ::: "memory");
    float sc;
    uint32_t tab_hi[4], tab_lo[4];
    codebook_tables(codebook, C, sc, tab_hi, tab_lo);

    // per-row powers of two (a row's two halves sit in lanes col and col + 32),
    // then the f16 hi/lo operands in contraction order
    Op8 ahi[QT][KS], alo[QT][KS], thi[QT][KS], tlo[QT][KS];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        float ma = 0.f, mt = 0.f;
#pragma unroll
        for (int k = 0; k < HALF; ++k) {
            ma = fmaxf(ma, fabsf(a[qt][k]));
            mt = fmaxf(mt, fabsf(t[qt][k]));
        }
        ma = fmaxf(ma, __shfl_xor(ma, 32));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float sA = pow2_scale_for(ma);
        const float sT = pow2_scale_for(mt);
        if (g == 0) rowk[wave][qt * 32 + col] = make_float2(inv_scales(sA, sc), coef / sT);
#pragma unroll
        for (int j = 0; j < KS; ++j) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float xa = a[qt][mse_dim<LAYOUT, BITS>(j, e)] * sA;
                const _Float16 ha = (_Float16)xa;
                ahi[qt][j].h[e] = ha;
                alo[qt][j].h[e] = (_Float16)(xa - (float)ha);
                const float xt = t[qt][qjl_dim<LAYOUT>(j, e)] * sT;
                const _Float16 ht = (_Float16)xt;
                thi[qt][j].h[e] = ht;
                tlo[qt][j].h[e] = (_Float16)(xt - (float)ht);
            }
        }
    }
    // rowk is read back by other lanes of this wavefront only; LDS operations of
    // one wavefront complete in order
    __builtin_amdgcn_wave_barrier();

    __amdgpu_buffer_rsrc_t out_r[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
        out_r[qt] = score_rows(scores + ((int64_t)p * B + b0 + qt * 32) * S, max(0, min(32, rows - qt * 32)), S);

    // One tile: the key-side operands of k-step j + 1 are built while the MFMAs
    // of step j run (the scheduling groups below interleave each MFMA with a few
    // vector instructions), then the scores are scaled and stored.
    auto tile_scores = [&](const TileCodes<NI, NS>& c, int t) __attribute__((always_inline)) {
        f32x16 accM[QT], accR[QT];
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
            for (int v = 0; v < 16; ++v) { accM[qt][v] = 0.f; accR[qt][v] = 0.f; }
        }
        Op8 chi[2], clo[2], sg[2];
        key_operands<LAYOUT, BITS, NI, NS>(c, 0, tab_hi, tab_lo, chi[0], clo[0], sg[0]);
#pragma unroll
        for (int j = 0; j < KS; ++j) {
            const int u = j & 1;
            if (j + 1 < KS) key_operands<LAYOUT, BITS, NI, NS>(c, j + 1, tab_hi, tab_lo, chi[u ^ 1], clo[u ^ 1], sg[u ^ 1]);
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) {
                accM[qt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[qt][j].h, chi[u].h, accM[qt], 0, 0, 0);
                accR[qt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(thi[qt][j].h, sg[u].h, accR[qt], 0, 0, 0);
                accM[qt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo[qt][j].h, chi[u].h, accM[qt], 0, 0, 0);
                accR[qt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(tlo[qt][j].h, sg[u].h, accR[qt], 0, 0, 0);
                accM[qt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[qt][j].h, clo[u].h, accM[qt], 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 5 * QT; ++i) {
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kSchedValu, VPM, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        const uint32_t lo = lane_offset(t * kTileKeys + col, S, g);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float2 k = rowk[wave][qt * 32 + 8 * (v >> 2) + 4 * g + (v & 3)];
                store_score(out_r[qt], lo + row_offset(v, S), fmaf(k.y * c.gam, accR[qt][v], accM[qt][v] * k.x));
            }
        }
    };

    // Two code buffers in turn (no register copies between iterations, so a wait
    // for one buffer never waits for the other's loads); the next tile's codes
    // are requested before the current tile is computed, clamped and
    // unconditional like the first load.
    rotate_tiles<2>(
        codes, tile, stride, ntiles,
        [&](TileCodes<NI, NS>& c, int t) __attribute__((always_inline)) {
            load_tile_at<LAYOUT, BITS, D>(c, idx, sign, gamma, key0, t, S, col, g);
        },
        tile_scores);
}


// Query-stationary launch: each wavefront holds QT query tiles; a workgroup's
// four wavefronts cover QW groups of QT query tiles times 4 / QW key-tile
// streams; MINW wavefronts per SIMD are resident, so 256 * MINW workgroups fill
// the chip.
template <int LAYOUT, int BITS, int D, int QT, int QW, int MINW>
hipError_t launch_qs_cfg(const float* A, const float* T, KeyStreams k, const float* codebook, int C,
                         float* scores, int P, int B, int S, hipStream_t stream) {
    constexpr int KW = kWaves / QW;
    const int qgroups = (B + QT * 32 - 1) / (QT * 32);
    const int groups_y = (qgroups + QW - 1) / QW;
    const int ntiles = (S + kTileKeys - 1) / kTileKeys;
    int64_t gx = (ntiles + KW - 1) / KW;
    int64_t cap = 256LL * MINW / ((int64_t)groups_y * P);
    if (cap < 1) cap = 1;
    if (gx > cap) gx = cap;
    const float coef = (float)(kSqrtHalfPi / (double)D);
    hipLaunchKernelGGL((score_qs_kernel<LAYOUT, BITS, D, QT, QW, MINW>), dim3((unsigned)gx, groups_y, P),
                       dim3(kThreads), 0, stream, A, T, k.idx, k.sign, k.gamma, codebook, C,
                       scores, B, S, coef);
    return hipGetLastError();
}


int qw_for(int B, int qt) {
    const int groups = (B + qt * 32 - 1) / (qt * 32);
    return groups >= 3 ? 4 : groups;
}

template <int LAYOUT, int BITS, int D, int QT>
hipError_t launch_qs_qt(const float* A, const float* T, KeyStreams k, const float* codebook, int C,
                        float* scores, int P, int B, int S, hipStream_t stream) {
    constexpr int MINW = QT == 2 ? 1 : (D <= 64 ? 2 : (LAYOUT == 0 ? 1 : 2));   // fits the registers
    switch (qw_for(B, QT)) {
        case 4: return launch_qs_cfg<LAYOUT, BITS, D, QT, 4, MINW>(A, T, k, codebook, C, scores, P, B, S, stream);
        case 2: return launch_qs_cfg<LAYOUT, BITS, D, QT, 2, MINW>(A, T, k, codebook, C, scores, P, B, S, stream);
        default: return launch_qs_cfg<LAYOUT, BITS, D, QT, 1, MINW>(A, T, k, codebook, C, scores, P, B, S, stream);
    }
}

// One query tile per wavefront. Two (QT = 2, 400 registers, one wavefront per
// SIMD) halve the key decoding per MFMA but measured slower on the 128-query
// workloads than two wavefronts per SIMD with one tile each.
template <int LAYOUT, int BITS, int D>
hipError_t launch_qs_d(const float* A, const float* T, KeyStreams k, const float* codebook, int C,
                       float* scores, int P, int B, int S, hipStream_t stream) {
    return launch_qs_qt<LAYOUT, BITS, D, 1>(A, T, k, codebook, C, scores, P, B, S, stream);
}


template <int LAYOUT, int BITS>
hipError_t launch_qs_layout(const float* A, const float* T, KeyStreams k, const float* codebook,
                            int C, float* scores, int P, int B, int S, int D, hipStream_t stream) {
    switch (D) {
        case 32:
            if constexpr (LAYOUT == 0)
                return launch_qs_d<LAYOUT, BITS, 32>(A, T, k, codebook, C, scores, P, B, S, stream);
            break;
        case 64: return launch_qs_d<LAYOUT, BITS, 64>(A, T, k, codebook, C, scores, P, B, S, stream);
        case 128: return launch_qs_d<LAYOUT, BITS, 128>(A, T, k, codebook, C, scores, P, B, S, stream);
        default: break;
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_family_reg(int layout, int bits, const float* A, const float* T, KeyStreams k, const float* codebook,
                             int C, float* scores, int P, int B, int S, int D, hipStream_t stream) {
    if (layout == 0) return launch_qs_layout<0, 0>(A, T, k, codebook, C, scores, P, B, S, D, stream);
    if (bits == 2) return launch_qs_layout<1, 2>(A, T, k, codebook, C, scores, P, B, S, D, stream);
    return launch_qs_layout<1, 3>(A, T, k, codebook, C, scores, P, B, S, D, stream);
}

}  // namespace tq
