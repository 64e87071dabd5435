// tq_score on the matrix cores, LDS-staged query operands (CDNA4
// v_mfma_f32_32x32x16_f16): one to four 32-query tiles per workgroup.
//
// What it computes is the scoring identity of "TurboQuant Attention in CUDA:
// Transform the Query, Reuse the Work" (sections "Move the transforms to the
// query", "Two kernels, two jobs"):
//   scores[b,s] = M[b,s] + (sqrt(pi/2)/D) gamma_s R[b,s],
//   M = A C^T with C[s,d] = codebook[idx[s,d]],  R = T Sigma^T with Sigma = signs.
// Both M and R are dense contractions over D across a block of queries, so they
// run on the matrix cores: queries are the 32 MFMA rows, keys the 32 columns,
// coordinates the contraction. "Fitting 4.4x More Context on Jetson", section
// "v5: Extended 2D SDPA", writes the same score as one inner product of length
// 2D; here the two halves keep separate accumulators because gamma_s scales
// only the second.
//
// fp32 accuracy from f16 matrix cores. Each fp32 operand x is split into
// x_hi = f16(x) and x_lo = f16(x - x_hi) (after a power-of-two scale that keeps
// both in f16 range), giving 22 significant bits; products of f16 pairs are
// exact in the fp32 accumulator. Signs are exactly +-1 in f16. Five products
// per k-step: A_hi c_hi, A_lo c_hi, A_hi c_lo (the dropped A_lo c_lo is below
// 2^-22 relative) into M, and T_hi sigma, T_lo sigma into R.
//
// Data flow per workgroup (4 wavefronts):
//  * prologue: the query-side operands A_hi, A_lo, T_hi, T_lo of up to MT
//    32-query tiles are built once from fp32 A and T and stored in LDS in the
//    exact per-lane operand order, so the main loop reads them with one
//    conflict-free 16-byte LDS read per operand;
//  * main loop: each wavefront takes 32-key tiles. A lane owns one key
//    (column lane % 32) and one half of its coordinates (lane / 32), loads that
//    half's index and sign bytes with wide loads, and builds its key-side
//    operands in registers: byte-select (v_perm) lookups into the codebook's
//    f16 hi/lo byte tables, and sign bits moved into the f16 sign position of
//    1.0. Nothing is gathered from memory ("Fitting 4.4x More Context on
//    Jetson", section "Can TurboQuant Match Scaled Dot-Product Attention?",
//    found the per-coordinate centroid gather to be its largest cost);
//  * epilogue: scores = M * (1/(sA sc)) + (coef/sT) gamma R, written as full
//    128-byte rows of consecutive keys.
//
// The order in which a lane's coordinates enter the contraction is free (the
// query-side operands are built in the same order), so each key layout uses the
// order in which its bitstream unpacks with the fewest instructions; see
// mse_dim and qjl_dim.
#include <type_traits>

#include "score_families.hpp"

namespace tq {
namespace {

using namespace ops;
using namespace layout;

// QJL = false scores MSE-only keys: scores = norm_s * M (no T, no signs).
// F16 = true is the single-pass f16 form (with QJL): one product per
// contraction, A_hi c_hi into M and T_hi sigma into R, so the lo halves are
// neither stored nor read nor looked up.
template <int LAYOUT, int BITS, int D, int MT, bool QJL, bool F16 = false>
__global__ __launch_bounds__(kThreads) void score_mfma_kernel(
    const float* __restrict__ A, const float* __restrict__ T,
    const uint8_t* __restrict__ idx, const uint8_t* __restrict__ sign,
    const void* __restrict__ gamma, const float* __restrict__ codebook, int C,
    float* __restrict__ scores, int B, int S, float coef) {
    using F = Fmt<LAYOUT, BITS>;
    constexpr int HALF = D / 2;                // coordinates per lane segment
    constexpr int KS = D / 16;                 // k-steps (16 coordinates each)
    constexpr int NI = F::template idx_dw<D>();
    constexpr int NS = F::template sign_dw<D>();
    constexpr int BLOCK = 64 * 16;             // one operand block: 64 lanes x 16 bytes
    constexpr int OPS_BYTES = MT * KS * 4 * BLOCK;
    constexpr int SEG = 16;                    // coordinates each prologue lane converts
    constexpr int PER_ROW = D / SEG;           // prologue lanes per query row
    constexpr int ROWS_PER_PASS = kThreads / PER_ROW;
    static_assert(HALF % SEG == 0, "the prologue converts 16-coordinate blocks inside one lane segment");

    __shared__ __attribute__((aligned(16))) uint8_t ops[OPS_BYTES];
    __shared__ float2 rowk[MT * 32];           // per-row epilogue factors (M, R)

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: keeps the tile loop scalar
    const int p = blockIdx.z;
    const int b0 = blockIdx.y * MT * 32;
    const int rows = min(MT * 32, B - b0);
    const int col = lane & 31;
    const int g = lane >> 5;
    const int ntiles = (S + kTileKeys - 1) / kTileKeys;
    const int64_t key0 = (int64_t)p * S;

    int tile = blockIdx.x * kWaves + wave;
    const int stride = gridDim.x * kWaves;
    // Code buffers of the tile loop: packed tiles' codes (7-8 registers a lane)
    // are requested two tiles ahead (packed workload 11.4 -> 10.5 us against one
    // ahead); unpacked ones (33 registers) one tile ahead.
    constexpr int NBUF = LAYOUT == 1 ? 3 : 2;
    TileCodes<NI, NS> codes[NBUF];
    TileCodes<NI, NS>& cur = codes[0];

    // codebook byte tables for v_perm lookups and its scale, filled in the
    // prologue once A, T and the first tile's codes have been requested
    float sc = 1.f;
    uint32_t tab_hi[4] = {0u, 0u, 0u, 0u}, tab_lo[4] = {0u, 0u, 0u, 0u};

    // ---- query-side operands: each row of A and T is scaled by its own power of
    //      two (row max found by the lanes that hold the row), split into f16
    //      hi/lo and stored at the slot its coordinate occupies in the operands
    const float* Ap = A + ((int64_t)p * B + b0) * D;
    const float* Tp = T + ((int64_t)p * B + b0) * D;
    for (int r0 = 0; r0 < MT * 32; r0 += ROWS_PER_PASS) {
        const int row = r0 + tid / PER_ROW;            // row within this workgroup's tiles
        const int pl = tid % PER_ROW;                  // coordinates 16*pl .. 16*pl+15
        float a[SEG], t[SEG];
        float ma = 0.f, mt = 0.f;
        // Loads are unconditional (rows past the end re-read the last row and are
        // zeroed below) so that the compiler's wait counts stay exact.
        const int rowc = min(row, rows - 1);
#pragma unroll
        for (int k = 0; k < SEG; k += 4) {
            const float4 va = *reinterpret_cast<const float4*>(Ap + (int64_t)rowc * D + pl * SEG + k);
            a[k] = va.x; a[k + 1] = va.y; a[k + 2] = va.z; a[k + 3] = va.w;
            if constexpr (QJL) {
                const float4 vt = *reinterpret_cast<const float4*>(Tp + (int64_t)rowc * D + pl * SEG + k);
                t[k] = vt.x; t[k + 1] = vt.y; t[k + 2] = vt.z; t[k + 3] = vt.w;
            } else {
                t[k] = t[k + 1] = t[k + 2] = t[k + 3] = 0.f;
            }
        }
        // The first tile's codes are requested right behind the first rows of A
        // and T: vector loads retire in issue order, so converting A and T waits
        // only for them while the key bytes are still in flight from HBM. An empty
        // asm with a memory clobber keeps the compiler from moving the key loads
        // above the A and T loads (it emits no instruction); the key load is
        // unconditional too (a wave without a tile loads nothing through it).
        if (r0 == 0) {
            asm volatile("" ::: "memory");
            load_tile_at<LAYOUT, BITS, D, QJL>(cur, idx, sign, gamma, key0, tile, S, col, g);
            if constexpr (NBUF == 3)
                load_tile_at<LAYOUT, BITS, D, QJL>(codes[1], idx, sign, gamma, key0, tile + stride, S, col, g);
            asm volatile("" ::: "memory");
            // codebook tables; their loads come after the vector loads above so
            // their latency is not paid first
            codebook_tables(codebook, C, sc, tab_hi, tab_lo);
        }
        if (row >= rows) {
#pragma unroll
            for (int k = 0; k < SEG; ++k) a[k] = t[k] = 0.f;
        }
#pragma unroll
        for (int k = 0; k < SEG; ++k) {
            ma = fmaxf(ma, fabsf(a[k]));
            mt = fmaxf(mt, fabsf(t[k]));
        }
#pragma unroll
        for (int o = 1; o < PER_ROW; o <<= 1) {
            ma = fmaxf(ma, __shfl_xor(ma, o));
            mt = fmaxf(mt, __shfl_xor(mt, o));
        }
        const float sA = pow2_scale_for(ma);
        const float sT = pow2_scale_for(mt);
        // sA, sT and sc are powers of two, so these factors are exact
        if (row < MT * 32 && pl == 0) rowk[row] = make_float2(inv_scales(sA, sc), coef / sT);
        const int mtile = row / 32, rl = row % 32;
        const int d0 = pl * SEG;
        const int gg = d0 / HALF;                               // lane segment holding these coordinates
        const int blk16 = (d0 % HALF) / SEG;                    // their 16-coordinate block in it
        prologue_store<LAYOUT, BITS, QJL, SEG, !F16>(ops + (mtile * KS * 4) * BLOCK, gg * 32 + rl, blk16, a, t, sA,
                                                     sT, row < MT * 32);
    }
    __syncthreads();


    // One tile: the key-side operands of k-step j + 1 are built while the LDS
    // reads and MFMAs of step j are in flight, then the scores are scaled and
    // stored (the same pipeline as score_qs_kernel, with the query operands read
    // from LDS).
    auto tile_scores = [&](const TileCodes<NI, NS>& c, int t) __attribute__((always_inline)) {
        f32x16 accM[MT], accR[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int v = 0; v < 16; ++v) { accM[mt][v] = 0.f; accR[mt][v] = 0.f; }
        }
        Op8 chi[2], clo[2], sg[2];
        key_operands<LAYOUT, BITS, NI, NS, QJL, !F16>(c, 0, tab_hi, tab_lo, chi[0], clo[0], sg[0]);
        // LDS operand blocks read and products per 32-query tile and k-step
        constexpr int NOPS = F16 ? 2 : QJL ? 4 : 2;
        constexpr int NMFMA = F16 ? 2 : QJL ? 5 : 3;
#pragma unroll
        for (int j = 0; j < KS; ++j) {
            const int u = j & 1;
            Op8 ahi[MT], alo[MT], thi[MT], tlo[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const uint8_t* base = ops + ((mt * KS + j) * 4) * BLOCK + slot_pos(lane, j) * 16;
                *reinterpret_cast<uint4*>(ahi[mt].u) = *reinterpret_cast<const uint4*>(base + 0 * BLOCK);
                if constexpr (!F16)
                    *reinterpret_cast<uint4*>(alo[mt].u) = *reinterpret_cast<const uint4*>(base + 1 * BLOCK);
                if constexpr (QJL) {
                    *reinterpret_cast<uint4*>(thi[mt].u) = *reinterpret_cast<const uint4*>(base + 2 * BLOCK);
                    if constexpr (!F16)
                        *reinterpret_cast<uint4*>(tlo[mt].u) = *reinterpret_cast<const uint4*>(base + 3 * BLOCK);
                }
            }
            if (j + 1 < KS)
                key_operands<LAYOUT, BITS, NI, NS, QJL, !F16>(c, j + 1, tab_hi, tab_lo, chi[u ^ 1], clo[u ^ 1],
                                                             sg[u ^ 1]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                accM[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[mt].h, chi[u].h, accM[mt], 0, 0, 0);
                if constexpr (QJL)
                    accR[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(thi[mt].h, sg[u].h, accR[mt], 0, 0, 0);
                if constexpr (!F16) {
                    accM[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo[mt].h, chi[u].h, accM[mt], 0, 0, 0);
                    if constexpr (QJL)
                        accR[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(tlo[mt].h, sg[u].h, accR[mt], 0, 0, 0);
                    accM[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[mt].h, clo[u].h, accM[mt], 0, 0, 0);
                }
            }
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, NOPS * MT, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedValu, kValuPerMfma, 0);
#pragma unroll
            for (int i = 0; i < NMFMA * MT; ++i) {
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kSchedValu, MT == 1 ? 5 : 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        const uint32_t lo = lane_offset(t * kTileKeys + col, S, g);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const __amdgpu_buffer_rsrc_t out_r =
                score_rows(scores + ((int64_t)p * B + b0 + mt * 32) * S, max(0, min(32, rows - mt * 32)), S);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float2 k = rowk[mt * 32 + 8 * (v >> 2) + 4 * g + (v & 3)];
                if constexpr (QJL)
                    store_score(out_r, lo + row_offset(v, S), fmaf(k.y * c.gam, accR[mt][v], accM[mt][v] * k.x));
                else
                    store_score(out_r, lo + row_offset(v, S), (accM[mt][v] * k.x) * c.gam);
            }
        }
    };

    // Two code buffers in turn. Wavefronts without a tile took part in the
    // prologue (it ends in a barrier) and leave here.
    if (tile < ntiles) {
        rotate_tiles<NBUF>(
            codes, tile, stride, ntiles,
            [&](TileCodes<NI, NS>& c, int t) __attribute__((always_inline)) {
                load_tile_at<LAYOUT, BITS, D, QJL>(c, idx, sign, gamma, key0, t, S, col, g);
            },
            tile_scores);
    }
}


template <int LAYOUT, int BITS, int D, int MT, bool QJL, bool F16 = false>
hipError_t launch_mt(const float* A, const float* T, KeyStreams k, const float* codebook, int C,
                     float* scores, int P, int B, int S, hipStream_t stream) {
    const int groups_y = (B + MT * 32 - 1) / (MT * 32);
    const int ntiles = (S + kTileKeys - 1) / kTileKeys;
    const int tpg = kWaves;
    const int lds = (D / 16) * 4 * 1024 * MT + MT * 32 * 8;
    int resident = (160 * 1024) / lds;                // workgroups a CU can hold by LDS
    // Two per CU at most: each workgroup builds the query operands once, so more,
    // shorter-lived workgroups repeat that work (measured: the packed workload runs
    // faster with 384-768 workgroups than with 1024).
    if (resident > 2) resident = 2;
    if (resident < 1) resident = 1;
    const int64_t target = 256LL * resident;           // 256 compute units
    int64_t gx = (ntiles + tpg - 1) / tpg;
    int64_t cap = target / ((int64_t)groups_y * P);
    if (cap < 1) cap = 1;
    if (gx > cap) gx = cap;
    const float coef = (float)(kSqrtHalfPi / (double)D);
    hipLaunchKernelGGL((score_mfma_kernel<LAYOUT, BITS, D, MT, QJL, F16>), dim3((unsigned)gx, groups_y, P),
                       dim3(kThreads), 0, stream, A, T, k.idx, k.sign, k.gamma, codebook, C,
                       scores, B, S, coef);
    return hipGetLastError();
}


template <int LAYOUT, int BITS, int D, bool QJL, bool F16 = false>
hipError_t launch_d(const float* A, const float* T, KeyStreams k, const float* codebook, int C,
                    float* scores, int P, int B, int S, hipStream_t stream) {
    switch (mt_for(B, D)) {
        case 4:
            if constexpr (D <= 128)
                return launch_mt<LAYOUT, BITS, D, 4, QJL, F16>(A, T, k, codebook, C, scores, P, B, S, stream);
            [[fallthrough]];
        case 2:
            return launch_mt<LAYOUT, BITS, D, 2, QJL, F16>(A, T, k, codebook, C, scores, P, B, S, stream);
        default:
            return launch_mt<LAYOUT, BITS, D, 1, QJL, F16>(A, T, k, codebook, C, scores, P, B, S, stream);
    }
}

template <int LAYOUT, int BITS, bool QJL = true, bool F16 = false>
hipError_t launch_layout(const float* A, const float* T, KeyStreams k, const float* codebook,
                         int C, float* scores, int P, int B, int S, int D, hipStream_t stream) {
    switch (D) {
        case 32:
            if constexpr (LAYOUT == 0)
                return launch_d<LAYOUT, BITS, 32, QJL, F16>(A, T, k, codebook, C, scores, P, B, S, stream);
            break;
        case 64: return launch_d<LAYOUT, BITS, 64, QJL, F16>(A, T, k, codebook, C, scores, P, B, S, stream);
        case 128: return launch_d<LAYOUT, BITS, 128, QJL, F16>(A, T, k, codebook, C, scores, P, B, S, stream);
        case 256: return launch_d<LAYOUT, BITS, 256, QJL, F16>(A, T, k, codebook, C, scores, P, B, S, stream);
        default: break;
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_family_lds(ScoreForm form, int layout, int bits, const float* A, const float* T, KeyStreams k,
                             const float* codebook, int C, float* scores, int P, int B, int S, int D,
                             hipStream_t stream) {
    auto by_layout = [&](auto qjl, auto f16) {
        constexpr bool QJL = decltype(qjl)::value, F16 = decltype(f16)::value;
        if (layout == 0) return launch_layout<0, 0, QJL, F16>(A, T, k, codebook, C, scores, P, B, S, D, stream);
        if (bits == 2) return launch_layout<1, 2, QJL, F16>(A, T, k, codebook, C, scores, P, B, S, D, stream);
        return launch_layout<1, 3, QJL, F16>(A, T, k, codebook, C, scores, P, B, S, D, stream);
    };
    switch (form) {
        case ScoreForm::kF16: return by_layout(std::true_type{}, std::true_type{});
        case ScoreForm::kMse: return by_layout(std::false_type{}, std::false_type{});
        default: return by_layout(std::true_type{}, std::false_type{});
    }
}

}  // namespace tq
