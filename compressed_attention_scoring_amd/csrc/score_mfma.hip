// Scoring kernel, matrix-core family (CDNA4 v_mfma_f32_32x32x16_f16).
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

#include "mfma_layout.hpp"
#include "score_i8.hpp"
#include "value_sel.hpp"

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

// ---------------------------------------------------------------------------
// Outlier split on the matrix cores ("TurboQuant: Rotate-then-Quantize KV
// Caches at 3 Bits", section 7: two MSE-only instances per head, the hot
// channels with one bit more). This kernel takes the page's 2.5-bit setting at
// D = 128: 32 hot channels at 3 bits (8 centroids) and 96 at 2 bits (4), both
// packed LSB-first with fp16 norms; a key's score is
// rho_hi M_hi + rho_lo M_lo with M = <A, c[idx]> per instance.
//
// The LDS-staged layout of score_mfma_kernel with two contractions in one
// 128-coordinate operand: lane half g holds hot coordinates [16 g, 16 g + 16)
// in k-steps 0-1 (k-step j, element e: coordinate 16 g + 8 j + e) and the other
// instance's [48 g, 48 g + 48) in k-steps 2-7 (the 2-bit order of the other
// kernels over those 48). So every k-step belongs to one instance for both lane
// halves: k-steps 0-1 accumulate M_hi, 2-7 M_lo, three split-f16 products each
// (24 MFMAs per 32 x 32 tile). A lane's hot codes are 6 bytes (16 3-bit fields,
// two 24-bit groups, one per k-step); its other codes 12 bytes (48 2-bit fields).
// ---------------------------------------------------------------------------
constexpr int kSplitDHi = 32;
constexpr int kSplitDLo = 96;

struct SplitTileCodes {
    uint32_t h0, h1;        // dwords holding this lane's hot fields (see split_hot_groups)
    uint32_t lw[3];         // this lane's 48 2-bit fields
    float rho_hi, rho_lo;
};

// Codes of key `key` for lane half g: hot row 12 bytes (the lane's 6 start at
// byte 6 g, read as the dwords at 4 g and 4 g + 4), other row 24 bytes (the
// lane's 12 at byte 12 g).
__device__ __forceinline__ void load_split_tile(SplitTileCodes& c, const uint8_t* __restrict__ idx_hi,
                                                const void* __restrict__ norm_hi, const uint8_t* __restrict__ idx_lo,
                                                const void* __restrict__ norm_lo, int64_t key, int g) {
    const uint32_t* hp = reinterpret_cast<const uint32_t*>(idx_hi + key * 12 + 4 * g);
    c.h0 = hp[0];
    c.h1 = hp[1];
    const uint32_t* lp = reinterpret_cast<const uint32_t*>(idx_lo + key * 24 + 12 * g);
    c.lw[0] = lp[0];
    c.lw[1] = lp[1];
    c.lw[2] = lp[2];
    c.rho_hi = (float)reinterpret_cast<const _Float16*>(norm_hi)[key];
    c.rho_lo = (float)reinterpret_cast<const _Float16*>(norm_lo)[key];
}

// The two 24-bit groups of the lane's hot fields (fields 8 j .. 8 j + 7 in
// group j): lane half 0's 48 bits start at bit 0 of h0, lane half 1's at bit 16.
__device__ __forceinline__ void split_hot_groups(const SplitTileCodes& c, int g, uint32_t& v0, uint32_t& v1) {
    v0 = __builtin_amdgcn_alignbit(c.h1, c.h0, g ? 16u : 0u) & 0xFFFFFFu;
    v1 = (g ? (c.h1 >> 8) : __builtin_amdgcn_alignbit(c.h1, c.h0, 24u)) & 0xFFFFFFu;
}

template <int MT>
__global__ __launch_bounds__(kThreads) void score_split_mfma_kernel(
    const float* __restrict__ A_hi, const float* __restrict__ A_lo,
    const uint8_t* __restrict__ idx_hi, const void* __restrict__ norm_hi,
    const uint8_t* __restrict__ idx_lo, const void* __restrict__ norm_lo,
    const float* __restrict__ cb_hi, int C_hi, const float* __restrict__ cb_lo, int C_lo,
    float* __restrict__ scores, int B, int S) {
    constexpr int D = kSplitDHi + kSplitDLo;
    constexpr int KS = D / 16;                 // 2 hot k-steps, then 6
    constexpr int BLOCK = 64 * 16;
    constexpr int OPS_BYTES = MT * KS * 2 * BLOCK;
    constexpr int SEG = 16;                    // coordinates each prologue lane converts
    constexpr int PER_ROW = D / SEG;           // 2 hot blocks, 6 others
    constexpr int ROWS_PER_PASS = kThreads / PER_ROW;

    __shared__ __attribute__((aligned(16))) uint8_t ops[OPS_BYTES];
    __shared__ float2 rowk[MT * 32];           // per-row epilogue factors (hot, other)

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int p = blockIdx.z;
    const int b0 = blockIdx.y * MT * 32;
    const int rows = min(MT * 32, B - b0);
    const int col = lane & 31;
    const int g = lane >> 5;
    const int ntiles = (S + kTileKeys - 1) / kTileKeys;
    const int64_t key0 = (int64_t)p * S;
    int tile = blockIdx.x * kWaves + wave;
    const int stride = gridDim.x * kWaves;

    SplitTileCodes codes[2];                   // code buffers of the tile loop
    SplitTileCodes& cur = codes[0];
    float sch = 1.f, scl = 1.f;
    uint32_t th_hi[4], th_lo[4], tl_hi[4], tl_lo[4];

    // ---- query operands: lane pl of a row converts hot block pl (pl < 2) or
    //      block pl - 2 of the others, scaled per row and instance by a power of two
    for (int r0 = 0; r0 < MT * 32; r0 += ROWS_PER_PASS) {
        const int row = r0 + tid / PER_ROW;
        const int pl = tid % PER_ROW;
        const bool hot = pl < 2;
        const int rowc = min(row, rows - 1);
        const float* src = hot ? A_hi + ((int64_t)p * B + b0 + rowc) * kSplitDHi + SEG * pl
                               : A_lo + ((int64_t)p * B + b0 + rowc) * kSplitDLo + SEG * (pl - 2);
        float a[SEG];
#pragma unroll
        for (int k = 0; k < SEG; k += 4) {
            const float4 v = *reinterpret_cast<const float4*>(src + k);
            a[k] = v.x; a[k + 1] = v.y; a[k + 2] = v.z; a[k + 3] = v.w;
        }
        if (r0 == 0) {
            asm volatile("" ::: "memory");
            const int s = min(min(tile, ntiles - 1) * kTileKeys + col, S - 1);
            load_split_tile(cur, idx_hi, norm_hi, idx_lo, norm_lo, key0 + s, g);
            asm volatile("" ::: "memory");
            codebook_tables(cb_hi, C_hi, sch, th_hi, th_lo);
            codebook_tables(cb_lo, C_lo, scl, tl_hi, tl_lo);
        }
        if (row >= rows) {
#pragma unroll
            for (int k = 0; k < SEG; ++k) a[k] = 0.f;
        }
        float m = 0.f;
#pragma unroll
        for (int k = 0; k < SEG; ++k) m = fmaxf(m, fabsf(a[k]));
        float mh = hot ? m : 0.f, ml = hot ? 0.f : m;
#pragma unroll
        for (int o = 1; o < PER_ROW; o <<= 1) {
            mh = fmaxf(mh, __shfl_xor(mh, o));
            ml = fmaxf(ml, __shfl_xor(ml, o));
        }
        const float sh = pow2_scale_for(mh);
        const float sl = pow2_scale_for(ml);
        if (row < MT * 32 && pl == 0) rowk[row] = make_float2(inv_scales(sh, sch), inv_scales(sl, scl));
        if (row < MT * 32) {
            const int mtile = row / 32, rl = row % 32;
            const float sr = hot ? sh : sl;
            int gg, blk16;
            if (hot) {
                gg = pl;                                  // hot coordinates 16 pl .. 16 pl + 15
                blk16 = 0;
            } else {
                const int d0 = SEG * (pl - 2);            // other coordinates d0 .. d0 + 15
                gg = d0 / (kSplitDLo / 2);
                blk16 = (d0 % (kSplitDLo / 2)) / SEG;
            }
            // whole 16-byte slots (as prologue_store): the hot block fills slots 0 and 1
            // in coordinate order, an other-instance block slots 2 + 2 blk16 + {0, 1} in
            // the 2-bit order; slot positions swizzled by slot_pos
            uint8_t* tile_base = ops + (mtile * KS * 2) * BLOCK;
            const int pp = gg * 32 + rl;
            uint16_t ah[SEG], al[SEG];
#pragma unroll
            for (int k = 0; k < SEG; ++k) split_f16(a[k] * sr, ah[k], al[k]);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int j = (hot ? 0 : 2 + 2 * blk16) + q;
                uint8_t* base = tile_base + (j * 2) * BLOCK + slot_pos(pp, j) * 16;
                const uint4 vh = hot ? whole_slot<0, 0, true>(ah, q) : whole_slot<1, 2, true>(ah, q);
                const uint4 vl = hot ? whole_slot<0, 0, true>(al, q) : whole_slot<1, 2, true>(al, q);
                *reinterpret_cast<uint4*>(base + 0 * BLOCK) = vh;
                *reinterpret_cast<uint4*>(base + 1 * BLOCK) = vl;
            }
        }
    }
    __syncthreads();

    auto tile_scores = [&](const SplitTileCodes& c, int t) __attribute__((always_inline)) {
        f32x16 accH[MT], accL[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int v = 0; v < 16; ++v) { accH[mt][v] = 0.f; accL[mt][v] = 0.f; }
        }
        uint32_t hv[2];
        split_hot_groups(c, g, hv[0], hv[1]);
        // key-side operands of k-step j (hot table for j < 2)
        auto key_ops = [&](int j, Op8& chi, Op8& clo) __attribute__((always_inline)) {
            uint32_t x0, x1;
            if (j < 2) {
                x0 = sel3x4(hv[j]);
                x1 = sel3x4(hv[j] >> 12);
                lut4(x0, th_hi, chi.u[0], chi.u[1]);
                lut4(x1, th_hi, chi.u[2], chi.u[3]);
                lut4(x0, th_lo, clo.u[0], clo.u[1]);
                lut4(x1, th_lo, clo.u[2], clo.u[3]);
            } else {
                Fmt<1, 2>::selectors<3>(c.lw, j - 2, x0, x1);
                lut4(x0, tl_hi, chi.u[0], chi.u[1]);
                lut4(x1, tl_hi, chi.u[2], chi.u[3]);
                lut4(x0, tl_lo, clo.u[0], clo.u[1]);
                lut4(x1, tl_lo, clo.u[2], clo.u[3]);
            }
        };
        // as in score_mfma_kernel: k-step j + 1's key operands are built while
        // k-step j's LDS reads and MFMAs are in flight
        Op8 chi[2], clo[2];
        key_ops(0, chi[0], clo[0]);
#pragma unroll
        for (int j = 0; j < KS; ++j) {
            const int u = j & 1;
            Op8 ahi[MT], alo[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const uint8_t* base = ops + ((mt * KS + j) * 2) * BLOCK + slot_pos(lane, j) * 16;
                *reinterpret_cast<uint4*>(ahi[mt].u) = *reinterpret_cast<const uint4*>(base + 0 * BLOCK);
                *reinterpret_cast<uint4*>(alo[mt].u) = *reinterpret_cast<const uint4*>(base + 1 * BLOCK);
            }
            if (j + 1 < KS) key_ops(j + 1, chi[u ^ 1], clo[u ^ 1]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                f32x16& acc = j < 2 ? accH[mt] : accL[mt];
                acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[mt].h, chi[u].h, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo[mt].h, chi[u].h, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[mt].h, clo[u].h, acc, 0, 0, 0);
            }
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * MT, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedValu, kValuPerMfma, 0);
#pragma unroll
            for (int i = 0; i < 3 * MT; ++i) {
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
                store_score(out_r, lo + row_offset(v, S),
                            fmaf(k.y * c.rho_lo, accL[mt][v], (k.x * c.rho_hi) * accH[mt][v]));
            }
        }
    };

    if (tile < ntiles) {
        rotate_tiles<2>(
            codes, tile, stride, ntiles,
            [&](SplitTileCodes& c, int t) __attribute__((always_inline)) {
                load_split_tile(c, idx_hi, norm_hi, idx_lo, norm_lo,
                                key0 + min(min(t, ntiles - 1) * kTileKeys + col, S - 1), g);
            },
            tile_scores);
    }
}

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

// ---------------------------------------------------------------------------
// Shared-decode variant (B > 96): the four wavefronts of a workgroup hold four
// different 32-query tiles in registers (as in score_qs_kernel) and walk the
// same key tiles. Each key tile is unpacked once per workgroup: wavefront w
// builds the key-side operands of k-steps [w KS/4, (w+1) KS/4) into one of two
// LDS buffers while the MFMAs of the previous tile read the other, with one
// workgroup barrier per tile. This removes the fourfold key decoding of the
// register variant, whose main loop was bound by vector-ALU issue.
// ---------------------------------------------------------------------------
// Coalesced loading of one wavefront's 32 query rows into the register layout
// in which lane (col, g) holds row col's coordinates [g D/2, (g+1) D/2). Loading
// that half row directly makes each load instruction touch 64 different
// 128-byte lines, one per lane; with every workgroup re-reading all of A and T
// that prologue took about a fifth of the long launch (timeline stamps: operands
// ready ~8 us after the first wave starts). Here each instruction reads whole
// lines of consecutive rows, and a transpose through the wavefront's own LDS
// region hands every lane its half row. Chunk c holds the CW/2 columns from
// c CW/2 on of both halves of all 32 rows; 16-byte slots are XOR-swizzled by row
// so that neither the writes nor the reads conflict on banks.
template <int D, int CW>
struct RowStage {
    static constexpr int HALF = D / 2;
    static constexpr int NSL = CW / 4;            // 16-byte slots per staged row
    static constexpr int NCH = HALF / (CW / 2);   // chunks per matrix
    static constexpr int PER = CW / 8;            // 16-byte loads per lane per chunk
    static constexpr int BYTES = 32 * CW * 4;     // LDS region per wavefront
    static_assert(CW == 32 || CW == 64, "16 or 8 slots per staged row");
    static_assert(HALF % (CW / 2) == 0, "chunks tile each half row");

    // slot of (row r, slot q): rows that one 16-lane LDS pass touches land on
    // distinct 4-bank groups (two rows share the 64 banks when CW = 32)
    __device__ static __forceinline__ int swz(int r, int q) { return q ^ ((r / (16 / NSL)) % NSL); }

    // Requests this lane's part of chunk c of the matrix whose wavefront rows
    // start at `rows`; row r reads row min(r, last) (rows past the end re-read
    // a valid one and are never stored).
    __device__ static __forceinline__ void load(const float* rows, int last, int lane, int c, float (&v)[4 * PER]) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int f = i * 64 + lane;
            const int r = f / NSL, q = f % NSL;
            const int h = q / (NSL / 2), w = q % (NSL / 2);
            const float4 x = *reinterpret_cast<const float4*>(rows + (int64_t)min(r, last) * D + h * HALF + c * (CW / 2) + w * 4);
            v[4 * i] = x.x; v[4 * i + 1] = x.y; v[4 * i + 2] = x.z; v[4 * i + 3] = x.w;
        }
    }

    // Writes chunk c to the wavefront's region and reads back this lane's
    // columns of it into dst[c CW/2 ...]. The region is private to the
    // wavefront, so wavefront-scope ordering suffices; the second fence keeps
    // the next chunk's writes behind this chunk's reads.
    __device__ static __forceinline__ void transpose(uint8_t* region, int lane, int c, const float (&v)[4 * PER],
                                                     float (&dst)[HALF]) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int f = i * 64 + lane;
            const int r = f / NSL, q = f % NSL;
            *reinterpret_cast<float4*>(region + r * CW * 4 + swz(r, q) * 16) =
                make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int col = lane & 31, g = lane >> 5;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const float4 x = *reinterpret_cast<const float4*>(region + col * CW * 4 + swz(col, g * (NSL / 2) + i) * 16);
            dst[c * (CW / 2) + 4 * i] = x.x;
            dst[c * (CW / 2) + 4 * i + 1] = x.y;
            dst[c * (CW / 2) + 4 * i + 2] = x.z;
            dst[c * (CW / 2) + 4 * i + 3] = x.w;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
};

// Per k-step LDS blocks: the codebook's hi part, its lo part unless F16, and
// the signs with QJL.
template <int LAYOUT, int BITS, int D, bool QJL = true, bool F16 = false>
struct SharedLds {
    static constexpr int KS = D / 16;
    static constexpr int BLOCK = 64 * 16;                       // one operand: 64 lanes x 16 bytes
    static constexpr int CLO = 1;                               // block of the codebook lo part (not F16)
    static constexpr int SG = F16 ? 1 : 2;                      // block of the signs (QJL)
    static constexpr int NB = (F16 ? 1 : 2) + (QJL ? 1 : 0);    // operands per k-step
    static constexpr int BUF = KS * NB * BLOCK;
};

template <int LAYOUT, int BITS, int D, int W, bool QJL = true, bool F16 = false>
__device__ __forceinline__ void decode_share(const TileCodes<Fmt<LAYOUT, BITS>::template idx_dw<D>(),
                                                         Fmt<LAYOUT, BITS>::template sign_dw<D>()>& c,
                                             const uint32_t (&tab_hi)[4], const uint32_t (&tab_lo)[4],
                                             uint8_t* buf, int lane) {
    using F = Fmt<LAYOUT, BITS>;
    constexpr int NI = F::template idx_dw<D>(), NS = F::template sign_dw<D>();
    using L = SharedLds<LAYOUT, BITS, D, QJL, F16>;
    constexpr int KS = D / 16, JW = KS / kWaves, BLOCK = L::BLOCK;
#pragma unroll
    for (int jj = 0; jj < JW; ++jj) {
        const int j = W * JW + jj;
        Op8 chi, clo, sg;
        key_operands<LAYOUT, BITS, NI, NS, QJL, !F16>(c, j, tab_hi, tab_lo, chi, clo, sg);
        uint8_t* base = buf + (j * L::NB) * BLOCK + lane * 16;
        *reinterpret_cast<uint4*>(base + 0 * BLOCK) = *reinterpret_cast<const uint4*>(chi.u);
        if constexpr (!F16) *reinterpret_cast<uint4*>(base + L::CLO * BLOCK) = *reinterpret_cast<const uint4*>(clo.u);
        if constexpr (QJL) *reinterpret_cast<uint4*>(base + L::SG * BLOCK) = *reinterpret_cast<const uint4*>(sg.u);
    }
}

// QJL = false: MSE-only keys (no sign stream, no T, gamma = the key's norm).
// F16 = true (with QJL): the single-pass f16 form, two products per k-step
// (A_hi c_hi, T_hi sigma) and no lo halves in registers or LDS.
template <int LAYOUT, int BITS, int D, bool QJL = true, bool F16 = false>
__global__ __launch_bounds__(kThreads, 2) void score_shared_kernel(
    const float* __restrict__ A, const float* __restrict__ T,
    const uint8_t* __restrict__ idx, const uint8_t* __restrict__ sign,
    const void* __restrict__ gamma, const float* __restrict__ codebook, int C,
    float* __restrict__ scores, int B, int S, float coef) {
    using F = Fmt<LAYOUT, BITS>;
    using L = SharedLds<LAYOUT, BITS, D, QJL, F16>;
    constexpr int HALF = D / 2;
    constexpr int KS = D / 16;
    constexpr int NI = F::template idx_dw<D>();
    constexpr int NS = F::template sign_dw<D>();
    constexpr int QT = QJL ? KS : 1;            // T operands kept (none without QJL)
    constexpr int LT = F16 ? 1 : KS;            // lo halves kept (none in the f16 form)
    static_assert(KS % kWaves == 0, "each wavefront unpacks the same number of k-steps");

    __shared__ __attribute__((aligned(16))) uint8_t kops[2 * L::BUF];
    __shared__ float2 rowk[kWaves][32];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int p = blockIdx.z;
    const int b0 = (blockIdx.y * kWaves + wave) * 32;
    const bool has_q = b0 < B;                 // uniform per wavefront; others only unpack keys
    const int rows = has_q ? min(32, B - b0) : 0;
    const int col = lane & 31;
    const int g = lane >> 5;
    const int ntiles = (S + kTileKeys - 1) / kTileKeys;
    const int64_t key0 = (int64_t)p * S;
    int tile = blockIdx.x;                     // uniform per workgroup: every barrier is reached by all
    const int stride = gridDim.x;
    if (tile >= ntiles) return;

    // Query half rows (rows past B re-read row B - 1; wavefronts past B never
    // store). Both LDS buffers serve as the staging area of the coalesced load
    // when they hold a 4 KiB region per wavefront; one barrier then frees them
    // for the first tile.
    constexpr bool STAGED = 2 * L::BUF / kWaves >= RowStage<D, 32>::BYTES;
    using RS = RowStage<D, (2 * L::BUF / kWaves >= RowStage<D, 64>::BYTES) ? 64 : 32>;
    static_assert(!STAGED || kWaves * RS::BYTES <= 2 * L::BUF, "staging regions fit the LDS buffers");
    float a[HALF], t[HALF];
    float va[RS::NCH][4 * RS::PER], vt[RS::NCH][4 * RS::PER];
    const int last = B - 1 - b0;
    if constexpr (STAGED) {
#pragma unroll
        for (int c = 0; c < RS::NCH; ++c) RS::load(A + ((int64_t)p * B + b0) * D, last, lane, c, va[c]);
        if constexpr (QJL) {
#pragma unroll
            for (int c = 0; c < RS::NCH; ++c) RS::load(T + ((int64_t)p * B + b0) * D, last, lane, c, vt[c]);
        }
    } else {
        const int64_t roff = ((int64_t)p * B + min(b0 + col, B - 1)) * D + g * HALF;
#pragma unroll
        for (int k = 0; k < HALF; k += 4) {
            const float4 x = *reinterpret_cast<const float4*>(A + roff + k);
            a[k] = x.x; a[k + 1] = x.y; a[k + 2] = x.z; a[k + 3] = x.w;
            if constexpr (QJL) {
                const float4 y = *reinterpret_cast<const float4*>(T + roff + k);
                t[k] = y.x; t[k + 1] = y.y; t[k + 2] = y.z; t[k + 3] = y.w;
            }
        }
    }
    if constexpr (!QJL) {
#pragma unroll
        for (int k = 0; k < HALF; ++k) t[k] = 0.f;
    }
    TileCodes<NI, NS> c0, c1;
    asm volatile("" ::: "memory");
    load_tile_at<LAYOUT, BITS, D, QJL>(c0, idx, sign, gamma, key0, tile, S, col, g);
    load_tile_at<LAYOUT, BITS, D, QJL>(c1, idx, sign, gamma, key0, tile + stride, S, col, g);
    asm volatile("" ::: "memory");
    float sc;
    uint32_t tab_hi[4], tab_lo[4];
    codebook_tables(codebook, C, sc, tab_hi, tab_lo);
    if constexpr (STAGED) {
        uint8_t* region = kops + wave * RS::BYTES;
#pragma unroll
        for (int c = 0; c < RS::NCH; ++c) RS::transpose(region, lane, c, va[c], a);
        if constexpr (QJL) {
#pragma unroll
            for (int c = 0; c < RS::NCH; ++c) RS::transpose(region, lane, c, vt[c], t);
        }
        __syncthreads();
    }

    float ma = 0.f, mt = 0.f;
#pragma unroll
    for (int k = 0; k < HALF; ++k) {
        ma = fmaxf(ma, fabsf(a[k]));
        mt = fmaxf(mt, fabsf(t[k]));
    }
    ma = fmaxf(ma, __shfl_xor(ma, 32));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float sA = pow2_scale_for(ma);
    const float sT = pow2_scale_for(mt);
    if (g == 0) rowk[wave][col] = make_float2(inv_scales(sA, sc), coef / sT);
    Op8 ahi[KS], alo[LT], thi[QT], tlo[F16 ? 1 : QT];
#pragma unroll
    for (int j = 0; j < KS; ++j) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float xa = a[mse_dim<LAYOUT, BITS>(j, e)] * sA;
            const _Float16 ha = (_Float16)xa;
            ahi[j].h[e] = ha;
            if constexpr (!F16) alo[j].h[e] = (_Float16)(xa - (float)ha);
            if constexpr (QJL) {
                const float xt = t[qjl_dim<LAYOUT>(j, e)] * sT;
                const _Float16 ht = (_Float16)xt;
                thi[j].h[e] = ht;
                if constexpr (!F16) tlo[j].h[e] = (_Float16)(xt - (float)ht);
            }
        }
    }

    auto decode = [&](const TileCodes<NI, NS>& c, uint8_t* buf) __attribute__((always_inline)) {
        switch (wave) {
            case 0: decode_share<LAYOUT, BITS, D, 0, QJL, F16>(c, tab_hi, tab_lo, buf, lane); break;
            case 1: decode_share<LAYOUT, BITS, D, 1, QJL, F16>(c, tab_hi, tab_lo, buf, lane); break;
            case 2: decode_share<LAYOUT, BITS, D, 2, QJL, F16>(c, tab_hi, tab_lo, buf, lane); break;
            default: decode_share<LAYOUT, BITS, D, 3, QJL, F16>(c, tab_hi, tab_lo, buf, lane); break;
        }
    };
    decode(c0, kops);
    __syncthreads();
    // epilogue factors of the 16 rows this lane's accumulators hold, read once
    // (long workload 49.2 -> 48.0 us against an LDS read per row and tile)
    float2 rk[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) rk[v] = rowk[wave][8 * (v >> 2) + 4 * g + (v & 3)];

    // wavefronts past B compute too (no branch around the stores keeps the wait
    // counts exact); their descriptor covers no rows, so every store is dropped
    const __amdgpu_buffer_rsrc_t out_r = score_rows(scores + ((int64_t)p * B + (has_q ? b0 : 0)) * S, rows, S);
    float gam_cur = c0.gam;

    // One tile from LDS buffer `buf`: `cr` is refilled two tiles ahead, this
    // tile's MFMAs are issued, and then the next tile's codes `cn` are unpacked
    // into the other buffer (its gamma kept for the next step), so the wait for
    // those codes comes after this tile's matrix work rather than before it;
    // one barrier ends the step. Past the last tile `cn` holds zeros whose
    // unpacking nobody reads.
    auto step = [&](int t, uint8_t* buf, uint8_t* other, const TileCodes<NI, NS>& cn, TileCodes<NI, NS>& cr)
        __attribute__((always_inline)) {
        load_tile_at<LAYOUT, BITS, D, QJL>(cr, idx, sign, gamma, key0, t + 2 * stride, S, col, g);
        f32x16 accM, accR;
#pragma unroll
        for (int v = 0; v < 16; ++v) { accM[v] = 0.f; accR[v] = 0.f; }
        // key operands of k-step j + 1 are read from LDS while the MFMAs of k-step
        // j run (two register sets in turn), so LDS latency does not stall the chain
        const uint8_t* my = buf + lane * 16;
        Op8 kop[2][3];
        // o[0]: codebook hi, o[1]: codebook lo (not F16), o[2]: signs (QJL)
        auto read_ops = [&](int j, Op8 (&o)[3]) __attribute__((always_inline)) {
            *reinterpret_cast<uint4*>(o[0].u) = *reinterpret_cast<const uint4*>(my + (j * L::NB + 0) * L::BLOCK);
            if constexpr (!F16)
                *reinterpret_cast<uint4*>(o[1].u) =
                    *reinterpret_cast<const uint4*>(my + (j * L::NB + L::CLO) * L::BLOCK);
            if constexpr (QJL)
                *reinterpret_cast<uint4*>(o[2].u) =
                    *reinterpret_cast<const uint4*>(my + (j * L::NB + L::SG) * L::BLOCK);
        };
        read_ops(0, kop[0]);
#pragma unroll
        for (int j = 0; j < KS; ++j) {
            const Op8(&o)[3] = kop[j & 1];
            if (j + 1 < KS) read_ops(j + 1, kop[(j + 1) & 1]);
            accM = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[j].h, o[0].h, accM, 0, 0, 0);
            if constexpr (F16) {
                accR = __builtin_amdgcn_mfma_f32_32x32x16_f16(thi[j].h, o[2].h, accR, 0, 0, 0);
            } else if constexpr (QJL) {
                accR = __builtin_amdgcn_mfma_f32_32x32x16_f16(thi[j].h, o[2].h, accR, 0, 0, 0);
                accM = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo[j].h, o[0].h, accM, 0, 0, 0);
                accR = __builtin_amdgcn_mfma_f32_32x32x16_f16(tlo[j].h, o[2].h, accR, 0, 0, 0);
            } else {
                accM = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo[j].h, o[0].h, accM, 0, 0, 0);
            }
            if constexpr (!F16) accM = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[j].h, o[1].h, accM, 0, 0, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, L::NB, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, F16 ? 2 : QJL ? 5 : 3, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        decode(cn, other);
        const float gam_next = cn.gam;
        const uint32_t lo = lane_offset(t * kTileKeys + col, S, g);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float2 k = rk[v];
            if constexpr (QJL)
                store_score(out_r, lo + row_offset(v, S), fmaf(k.y * gam_cur, accR[v], accM[v] * k.x));
            else
                store_score(out_r, lo + row_offset(v, S), (k.x * gam_cur) * accM[v]);
        }
        gam_cur = gam_next;
        __syncthreads();
    };
    alternate_tiles(tile, stride, ntiles, [&](auto phase, int t) __attribute__((always_inline)) {
        if constexpr (decltype(phase)::value == 0)
            step(t, kops, kops + L::BUF, c1, c0);
        else
            step(t, kops + L::BUF, kops, c0, c1);
    });
}

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

// ---------------------------------------------------------------------------
// host side: shape support and launch
// ---------------------------------------------------------------------------

constexpr int kMaxLdsBytes = 128 * 1024;

// ---------------------------------------------------------------------------
// Outlier split, four queries (B <= 4 over many keys): v_mfma_f32_16x16x32_f16
// with the 16 keys of a tile as columns and, as rows, four queries times four
// operand types: row 4 b + type holds, for query b, the hot instance's A_hi
// (type 0) or A_lo (1) part, or the other instance's A_hi (2) or A_lo (3)
// part, each zero outside its instance's coordinates. Lane group gq = lane / 16
// owns 32 coordinates of its key: group 0 the 32 hot ones (3-bit, the key's
// whole 12-byte row, the 3-bit order of the other kernels), groups 1-3 the
// other instance's 32 (gq - 1) .. 32 gq - 1 (2-bit, 8 bytes, the 2-bit order),
// each against its own instance's codebook. Two MFMAs per k-step: the
// codebook's hi parts, then its lo parts, against the same rows (the lo rows
// then add the A_lo c_lo term too). Lane 16 b + key ends with the four types of
// (query b, key): rho_hi (t0 + t1) and rho_lo (t2 + t3) scaled back.
// ---------------------------------------------------------------------------
template <int MINW>
__global__ __launch_bounds__(kThreads, MINW) void score_split16_kernel(
    const float* __restrict__ A_hi, const float* __restrict__ A_lo,
    const uint8_t* __restrict__ idx_hi, const void* __restrict__ norm_hi,
    const uint8_t* __restrict__ idx_lo, const void* __restrict__ norm_lo,
    const float* __restrict__ cb_hi, int C_hi, const float* __restrict__ cb_lo, int C_lo,
    float* __restrict__ scores, int B, int S) {
    constexpr int Q = 32;                          // coordinates per lane
    constexpr int NJ = Q / 8;                      // k-steps
    struct Codes {
        uint32_t w[3];                             // hot row (group 0) or 8 bytes of the other row
        float rho_hi, rho_lo;
    };
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int p = blockIdx.z;
    const int b0 = blockIdx.y * 4;
    const int nb = min(4, B - b0);
    const int ntiles = (S + kTileKeys16 - 1) / kTileKeys16;
    int tile = blockIdx.x * kWaves + wave;
    const int stride = gridDim.x * kWaves;
    if (tile >= ntiles) return;                    // no barrier in this kernel
    const int gq = lane >> 4;
    const int kc = lane & 15;
    const int r = lane & 15;
    const int rb = r >> 2, rtype = r & 3;
    const bool hot = gq == 0;
    const int64_t key0 = (int64_t)p * S;

    // Branch-free: every lane reads three dwords; in groups 1-3 the third read
    // repeats the first address (in bounds, unused).
    auto load = [&](Codes& c, int64_t key) __attribute__((always_inline)) {
        const uint32_t* a01 = reinterpret_cast<const uint32_t*>(hot ? idx_hi + key * 12
                                                                    : idx_lo + key * 24 + 8 * (gq - 1));
        const uint32_t* a2 = hot ? a01 + 2 : a01;
        c.w[0] = a01[0];
        c.w[1] = a01[1];
        c.w[2] = a2[0];
        c.rho_hi = (float)reinterpret_cast<const _Float16*>(norm_hi)[key];
        c.rho_lo = (float)reinterpret_cast<const _Float16*>(norm_lo)[key];
    };

    // this lane's 32 query coordinates (query rb, clamped: queries past B are
    // computed but never stored)
    const int qb = b0 + min(rb, nb - 1);
    const float* src = hot ? A_hi + ((int64_t)p * B + qb) * kSplitDHi
                           : A_lo + ((int64_t)p * B + qb) * kSplitDLo + Q * (gq - 1);
    float x[Q];
#pragma unroll
    for (int k = 0; k < Q; k += 4) {
        const float4 v = *reinterpret_cast<const float4*>(src + k);
        x[k] = v.x; x[k + 1] = v.y; x[k + 2] = v.z; x[k + 3] = v.w;
    }
    Codes codes[3];                            // code buffers of the tile loop
    Codes& cur = codes[0];
    asm volatile("" ::: "memory");
    load(cur, key0 + min(tile * kTileKeys16 + kc, S - 1));
    asm volatile("" ::: "memory");
    float sch, scl;
    uint32_t th_hi[4], th_lo[4], tl_hi[4], tl_lo[4];
    codebook_tables(cb_hi, C_hi, sch, th_hi, th_lo);
    codebook_tables(cb_lo, C_lo, scl, tl_hi, tl_lo);
    uint32_t tab_hi[4], tab_lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        tab_hi[i] = hot ? th_hi[i] : tl_hi[i];
        tab_lo[i] = hot ? th_lo[i] : tl_lo[i];
    }

    // per-query, per-instance scales: maxima over lane group 0 (hot) and groups 1-3
    float m = 0.f;
#pragma unroll
    for (int k = 0; k < Q; ++k) m = fmaxf(m, fabsf(x[k]));
    float mh = hot ? m : 0.f, ml = hot ? 0.f : m;
    mh = fmaxf(mh, __shfl_xor(mh, 16));
    mh = fmaxf(mh, __shfl_xor(mh, 32));
    ml = fmaxf(ml, __shfl_xor(ml, 16));
    ml = fmaxf(ml, __shfl_xor(ml, 32));
    const float sh = pow2_scale_for(mh);
    const float sl = pow2_scale_for(ml);
    const float s_own = hot ? sh : sl;
    // epilogue factors of output query gq (held by every lane with r = 4 gq)
    const float kh = 1.f / (__shfl(sh, 4 * gq) * sch);
    const float kl = 1.f / (__shfl(sl, 4 * gq) * scl);

    // row operands: types 0/1 carry the hot coordinates (group 0 only), 2/3 the others
    const bool live_hi = hot && rtype < 2, live_lo = !hot && rtype >= 2;
    const bool part_lo = (rtype & 1) != 0;
    Op8 ops[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float xv = (hot ? x[mse_dim<1, 3>(j, e)] : x[mse_dim<1, 2>(j, e)]) * s_own;
            const _Float16 h = (_Float16)xv;
            const _Float16 l = (_Float16)(xv - (float)h);
            ops[j].h[e] = (live_hi || live_lo) ? (part_lo ? l : h) : (_Float16)0.f;
        }
    }

    const __amdgpu_buffer_rsrc_t out_r = score_rows(scores + ((int64_t)p * B + b0) * S, nb, S);

    auto tile_scores = [&](const Codes& c, int t) __attribute__((always_inline)) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            uint32_t h0, h1, l0, l1;
            Fmt<1, 3>::selectors<3>(c.w, j, h0, h1);
            Fmt<1, 2>::selectors<3>(c.w, j, l0, l1);
            const uint32_t x0 = hot ? h0 : l0, x1 = hot ? h1 : l1;
            Op8 kh8, kl8;
            lut4(x0, tab_hi, kh8.u[0], kh8.u[1]);
            lut4(x1, tab_hi, kh8.u[2], kh8.u[3]);
            lut4(x0, tab_lo, kl8.u[0], kl8.u[1]);
            lut4(x1, tab_lo, kl8.u[2], kl8.u[3]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ops[j].h, kh8.h, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ops[j].h, kl8.h, acc, 0, 0, 0);
        }
        const int s = t * kTileKeys16 + kc;
        const uint32_t off = s < S ? ((uint32_t)gq * (uint32_t)S + (uint32_t)s) * 4u : kDropKey;
        store_score(out_r, off, fmaf(kl * c.rho_lo, acc[2] + acc[3], (kh * c.rho_hi) * (acc[0] + acc[1])));
    };

    // three code buffers in turn: each tile's codes are requested two tiles ahead
    auto load_tile_codes = [&](Codes& c, int t) __attribute__((always_inline)) {
        load(c, key0 + min(min(t, ntiles - 1) * kTileKeys16 + kc, S - 1));
    };
    load_tile_codes(codes[1], tile + stride);
    rotate_tiles<3>(codes, tile, stride, ntiles, load_tile_codes, tile_scores);
}

// ---------------------------------------------------------------------------
// Fused decode step: scores, online softmax and value aggregation in one pass,
// so no score reaches HBM ("Fitting 4.4x More Context on Jetson", section "v6:
// Fused Vectorized Hybrid" and its online-softmax FAQ; "TurboQuant:
// Rotate-then-Quantize KV Caches at 3 Bits", section 8, kernel view). One
// workgroup of four wavefronts per (key chunk, 32-query tile, problem); each
// wavefront takes every fourth 32-key tile of the chunk.
//
// Scores come from the same split-f16 products as score_mfma_kernel (query
// operands staged once per workgroup in LDS) with the operands swapped, so the
// accumulators hold keys as rows and queries as columns: lane (query n, half g)
// holds the scores of keys 8(v/4) + 4g + (v%4), v = 0..15, for query n. That is
// the layout the value product wants: with keys as the contraction, lane
// (n, g) supplies its 16 keys' weights in two 16-key steps (slot e of step s is
// its key v = 8s + e), and the value operand of lane (coordinate row, g) takes
// the same keys in the same slots. The online softmax, the norm scaling and the
// split-f16 value products follow attend_partial_kernel's wide mode (value
// coordinates NT*n + t of tile t in lane n). gamma and the value norms of a
// tile's keys are regrouped from the lanes that loaded them through a small
// per-wavefront LDS slot. The workgroup merges its four wavefronts and writes
// (m, l, acc) per query into the attend workspace layout; the attend combine
// kernel finishes.
// ---------------------------------------------------------------------------
constexpr float kFusedTau = 5.5f;   // rescale when a tile's maximum passes the reference by more
constexpr int kFusedNormBits = 4;   // scaled value norms stay below 2^(kFusedNormBits + 2)

template <int LAYOUT, int BITS, int D, int VLAYOUT, int VBITS>
__global__ __launch_bounds__(kThreads) void score_attend_kernel(
    const float* __restrict__ A, const float* __restrict__ T,
    const uint8_t* __restrict__ idx, const uint8_t* __restrict__ sign,
    const void* __restrict__ gamma, const float* __restrict__ codebook, int C,
    const uint8_t* __restrict__ vidx, const void* __restrict__ vnorm,
    const float* __restrict__ vcodebook, int VC, float scale, float* __restrict__ ws,
    int B, int S, int chunk, int nch, float coef) {
    using F = Fmt<LAYOUT, BITS>;
    constexpr int HALF = D / 2;
    constexpr int KS = D / 16;
    constexpr int NI = F::template idx_dw<D>();
    constexpr int NS = F::template sign_dw<D>();
    constexpr int BLOCK = 64 * 16;
    constexpr int OPS_BYTES = KS * 4 * BLOCK;
    constexpr int SEG = 16;
    constexpr int PER_ROW = D / SEG;
    constexpr int ROWS_PER_PASS = kThreads / PER_ROW;
    constexpr int NT = D / 32;                     // value coordinates per lane = tiles of the value product
    constexpr int VBW = VLAYOUT == 0 ? 8 : VBITS;  // value index bits per coordinate
    constexpr int VW = NT * VBW;                   // value bits per lane per key
    constexpr int VROWB = D * VBW / 8;             // bytes per value row
    constexpr int VCROSS = VW > 32 ? 2 : (32 % VW == 0 ? 0 : 1);
    constexpr int DP = D + 1;
    constexpr int MERGE_BYTES = kWaves * 32 * DP * 4;
    constexpr int LDS_BYTES = OPS_BYTES > MERGE_BYTES ? OPS_BYTES : MERGE_BYTES;
    static_assert(HALF % SEG == 0 && VW <= 64 && VROWB % 4 == 0, "fused tiling");

    // the query operands, then (after a barrier) the wavefronts' partial sums
    __shared__ __attribute__((aligned(16))) uint8_t lds_raw[LDS_BYTES];
    __shared__ float2 rowk[32];
    __shared__ __attribute__((aligned(16))) float kv[kWaves][2][32];   // gamma, value norm per tile key
    __shared__ float red_m[kWaves][32];
    __shared__ float red_l[kWaves][32];
    uint8_t* ops = lds_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int p = blockIdx.z;
    const int b0 = blockIdx.y * 32;
    const int rows = min(32, B - b0);
    const int c = blockIdx.x;
    const int col = lane & 31;
    const int g = lane >> 5;
    const int s_begin = c * chunk;
    const int s_end = min(S, s_begin + chunk);
    const int ntl = (s_end - s_begin + kTileKeys - 1) / kTileKeys;   // tiles in this chunk
    const int64_t key0 = (int64_t)p * S;
    const bool qvalid = col < rows;

    float sc = 1.f;
    uint32_t tab_hi[4] = {0u, 0u, 0u, 0u}, tab_lo[4] = {0u, 0u, 0u, 0u};
    TileCodes<NI, NS> codes[2];                  // key code buffers of the tile loop
    TileCodes<NI, NS>& cur = codes[0];
    int tl = wave;                                 // this wavefront's tiles: wave, wave + 4, ...
    auto tile_key = [&](int t) { return min(s_begin + min(t, ntl - 1) * kTileKeys + col, S - 1); };

    // ---- query operands into LDS (as score_mfma_kernel with one query tile)
    const float* Ap = A + ((int64_t)p * B + b0) * D;
    const float* Tp = T + ((int64_t)p * B + b0) * D;
    for (int r0 = 0; r0 < 32; r0 += ROWS_PER_PASS) {
        const int row = r0 + tid / PER_ROW;
        const int pl = tid % PER_ROW;
        float a[SEG], t[SEG];
        float ma = 0.f, mt = 0.f;
        const int rowc = min(row, rows - 1);
#pragma unroll
        for (int k = 0; k < SEG; k += 4) {
            const float4 va = *reinterpret_cast<const float4*>(Ap + (int64_t)rowc * D + pl * SEG + k);
            const float4 vt = *reinterpret_cast<const float4*>(Tp + (int64_t)rowc * D + pl * SEG + k);
            a[k] = va.x; a[k + 1] = va.y; a[k + 2] = va.z; a[k + 3] = va.w;
            t[k] = vt.x; t[k + 1] = vt.y; t[k + 2] = vt.z; t[k + 3] = vt.w;
        }
        if (r0 == 0) {
            asm volatile("" ::: "memory");
            load_tile<LAYOUT, BITS, D>(cur, idx, sign, gamma, key0 + tile_key(tl), g);
            asm volatile("" ::: "memory");
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
        if (row < 32 && pl == 0) rowk[row] = make_float2(inv_scales(sA, sc), coef / sT);
        {
            const int d0 = pl * SEG;
            const int gg = d0 / HALF;
            const int blk16 = (d0 % HALF) / SEG;
            prologue_store<LAYOUT, BITS, true, SEG>(ops, gg * 32 + row, blk16, a, t, sA, sT, row < 32);
        }
    }

    // value codebook tables (f16 hi and lo parts times a power of two)
    float vsc;
    uint32_t vtab_hi[4], vtab_lo[4];
    codebook_tables(vcodebook, VC, vsc, vtab_hi, vtab_lo);
    // value bits of coordinates NT*col .. NT*col+NT-1: dword k0 of the row, and
    // the next one when the field runs into it
    const int vbit = VBW * NT * col;
    const int vk0 = vbit >> 5;
    const int vsh = vbit & 31;
    const bool vtwo = VCROSS == 2 || (VCROSS == 1 && vsh + VW > 32);
    const uint8_t* vbase = vidx + key0 * VROWB + 4 * vk0;
    __syncthreads();
    const float2 kq = rowk[col];     // this lane's query's factors (M, R)

    // raw value loads of a tile: this lane's 16 keys 8(v/4) + 4g + (v%4)
    struct VRaw {
        uint32_t lo[16], hi[16];
        uint32_t nrm;                  // value norm bits of this lane's own key (col)
    };
    auto vkey = [&](int t, int v) {
        return min(s_begin + min(t, ntl - 1) * kTileKeys + 8 * (v >> 2) + 4 * g + (v & 3), S - 1);
    };
    auto load_values = [&](VRaw& r, int t) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const uint32_t* w = reinterpret_cast<const uint32_t*>(vbase + (int64_t)vkey(t, v) * VROWB);
            r.lo[v] = w[0];
            r.hi[v] = w[vtwo ? 1 : 0];
        }
        if constexpr (VLAYOUT == 0) r.nrm = reinterpret_cast<const uint32_t*>(vnorm)[key0 + tile_key(t)];
        else r.nrm = reinterpret_cast<const uint16_t*>(vnorm)[key0 + tile_key(t)];
    };

    f32x16 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[t][v] = 0.f;
    float M = -INFINITY;       // reference maximum of scale*score for query col
    float lsum = 0.f;          // sum of exp(scale*score - M) over this lane's keys
    float nexp = -1000.f;      // value norms are scaled by 2^-nexp ...
    float nlim = 0.f;          // ... and must stay below nlim

    auto tile_attend = [&](const TileCodes<NI, NS>& cd, const VRaw& vr, int t) __attribute__((always_inline)) {
        // ---- scores, keys as rows
        f32x16 accM, accR;
#pragma unroll
        for (int v = 0; v < 16; ++v) { accM[v] = 0.f; accR[v] = 0.f; }
        Op8 chi[2], clo[2], sg[2];
        key_operands<LAYOUT, BITS, NI, NS>(cd, 0, tab_hi, tab_lo, chi[0], clo[0], sg[0]);
#pragma unroll
        for (int j = 0; j < KS; ++j) {
            const int u = j & 1;
            Op8 ahi, alo, thi, tlo;
            const uint8_t* base = ops + (j * 4) * BLOCK + slot_pos(lane, j) * 16;
            *reinterpret_cast<uint4*>(ahi.u) = *reinterpret_cast<const uint4*>(base + 0 * BLOCK);
            *reinterpret_cast<uint4*>(alo.u) = *reinterpret_cast<const uint4*>(base + 1 * BLOCK);
            *reinterpret_cast<uint4*>(thi.u) = *reinterpret_cast<const uint4*>(base + 2 * BLOCK);
            *reinterpret_cast<uint4*>(tlo.u) = *reinterpret_cast<const uint4*>(base + 3 * BLOCK);
            if (j + 1 < KS) key_operands<LAYOUT, BITS, NI, NS>(cd, j + 1, tab_hi, tab_lo, chi[u ^ 1], clo[u ^ 1], sg[u ^ 1]);
            accM = __builtin_amdgcn_mfma_f32_32x32x16_f16(chi[u].h, ahi.h, accM, 0, 0, 0);
            accR = __builtin_amdgcn_mfma_f32_32x32x16_f16(sg[u].h, thi.h, accR, 0, 0, 0);
            accM = __builtin_amdgcn_mfma_f32_32x32x16_f16(chi[u].h, alo.h, accM, 0, 0, 0);
            accR = __builtin_amdgcn_mfma_f32_32x32x16_f16(sg[u].h, tlo.h, accR, 0, 0, 0);
            accM = __builtin_amdgcn_mfma_f32_32x32x16_f16(clo[u].h, ahi.h, accM, 0, 0, 0);
        }
        // ---- gamma and value norm of the keys this lane holds, regrouped
        if (g == 0) {
            kv[wave][0][col] = cd.gam;
            kv[wave][1][col] = VLAYOUT == 0 ? __builtin_bit_cast(float, vr.nrm)
                                            : (float)__builtin_bit_cast(_Float16, (uint16_t)vr.nrm);
        }
        __builtin_amdgcn_wave_barrier();
        float gm[16], vn[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const float4 a4 = *reinterpret_cast<const float4*>(&kv[wave][0][8 * q4 + 4 * g]);
            const float4 b4 = *reinterpret_cast<const float4*>(&kv[wave][1][8 * q4 + 4 * g]);
            gm[4 * q4 + 0] = a4.x; gm[4 * q4 + 1] = a4.y; gm[4 * q4 + 2] = a4.z; gm[4 * q4 + 3] = a4.w;
            vn[4 * q4 + 0] = b4.x; vn[4 * q4 + 1] = b4.y; vn[4 * q4 + 2] = b4.z; vn[4 * q4 + 3] = b4.w;
        }
        __builtin_amdgcn_wave_barrier();
        // ---- online softmax over this tile's keys for query col
        const int ts = s_begin + t * kTileKeys;
        float z[16];
        float ms = -INFINITY, nm = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int key = ts + 8 * (v >> 2) + 4 * g + (v & 3);
            const float sco = fmaf(kq.y * gm[v], accR[v], accM[v] * kq.x);
            z[v] = (qvalid && key < s_end) ? scale * sco : -INFINITY;
            ms = fmaxf(ms, z[v]);
            nm = fmaxf(nm, fabsf(vn[v]));
        }
        ms = fmaxf(ms, __shfl_xor(ms, 32));
        const bool need_m = ms > M + kFusedTau;
        if (__any(need_m || nm >= nlim)) {
            float nw = nm;
#pragma unroll
            for (int m = 1; m < 64; m <<= 1) nw = fmaxf(nw, __shfl_xor(nw, m));
            float fac = 1.f;
            if (nw >= nlim) {
                int e2;
                (void)frexpf(nw, &e2);
                const float ne = nw > 0.f ? (float)(e2 - kFusedNormBits) : 0.f;
                fac = exp2f(nexp - ne);
                nexp = ne;
                nlim = exp2f(ne + kFusedNormBits + 2);
            }
            const float Mn = need_m ? ms : M;
            const float fm = need_m ? __expf(M - Mn) : 1.f;
            M = Mn;
            lsum *= fm;
            fac *= fm;
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[tt][v] *= fac;
        }
        const float nscale = exp2f(-nexp);
        Op8 whi[2], wlo[2];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float w = z[v] == -INFINITY ? 0.f : __expf(z[v] - M);
            lsum += w;
            const float x = w * vn[v] * nscale;
            const _Float16 h = (_Float16)x;
            whi[v >> 3].h[v & 7] = h;
            wlo[v >> 3].h[v & 7] = (_Float16)(x - (float)h);
        }
        // ---- value products: step st takes keys v = 8 st + e in slot e
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            uint64_t vb[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int v = 8 * st + e;
                vb[e] = ((vtwo ? (uint64_t)vr.hi[v] << 32 : 0ull) | vr.lo[v]) >> vsh;
            }
            // packed fields (VW <= 32 bits per key): selectors from byte-transposed bits
            constexpr bool BYTES = VLAYOUT == 1 && VW <= 32;
            using VS = typename std::conditional<BYTES, ValueSelectors<VBW, VW>, NoValueSelectors>::type;
            const VS vs(vb);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                uint32_t sel0 = 0, sel1 = 0;
                if constexpr (BYTES) {
                    vs.tile(tt, sel0, sel1);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        sel0 |= ((uint32_t)(vb[e] >> (VBW * tt)) & ((1u << VBW) - 1u)) << (8 * e);
                        sel1 |= ((uint32_t)(vb[4 + e] >> (VBW * tt)) & ((1u << VBW) - 1u)) << (8 * e);
                    }
                }
                Op8 vhi, vlo;
                lut4(sel0, vtab_hi, vhi.u[0], vhi.u[1]);
                lut4(sel1, vtab_hi, vhi.u[2], vhi.u[3]);
                lut4(sel0, vtab_lo, vlo.u[0], vlo.u[1]);
                lut4(sel1, vtab_lo, vlo.u[2], vlo.u[3]);
                acc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vhi.h, whi[st].h, acc[tt], 0, 0, 0);
                acc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vlo.h, whi[st].h, acc[tt], 0, 0, 0);
                acc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vhi.h, wlo[st].h, acc[tt], 0, 0, 0);
            }
        }
    };

    if (tl < ntl) {
        VRaw vals[2];                                // the raw values travel with the key codes
        load_values(vals[0], tl);
        rotate_tiles<2>(
            tl, kWaves, ntl,
            [&](auto ph, int t) __attribute__((always_inline)) {
                load_tile<LAYOUT, BITS, D>(codes[decltype(ph)::value], idx, sign, gamma, key0 + tile_key(t), g);
                load_values(vals[decltype(ph)::value], t);
            },
            [&](auto ph, int t) __attribute__((always_inline)) {
                tile_attend(codes[decltype(ph)::value], vals[decltype(ph)::value], t);
            });
    }

    // ---- this wavefront's (m, l, acc) to LDS (true scale), then merge the four
    lsum += __shfl_xor(lsum, 32);
    const float unscale = exp2f(nexp) / vsc;
    __syncthreads();                                   // every wavefront is done with the query operands
    float* red_acc = reinterpret_cast<float*>(lds_raw);   // [kWaves][32][DP]
    if (g == 0) {
        red_m[wave][col] = M;
        red_l[wave][col] = lsum;
    }
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int row = 8 * (v >> 2) + 4 * g + (v & 3);
            red_acc[(wave * 32 + col) * DP + NT * row + tt] = acc[tt][v] * unscale;
        }
    __syncthreads();
    for (int i = tid; i < 32 * D; i += kThreads) {
        const int d = i % D;
        const int qi = i / D;
        if (qi >= rows) continue;
        float Mx = -INFINITY;
#pragma unroll
        for (int k = 0; k < kWaves; ++k) Mx = fmaxf(Mx, red_m[k][qi]);
        float a = 0.f, l = 0.f;
#pragma unroll
        for (int k = 0; k < kWaves; ++k) {
            const float f = red_m[k][qi] == -INFINITY ? 0.f : __expf(red_m[k][qi] - Mx);
            a = fmaf(red_acc[(k * 32 + qi) * DP + d], f, a);
            l = fmaf(red_l[k][qi], f, l);
        }
        float* rec = ws + (((int64_t)p * B + b0 + qi) * nch + c) * (D + 2);
        rec[2 + d] = a;
        if (d == 0) {
            rec[0] = Mx;
            rec[1] = l;
        }
    }
}

int mt_for(int B, int D) {
    const int tiles = (B + 31) / 32;
    const int per_tile = (D / 16) * 4 * 1024;        // LDS bytes per 32-query tile
    int cap = kMaxLdsBytes / per_tile;
    if (cap > 4) cap = 4;
    if (cap < 1) cap = 1;
    if (tiles >= 4 && cap >= 4) return 4;
    if (tiles >= 2 && cap >= 2) return 2;
    return 1;
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

// Shared-decode launch: workgroup rows are groups of four 32-query tiles; two
// workgroups per CU are resident (registers), so 512 workgroups fill the chip.
template <int LAYOUT, int BITS, int D, bool QJL = true, bool F16 = false>
hipError_t launch_shared_d(const float* A, const float* T, KeyStreams k, const float* codebook, int C,
                           float* scores, int P, int B, int S, hipStream_t stream) {
    const int groups_y = (B + 127) / 128;
    const int ntiles = (S + kTileKeys - 1) / kTileKeys;
    int64_t gx = ntiles;
    int64_t cap = 512 / ((int64_t)groups_y * P);
    if (cap < 1) cap = 1;
    if (gx > cap) gx = cap;
    const float coef = (float)(kSqrtHalfPi / (double)D);
    hipLaunchKernelGGL((score_shared_kernel<LAYOUT, BITS, D, QJL, F16>), dim3((unsigned)gx, groups_y, P),
                       dim3(kThreads), 0, stream, A, T, k.idx, k.sign, k.gamma, codebook, C,
                       scores, B, S, coef);
    return hipGetLastError();
}

template <int LAYOUT, int BITS, bool QJL = true, bool F16 = false>
hipError_t launch_shared_layout(const float* A, const float* T, KeyStreams k, const float* codebook,
                                int C, float* scores, int P, int B, int S, int D, hipStream_t stream) {
    if (D == 64) return launch_shared_d<LAYOUT, BITS, 64, QJL, F16>(A, T, k, codebook, C, scores, P, B, S, stream);
    if (D == 128) return launch_shared_d<LAYOUT, BITS, 128, QJL, F16>(A, T, k, codebook, C, scores, P, B, S, stream);
    return hipErrorInvalidValue;
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

namespace {

bool lds_supported(int layout, int bits, int C, int D) {
    if (C < 1 || C > 8) return false;          // byte-select lookup tables hold 8 entries
    if (layout == 0) return D == 32 || D == 64 || D == 128 || D == 256;
    if (bits != 2 && bits != 3) return false;
    return D == 64 || D == 128 || D == 256;
}

bool reg_supported(int layout, int bits, int C, int D) {
    return lds_supported(layout, bits, C, D) && D <= 128;   // D = 256 would need 256 operand registers
}

bool shared_supported(int layout, int bits, int C, int D) {
    return lds_supported(layout, bits, C, D) && (D == 64 || D == 128);   // k-steps split over 4 wavefronts
}

bool small_supported(int layout, int bits, int C, int D) {
    return lds_supported(layout, bits, C, D) && (D == 128 || D == 256);   // a lane owns D/4 >= 32 coordinates
}

// Automatic choice, from measurements on the five workload shapes: with a single
// 32-query tile (B <= 32) the workgroup-shared LDS staging wins (its one-time
// operand build is split over 256 threads); with more query tiles the
// register-resident operands win (no LDS traffic in the main loop).
int pick_variant(int layout, int bits, int C, int B, int64_t keys, int D) {
    // One group of four queries: 12 16x16 MFMAs per 16 keys against 40 32x32
    // ones per 32 keys padded. Each wavefront builds its own query operands, so
    // this pays once wavefronts see many tiles (measured: GQA's 4.2 M keys run
    // 1.6x faster, one problem of 32 K keys runs slower). With two groups of
    // four the key decoding doubles and the padded 32x32 tile measured faster.
    if (B <= 4 && keys >= (int64_t(1) << 20) && small_supported(layout, bits, C, D)) return kMfmaSmall;
    // Four or more query tiles: the shared-decode variant unpacks each key tile
    // once for all four (long workload 51.3 -> 48.3 us against the register
    // variant); with three, one of its four wavefronts would idle.
    if (B > 96 && shared_supported(layout, bits, C, D)) return kMfmaShared;
    if (B > 32 && reg_supported(layout, bits, C, D)) return kMfmaReg;
    return kMfmaLds;
}

}  // namespace

namespace {

// The single-pass f16 form takes the automatic choice's family, with the
// LDS-staged kernel where that choice is the register-resident one.
int pick_f16_variant(int layout, int bits, int C, int B, int64_t keys, int D) {
    const int v = pick_variant(layout, bits, C, B, keys, D);
    return v == kMfmaReg ? kMfmaLds : v;
}

// The name of a kernel's single-pass f16 form (static strings).
const char* with_f16_suffix(const char* base) {
    if (!base) return nullptr;
    static const char* const names[][2] = {
        {"mfma32_unpacked_mt1", "mfma32_unpacked_mt1_f16"}, {"mfma32_unpacked_mt2", "mfma32_unpacked_mt2_f16"},
        {"mfma32_unpacked_mt4", "mfma32_unpacked_mt4_f16"}, {"mfma32_packed2_mt1", "mfma32_packed2_mt1_f16"},
        {"mfma32_packed2_mt2", "mfma32_packed2_mt2_f16"}, {"mfma32_packed2_mt4", "mfma32_packed2_mt4_f16"},
        {"mfma32_packed3_mt1", "mfma32_packed3_mt1_f16"}, {"mfma32_packed3_mt2", "mfma32_packed3_mt2_f16"},
        {"mfma32_packed3_mt4", "mfma32_packed3_mt4_f16"}, {"mfma16_unpacked", "mfma16_unpacked_f16"},
        {"mfma16i8_packed2", "mfma16_packed2_f16"}, {"mfma16i8_packed3", "mfma16_packed3_f16"},
        {"mfma32shared_unpacked", "mfma32shared_unpacked_f16"}, {"mfma32shared_packed2", "mfma32shared_packed2_f16"},
        {"mfma32shared_packed3", "mfma32shared_packed3_f16"},
    };
    for (const auto& n : names)
        if (__builtin_strcmp(n[0], base) == 0) return n[1];
    return nullptr;
}
}  // namespace

bool score_mfma_supported(int layout, int bits, int C, int B, int D, int variant) {
    (void)B;
    if (variant == kMfmaAuto || variant == kMfmaF16) return lds_supported(layout, bits, C, D);
    if (variant == kMfmaLds) return lds_supported(layout, bits, C, D);
    if (variant == kMfmaReg) return reg_supported(layout, bits, C, D);
    if (variant == kMfmaSmall) return small_supported(layout, bits, C, D);
    if (variant == kMfmaShared) return shared_supported(layout, bits, C, D);
    return false;
}

const char* score_mfma_name(int layout, int bits, int C, int P, int B, int S, int D, int variant) {
    if (!score_mfma_supported(layout, bits, C, B, D, variant)) return nullptr;
    if (variant == kMfmaF16)
        return with_f16_suffix(score_mfma_name(layout, bits, C, P, B, S, D,
                                               pick_f16_variant(layout, bits, C, B, (int64_t)P * S, D)));
    if (variant == kMfmaAuto) variant = pick_variant(layout, bits, C, B, (int64_t)P * S, D);
    if (variant == kMfmaReg) return layout == 0 ? "mfma32reg_unpacked" : bits == 2 ? "mfma32reg_packed2" : "mfma32reg_packed3";
    if (variant == kMfmaSmall) return layout == 0 ? "mfma16_unpacked" : bits == 2 ? "mfma16i8_packed2" : "mfma16i8_packed3";
    if (variant == kMfmaShared) return layout == 0 ? "mfma32shared_unpacked" : bits == 2 ? "mfma32shared_packed2" : "mfma32shared_packed3";
    const int mt = mt_for(B, D);
    if (layout == 0) return mt == 4 ? "mfma32_unpacked_mt4" : mt == 2 ? "mfma32_unpacked_mt2" : "mfma32_unpacked_mt1";
    if (bits == 2) return mt == 4 ? "mfma32_packed2_mt4" : mt == 2 ? "mfma32_packed2_mt2" : "mfma32_packed2_mt1";
    return mt == 4 ? "mfma32_packed3_mt4" : mt == 2 ? "mfma32_packed3_mt2" : "mfma32_packed3_mt1";
}

hipError_t launch_score_mfma(const float* A, const float* T, KeyStreams keys,
                             int layout, int bits, const float* codebook, int C,
                             float* scores, int P, int B, int S, int D, int variant,
                             hipStream_t stream) {
    if (!score_mfma_supported(layout, bits, C, B, D, variant)) return hipErrorInvalidValue;
    if (variant == kMfmaF16) {
        const int v = pick_f16_variant(layout, bits, C, B, (int64_t)P * S, D);
        if (v == kMfmaShared) {
            if (layout == 0) return launch_shared_layout<0, 0, true, true>(A, T, keys, codebook, C, scores, P, B, S, D, stream);
            if (bits == 2) return launch_shared_layout<1, 2, true, true>(A, T, keys, codebook, C, scores, P, B, S, D, stream);
            return launch_shared_layout<1, 3, true, true>(A, T, keys, codebook, C, scores, P, B, S, D, stream);
        }
        if (v == kMfmaSmall) {
            if (layout == 0) return launch_small_layout<0, 0, true, true>(A, T, keys, codebook, C, scores, P, B, S, D, stream);
            if (bits == 2) return launch_small_layout<1, 2, true, true>(A, T, keys, codebook, C, scores, P, B, S, D, stream);
            return launch_small_layout<1, 3, true, true>(A, T, keys, codebook, C, scores, P, B, S, D, stream);
        }
        if (layout == 0) return launch_layout<0, 0, true, true>(A, T, keys, codebook, C, scores, P, B, S, D, stream);
        if (bits == 2) return launch_layout<1, 2, true, true>(A, T, keys, codebook, C, scores, P, B, S, D, stream);
        return launch_layout<1, 3, true, true>(A, T, keys, codebook, C, scores, P, B, S, D, stream);
    }
    if (variant == kMfmaAuto) variant = pick_variant(layout, bits, C, B, (int64_t)P * S, D);
    if (variant == kMfmaShared) {
        if (layout == 0) return launch_shared_layout<0, 0>(A, T, keys, codebook, C, scores, P, B, S, D, stream);
        if (bits == 2) return launch_shared_layout<1, 2>(A, T, keys, codebook, C, scores, P, B, S, D, stream);
        return launch_shared_layout<1, 3>(A, T, keys, codebook, C, scores, P, B, S, D, stream);
    }
    if (variant == kMfmaSmall) {
        if (layout == 0) return launch_small_layout<0, 0>(A, T, keys, codebook, C, scores, P, B, S, D, stream);
        if (bits == 2) return launch_small_layout<1, 2>(A, T, keys, codebook, C, scores, P, B, S, D, stream);
        return launch_small_layout<1, 3>(A, T, keys, codebook, C, scores, P, B, S, D, stream);
    }
    if (variant == kMfmaReg) {
        if (layout == 0) return launch_qs_layout<0, 0>(A, T, keys, codebook, C, scores, P, B, S, D, stream);
        if (bits == 2) return launch_qs_layout<1, 2>(A, T, keys, codebook, C, scores, P, B, S, D, stream);
        return launch_qs_layout<1, 3>(A, T, keys, codebook, C, scores, P, B, S, D, stream);
    }
    if (layout == 0) return launch_layout<0, 0>(A, T, keys, codebook, C, scores, P, B, S, D, stream);
    if (bits == 2) return launch_layout<1, 2>(A, T, keys, codebook, C, scores, P, B, S, D, stream);
    return launch_layout<1, 3>(A, T, keys, codebook, C, scores, P, B, S, D, stream);
}

bool score_mse_supported(int layout, int bits, int C, int D) { return lds_supported(layout, bits, C, D); }

bool split_mfma_supported(int bits_hi, int C_hi, int bits_lo, int C_lo, int D_hi, int D_lo, int S) {
    return bits_hi == 3 && C_hi == 8 && bits_lo == 2 && C_lo == 4 && D_hi == kSplitDHi && D_lo == kSplitDLo &&
           S < (1 << 24);
}

namespace {
template <int MT>
hipError_t launch_split_mt(const float* A_hi, const float* A_lo, SplitStreams k, const float* cb_hi, int C_hi,
                           const float* cb_lo, int C_lo, float* scores, int P, int B, int S, hipStream_t stream) {
    // the grid of launch_mt: at most two workgroups per CU
    const int groups_y = (B + MT * 32 - 1) / (MT * 32);
    const int ntiles = (S + kTileKeys - 1) / kTileKeys;
    int64_t gx = (ntiles + kWaves - 1) / kWaves;
    int64_t cap = 512 / ((int64_t)groups_y * P);
    if (cap < 1) cap = 1;
    if (gx > cap) gx = cap;
    hipLaunchKernelGGL((score_split_mfma_kernel<MT>), dim3((unsigned)gx, groups_y, P), dim3(kThreads), 0, stream,
                       A_hi, A_lo, k.idx_hi, k.norm_hi, k.idx_lo, k.norm_lo, cb_hi, C_hi, cb_lo, C_lo, scores, B, S);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_score_split_mfma(const float* A_hi, const float* A_lo, SplitStreams k, const float* cb_hi, int C_hi,
                                   const float* cb_lo, int C_lo, float* scores, int P, int B, int S,
                                   hipStream_t stream) {
    if (B <= 4 && (int64_t)P * S >= (int64_t(1) << 20)) {
        // four queries over many keys: the 16x16 tiles (the rule tq_score uses);
        // six wavefronts per SIMD fit its registers
        constexpr int MINW = 6;
        const int ntiles = (S + kTileKeys16 - 1) / kTileKeys16;
        int64_t gx = (ntiles + kWaves - 1) / kWaves;
        int64_t cap = 256LL * MINW / P;
        if (cap < 1) cap = 1;
        if (gx > cap) gx = cap;
        hipLaunchKernelGGL((score_split16_kernel<MINW>), dim3((unsigned)gx, 1, P), dim3(kThreads), 0, stream, A_hi,
                           A_lo, k.idx_hi, k.norm_hi, k.idx_lo, k.norm_lo, cb_hi, C_hi, cb_lo, C_lo, scores, B, S);
        return hipGetLastError();
    }
    switch (mt_for(B, kSplitDHi + kSplitDLo)) {
        case 4: return launch_split_mt<4>(A_hi, A_lo, k, cb_hi, C_hi, cb_lo, C_lo, scores, P, B, S, stream);
        case 2: return launch_split_mt<2>(A_hi, A_lo, k, cb_hi, C_hi, cb_lo, C_lo, scores, P, B, S, stream);
        default: return launch_split_mt<1>(A_hi, A_lo, k, cb_hi, C_hi, cb_lo, C_lo, scores, P, B, S, stream);
    }
}

namespace {

template <int LAYOUT, int BITS, int VLAYOUT, int VBITS>
hipError_t launch_fused(const float* A, const float* T, KeyStreams k, const float* codebook, int C,
                        ValueStreams v, const float* vcodebook, int VC, float scale, float* ws, int P, int B, int S,
                        int chunk, int nch, hipStream_t stream) {
    constexpr int D = 128;
    const float coef = (float)(kSqrtHalfPi / (double)D);
    hipLaunchKernelGGL((score_attend_kernel<LAYOUT, BITS, D, VLAYOUT, VBITS>), dim3((unsigned)nch, (B + 31) / 32, P),
                       dim3(kThreads), 0, stream, A, T, k.idx, k.sign, k.gamma, codebook, C, v.idx, v.norm,
                       vcodebook, VC, scale, ws, B, S, chunk, nch, coef);
    return hipGetLastError();
}

template <int LAYOUT, int BITS>
hipError_t launch_fused_v(int vlayout, int vbits, const float* A, const float* T, KeyStreams k, const float* codebook,
                          int C, ValueStreams v, const float* vcodebook, int VC, float scale, float* ws, int P, int B,
                          int S, int chunk, int nch, hipStream_t stream) {
    if (vlayout == 0)
        return launch_fused<LAYOUT, BITS, 0, 0>(A, T, k, codebook, C, v, vcodebook, VC, scale, ws, P, B, S, chunk, nch, stream);
    if (vbits == 2)
        return launch_fused<LAYOUT, BITS, 1, 2>(A, T, k, codebook, C, v, vcodebook, VC, scale, ws, P, B, S, chunk, nch, stream);
    return launch_fused<LAYOUT, BITS, 1, 3>(A, T, k, codebook, C, v, vcodebook, VC, scale, ws, P, B, S, chunk, nch, stream);
}

}  // namespace

// Chunks of the fused step: multiples of four 32-key tiles (one per wavefront),
// about 256 workgroups in all (one per compute unit: the kernel holds about
// 66 KB of LDS).
void score_attend_plan(int P, int B, int S, int& chunk, int& nch) {
    const int64_t blocks = (int64_t)P * ((B + 31) / 32);
    int64_t n = (256 + blocks - 1) / blocks;
    const int64_t most = ((int64_t)S + 4 * kTileKeys - 1) / (4 * kTileKeys);
    if (n > most) n = most;
    if (n < 1) n = 1;
    const int64_t per = ((int64_t)S + n - 1) / n;
    chunk = (int)((per + 4 * kTileKeys - 1) / (4 * kTileKeys) * (4 * kTileKeys));
    nch = (S + chunk - 1) / chunk;
}

bool score_attend_supported(int layout, int bits, int C, int vlayout, int vbits, int VC, int D) {
    return D == 128 && lds_supported(layout, bits, C, D) && VC >= 1 && VC <= 8 &&
           (vlayout == 0 || vbits == 2 || vbits == 3);
}

hipError_t launch_score_attend_partial(const float* A, const float* T, KeyStreams keys, int layout, int bits,
                                       const float* codebook, int C, ValueStreams v, int vlayout, int vbits,
                                       const float* vcodebook, int VC, float scale, float* ws, int P, int B, int S,
                                       int chunk, int nch, hipStream_t stream) {
    if (layout == 0)
        return launch_fused_v<0, 0>(vlayout, vbits, A, T, keys, codebook, C, v, vcodebook, VC, scale, ws, P, B, S, chunk, nch, stream);
    if (bits == 2)
        return launch_fused_v<1, 2>(vlayout, vbits, A, T, keys, codebook, C, v, vcodebook, VC, scale, ws, P, B, S, chunk, nch, stream);
    return launch_fused_v<1, 3>(vlayout, vbits, A, T, keys, codebook, C, v, vcodebook, VC, scale, ws, P, B, S, chunk, nch, stream);
}

hipError_t launch_score_mse(const float* A, const uint8_t* idx, const void* norm, int layout, int bits,
                            const float* codebook, int C, float* scores, int P, int B, int S, int D,
                            hipStream_t stream) {
    if (!score_mse_supported(layout, bits, C, D)) return hipErrorInvalidValue;
    const KeyStreams k{idx, nullptr, norm};
    // as for tq_score: one group of four queries over many keys takes the 16x16
    // tiles, four or more query tiles the shared decode
    const int variant = pick_variant(layout, bits, C, B, (int64_t)P * S, D);
    if (variant == kMfmaSmall) {
        if (layout == 0) return launch_small_layout<0, 0, false>(A, nullptr, k, codebook, C, scores, P, B, S, D, stream);
        if (bits == 2) return launch_small_layout<1, 2, false>(A, nullptr, k, codebook, C, scores, P, B, S, D, stream);
        return launch_small_layout<1, 3, false>(A, nullptr, k, codebook, C, scores, P, B, S, D, stream);
    }
    if (variant == kMfmaShared) {
        if (layout == 0) return launch_shared_layout<0, 0, false>(A, nullptr, k, codebook, C, scores, P, B, S, D, stream);
        if (bits == 2) return launch_shared_layout<1, 2, false>(A, nullptr, k, codebook, C, scores, P, B, S, D, stream);
        return launch_shared_layout<1, 3, false>(A, nullptr, k, codebook, C, scores, P, B, S, D, stream);
    }
    if (layout == 0) return launch_layout<0, 0, false>(A, nullptr, k, codebook, C, scores, P, B, S, D, stream);
    if (bits == 2) return launch_layout<1, 2, false>(A, nullptr, k, codebook, C, scores, P, B, S, D, stream);
    return launch_layout<1, 3, false>(A, nullptr, k, codebook, C, scores, P, B, S, D, stream);
}

}  // namespace tq
