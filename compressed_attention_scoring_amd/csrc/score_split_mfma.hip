// The outlier split's scorers on the matrix cores ("TurboQuant: Rotate-then-
// Quantize KV Caches at 3 Bits", section 7): the 32 x 32 LDS-staged form and
// the four-query 16 x 16 form.
#include "score_families.hpp"

namespace tq {
namespace {

using namespace ops;
using namespace layout;

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

}  // namespace

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

}  // namespace tq
