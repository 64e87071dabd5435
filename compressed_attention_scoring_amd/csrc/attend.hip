// Decode attention output over compressed values, the step downstream of
// scoring ("TurboQuant: Rotate-then-Quantize KV Caches at 3 Bits", section 8,
// "Kernel view: never un-rotate a key"; "Fitting 4.4x More Context on Jetson",
// the online-softmax FAQ): values are stored by the MSE quantizer (rotation
// Pi_v, codebook, one norm per vector), and
//   o_b = Pi_v^T sum_s p_bs ||v_s|| c[idx_s],   p_b = softmax(scale * scores_b).
//
// Split over key ranges (split-KV). attend_partial_kernel: one workgroup of four
// wavefronts per (key chunk, group of query tiles, block of coordinates,
// problem). A wavefront owns one query tile and a share of the chunk's keys and runs an online softmax over
// them: a running reference maximum per query, raised (and the accumulator
// rescaled) only when a step's maximum exceeds it by more than kTau, so the
// rescale is rare. The weighted sum
//   acc[d][b] = sum_s exp(scale*score_bs - m_b) ||v_s|| c[idx_sd]
// runs on the matrix cores with the value coordinates as rows, the queries as
// columns and keys as the contraction, so that each lane's accumulators belong
// to one query:
//  - wide (B > 8): v_mfma_f32_32x32x16_f16, 32 queries per tile, three products
//    of f16 hi/lo parts (V_hi W_hi, V_lo W_hi, V_hi W_lo);
//  - narrow (B <= 8): v_mfma_f32_16x16x32_f16, the weights' hi parts in
//    columns 0-7 and lo parts in columns 8-15, so two products cover all three
//    terms.
// Weights carry the value norms, scaled by a power of two that tracks the
// largest norm seen, and codebook entries are scaled by a power of two, so
// every f16 operand stays in the normal range. The wavefronts sharing a query
// tile merge through LDS and the workgroup writes (m, l, acc) per query and
// chunk. attend_combine_kernel merges the chunks of one query and applies
// Pi_v^T once.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "tq_common.hpp"
#include "value_sel.hpp"

namespace tq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4u __attribute__((ext_vector_type(4), aligned(4)));
typedef _Float16 f16x8u __attribute__((ext_vector_type(8), aligned(2)));

enum AttendMode { kWide = 0, kNarrow = 1 };

// MFMA geometry: ROWS coordinates per tile (lanes n = lane % ROWS), KG lane
// groups along the contraction (g = lane / ROWS), KSTEP keys per product, Q
// queries per tile.
template <int MODE> struct Geo;
template <> struct Geo<kWide> {
    static constexpr int ROWS = 32, KG = 2, KSTEP = 16, Q = 32;
};
template <> struct Geo<kNarrow> {
    static constexpr int ROWS = 16, KG = 4, KSTEP = 32, Q = 8;
};

constexpr int kWaves = 4;          // wavefronts per workgroup
constexpr float kTau = 5.5f;       // rescale when a step max passes the reference by more (e^5.5 < 2^8)
constexpr int kNormBits = 4;       // scaled norms stay below 2^(kNormBits + 2) until the next rescale
constexpr int kTargetBlocks = 512; // workgroups one call aims for (two per compute unit)
constexpr int kComputeUnits = 256; // MI355X
// Partial results at most 1/kPartialShare of the bytes a chunk reads, or
// 1/kPartialShareWide where the smaller share would leave fewer workgroups.
constexpr int kPartialShare = 8;
constexpr int kPartialShareWide = 4;

union H8 {
    f16x8 h;
    uint32_t u[4];
};

__device__ __forceinline__ float pow2_below(float maxabs, int top) {
    // a power of two bringing maxabs into [2^(top-1), 2^top); 1 if maxabs is 0 or not finite
    if (!(maxabs > 0.f) || !(maxabs < 3.0e38f)) return 1.f;
    int e;
    (void)frexpf(maxabs, &e);
    return ldexpf(1.f, min(126, max(-126, top - e)));
}

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// four selector bytes (< 8) -> two dwords of f16 pairs from byte tables
// {low bytes of entries 0-3, 4-7, high bytes of 0-3, 4-7}
__device__ __forceinline__ void lut4(uint32_t x, const uint32_t (&tab)[4], uint32_t& o0, uint32_t& o1) {
    const uint32_t lo = perm(tab[1], tab[0], x);
    const uint32_t hi = perm(tab[3], tab[2], x);
    o0 = perm(hi, lo, 0x05010400u);
    o1 = perm(hi, lo, 0x07030602u);
}

__device__ __forceinline__ float xor_max(float v, int m) { return fmaxf(v, __shfl_xor(v, m)); }

// Raw loads of one step for one lane: 8 scores of its query, 8 norms (fp32
// bits, or fp16 pairs), and per key the one or two dwords holding its value
// bits. Kept as loaded, so that the loads of the next step can be in flight
// while this one is computed.
template <int LAYOUT>
struct Raw {
    float sc[8];
    uint32_t nr[8];
    uint32_t vlo[8], vhi[8];
};

template <int LAYOUT, int BITS, int D, int MODE, int QTW, int NT>
__global__ __launch_bounds__(kWaves * 64) void attend_partial_kernel(
    const float* __restrict__ scores, const uint8_t* __restrict__ vidx, const void* __restrict__ vnorm,
    const float* __restrict__ codebook, int C, float scale, float* __restrict__ ws,
    int B, int S, int chunk, int nch) {
    using G = Geo<MODE>;
    constexpr int DB = NT * G::ROWS;               // coordinates per workgroup
    constexpr int DBLK = D / DB;                   // workgroups along the coordinates
    constexpr int NW = kWaves;
    constexpr int KW = NW / QTW;                   // wavefronts sharing one query tile
    constexpr int DP = DB + 1;                     // LDS row stride (consecutive queries on distinct banks)
    constexpr int BW = LAYOUT == 0 ? 8 : BITS;     // bits per coordinate
    constexpr int W = NT * BW;                     // value bits per lane per key
    constexpr int ROWB = D * BW / 8;               // bytes per value row
    // 0: a lane's field never leaves its dword; 2: it always spans two; 1: it depends on the lane
    constexpr int CROSS = W > 32 ? 2 : (32 % W == 0 ? 0 : 1);
    static_assert(DBLK * DB == D && W <= 64 && ROWB % 4 == 0, "tiling");
    __shared__ float red_acc[NW][G::Q][DP];
    __shared__ float red_m[NW][G::Q];
    __shared__ float red_l[NW][G::Q];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qtw = wave % QTW;
    const int kw = wave / QTW;
    const int p = blockIdx.z;
    const int c = blockIdx.x;
    const int tg = blockIdx.y / DBLK;                  // group of query tiles
    const int db = blockIdx.y % DBLK;                  // coordinate block
    const int q0 = (tg * QTW + qtw) * G::Q;            // first query of this wavefront's tile
    const int n = lane % G::ROWS;
    const int g = lane / G::ROWS;
    const int ql = MODE == kWide ? n : (n & 7);        // query of this lane's weight column
    const int part = MODE == kWide ? 0 : (n >> 3);     // narrow: 0 = hi column, 1 = lo column
    const bool qvalid = q0 + ql < B;
    const float* srow = scores + ((int64_t)p * B + min(q0 + ql, B - 1)) * S;
    const int s_begin = c * chunk;
    const int s_end = min(S, s_begin + chunk);
    const int64_t key0 = (int64_t)p * S;
    // value bits of coordinates db*DB + NT*n .. + NT-1: dword k0 of the row, and
    // the next one when the field runs into it
    const int vbit = BW * (db * DB + NT * n);
    const int k0 = vbit >> 5;
    const int vsh = vbit & 31;
    const bool two = CROSS == 2 || (CROSS == 1 && vsh + W > 32);
    const uint8_t* vbase = vidx + key0 * ROWB + 4 * k0;

    // codebook tables (hi and lo f16 parts of the entries times a power of two)
    float cbv[8];
    float mc = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        cbv[k] = k < C ? codebook[k] : 0.f;
        mc = fmaxf(mc, fabsf(cbv[k]));
    }
    const float cscale = pow2_below(mc, 14);
    uint32_t tab_hi[4] = {0u, 0u, 0u, 0u}, tab_lo[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float x = cbv[k] * cscale;
        const _Float16 h = (_Float16)x;
        const _Float16 l = (_Float16)(x - (float)h);
        const uint16_t hb = __builtin_bit_cast(uint16_t, h), lb = __builtin_bit_cast(uint16_t, l);
        const int w = k >> 2, sh = 8 * (k & 3);
        tab_hi[w] |= (uint32_t)(hb & 0xffu) << sh;
        tab_hi[2 + w] |= (uint32_t)(hb >> 8) << sh;
        tab_lo[w] |= (uint32_t)(lb & 0xffu) << sh;
        tab_lo[2 + w] |= (uint32_t)(lb >> 8) << sh;
    }

    using Acc = typename std::conditional<MODE == kWide, f32x16, f32x4>::type;
    constexpr int NV = MODE == kWide ? 16 : 4;
    Acc acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[t][v] = 0.f;
    float M = -INFINITY;      // reference maximum of scale*score for query ql
    float lsum = 0.f;         // sum of exp(scale*score - M) over this lane's keys
    float nexp = -1000.f;     // norms are scaled by 2^-nexp ...
    float nlim = 0.f;         // ... and must stay below nlim = 2^(nexp + kNormBits + 2)

    // this wavefront's steps: keys s_begin + (kw + KW*i)*KSTEP + [0, KSTEP)
    const int span = s_end - s_begin - kw * G::KSTEP;
    const int ntot = span > 0 ? (span + KW * G::KSTEP - 1) / (KW * G::KSTEP) : 0;
    const int nfull = span >= G::KSTEP ? (span - G::KSTEP) / (KW * G::KSTEP) + 1 : 0;
    auto first_key = [&](int i) { return s_begin + (kw + KW * i) * G::KSTEP + 8 * g; };

    auto load_full = [&](Raw<LAYOUT>& r, int sk) {
        const f32x4u a = *reinterpret_cast<const f32x4u*>(srow + sk);
        const f32x4u b = *reinterpret_cast<const f32x4u*>(srow + sk + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            r.sc[e] = a[e];
            r.sc[4 + e] = b[e];
        }
        if constexpr (LAYOUT == 0) {
            const uint32_t* np = reinterpret_cast<const uint32_t*>(vnorm) + key0 + sk;
            typedef uint32_t u32x4u __attribute__((ext_vector_type(4), aligned(4)));
            const u32x4u x = *reinterpret_cast<const u32x4u*>(np);
            const u32x4u y = *reinterpret_cast<const u32x4u*>(np + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                r.nr[e] = x[e];
                r.nr[4 + e] = y[e];
            }
        } else {
            typedef uint32_t u32x4h __attribute__((ext_vector_type(4), aligned(2)));
            const u32x4h x = *reinterpret_cast<const u32x4h*>(reinterpret_cast<const uint16_t*>(vnorm) + key0 + sk);
#pragma unroll
            for (int e = 0; e < 4; ++e) r.nr[e] = x[e];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t* w = reinterpret_cast<const uint32_t*>(vbase + (int64_t)(sk + e) * ROWB);
            r.vlo[e] = w[0];
            r.vhi[e] = w[two ? 1 : 0];     // in-row either way
        }
    };
    auto load_tail = [&](Raw<LAYOUT>& r, int sk) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int s = min(sk + e, s_end - 1);
            r.sc[e] = srow[s];
            if constexpr (LAYOUT == 0) {
                r.nr[e] = reinterpret_cast<const uint32_t*>(vnorm)[key0 + s];
            } else {
                const uint32_t h = reinterpret_cast<const uint16_t*>(vnorm)[key0 + s];
                if (e % 2 == 0) r.nr[e / 2] = h;
                else r.nr[e / 2] |= h << 16;
            }
            const uint32_t* w = reinterpret_cast<const uint32_t*>(vbase + (int64_t)s * ROWB);
            r.vlo[e] = w[0];
            r.vhi[e] = w[two ? 1 : 0];
        }
    };
    auto compute = [&](const Raw<LAYOUT>& r, int sk, int lim) {
        // step maximum of the lane's query over the step's keys
        float z[8], nv[8];
        float ms = -INFINITY, nm = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            z[e] = (qvalid && sk + e < lim) ? scale * r.sc[e] : -INFINITY;
            if constexpr (LAYOUT == 0) nv[e] = __builtin_bit_cast(float, r.nr[e]);
            else nv[e] = (float)__builtin_bit_cast(_Float16, (uint16_t)(r.nr[e / 2] >> (16 * (e % 2))));
            ms = fmaxf(ms, z[e]);
            nm = fmaxf(nm, fabsf(nv[e]));
        }
        ms = xor_max(ms, 32);
        if constexpr (MODE == kNarrow) ms = xor_max(ms, 16);
        const bool need_m = ms > M + kTau;
        if (__any(need_m || nm >= nlim)) {
            // rescale: new reference maximum for the lanes that need it, and a new
            // norm scale for the whole wavefront if a norm outgrew the current one
            float nw = nm;
#pragma unroll
            for (int m = 1; m < 64; m <<= 1) nw = xor_max(nw, m);
            float fac = 1.f;
            if (nw >= nlim) {
                int e2;
                (void)frexpf(nw, &e2);
                const float ne = nw > 0.f ? (float)(e2 - kNormBits) : 0.f;
                fac = exp2f(nexp - ne);
                nexp = ne;
                nlim = exp2f(ne + kNormBits + 2);
            }
            const float Mn = need_m ? ms : M;
            const float fm = need_m ? __expf(M - Mn) : 1.f;
            M = Mn;
            lsum *= fm;
            fac *= fm;
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int v = 0; v < NV; ++v) acc[t][v] *= fac;
        }
        const float nscale = exp2f(-nexp);
        H8 whi, wlo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float w = z[e] == -INFINITY ? 0.f : __expf(z[e] - M);
            lsum += w;
            const float x = w * nv[e] * nscale;
            const _Float16 h = (_Float16)x;
            whi.h[e] = h;
            wlo.h[e] = (_Float16)(x - (float)h);
        }
        uint64_t vb[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) vb[e] = ((two ? (uint64_t)r.vhi[e] << 32 : 0ull) | r.vlo[e]) >> vsh;
        // packed fields (W <= 32 bits per key): selectors from byte-transposed bits
        constexpr bool BYTES = LAYOUT == 1 && W <= 32;
        using VS = typename std::conditional<BYTES, ValueSelectors<BW, W>, NoValueSelectors>::type;
        const VS vs(vb);
        // value operands per tile and the products
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            uint32_t sel0 = 0, sel1 = 0;
            if constexpr (BYTES) {
                vs.tile(t, sel0, sel1);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sel0 |= ((uint32_t)(vb[e] >> (BW * t)) & ((1u << BW) - 1u)) << (8 * e);
                    sel1 |= ((uint32_t)(vb[4 + e] >> (BW * t)) & ((1u << BW) - 1u)) << (8 * e);
                }
            }
            H8 vhi, vlo;
            lut4(sel0, tab_hi, vhi.u[0], vhi.u[1]);
            lut4(sel1, tab_hi, vhi.u[2], vhi.u[3]);
            lut4(sel0, tab_lo, vlo.u[0], vlo.u[1]);
            lut4(sel1, tab_lo, vlo.u[2], vlo.u[3]);
            if constexpr (MODE == kWide) {
                acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vhi.h, whi.h, acc[t], 0, 0, 0);
                acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vlo.h, whi.h, acc[t], 0, 0, 0);
                acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vhi.h, wlo.h, acc[t], 0, 0, 0);
            } else {
                H8 wb, wh;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    wb.u[k] = part ? wlo.u[k] : whi.u[k];
                    wh.u[k] = part ? 0u : whi.u[k];
                }
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vhi.h, wb.h, acc[t], 0, 0, 0);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vlo.h, wh.h, acc[t], 0, 0, 0);
            }
        }
    };

    if (q0 < B) {
        // full steps, two buffers: the next step's loads are in flight while a step
        // is computed (a prefetch past the last full step re-reads that step)
        if (nfull > 0) {
            Raw<LAYOUT> ra, rb;
            load_full(ra, first_key(0));
            int i = 0;
            for (; i + 1 < nfull; i += 2) {
                load_full(rb, first_key(i + 1));
                compute(ra, first_key(i), INT32_MAX);
                load_full(ra, first_key(min(i + 2, nfull - 1)));
                compute(rb, first_key(i + 1), INT32_MAX);
            }
            if (i < nfull) compute(ra, first_key(i), INT32_MAX);
        }
        if (ntot > nfull) {
            Raw<LAYOUT> rt;
            load_tail(rt, first_key(nfull));
            compute(rt, first_key(nfull), s_end);
        }
    }

    // ---- per-wavefront results to LDS: query ql's m, l and acc (true scale)
    lsum += __shfl_xor(lsum, 32);
    if constexpr (MODE == kNarrow) {
        lsum += __shfl_xor(lsum, 16);
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int v = 0; v < NV; ++v) acc[t][v] += __shfl_xor(acc[t][v], 8);   // hi + lo columns
    }
    const float unscale = exp2f(nexp) / cscale;
    if (g == 0 && part == 0) {
        red_m[wave][ql] = M;
        red_l[wave][ql] = lsum;
    }
    if (part == 0) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int row = MODE == kWide ? 8 * (v >> 2) + 4 * g + (v & 3) : 4 * g + v;
                red_acc[wave][ql][NT * row + t] = acc[t][v] * unscale;
            }
    }
    __syncthreads();

    // ---- merge the KW wavefronts of each query tile and write the records
    for (int i = tid; i < QTW * G::Q * DB; i += NW * 64) {
        const int d = i % DB;
        const int qi = (i / DB) % G::Q;
        const int tq = i / (DB * G::Q);
        const int q = (tg * QTW + tq) * G::Q + qi;
        if (q >= B) continue;
        float Mx = -INFINITY;
#pragma unroll
        for (int k = 0; k < KW; ++k) Mx = fmaxf(Mx, red_m[k * QTW + tq][qi]);
        float a = 0.f, l = 0.f;
#pragma unroll
        for (int k = 0; k < KW; ++k) {
            const int w = k * QTW + tq;
            const float f = red_m[w][qi] == -INFINITY ? 0.f : __expf(red_m[w][qi] - Mx);
            a = fmaf(red_acc[w][qi][d], f, a);
            l = fmaf(red_l[w][qi], f, l);
        }
        float* rec = ws + (((int64_t)p * B + q) * nch + c) * (D + 2);
        rec[2 + db * DB + d] = a;
        if (db == 0 && d == 0) {
            rec[0] = Mx;
            rec[1] = l;
        }
    }
}

// One workgroup per (query, problem): merge the chunks' (m, l, acc) and apply
// Pi_v^T: out_j = sum_d Pi_v[d][j] a_d with a = sum_c acc_c e^(m_c - M) / sum_c l_c e^(m_c - M).
// The kernel is a chain of memory round trips, so it is shaped for as few as
// possible: the thread's share of Pi_v is requested first, then every
// wavefront requests its chunk records (wavefront w takes chunks w, w + 16, ...,
// NB of them per batch of loads, one batch for up to NW NB chunks) and merges
// them with a running maximum of its own; the wavefront results are merged
// through LDS.
constexpr int kCombineBatch = 16;   // chunk records per wavefront per batch of loads

// NW wavefronts (4 or 16: launch_attend_combine takes sixteen only when there
// are more chunk records than four wavefronts take in one batch).
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void attend_combine_kernel(const float* __restrict__ ws, const float* __restrict__ Pi_v,
                                                                 float* __restrict__ out, int H, int B, int nch) {
    constexpr int DL = (D + 63) / 64;      // coordinates per lane
    constexpr int NB = kCombineBatch;
    constexpr int JP = NW * 64 / D;        // threads per output coordinate in the product with Pi_v
    constexpr int DJ = D / JP;             // coordinates each of them sums
    __shared__ float part_a[NW][D];
    __shared__ float part_l[NW];
    __shared__ float part_m[NW];
    __shared__ float a[D];
    __shared__ float po[JP][D];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int b = blockIdx.x;
    const int p = blockIdx.y;
    const float* rec = ws + ((int64_t)p * B + b) * nch * (D + 2);

    // this thread's share of Pi_v (column j, rows h DJ .. h DJ + DJ - 1)
    const int j = tid % D;
    const int h = tid / D;
    const float* P = Pi_v + (int64_t)(p % H) * D * D + (int64_t)h * DJ * D + j;
    float pv[DJ];
#pragma unroll
    for (int d = 0; d < DJ; ++d) pv[d] = P[(int64_t)d * D];

    float mw = -INFINITY, den = 0.f;
    float acc[DL];
#pragma unroll
    for (int k = 0; k < DL; ++k) acc[k] = 0.f;
    for (int c0 = wave; c0 < nch; c0 += NW * NB) {
        float mv[NB], lv[NB], av[NB][DL];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int c = min(c0 + NW * i, nch - 1);
            const float* r = rec + (int64_t)c * (D + 2);
            mv[i] = r[0];
            lv[i] = r[1];
#pragma unroll
            for (int k = 0; k < DL; ++k) av[i][k] = r[2 + min(lane + 64 * k, D - 1)];
        }
        float bm = mw;
#pragma unroll
        for (int i = 0; i < NB; ++i)
            if (c0 + NW * i < nch) bm = fmaxf(bm, mv[i]);
        const float f0 = mw == -INFINITY ? 0.f : __expf(mw - bm);   // rescale what was merged so far
        den *= f0;
#pragma unroll
        for (int k = 0; k < DL; ++k) acc[k] *= f0;
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const float f = (c0 + NW * i < nch && mv[i] != -INFINITY) ? __expf(mv[i] - bm) : 0.f;
            den = fmaf(lv[i], f, den);
#pragma unroll
            for (int k = 0; k < DL; ++k) acc[k] = fmaf(av[i][k], f, acc[k]);
        }
        mw = bm;
    }
#pragma unroll
    for (int k = 0; k < DL; ++k) {
        const int d = lane + 64 * k;
        if (d < D) part_a[wave][d] = acc[k];
    }
    if (lane == 0) {
        part_l[wave] = den;
        part_m[wave] = mw;
    }
    __syncthreads();
    if (tid < D) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, part_m[w]);
        float l = 0.f, v = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float f = part_m[w] == -INFINITY ? 0.f : __expf(part_m[w] - M);
            l = fmaf(part_l[w], f, l);
            v = fmaf(part_a[w][tid], f, v);
        }
        a[tid] = v / l;
    }
    __syncthreads();
    float o = 0.f;
#pragma unroll
    for (int d = 0; d < DJ; ++d) o = fmaf(pv[d], a[h * DJ + d], o);
    po[h][j] = o;
    __syncthreads();
    if (tid < D) {
        float r = 0.f;
#pragma unroll
        for (int k = 0; k < JP; ++k) r += po[k][tid];
        out[((int64_t)p * B + b) * D + tid] = r;
    }
}

struct Plan {
    int mode;    // kWide or kNarrow
    int qtw;     // query tiles per workgroup (1, 2 or 4)
    int gy;      // groups of query tiles
    int nt;      // tiles (coordinates per lane) per wavefront
    int dblk;    // workgroups along the coordinates
    int nch;     // key chunks
    int chunk;   // keys per chunk
    int nmax;    // chunk count before rounding (an upper bound on nch)
};

Plan make_plan_share(int P, int B, int S, int D, int layout, int bits, int share) {
    Plan pl;
    pl.mode = B <= 8 ? kNarrow : kWide;
    const int Q = pl.mode == kWide ? Geo<kWide>::Q : Geo<kNarrow>::Q;
    const int rows = pl.mode == kWide ? Geo<kWide>::ROWS : Geo<kNarrow>::ROWS;
    const int kstep = pl.mode == kWide ? Geo<kWide>::KSTEP : Geo<kNarrow>::KSTEP;
    const int ntiles = (B + Q - 1) / Q;
    pl.qtw = ntiles >= 4 ? 4 : ntiles >= 2 ? 2 : 1;
    pl.gy = (ntiles + pl.qtw - 1) / pl.qtw;
    const int unit = kstep * (kWaves / pl.qtw);      // keys of one step of every wavefront sharing a tile
    // keys per chunk at least: the partial results stay under 1/share of
    // the bytes the chunk reads (its scores and values)
    const int64_t bq = std::min<int64_t>(B, (int64_t)Q * pl.qtw);
    const int64_t vbytes = (layout == 0 ? D + 4 : (int64_t)D * bits / 8 + 2);
    int64_t cmin = (share * bq * (D + 2) * 4 + bq * 4 + vbytes - 1) / (bq * 4 + vbytes);
    cmin = (cmin + unit - 1) / unit * unit;
    const int64_t blocks = (int64_t)P * pl.gy;
    int64_t n = (kTargetBlocks + blocks - 1) / blocks;
    const int64_t most = (S + cmin - 1) / cmin;
    if (n > most) n = most;
    // a grid past a whole number of rounds of one workgroup per compute unit
    // doubles up the CUs of the partial round, which then finish last
    // (measured: the packed workload's 293 chunks ran 27.4 us, 256 ran 21.3)
    if (blocks * n > kComputeUnits) n = blocks * n / kComputeUnits * kComputeUnits / blocks;
    if (n < 1) n = 1;
    // split the coordinates (which repeats the weights' arithmetic in every
    // block) only until there is about one workgroup per compute unit
    const int ntfull = D / rows;
    pl.dblk = 1;
    while (pl.dblk < 4 && ntfull / (2 * pl.dblk) >= 1 && blocks * n * pl.dblk < kComputeUnits) pl.dblk *= 2;
    // and past one round, whole rounds again (fewer, longer chunks rather than a
    // partial round: packed workload 320 -> 256 workgroups)
    const int64_t wgs = blocks * n * pl.dblk;
    if (wgs > kComputeUnits && wgs % kComputeUnits != 0) {
        const int64_t n2 = wgs / kComputeUnits * kComputeUnits / (blocks * pl.dblk);
        if (n2 >= 1) n = n2;
    }
    pl.nt = ntfull / pl.dblk;
    const int64_t per = (S + n - 1) / n;
    pl.chunk = (int)((per + unit - 1) / unit * unit);
    pl.nch = (int)(((int64_t)S + pl.chunk - 1) / pl.chunk);
    pl.nmax = (int)n;
    return pl;
}

// The smaller record share where it keeps the workgroup count (decode: 64
// chunks x 4 coordinate blocks instead of 128 x 2), the larger one where it
// would halve it (long: 256 workgroups instead of 512 ran no faster and fetched
// 229 MB instead of 165 MB of scores and values).
Plan make_plan(int P, int B, int S, int D, int layout, int bits) {
    const Plan narrow = make_plan_share(P, B, S, D, layout, bits, kPartialShare);
    const Plan wide = make_plan_share(P, B, S, D, layout, bits, kPartialShareWide);
    const int64_t wg_narrow = (int64_t)narrow.nch * narrow.gy * narrow.dblk;
    const int64_t wg_wide = (int64_t)wide.nch * wide.gy * wide.dblk;
    Plan pl = wg_narrow >= wg_wide ? narrow : wide;
    pl.nmax = narrow.nmax > wide.nmax ? narrow.nmax : wide.nmax;   // an upper bound on either's chunks
    return pl;
}

template <int LAYOUT, int BITS, int D, int MODE, int QTW>
hipError_t launch_partial_q(const Plan& pl, const float* scores, ValueStreams v, const float* codebook, int C,
                            float scale, float* ws, int P, int B, int S, hipStream_t stream) {
    constexpr int NTF = D / Geo<MODE>::ROWS;
    const dim3 grid((unsigned)pl.nch, (unsigned)(pl.gy * pl.dblk), (unsigned)P);
#define TQ_PARTIAL(NTV)                                                                                       \
    hipLaunchKernelGGL((attend_partial_kernel<LAYOUT, BITS, D, MODE, QTW, NTV>), grid,                         \
                       dim3(kWaves * 64), 0, stream, scores, v.idx, v.norm, codebook, C, scale, ws, \
                       B, S, pl.chunk, pl.nch)
    constexpr int NT2 = NTF / 2 > 0 ? NTF / 2 : 1;
    constexpr int NT4 = NTF / 4 > 0 ? NTF / 4 : 1;
    if (pl.nt == NTF) TQ_PARTIAL(NTF);
    else if (pl.nt == NT2) TQ_PARTIAL(NT2);
    else TQ_PARTIAL(NT4);
#undef TQ_PARTIAL
    return hipGetLastError();
}

template <int LAYOUT, int BITS, int D, int MODE>
hipError_t launch_partial(const Plan& pl, const float* scores, ValueStreams v, const float* codebook, int C,
                          float scale, float* ws, int P, int B, int S, hipStream_t stream) {
    if (pl.qtw == 4) return launch_partial_q<LAYOUT, BITS, D, MODE, 4>(pl, scores, v, codebook, C, scale, ws, P, B, S, stream);
    if (pl.qtw == 2) return launch_partial_q<LAYOUT, BITS, D, MODE, 2>(pl, scores, v, codebook, C, scale, ws, P, B, S, stream);
    return launch_partial_q<LAYOUT, BITS, D, MODE, 1>(pl, scores, v, codebook, C, scale, ws, P, B, S, stream);
}

template <int LAYOUT, int BITS, int D>
hipError_t launch_attend_d(const float* scores, ValueStreams v, const float* codebook, int C, const float* Pi_v,
                           float scale, float* out, float* ws, int P, int H, int B, int S, hipStream_t stream) {
    const Plan pl = make_plan(P, B, S, D, LAYOUT, BITS);
    const hipError_t e = pl.mode == kWide
                             ? launch_partial<LAYOUT, BITS, D, kWide>(pl, scores, v, codebook, C, scale, ws, P, B, S, stream)
                             : launch_partial<LAYOUT, BITS, D, kNarrow>(pl, scores, v, codebook, C, scale, ws, P, B, S, stream);
    if (e != hipSuccess) return e;
    return launch_attend_combine(ws, Pi_v, out, P, H, B, D, pl.nch, stream);
}

template <int LAYOUT, int BITS>
hipError_t launch_attend_layout(const float* scores, ValueStreams v, const float* codebook, int C, const float* Pi_v,
                                float scale, float* out, float* ws, int P, int H, int B, int S, int D,
                                hipStream_t stream) {
    if (D == 64) return launch_attend_d<LAYOUT, BITS, 64>(scores, v, codebook, C, Pi_v, scale, out, ws, P, H, B, S, stream);
    return launch_attend_d<LAYOUT, BITS, 128>(scores, v, codebook, C, Pi_v, scale, out, ws, P, H, B, S, stream);
}

}  // namespace

hipError_t launch_attend_combine(const float* ws, const float* Pi_v, float* out, int P, int H, int B, int D, int nch,
                                 hipStream_t stream) {
    const dim3 grid((unsigned)B, P);
    const bool wide = nch > 4 * kCombineBatch;   // more records than four wavefronts take in one batch
    if (D == 64) {
        if (wide) hipLaunchKernelGGL((attend_combine_kernel<64, 16>), grid, dim3(1024), 0, stream, ws, Pi_v, out, H, B, nch);
        else hipLaunchKernelGGL((attend_combine_kernel<64, 4>), grid, dim3(256), 0, stream, ws, Pi_v, out, H, B, nch);
    } else if (D == 128) {
        if (wide) hipLaunchKernelGGL((attend_combine_kernel<128, 16>), grid, dim3(1024), 0, stream, ws, Pi_v, out, H, B, nch);
        else hipLaunchKernelGGL((attend_combine_kernel<128, 4>), grid, dim3(256), 0, stream, ws, Pi_v, out, H, B, nch);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// The unpacked layout reads the most bytes per key, so it has the shortest
// chunks and the most of them: its count bounds every layout's.
int attend_chunks(int P, int B, int S, int D) { return make_plan(P, B, S, D, 0, 0).nmax; }

bool attend_supported(int layout, int bits, int C, int D) {
    if (C < 1 || C > 8) return false;
    if (D != 64 && D != 128) return false;
    return layout == 0 || bits == 2 || bits == 3;
}

hipError_t launch_attend(const float* scores, ValueStreams v, int layout, int bits, const float* codebook, int C,
                         const float* Pi_v, float scale, float* out, float* ws, int P, int H, int B, int S, int D,
                         hipStream_t stream) {
    if (!attend_supported(layout, bits, C, D)) return hipErrorInvalidValue;
    if (layout == 0) return launch_attend_layout<0, 0>(scores, v, codebook, C, Pi_v, scale, out, ws, P, H, B, S, D, stream);
    if (bits == 2) return launch_attend_layout<1, 2>(scores, v, codebook, C, Pi_v, scale, out, ws, P, H, B, S, D, stream);
    return launch_attend_layout<1, 3>(scores, v, codebook, C, Pi_v, scale, out, ws, P, H, B, S, D, stream);
}

}  // namespace tq
