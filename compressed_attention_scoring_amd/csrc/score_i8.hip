// tq_score for up to four queries per problem over packed keys, on the integer
// matrix cores of gfx950 (v_mfma_i32_16x16x64_i8).
//
// What it computes is the scorer of "TurboQuant Attention in CUDA" (section
// "What the rearrangement saves"): scores = M + (sqrt(pi/2)/D) gamma R with
// M = A . c[idx] and R = T . sigma, A = Pi q and T = S q the transformed query
// ("TurboQuant: Rotate-then-Quantize KV Caches at 3 Bits", section 3).
//
// Why integers. With four queries per problem each decoded key serves only four
// rows, so the f16 four-query kernel is bound by vector-ALU key decoding: every
// codebook value needs an f16 hi and an f16 lo part (two byte-table lookups plus
// two interleaving permutes per four values) and every sign an f16 +-1. Here:
// - the codebook entries, scaled so the largest is 127, are written as three
//   int8 limbs c = c0 + c1/2^7 + c2/2^14; an 8-entry table of one limb is eight
//   bytes, so one v_perm looks up four coordinates' limb directly;
// - a sign enters as its bit b in {0, 1} (sigma = 2b - 1): one shift and one
//   mask give four coordinates' bytes;
// - the query rows A and T, each scaled so its largest magnitude is 127, are
//   split into four int8 limbs in the prologue, once per wavefront: a fixed
//   point of 28 bits below the row's largest coordinate, so that coordinates
//   many decades smaller than it keep their precision (three limbs gave
//   4.5e-4 of error on rows spanning 1e-6 .. 1e3).
// The products are exact in int32. Limb products of weight 2^-7(l+m) with
// l + m <= 3 are kept, summed by weight in the accumulator: operand row 4 q + t
// holds, for the MFMA against codebook limb m, query q's limb t - m (zero when
// t < m), so accumulator row 4 q + t collects every product of weight 2^-7t.
// The sign MFMA's row 4 q + t holds T's limb t.
//
// Layout (v_mfma_i32_16x16x64_i8): lane l supplies row (A) or column (keys)
// l % 16 and contraction bytes 16 (l / 16) .. 16 (l / 16) + 15; output register
// v of lane l is row 4 (l / 16) + v, column l % 16. Lane group gq = l / 16 owns
// coordinates [gq D/4, (gq + 1) D/4) of each key (as in the f16 four-query
// kernel). In a codebook k-step v of 16 coordinates, operand dword w holds the
// selectors of k-steps 2v + w/2 (elements 4 (w % 2) .. +3) of the f16 kernels'
// order (mse_dim); in a sign k-step u, byte k of dword d is bit
// 4 (u % 2) + d + 8 k of the lane's sign dword u / 2.
#include "score_i8.hpp"

#include "mfma_layout.hpp"

namespace tq {
namespace {

using namespace ops;
using namespace layout;

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Scale that brings a row's largest magnitude to 127 (1 when it is 0 or not
// finite; capped so that rows of tiny values stay finite and round to zero).
__device__ __forceinline__ float limb_scale(float maxabs) {
    if (!(maxabs > 0.f) || !(maxabs < 3.0e38f)) return 1.f;
    const float s = 127.f / maxabs;
    return s < 1.0e30f ? s : 1.0e30f;
}

// x (|x| <= 127) as sum over n < N of l[n] / 2^7n, with int8 limbs (|l[n]| <= 64
// for n >= 1). Every step is exact in fp32 until the residual is below its ulp.
template <int N>
__device__ __forceinline__ void int8_limbs(float x, int (&l)[N]) {
#pragma unroll
    for (int n = 0; n < N; ++n) {
        const float r = rintf(x);
        l[n] = (int)r;
        x = (x - r) * 128.f;
    }
}

// Four int8 limbs as the bytes of a dword.
__device__ __forceinline__ uint32_t pack_limbs(const int (&l)[4]) {
    return ((uint32_t)l[0] & 0xffu) | (((uint32_t)l[1] & 0xffu) << 8) | (((uint32_t)l[2] & 0xffu) << 16) |
           ((uint32_t)l[3] << 24);
}

// i0 + i1/2^7 + i2/2^14 + i3/2^21, smallest weights first.
__device__ __forceinline__ float weighted(int i0, int i1, int i2, int i3) {
    return fmaf((float)i1, 1.f / 128.f, fmaf((float)i2, 1.f / 16384.f, (float)i3 * (1.f / 2097152.f))) + (float)i0;
}

__device__ __forceinline__ uint32_t put_byte(uint32_t w, int k, int v) {
    return w | (((uint32_t)v & 0xffu) << (8 * k));
}

// QJL = false scores MSE-only keys (no sign stream, no T, gamma = the key's
// norm): scores = norm M.
template <int BITS, int D, int MINW, bool QJL>
__global__ __launch_bounds__(kThreads, MINW) void score_i8_kernel(
    const float* __restrict__ A, const float* __restrict__ T,
    const uint8_t* __restrict__ idx, const uint8_t* __restrict__ sign,
    const void* __restrict__ gamma, const float* __restrict__ codebook, int C,
    float* __restrict__ scores, int B, int S, float coef) {
    using SF = SmallFmt<1, BITS, D>;
    using F = Fmt<1, BITS>;
    constexpr int NI = SF::NI, NS = SF::NS, Q = SF::Q;
    constexpr int NV = Q / 16;                     // 16-coordinate k-steps per lane, each contraction
    static_assert(Q % 32 == 0, "whole sign dwords per lane");

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
    const int r = lane & 15;                       // operand row = 4 q + limb
    const int rq = r >> 2, rt = r & 3;
    const int64_t key0 = (int64_t)p * S;

    // this lane's quarter of query rq's rows of A and T (queries past B are
    // computed from the last one and never stored)
    const int64_t qoff = ((int64_t)p * B + b0 + min(rq, nb - 1)) * D + gq * Q;
    float xa[Q], xt[Q];
#pragma unroll
    for (int k = 0; k < Q; k += 4) {
        const float4 va = *reinterpret_cast<const float4*>(A + qoff + k);
        xa[k] = va.x; xa[k + 1] = va.y; xa[k + 2] = va.z; xa[k + 3] = va.w;
        if constexpr (QJL) {
            const float4 vt = *reinterpret_cast<const float4*>(T + qoff + k);
            xt[k] = vt.x; xt[k + 1] = vt.y; xt[k + 2] = vt.z; xt[k + 3] = vt.w;
        } else {
            xt[k] = xt[k + 1] = xt[k + 2] = xt[k + 3] = 0.f;
        }
    }
    // Code buffers: each tile's codes are requested four tiles ahead (a packed
    // tile's codes are 3-5 registers a lane).
    constexpr int NBUF = 5;
    TileCodes<NI, NS> codes[NBUF];
    asm volatile("" ::: "memory");
    load_quarter<1, BITS, D, QJL>(codes[0], idx, sign, gamma, key0 + min(tile * kTileKeys16 + kc, S - 1), gq);
    asm volatile("" ::: "memory");

    // codebook limb tables: tab[m] = limb m of entries 0-3 (dword 0) and 4-7
    float cbv[8], mc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        cbv[e] = e < C ? codebook[e] : 0.f;
        mc = fmaxf(mc, fabsf(cbv[e]));
    }
    const float sc = limb_scale(mc);
    uint32_t tab[3][2] = {{0u, 0u}, {0u, 0u}, {0u, 0u}};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        int l[3];
        int8_limbs(cbv[e] * sc, l);
        tab[0][e >> 2] = put_byte(tab[0][e >> 2], e & 3, l[0]);
        tab[1][e >> 2] = put_byte(tab[1][e >> 2], e & 3, l[1]);
        tab[2][e >> 2] = put_byte(tab[2][e >> 2], e & 3, l[2]);
    }

    // row scales: maxima over the row's four quarters (lanes r, r + 16, r + 32, r + 48)
    float ma = 0.f, mt = 0.f;
#pragma unroll
    for (int k = 0; k < Q; ++k) {
        ma = fmaxf(ma, fabsf(xa[k]));
        mt = fmaxf(mt, fabsf(xt[k]));
    }
    ma = fmaxf(ma, __shfl_xor(ma, 16));
    ma = fmaxf(ma, __shfl_xor(ma, 32));
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float sA = limb_scale(ma), sT = limb_scale(mt);

    // Query operands. ca[m][v]: against codebook limb m in k-step v, row type t
    // holds limb t - m of A (zero when t < m). ts[v]: row type t holds limb t of
    // T. The four limbs of a value are packed as the bytes of a dword and picked
    // by a per-lane shift and mask, so that the selection is arithmetic. Sums of
    // T's limbs over the whole row (for sigma = 2b - 1) are reduced over the
    // quarters.
    const int sh1 = 8 * max(rt - 1, 0), sh2 = 8 * max(rt - 2, 0);
    const uint32_t mk1 = rt >= 1 ? 0xffu : 0u, mk2 = rt >= 2 ? 0xffu : 0u;
    uint32_t ca[3][NV][4], ts[NV][4];
    int tsum[4] = {0, 0, 0, 0};
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t o0 = 0u, o1 = 0u, o2 = 0u, ot = 0u;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                int la[4], lt[4];
                int8_limbs(xa[mse_dim<1, BITS>(2 * v + w / 2, 4 * (w % 2) + k)] * sA, la);
                int8_limbs(xt[32 * (v / 2) + 4 * (v % 2) + w + 8 * k] * sT, lt);
#pragma unroll
                for (int n = 0; n < 4; ++n) tsum[n] += lt[n];
                const uint32_t pa = pack_limbs(la), pt = pack_limbs(lt);
                o0 |= ((pa >> (8 * rt)) & 0xffu) << (8 * k);
                o1 |= ((pa >> sh1) & mk1) << (8 * k);
                o2 |= ((pa >> sh2) & mk2) << (8 * k);
                ot |= ((pt >> (8 * rt)) & 0xffu) << (8 * k);
            }
            ca[0][v][w] = o0;
            ca[1][v][w] = o1;
            ca[2][v][w] = o2;
            ts[v][w] = ot;
        }
#pragma unroll
    for (int n = 0; n < 4; ++n) {
        tsum[n] += __shfl_xor(tsum[n], 16);
        tsum[n] += __shfl_xor(tsum[n], 32);
    }
    // epilogue factors of output query gq (row scales of lane 4 gq, whose row is
    // query gq's): M / (sA sc) and (coef / sT) gamma (2 R_b - sum T)
    const float kx = inv_scales(__shfl(sA, 4 * gq), sc);
    const float ky = coef / __shfl(sT, 4 * gq);
    const float tsum_out = weighted(__shfl(tsum[0], 4 * gq), __shfl(tsum[1], 4 * gq), __shfl(tsum[2], 4 * gq),
                                    __shfl(tsum[3], 4 * gq));

    const __amdgpu_buffer_rsrc_t out_r = score_rows(scores + ((int64_t)p * B + b0) * S, nb, S);

    auto tile_scores = [&](const TileCodes<NI, NS>& c, int t) __attribute__((always_inline)) {
        i32x4 acc = {0, 0, 0, 0}, accs = {0, 0, 0, 0};
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            uint32_t x[4];
            F::template selectors<NI>(c.iw, 2 * v, x[0], x[1]);
            F::template selectors<NI>(c.iw, 2 * v + 1, x[2], x[3]);
#pragma unroll
            for (int m = 0; m < 3; ++m) {
                i32x4 key, q;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    key[w] = (int)perm(tab[m][1], tab[m][0], x[w]);
                    q[w] = (int)ca[m][v][w];
                }
                acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(q, key, acc, 0, 0, 0);
            }
            if constexpr (QJL) {
                const uint32_t sw = c.sw[v / 2] >> (4 * (v % 2));
                i32x4 bits, q;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    bits[d] = (int)((sw >> d) & 0x01010101u);
                    q[d] = (int)ts[v][d];
                }
                accs = __builtin_amdgcn_mfma_i32_16x16x64_i8(q, bits, accs, 0, 0, 0);
            }
        }
        // lane 16 q + key holds rows 4 q .. 4 q + 3 of column key: the weights 2^-7t
        const float M = weighted(acc[0], acc[1], acc[2], acc[3]);
        const int s = t * kTileKeys16 + kc;
        const uint32_t off = s < S ? ((uint32_t)gq * (uint32_t)S + (uint32_t)s) * 4u : kDropKey;
        if constexpr (QJL) {
            const float Rb = weighted(accs[0], accs[1], accs[2], accs[3]);
            store_score(out_r, off, fmaf(ky * c.gam, fmaf(2.f, Rb, -tsum_out), kx * M));
        } else {
            store_score(out_r, off, (kx * c.gam) * M);
        }
    };

    auto load = [&](TileCodes<NI, NS>& c, int t) __attribute__((always_inline)) {
        load_quarter<1, BITS, D, QJL>(c, idx, sign, gamma, key0 + min(min(t, ntiles - 1) * kTileKeys16 + kc, S - 1),
                                      gq);
    };
#pragma unroll
    for (int k = 1; k < NBUF - 1; ++k) load(codes[k], tile + k * stride);
    rotate_tiles<NBUF>(codes, tile, stride, ntiles, load, tile_scores);
}

template <int BITS, int D, bool QJL>
hipError_t launch_bits_d(const float* A, const float* T, KeyStreams k, const float* codebook, int C, float* scores,
                         int P, int B, int S, hipStream_t stream) {
    // without signs about 77 registers at D = 128: six wavefronts per SIMD
    constexpr int MINW = D <= 128 ? (QJL ? 4 : 6) : 2;
    const int groups_y = (B + 3) / 4;
    const int ntiles = (S + kTileKeys16 - 1) / kTileKeys16;
    int64_t gx = (ntiles + kWaves - 1) / kWaves;
    int64_t cap = 256LL * MINW / ((int64_t)groups_y * P);
    if (cap < 1) cap = 1;
    if (gx > cap) gx = cap;
    const float coef = (float)(kSqrtHalfPi / (double)D);
    hipLaunchKernelGGL((score_i8_kernel<BITS, D, MINW, QJL>), dim3((unsigned)gx, groups_y, P), dim3(kThreads), 0, stream,
                       A, T, k.idx, k.sign, k.gamma, codebook, C, scores, B, S, coef);
    return hipGetLastError();
}


template <bool QJL>
hipError_t launch_qjl(const float* A, const float* T, KeyStreams k, const float* codebook, int C, float* scores,
                      int P, int B, int S, int D, int bits, hipStream_t stream) {
    if (bits == 2 && D == 128) return launch_bits_d<2, 128, QJL>(A, T, k, codebook, C, scores, P, B, S, stream);
    if (bits == 2 && D == 256) return launch_bits_d<2, 256, QJL>(A, T, k, codebook, C, scores, P, B, S, stream);
    if (bits == 3 && D == 128) return launch_bits_d<3, 128, QJL>(A, T, k, codebook, C, scores, P, B, S, stream);
    if (bits == 3 && D == 256) return launch_bits_d<3, 256, QJL>(A, T, k, codebook, C, scores, P, B, S, stream);
    return hipErrorInvalidValue;
}

}  // namespace

bool score_i8_supported(int layout, int bits, int C, int D) {
    return layout == 1 && (bits == 2 || bits == 3) && C >= 1 && C <= 8 && (D == 128 || D == 256);
}

hipError_t launch_score_i8(const float* A, const float* T, KeyStreams k, const float* codebook, int C,
                           float* scores, int P, int B, int S, int D, int bits, bool qjl, hipStream_t stream) {
    return qjl ? launch_qjl<true>(A, T, k, codebook, C, scores, P, B, S, D, bits, stream)
               : launch_qjl<false>(A, T, k, codebook, C, scores, P, B, S, D, bits, stream);
}

}  // namespace tq
