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
    const int gq = lane >> 4;                      // lane group: coordinate quarter / output query
    const int kc = lane & 15;                      // key column
    const int r = lane & 15;                       // operand row = 4 q + limb
    const int rq = r >> 2, rt = r & 3;
    const int64_t key0 = (int64_t)p * S;

    constexpr int NBUF = 5;
    TileCodes<NI, NS> codes[NBUF];
    // This lane's quarter of tile t's codes, through descriptors that cover the
    // tile's keys: a tile past the end, and keys past S, load nothing.
    constexpr int IQ = SF::IDX_ROW / 4, SQ = SF::SIGN_ROW / 4;
    const uint32_t ioff = (uint32_t)(kc * SF::IDX_ROW + gq * IQ);
    const uint32_t soff = (uint32_t)(kc * SF::SIGN_ROW + gq * SQ);
    auto load = [&](TileCodes<NI, NS>& c, int t) __attribute__((always_inline)) {
        const int nk = __builtin_amdgcn_readfirstlane(max(0, min(kTileKeys16, S - t * kTileKeys16)));
        const int64_t k0 = key0 + (nk > 0 ? (int64_t)t * kTileKeys16 : 0);
        buffer_dwords<NI>(key_rows(idx + k0 * SF::IDX_ROW, nk, SF::IDX_ROW), ioff, c.iw);
        if constexpr (QJL) buffer_dwords<NS>(key_rows(sign + k0 * SF::SIGN_ROW, nk, SF::SIGN_ROW), soff, c.sw);
        const uint16_t h = __builtin_amdgcn_raw_buffer_load_b16(
            key_rows(static_cast<const _Float16*>(gamma) + k0, nk, 2), (uint32_t)kc * 2u, 0, 0);
        c.gam = (float)__builtin_bit_cast(_Float16, h);
    };

    // The query operands are the same for the four wavefronts of the workgroup,
    // and a limb decomposition serves the four lanes that differ only in the
    // limb they take; so the workgroup decomposes each of the 8 D values of its
    // four rows of A and T once into a shared table, and every lane then
    // gathers its operand bytes from it. Thread t takes VPT consecutive
    // coordinates of row (t / 32) % 4 of A (t < 128) or T; a row's 32 threads
    // share a half wavefront, so its maximum and its limb sums reduce over it.
    // Rows past B re-read the last query and are never stored.
    constexpr int VPT = D / 32;                    // values per thread
    constexpr int QP = Q + 1;                      // table stride of a quarter row (bank spread)
    constexpr int RS = 4 * QP + 4;                 // table stride of a row
    __shared__ uint32_t limbs[2][4 * RS];          // [A or T][row, quarter, coordinate]: four int8 limbs
    __shared__ float row_scale[2][4];
    __shared__ int row_tsum[4][4];
    {
        const int t = threadIdx.x;
        const int type = t >> 7, row = (t >> 5) & 3, c0 = (t & 31) * VPT;
        const float* src = (type == 0 ? A : T) + ((int64_t)p * B + b0 + min(row, nb - 1)) * D + c0;
        float x[VPT];
        if (type == 0 || QJL) {
#pragma unroll
            for (int k = 0; k < VPT; k += 4) {
                const float4 v = *reinterpret_cast<const float4*>(src + k);
                x[k] = v.x; x[k + 1] = v.y; x[k + 2] = v.z; x[k + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int k = 0; k < VPT; ++k) x[k] = 0.f;
        }
        // Code buffers: each tile's codes are requested four tiles ahead (a
        // packed tile's codes are 3-5 registers a lane); the first tile's right
        // behind this thread's row values, so the table waits for those only.
        asm volatile("" ::: "memory");
        load(codes[0], tile);
        asm volatile("" ::: "memory");
        float m = 0.f;
#pragma unroll
        for (int k = 0; k < VPT; ++k) m = fmaxf(m, fabsf(x[k]));
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
        const float sx = limb_scale(m);
        int ls[4] = {0, 0, 0, 0};
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            int l[4];
            int8_limbs(x[k] * sx, l);
#pragma unroll
            for (int n = 0; n < 4; ++n) ls[n] += l[n];
            const int c = c0 + k;
            limbs[type][row * RS + (c / Q) * QP + c % Q] = pack_limbs(l);
        }
        if (type == 1) {                           // uniform: wavefronts 2 and 3
#pragma unroll
            for (int n = 0; n < 4; ++n)
#pragma unroll
                for (int o = 1; o < 32; o <<= 1) ls[n] += __shfl_xor(ls[n], o);
        }
        if ((t & 31) == 0) {
            row_scale[type][row] = sx;
            if (type == 1) {
#pragma unroll
                for (int n = 0; n < 4; ++n) row_tsum[row][n] = ls[n];
            }
        }
    }

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
    __syncthreads();
    if (tile >= ntiles) return;                    // after the only barrier of this kernel

    // Query operands. ca[m][v]: against codebook limb m in k-step v, row type t
    // holds limb t - m of A (zero when t < m). ts[v]: row type t holds limb t of
    // T. Byte k of an operand dword is a byte of coordinate k's limb dword:
    // two byte permutes pick it from four table words (selector byte 12 gives 0).
    auto gather = [](const uint32_t (&d)[4], uint32_t sel_lo, uint32_t sel_hi) __attribute__((always_inline)) {
        return perm(d[1], d[0], sel_lo) | perm(d[3], d[2], sel_hi);
    };
    auto sels = [](int b, uint32_t& lo, uint32_t& hi) __attribute__((always_inline)) {
        lo = b < 0 ? 0x0C0C0C0Cu : (uint32_t)b | ((uint32_t)(4 + b) << 8) | 0x0C0C0000u;
        hi = b < 0 ? 0x0C0C0C0Cu : 0x00000C0Cu | ((uint32_t)b << 16) | ((uint32_t)(4 + b) << 24);
    };
    uint32_t sl[3], sh[3];
#pragma unroll
    for (int m = 0; m < 3; ++m) sels(rt - m, sl[m], sh[m]);
    const uint32_t* la_row = &limbs[0][rq * RS + gq * QP];
    const uint32_t* lt_row = &limbs[1][rq * RS + gq * QP];
    uint32_t ca[3][NV][4], ts[NV][4];
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t da[4], dt[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                da[k] = la_row[mse_dim<1, BITS>(2 * v + w / 2, 4 * (w % 2) + k)];
                if constexpr (QJL) dt[k] = lt_row[32 * (v / 2) + 4 * (v % 2) + w + 8 * k];
            }
#pragma unroll
            for (int m = 0; m < 3; ++m) ca[m][v][w] = gather(da, sl[m], sh[m]);
            if constexpr (QJL) ts[v][w] = gather(dt, sl[0], sh[0]);
        }
    // epilogue factors of output query gq: M / (sA sc) and (coef / sT) gamma (2 R_b - sum T)
    const float kx = inv_scales(row_scale[0][gq], sc);
    const float ky = coef / row_scale[1][gq];
    float tsum_out = 0.f;
    if constexpr (QJL) tsum_out = weighted(row_tsum[gq][0], row_tsum[gq][1], row_tsum[gq][2], row_tsum[gq][3]);

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
