// Decode attention output over compressed values, the step downstream of
// scoring ("TurboQuant: Rotate-then-Quantize KV Caches at 3 Bits", section 8,
// "Kernel view: never un-rotate a key"; "Fitting 4.4x More Context on Jetson",
// the online-softmax FAQ): values are stored by the MSE quantizer (rotation
// Pi_v, codebook, one norm per vector), and
//   o_b = Pi_v^T sum_s p_bs ||v_s|| c[idx_s],   p_b = softmax(scale * scores_b).
//
// Split over key ranges (split-KV). attend_partial_kernel: one workgroup per
// (key chunk, 32-query block, problem); it finds the chunk's maximum of
// scale*score per query and the chunk's largest norm, then each wavefront owns
// 32 output coordinates and accumulates, over the chunk's 32-key tiles,
//   acc[b][d] = sum_s exp(scale*score_bs - m_b) ||v_s|| c[idx_sd]
// on the matrix cores: v_mfma_f32_32x32x16_f16 with the queries as rows, the
// wavefront's coordinates as columns and 16 keys per contraction step. Both
// operands are split into f16 hi/lo parts (three products: P_hi V_hi, P_lo V_hi,
// P_hi V_lo) after power-of-two scales: the weights are scaled so the chunk's
// largest possible weight (its largest norm) sits just below 2^14, which keeps
// every weight that matters out of f16's subnormal range. It writes
// (m, l, acc) per (chunk, query). attend_combine_kernel merges the chunks of one
// query and applies Pi_v^T once.
#include "tq_common.hpp"

namespace tq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kAttendTile = 32;           // keys per contraction tile (two MFMA steps)

union H8 {
    f16x8 h;
    uint32_t u[4];
};

__device__ __forceinline__ float pow2_below_2e14(float maxabs) {
    // a power of two bringing maxabs into [2^13, 2^14); 1 if maxabs is 0 or not finite
    if (!(maxabs > 0.f) || !(maxabs < 3.0e38f)) return 1.f;
    int e;
    (void)frexpf(maxabs, &e);
    return ldexpf(1.f, min(126, max(-126, 14 - e)));
}

// Index of coordinate d of value s. Unpacked: one byte; packed: BITS bits at
// bit BITS*d of the value's LSB-first byte string.
template <int LAYOUT, int BITS, int D>
__device__ __forceinline__ uint32_t value_index(const uint8_t* __restrict__ idx, int64_t s, int d) {
    if constexpr (LAYOUT == 0) {
        return idx[s * D + d];
    } else {
        constexpr int ROW = D * BITS / 8;
        const int bit = BITS * d;
        // two aligned dwords cover any field (rows are multiples of 4 bytes for D % 32 == 0)
        const uint32_t* w = reinterpret_cast<const uint32_t*>(idx + s * ROW) + bit / 32;
        const uint64_t both = (uint64_t)w[0] | ((bit % 32 > 32 - BITS) ? (uint64_t)w[1] << 32 : 0ull);
        return (uint32_t)(both >> (bit % 32)) & ((1u << BITS) - 1u);
    }
}

template <int LAYOUT>
__device__ __forceinline__ float value_norm(const void* __restrict__ norm, int64_t s) {
    if constexpr (LAYOUT == 0) return reinterpret_cast<const float*>(norm)[s];
    else return (float)reinterpret_cast<const _Float16*>(norm)[s];
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

template <int LAYOUT, int BITS, int D>
__global__ __launch_bounds__(D * 2) void attend_partial_kernel(
    const float* __restrict__ scores, const uint8_t* __restrict__ idx, const void* __restrict__ norm,
    const float* __restrict__ codebook, int C, float scale, float* __restrict__ ws,
    int B, int S, int chunk, int nchunks) {
    constexpr int NW = D / 32;               // wavefronts: one per 32 output coordinates
    constexpr int NT = NW * 64;
    __shared__ float red[NT];
    __shared__ float rowmax[32];
    __shared__ float sh_nmax;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = blockIdx.x;
    const int b0 = blockIdx.y * 32;
    const int p = blockIdx.z;
    const int rows = min(32, B - b0);
    const int s_begin = c * chunk;
    const int s_end = min(S, s_begin + chunk);
    const int64_t key0 = (int64_t)p * S;
    const float* sc_p = scores + ((int64_t)p * B + b0) * S;

    // ---- chunk maxima: m_b = max scale*score (rows past B read row rows-1) and
    //      the largest norm
    {
        const int b = tid % 32, part = tid / 32;
        const float* row = sc_p + (int64_t)min(b, rows - 1) * S;
        float m = -INFINITY;
        for (int s = s_begin + part; s < s_end; s += NT / 32) m = fmaxf(m, scale * row[s]);
        red[tid] = m;
        float n = 0.f;
        for (int s = s_begin + tid; s < s_end; s += NT) n = fmaxf(n, fabsf(value_norm<LAYOUT>(norm, key0 + s)));
        __syncthreads();
        if (tid < 32) {
            float mm = red[tid];
            for (int k = 1; k < NT / 32; ++k) mm = fmaxf(mm, red[tid + 32 * k]);
            rowmax[tid] = mm;
        }
        __syncthreads();
        red[tid] = n;
        __syncthreads();
        if (tid == 0) {
            float nn = 0.f;
            for (int k = 0; k < NT; ++k) nn = fmaxf(nn, red[k]);
            sh_nmax = nn;
        }
        __syncthreads();
    }
    const float wscale = pow2_below_2e14(sh_nmax);    // weights p' * wscale stay below 2^14

    // codebook scale and byte tables (hi and lo f16 parts)
    float cbv[8];
    float mc = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        cbv[k] = k < C ? codebook[k] : 0.f;
        mc = fmaxf(mc, fabsf(cbv[k]));
    }
    const float cscale = pow2_below_2e14(mc);
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

    // ---- accumulate: lane (query r = lane % 32, key group g = lane / 32) for the
    //      A operand; lane (coordinate d = 32 wave + lane % 32, key group g) for B
    const int r = lane & 31;
    const int g = lane >> 5;
    const int d = 32 * wave + r;
    const float mr = rowmax[r];
    const float* srow = sc_p + (int64_t)min(r, rows - 1) * S;
    f32x16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;
    float lsum = 0.f;                          // sum of exp over this lane's keys (query r)
    for (int t0 = s_begin; t0 < s_end; t0 += kAttendTile) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int sb = t0 + 16 * ks + 8 * g;   // this lane's 8 keys of the step
            H8 phi, plo, vhi, vlo;
            uint32_t sel0 = 0, sel1 = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int s = sb + e;
                const bool in = s < s_end;
                const int sc_ = in ? s : s_end - 1;
                const float w = in ? __expf(scale * srow[sc_] - mr) : 0.f;
                lsum += w;
                const float x = w * value_norm<LAYOUT>(norm, key0 + sc_) * wscale;
                const _Float16 h = (_Float16)x;
                phi.h[e] = h;
                plo.h[e] = (_Float16)(x - (float)h);
                const uint32_t iv = value_index<LAYOUT, BITS, D>(idx, key0 + sc_, d);
                if (e < 4) sel0 |= iv << (8 * e);
                else sel1 |= iv << (8 * (e - 4));
            }
            lut4(sel0, tab_hi, vhi.u[0], vhi.u[1]);
            lut4(sel1, tab_hi, vhi.u[2], vhi.u[3]);
            lut4(sel0, tab_lo, vlo.u[0], vlo.u[1]);
            lut4(sel1, tab_lo, vlo.u[2], vlo.u[3]);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(phi.h, vhi.h, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(plo.h, vhi.h, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(phi.h, vlo.h, acc, 0, 0, 0);
        }
    }
    // l_b: the two key groups of query r sit in lanes r and r + 32
    lsum += __shfl_xor(lsum, 32);

    // ---- write (m, l, acc) of this chunk: ws layout [P][B][nchunks][D + 2]
    const float unscale = 1.f / (wscale * cscale);   // powers of two: exact
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int row = 8 * (v >> 2) + 4 * g + (v & 3);   // output element v: query row, coordinate d
        if (row < rows) {
            float* rec = ws + (((int64_t)p * B + b0 + row) * nchunks + c) * (D + 2);
            rec[2 + 32 * wave + r] = acc[v] * unscale;
        }
    }
    if (wave == 0 && g == 0 && r < rows) {
        float* rec = ws + (((int64_t)p * B + b0 + r) * nchunks + c) * (D + 2);
        rec[0] = mr;
        rec[1] = lsum;
    }
}

template <int D>
__global__ __launch_bounds__(D) void attend_combine_kernel(const float* __restrict__ ws, const float* __restrict__ Pi_v,
                                                           float* __restrict__ out, int H, int B, int nchunks) {
    __shared__ float a[D];
    const int j = threadIdx.x;
    const int b = blockIdx.x;
    const int p = blockIdx.y;
    const float* rec = ws + ((int64_t)p * B + b) * nchunks * (D + 2);
    float M = -INFINITY;
    for (int c = 0; c < nchunks; ++c) M = fmaxf(M, rec[c * (D + 2)]);
    float num = 0.f, den = 0.f;
    for (int c = 0; c < nchunks; ++c) {
        const float f = __expf(rec[c * (D + 2)] - M);
        den = fmaf(rec[c * (D + 2) + 1], f, den);
        num = fmaf(rec[c * (D + 2) + 2 + j], f, num);
    }
    a[j] = num / den;
    __syncthreads();
    // o_j = sum_d Pi_v[d][j] a_d
    const float* P = Pi_v + (int64_t)(p % H) * D * D;
    float o = 0.f;
    for (int dd = 0; dd < D; ++dd) o = fmaf(P[(int64_t)dd * D + j], a[dd], o);
    out[((int64_t)p * B + b) * D + j] = o;
}

template <int LAYOUT, int BITS, int D>
hipError_t launch_attend_d(const float* scores, ValueStreams v, const float* codebook, int C, const float* Pi_v,
                           float scale, float* out, float* ws, int P, int H, int B, int S, hipStream_t stream) {
    const int nch = attend_chunks(P, B, S);
    const int chunk = ((S + nch - 1) / nch + kAttendTile - 1) / kAttendTile * kAttendTile;
    const int used = (S + chunk - 1) / chunk;
    hipLaunchKernelGGL((attend_partial_kernel<LAYOUT, BITS, D>), dim3((unsigned)used, (B + 31) / 32, P), dim3(D * 2),
                       0, stream, scores, v.idx, v.norm, codebook, C, scale, ws, B, S, chunk, used);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attend_combine_kernel<D>), dim3((unsigned)B, P), dim3(D), 0, stream, ws, Pi_v, out, H, B,
                       used);
    return hipGetLastError();
}

template <int LAYOUT, int BITS>
hipError_t launch_attend_layout(const float* scores, ValueStreams v, const float* codebook, int C, const float* Pi_v,
                                float scale, float* out, float* ws, int P, int H, int B, int S, int D,
                                hipStream_t stream) {
    if (D == 64) return launch_attend_d<LAYOUT, BITS, 64>(scores, v, codebook, C, Pi_v, scale, out, ws, P, H, B, S, stream);
    return launch_attend_d<LAYOUT, BITS, 128>(scores, v, codebook, C, Pi_v, scale, out, ws, P, H, B, S, stream);
}

}  // namespace

// Key chunks per (problem, 32-query block): enough workgroups to fill the chip
// (about 512), each chunk at least one 32-key tile.
int attend_chunks(int P, int B, int S) {
    const int64_t blocks = (int64_t)P * ((B + 31) / 32);
    int64_t n = (512 + blocks - 1) / blocks;
    const int64_t tiles = (S + kAttendTile - 1) / kAttendTile;
    if (n > tiles) n = tiles;
    if (n < 1) n = 1;
    return (int)n;
}

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
