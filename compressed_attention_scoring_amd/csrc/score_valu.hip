// Scoring kernel, vector-ALU family: any D, any B, both key layouts.
//
// Computes, for one problem p and one key s per lane,
//   scores[p,b,s] = sum_d A[p,b,d] codebook[idx[s,d]]
//                 + (sqrt(pi/2)/D) gamma[s] sum_d T[p,b,d] sigma[s,d]
// ("TurboQuant Attention in CUDA: Transform the Query, Reuse the Work",
// sections "Two kernels, two jobs" and "Full CUDA solution"), in fp32 with
// fp32 accumulation.
//
// Differences from the page's kernel, which gives each (query, key) pair its
// own thread: a lane owns one key and QB queries, so the key's codes are read
// once per query group instead of once per query; A and T of the query group
// sit in LDS laid out [d][query] so one broadcast read serves the whole
// wavefront; the codebook sits in LDS. Packed indices are unpacked from their
// LSB-first bitstream in registers ("Fitting 4.4x More Context on Jetson",
// section "v6: Fused Vectorized Hybrid", extracts 2-bit fields the same way).
//
// This family is the general fallback (odd D, tiny problems); the matrix-core
// families (dispatched by score_mfma.hip) are the fast path where it applies.
#include "tq_common.hpp"

namespace tq {
namespace {

constexpr int kThreads = 256;

// Decode the 8 coordinates of chunk j of key `key` into byte indices and +-1 signs.
template <int LAYOUT, int BITS>
__device__ __forceinline__ void decode_chunk8(const uint8_t* __restrict__ idx,
                                              const uint8_t* __restrict__ sign,
                                              int64_t key, int D, int j,
                                              int (&code)[8], float (&sg)[8]) {
    if constexpr (LAYOUT == 0) {
        const uint64_t iv = *reinterpret_cast<const uint64_t*>(idx + key * D + 8 * j);
        const uint64_t sv = *reinterpret_cast<const uint64_t*>(sign + key * D + 8 * j);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            code[t] = (int)((iv >> (8 * t)) & 0xffu);
            const int8_t sb = (int8_t)((sv >> (8 * t)) & 0xffu);
            sg[t] = (float)sb;
        }
    } else {
        const int64_t row = (int64_t)D * BITS / 8;
        const uint8_t* ip = idx + key * row + (int64_t)BITS * j;
        uint32_t w = 0;
#pragma unroll
        for (int k = 0; k < BITS; ++k) w |= (uint32_t)ip[k] << (8 * k);
        const uint32_t sb = sign[key * (D / 8) + j];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            code[t] = (int)((w >> (BITS * t)) & ((1u << BITS) - 1u));
            sg[t] = ((sb >> t) & 1u) ? 1.0f : -1.0f;
        }
    }
}

template <int LAYOUT, int BITS, int QB>
__global__ __launch_bounds__(kThreads) void score_valu_kernel(
    const float* __restrict__ A, const float* __restrict__ T,
    const uint8_t* __restrict__ idx, const uint8_t* __restrict__ sign,
    const void* __restrict__ gamma, const float* __restrict__ codebook, int C,
    float* __restrict__ scores, int B, int S, int D, float coef) {
    extern __shared__ float lds[];
    float* At = lds;               // [D][QB]
    float* Tt = lds + D * QB;      // [D][QB]
    float* cb = lds + 2 * D * QB;  // [C]

    const int p = blockIdx.z;
    const int b0 = blockIdx.y * QB;
    for (int e = threadIdx.x; e < QB * D; e += kThreads) {
        const int i = e / D, d = e % D;
        const int b = b0 + i;
        float a = 0.f, t = 0.f;
        if (b < B) {
            const int64_t o = ((int64_t)p * B + b) * D + d;
            a = A[o];
            t = T[o];
        }
        At[d * QB + i] = a;
        Tt[d * QB + i] = t;
    }
    for (int e = threadIdx.x; e < C; e += kThreads) cb[e] = codebook[e];
    __syncthreads();

    const int s = blockIdx.x * kThreads + threadIdx.x;
    if (s >= S) return;
    const int64_t key = (int64_t)p * S + s;

    float m[QB], r[QB];
#pragma unroll
    for (int i = 0; i < QB; ++i) m[i] = r[i] = 0.f;

    const bool chunked = (D % 8) == 0;
    const int full = chunked ? D / 8 : 0;
    for (int j = 0; j < full; ++j) {
        int code[8];
        float sg[8];
        decode_chunk8<LAYOUT, BITS>(idx, sign, key, D, j, code, sg);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int d = 8 * j + t;
            const float c = cb[code[t]];
#pragma unroll
            for (int i = 0; i < QB; ++i) {
                m[i] = fmaf(At[d * QB + i], c, m[i]);
                r[i] = fmaf(Tt[d * QB + i], sg[t], r[i]);
            }
        }
    }
    if constexpr (LAYOUT == 0) {
        // coordinates not covered by whole 8-byte chunks (only when D % 8 != 0)
        for (int d = 8 * full; d < D; ++d) {
            const float c = cb[idx[key * D + d]];
            const float sgv = (float)(int8_t)sign[key * D + d];
#pragma unroll
            for (int i = 0; i < QB; ++i) {
                m[i] = fmaf(At[d * QB + i], c, m[i]);
                r[i] = fmaf(Tt[d * QB + i], sgv, r[i]);
            }
        }
    }

    float g;
    if constexpr (LAYOUT == 0) g = reinterpret_cast<const float*>(gamma)[key];
    else g = (float)reinterpret_cast<const _Float16*>(gamma)[key];
    const float scale = coef * g;
#pragma unroll
    for (int i = 0; i < QB; ++i) {
        const int b = b0 + i;
        if (b < B) scores[((int64_t)p * B + b) * S + s] = fmaf(scale, r[i], m[i]);
    }
}

template <int LAYOUT, int BITS, int QB>
hipError_t launch_qb(const float* A, const float* T, KeyStreams k, const float* codebook,
                     int C, float* scores, int P, int B, int S, int D, hipStream_t stream) {
    dim3 grid((S + kThreads - 1) / kThreads, (B + QB - 1) / QB, P);
    const size_t lds = (size_t)(2 * D * QB + C) * sizeof(float);
    const float coef = (float)(kSqrtHalfPi / (double)D);
    hipLaunchKernelGGL((score_valu_kernel<LAYOUT, BITS, QB>), grid, dim3(kThreads), lds, stream,
                       A, T, k.idx, k.sign, k.gamma, codebook, C, scores, B, S, D, coef);
    return hipGetLastError();
}

template <int LAYOUT, int BITS>
hipError_t launch_layout(const float* A, const float* T, KeyStreams k, const float* codebook,
                         int C, float* scores, int P, int B, int S, int D, hipStream_t stream) {
    // queries per lane: enough to cover small B without idle slots; LDS holds
    // 2*D*QB floats, so large D takes fewer queries per pass
    const int cap = D > 512 ? 4 : 8;
    if (B <= 1) return launch_qb<LAYOUT, BITS, 1>(A, T, k, codebook, C, scores, P, B, S, D, stream);
    if (B <= 2) return launch_qb<LAYOUT, BITS, 2>(A, T, k, codebook, C, scores, P, B, S, D, stream);
    if (B <= 4 || cap == 4)
        return launch_qb<LAYOUT, BITS, 4>(A, T, k, codebook, C, scores, P, B, S, D, stream);
    return launch_qb<LAYOUT, BITS, 8>(A, T, k, codebook, C, scores, P, B, S, D, stream);
}

}  // namespace

hipError_t launch_score_valu(const float* A, const float* T, KeyStreams keys,
                             int layout, int bits, const float* codebook, int C,
                             float* scores, int P, int B, int S, int D,
                             hipStream_t stream) {
    if (layout == 0)
        return launch_layout<0, 0>(A, T, keys, codebook, C, scores, P, B, S, D, stream);
    if (bits == 2)
        return launch_layout<1, 2>(A, T, keys, codebook, C, scores, P, B, S, D, stream);
    return launch_layout<1, 3>(A, T, keys, codebook, C, scores, P, B, S, D, stream);
}

}  // namespace tq
