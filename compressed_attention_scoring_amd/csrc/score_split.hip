// The outlier split ("TurboQuant: Rotate-then-Quantize KV Caches at 3 Bits",
// section 7): two MSE-only quantizer instances per head over disjoint channel
// sets, the hot channels with more bits, each with its own rotation and norm.
// A key's score is the sum of its instances' scores:
//   scores[p,b,s] = norm_hi[s] sum_i A_hi[b,i] cb_hi[idx_hi[s,i]]
//                 + norm_lo[s] sum_j A_lo[b,j] cb_lo[idx_lo[s,j]],
// with A_hi = Pi_hi q[hot channels] and A_lo = Pi_lo q[other channels].
//
// split_query_mfma_kernel: the two rotations' products on the fp32 matrix
// cores, 16x16 tiles, when both instance sizes are multiples of 16 (below).
// split_query_kernel, the other sizes: one workgroup per query; the query's
// channels, permuted so the hot ones come first, are staged in LDS and each
// output coordinate is one thread's dot product with its row of the instance's
// rotation (the instances are small and not powers of two, so a dense product).
//
// score_split_kernel: one key per lane and QB queries per pass, both instances
// in the same pass so each score is written once. The query operands are the
// same for every lane, so they are read with scalar loads and enter the FMAs
// from scalar registers; the codebooks sit in LDS; fp32 FMAs. Index rows are decoded
// eight coordinates at a time from either layout (bytes, or LSB-first 2- or
// 3-bit streams).
#include "tq_common.hpp"

namespace tq {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void split_query_kernel(const float* __restrict__ q,
                                                               const int32_t* __restrict__ perm,
                                                               const float* __restrict__ Pi_hi,
                                                               const float* __restrict__ Pi_lo,
                                                               float* __restrict__ A_hi, float* __restrict__ A_lo,
                                                               int H, int B, int D, int D_hi) {
    extern __shared__ float qs[];                 // [D] permuted query
    const int b = blockIdx.x;
    const int p = blockIdx.y;
    const int h = p % H;
    const float* src = q + ((int64_t)p * B + b) * D;
    for (int i = threadIdx.x; i < D; i += kThreads) qs[i] = src[perm[i]];
    __syncthreads();
    const int D_lo = D - D_hi;
    for (int i = threadIdx.x; i < D; i += kThreads) {
        const bool hi = i < D_hi;
        const int n = hi ? D_hi : D_lo;           // size of this coordinate's instance
        const int r = hi ? i : i - D_hi;          // its row in the instance's rotation
        const float* row = (hi ? Pi_hi + (int64_t)h * D_hi * D_hi : Pi_lo + (int64_t)h * D_lo * D_lo) + (int64_t)r * n;
        const float* x = qs + (hi ? 0 : D_hi);
        float acc = 0.f;
        for (int j = 0; j < n; ++j) acc = fmaf(row[j], x[j], acc);
        if (hi) A_hi[((int64_t)p * B + b) * D_hi + r] = acc;
        else A_lo[((int64_t)p * B + b) * D_lo + r] = acc;
    }
}

// Matrix-core form of the same products, for instance sizes that are multiples
// of 16 up to 256: one 16x16 output tile (16 query rows x 16 rows of one
// instance's rotation) per workgroup on v_mfma_f32_16x16x4_f32 (fp32 operands
// and accumulation). The instance's N coordinates are split over N / 16
// wavefronts, four consecutive coordinates per lane group of 16 lanes: lane l
// loads one 16-byte piece of rotation row l % 16, the matching four entries of
// perm and the four query values they name, for query row l % 16; the partial
// tiles are summed through LDS. Query rows are listed as in the plain
// transform: the P / H problems of a head form one list of rows when its tile
// count fits the grid (row k is query k % B of problem h + H (j0 + k / B)).
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kSplitMaxWaves = 16;                // instances up to 256 coordinates

__global__ __launch_bounds__(64 * kSplitMaxWaves) void split_query_mfma_kernel(
    const float* __restrict__ q, const int32_t* __restrict__ perm, const float* __restrict__ Pi_hi,
    const float* __restrict__ Pi_lo, float* __restrict__ A_hi, float* __restrict__ A_lo, int H, int B, int D,
    int D_hi, int PG) {
    __shared__ float part[kSplitMaxWaves][64][5];    // partial tiles, padded against bank conflicts
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int r0 = blockIdx.x * 16;               // output coordinate over [0, D): the hot instance first
    const bool hot = r0 < D_hi;
    const int N = hot ? D_hi : D - D_hi;          // the instance's size
    const int off = hot ? 0 : D_hi;               // its first entry of perm
    const int rr0 = r0 - off;                     // first row of its rotation in this tile
    const int nw = N / 16;                        // wavefronts with coordinates
    const int b0 = blockIdx.y * 16;
    const int grp = blockIdx.z;
    const int h = grp % H;
    const int64_t j0 = (int64_t)(grp / H) * PG;
    const int nrows = PG * B;
    const int i = lane & 15, g = lane >> 4;
    auto qrow = [&](int k) -> int64_t {
        return PG == 1 ? (int64_t)grp * B + k : (h + (int64_t)H * (j0 + k / B)) * B + k % B;
    };
    if (wave < nw) {
        const int k0 = wave * 16 + g * 4;         // this lane's four coordinates of the instance
        const float* rot = (hot ? Pi_hi : Pi_lo) + (int64_t)h * N * N;
        const float4 w = *reinterpret_cast<const float4*>(rot + (int64_t)(rr0 + i) * N + k0);
        const int4 c = *reinterpret_cast<const int4*>(perm + off + k0);
        const int b = b0 + i;
        const float* qr = q + qrow(b < nrows ? b : nrows - 1) * D;
        float x0 = qr[c.x], x1 = qr[c.y], x2 = qr[c.z], x3 = qr[c.w];
        if (b >= nrows) x0 = x1 = x2 = x3 = 0.f;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x0, w.x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x1, w.y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x2, w.z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x3, w.w, acc, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 4; ++v) part[wave][lane][v] = acc[v];
    }
    __syncthreads();
    // element e of the tile: lane l = e % 64 of the MFMA layout, slot v = e / 64,
    // query row 4 (l / 16) + v, rotation row rr0 + l % 16
    float* out = hot ? A_hi : A_lo;
    for (int e = tid; e < 256; e += blockDim.x) {
        const int l = e & 63, v = e >> 6;
        float y = part[0][l][v];
        for (int u = 1; u < nw; ++u) y += part[u][l][v];
        const int bb = b0 + 4 * (l >> 4) + v;
        if (bb < nrows) out[qrow(bb) * N + rr0 + (l & 15)] = y;
    }
}

// Eight consecutive coordinates (chunk j) of a key's index row in layout BITS
// (0: one byte per index).
template <int BITS>
__device__ __forceinline__ void indices8(const uint8_t* __restrict__ row, int j, int (&code)[8]) {
    if constexpr (BITS == 0) {
        const uint64_t v = *reinterpret_cast<const uint64_t*>(row + 8 * j);
#pragma unroll
        for (int t = 0; t < 8; ++t) code[t] = (int)((v >> (8 * t)) & 0xffu);
    } else {
        const uint8_t* b = row + BITS * j;        // 8 indices take BITS bytes
        uint32_t w = 0;
#pragma unroll
        for (int k = 0; k < BITS; ++k) w |= (uint32_t)b[k] << (8 * k);
#pragma unroll
        for (int t = 0; t < 8; ++t) code[t] = (int)((w >> (BITS * t)) & ((1u << BITS) - 1u));
    }
}

template <int BITS>
__device__ __forceinline__ float norm_of(const void* __restrict__ norm, int64_t key) {
    if constexpr (BITS == 0) return reinterpret_cast<const float*>(norm)[key];
    else return (float)reinterpret_cast<const _Float16*>(norm)[key];
}

// Accumulate one instance's dot products for QB queries. `A` points at row b0
// of the instance's query operands and `rows` clamps the row index; every
// address into A is the same for the whole wavefront, so those loads are scalar
// and the FMAs take their query operand from scalar registers.
template <int BITS, int QB>
__device__ __forceinline__ void instance_dots(const uint8_t* __restrict__ row, int n,
                                              const float* __restrict__ A, int rows,
                                              const float* __restrict__ cb, float (&m)[QB]) {
    for (int j = 0; j < n / 8; ++j) {
        int code[8];
        indices8<BITS>(row, j, code);
        float c[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) c[t] = cb[code[t]];
#pragma unroll
        for (int i = 0; i < QB; ++i) {
            const float* a = A + (int64_t)min(i, rows - 1) * n + 8 * j;
#pragma unroll
            for (int t = 0; t < 8; ++t) m[i] = fmaf(a[t], c[t], m[i]);
        }
    }
}

template <int BH, int BL, int QB>
__global__ __launch_bounds__(kThreads) void score_split_kernel(
    const float* __restrict__ A_hi, const float* __restrict__ A_lo, const uint8_t* __restrict__ idx_hi,
    const void* __restrict__ norm_hi, const uint8_t* __restrict__ idx_lo, const void* __restrict__ norm_lo,
    const float* __restrict__ cb_hi, int C_hi, const float* __restrict__ cb_lo, int C_lo,
    float* __restrict__ scores, int B, int S, int D_hi, int D_lo) {
    __shared__ float ch[256];
    __shared__ float cl[256];
    const int p = blockIdx.z;
    const int b0 = blockIdx.y * QB;
    const int rows = min(QB, B - b0);            // valid queries of this group
    for (int e = threadIdx.x; e < C_hi; e += kThreads) ch[e] = cb_hi[e];
    for (int e = threadIdx.x; e < C_lo; e += kThreads) cl[e] = cb_lo[e];
    __syncthreads();

    const int s = blockIdx.x * kThreads + threadIdx.x;
    if (s >= S) return;
    const int64_t key = (int64_t)p * S + s;
    const int64_t row_hi = BH == 0 ? D_hi : (int64_t)D_hi * BH / 8;
    const int64_t row_lo = BL == 0 ? D_lo : (int64_t)D_lo * BL / 8;
    float mh[QB], ml[QB];
#pragma unroll
    for (int i = 0; i < QB; ++i) mh[i] = ml[i] = 0.f;
    instance_dots<BH, QB>(idx_hi + key * row_hi, D_hi, A_hi + ((int64_t)p * B + b0) * D_hi, rows, ch, mh);
    instance_dots<BL, QB>(idx_lo + key * row_lo, D_lo, A_lo + ((int64_t)p * B + b0) * D_lo, rows, cl, ml);
    const float nh = norm_of<BH>(norm_hi, key);
    const float nl = norm_of<BL>(norm_lo, key);
#pragma unroll
    for (int i = 0; i < QB; ++i) {
        if (i < rows) scores[((int64_t)p * B + b0 + i) * S + s] = fmaf(nh, mh[i], nl * ml[i]);
    }
}

template <int BH, int BL, int QB>
hipError_t launch_split_qb(const float* A_hi, const float* A_lo, SplitStreams k, const float* cb_hi, int C_hi,
                           const float* cb_lo, int C_lo, float* scores, int P, int B, int S, int D_hi, int D_lo,
                           hipStream_t stream) {
    const dim3 grid((S + kThreads - 1) / kThreads, (B + QB - 1) / QB, P);
    hipLaunchKernelGGL((score_split_kernel<BH, BL, QB>), grid, dim3(kThreads), 0, stream, A_hi, A_lo, k.idx_hi,
                       k.norm_hi, k.idx_lo, k.norm_lo, cb_hi, C_hi, cb_lo, C_lo, scores, B, S, D_hi, D_lo);
    return hipGetLastError();
}

template <int BH, int BL>
hipError_t launch_split_bits(const float* A_hi, const float* A_lo, SplitStreams k, const float* cb_hi, int C_hi,
                             const float* cb_lo, int C_lo, float* scores, int P, int B, int S, int D_hi, int D_lo,
                             hipStream_t stream) {
    // Queries per lane: a codebook lookup serves QB FMAs, but fewer, longer query
    // groups mean fewer wavefronts. Take the largest QB that still gives about
    // 1024 workgroups (four wavefronts per SIMD); measured at B = 32, S = 32 768:
    // 10.6 us with QB = 4 against 20.2 us with QB = 16, while B = 128, S = 262 144
    // prefers 16 (144 us against 167).
    const int64_t kb = ((int64_t)S + kThreads - 1) / kThreads * P;
    if (B <= 1) return launch_split_qb<BH, BL, 1>(A_hi, A_lo, k, cb_hi, C_hi, cb_lo, C_lo, scores, P, B, S, D_hi, D_lo, stream);
    if (B <= 2) return launch_split_qb<BH, BL, 2>(A_hi, A_lo, k, cb_hi, C_hi, cb_lo, C_lo, scores, P, B, S, D_hi, D_lo, stream);
    if (B > 8 && kb * ((B + 15) / 16) >= 1024)
        return launch_split_qb<BH, BL, 16>(A_hi, A_lo, k, cb_hi, C_hi, cb_lo, C_lo, scores, P, B, S, D_hi, D_lo, stream);
    if (B > 4 && kb * ((B + 7) / 8) >= 1024)
        return launch_split_qb<BH, BL, 8>(A_hi, A_lo, k, cb_hi, C_hi, cb_lo, C_lo, scores, P, B, S, D_hi, D_lo, stream);
    return launch_split_qb<BH, BL, 4>(A_hi, A_lo, k, cb_hi, C_hi, cb_lo, C_lo, scores, P, B, S, D_hi, D_lo, stream);
}

template <int BH>
hipError_t launch_split_lo(int bits_lo, const float* A_hi, const float* A_lo, SplitStreams k, const float* cb_hi,
                           int C_hi, const float* cb_lo, int C_lo, float* scores, int P, int B, int S, int D_hi,
                           int D_lo, hipStream_t stream) {
    if (bits_lo == 0) return launch_split_bits<BH, 0>(A_hi, A_lo, k, cb_hi, C_hi, cb_lo, C_lo, scores, P, B, S, D_hi, D_lo, stream);
    if (bits_lo == 2) return launch_split_bits<BH, 2>(A_hi, A_lo, k, cb_hi, C_hi, cb_lo, C_lo, scores, P, B, S, D_hi, D_lo, stream);
    return launch_split_bits<BH, 3>(A_hi, A_lo, k, cb_hi, C_hi, cb_lo, C_lo, scores, P, B, S, D_hi, D_lo, stream);
}

}  // namespace

hipError_t launch_query_transform_split(const float* q, const int32_t* perm, const float* Pi_hi, const float* Pi_lo,
                                        float* A_hi, float* A_lo, int P, int H, int B, int D, int D_hi,
                                        hipStream_t stream) {
    const int D_lo = D - D_hi;
    if (D_hi % 16 == 0 && D_lo % 16 == 0 && D_hi <= 16 * kSplitMaxWaves && D_lo <= 16 * kSplitMaxWaves) {
        const int64_t per_head = (int64_t)(P / H) * B;
        const int PG = (per_head + 15) / 16 <= 65535 ? P / H : 1;
        const int64_t tiles = ((int64_t)PG * B + 15) / 16;
        if (tiles <= 65535) {
            const int waves = (D_hi > D_lo ? D_hi : D_lo) / 16;
            hipLaunchKernelGGL(split_query_mfma_kernel, dim3((unsigned)(D / 16), (unsigned)tiles, (unsigned)(P / PG)),
                               dim3(64 * waves), 0, stream, q, perm, Pi_hi, Pi_lo, A_hi, A_lo, H, B, D, D_hi, PG);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL(split_query_kernel, dim3((unsigned)B, (unsigned)P), dim3(kThreads), (size_t)D * sizeof(float),
                       stream, q, perm, Pi_hi, Pi_lo, A_hi, A_lo, H, B, D, D_hi);
    return hipGetLastError();
}

hipError_t launch_score_split(const float* A_hi, const float* A_lo, SplitStreams k, int bits_hi, int bits_lo,
                              const float* cb_hi, int C_hi, const float* cb_lo, int C_lo, float* scores, int P,
                              int B, int S, int D_hi, int D_lo, hipStream_t stream) {
    if (split_mfma_supported(bits_hi, C_hi, bits_lo, C_lo, D_hi, D_lo, S))
        return launch_score_split_mfma(A_hi, A_lo, k, cb_hi, C_hi, cb_lo, C_lo, scores, P, B, S, stream);
    if (bits_hi == 0) return launch_split_lo<0>(bits_lo, A_hi, A_lo, k, cb_hi, C_hi, cb_lo, C_lo, scores, P, B, S, D_hi, D_lo, stream);
    if (bits_hi == 2) return launch_split_lo<2>(bits_lo, A_hi, A_lo, k, cb_hi, C_hi, cb_lo, C_lo, scores, P, B, S, D_hi, D_lo, stream);
    return launch_split_lo<3>(bits_lo, A_hi, A_lo, k, cb_hi, C_hi, cb_lo, C_lo, scores, P, B, S, D_hi, D_lo, stream);
}

}  // namespace tq
