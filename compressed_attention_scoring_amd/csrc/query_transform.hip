// Query transform: A = Pi q and T = S_mat q, once per query.
//
// "TurboQuant Attention in CUDA: Transform the Query, Reuse the Work",
// section "Move the transforms to the query": the rotation and the QJL
// projection move onto the query side, so every cached key reuses A and T.
// "Fitting 4.4x More Context on Jetson", section "v3: Combined Transform",
// stacks both matrices into one operand; the same is done here: the rows of
// W_h = [Pi_h ; S_mat_h] (2D x D) produce [A | T] in one fp32 product
// Y[p, b, r] = sum_j W_h[r, j] q[p, b, j], r < 2D.
//
// The product is tiny (4 P B D^2 flops) and latency-bound, so both variants are
// shaped for few dependent memory rounds. D a multiple of 32 up to 256 runs on
// the matrix cores (query_transform_mfma16_kernel below). Other D use the vector
// kernel: a 256-lane workgroup owns 16 rows of W and 32 queries of one problem;
// its operands are requested in one round of loads into LDS per 256 columns,
// then every lane forms two outputs from broadcast LDS reads with eight
// independent fp32 FMA chains.
#include "tq_common.hpp"

namespace tq {
namespace {

constexpr int kRows = 16;      // rows of W per workgroup
constexpr int kQueries = 32;   // queries per workgroup
constexpr int kChunk = 256;    // K columns staged per round
constexpr int kPad = 4;        // LDS row padding (floats) against bank conflicts

__global__ __launch_bounds__(256) void query_transform_kernel(
    const float* __restrict__ q, const float* __restrict__ Pi,
    const float* __restrict__ S_mat, float* __restrict__ A, float* __restrict__ T,
    int H, int B, int D) {
    extern __shared__ float lds[];
    const int kc_max = D < kChunk ? D : kChunk;
    const int ld = ((kc_max + 3) & ~3) + kPad;   // a multiple of 4 floats: 16-byte LDS reads stay aligned
    float* Ws = lds;                    // [kRows][ld]
    float* Qs = lds + kRows * ld;       // [kQueries][ld]

    const int tid = threadIdx.x;
    const int r0 = blockIdx.x * kRows;
    const int b0 = blockIdx.y * kQueries;
    const int p = blockIdx.z;
    const int h = p % H;
    const int twoD = 2 * D;
    const float* Pi_h = Pi + (int64_t)h * D * D;
    const float* S_h = S_mat + (int64_t)h * D * D;
    const float* q_p = q + (int64_t)p * B * D;

    const int r = tid % kRows;          // W row of this lane
    const int bq = tid / kRows;         // queries bq and bq + 16
    float acc0[4] = {0.f, 0.f, 0.f, 0.f}, acc1[4] = {0.f, 0.f, 0.f, 0.f};

    for (int j0 = 0; j0 < D; j0 += kChunk) {
        const int kc = min(kChunk, D - j0);
        const bool vec = (kc % 4) == 0 && (D % 4) == 0;
        if (vec) {
            const int n4 = kc / 4;
            for (int e = tid; e < kRows * n4; e += 256) {
                const int row = e / n4, c4 = e % n4;
                const int rr = r0 + row;
                float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                if (rr < twoD) {
                    const float* src = rr < D ? Pi_h + (int64_t)rr * D : S_h + (int64_t)(rr - D) * D;
                    v = *reinterpret_cast<const float4*>(src + j0 + 4 * c4);
                }
                *reinterpret_cast<float4*>(Ws + row * ld + 4 * c4) = v;
            }
            for (int e = tid; e < kQueries * n4; e += 256) {
                const int row = e / n4, c4 = e % n4;
                const int b = b0 + row;
                float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                if (b < B) v = *reinterpret_cast<const float4*>(q_p + (int64_t)b * D + j0 + 4 * c4);
                *reinterpret_cast<float4*>(Qs + row * ld + 4 * c4) = v;
            }
        } else {
            for (int e = tid; e < kRows * kc; e += 256) {
                const int row = e / kc, c = e % kc;
                const int rr = r0 + row;
                float v = 0.f;
                if (rr < twoD) v = rr < D ? Pi_h[(int64_t)rr * D + j0 + c] : S_h[(int64_t)(rr - D) * D + j0 + c];
                Ws[row * ld + c] = v;
            }
            for (int e = tid; e < kQueries * kc; e += 256) {
                const int row = e / kc, c = e % kc;
                const int b = b0 + row;
                Qs[row * ld + c] = b < B ? q_p[(int64_t)b * D + j0 + c] : 0.f;
            }
            // zero the tail so the 4-wide loop below reads defined values
            for (int e = tid; e < (kRows + kQueries) * 4; e += 256) {
                const int row = e / 4, c = kc + e % 4;
                if (c < ld) lds[row * ld + c] = 0.f;
            }
        }
        __syncthreads();
        const float* w = Ws + r * ld;
        const float* qa = Qs + bq * ld;
        const float* qb = Qs + (bq + 16) * ld;
        for (int j = 0; j < kc; j += 4) {
            const float4 wv = *reinterpret_cast<const float4*>(w + j);
            const float4 av = *reinterpret_cast<const float4*>(qa + j);
            const float4 bv = *reinterpret_cast<const float4*>(qb + j);
            acc0[0] = fmaf(wv.x, av.x, acc0[0]);
            acc0[1] = fmaf(wv.y, av.y, acc0[1]);
            acc0[2] = fmaf(wv.z, av.z, acc0[2]);
            acc0[3] = fmaf(wv.w, av.w, acc0[3]);
            acc1[0] = fmaf(wv.x, bv.x, acc1[0]);
            acc1[1] = fmaf(wv.y, bv.y, acc1[1]);
            acc1[2] = fmaf(wv.z, bv.z, acc1[2]);
            acc1[3] = fmaf(wv.w, bv.w, acc1[3]);
        }
        __syncthreads();
    }

    const int rr = r0 + r;
    if (rr >= twoD) return;
    float* out = rr < D ? A : T;
    const int d = rr < D ? rr : rr - D;
    const float y0 = (acc0[0] + acc0[1]) + (acc0[2] + acc0[3]);
    const float y1 = (acc1[0] + acc1[1]) + (acc1[2] + acc1[3]);
    if (b0 + bq < B) out[((int64_t)p * B + b0 + bq) * D + d] = y0;
    if (b0 + bq + 16 < B) out[((int64_t)p * B + b0 + bq + 16) * D + d] = y1;
}

// Matrix-core variant for D a multiple of 32 up to 256: one 16x16 tile of Y
// (16 queries x 16 rows of W) per workgroup, contracted with fp32 MFMA
// (v_mfma_f32_16x16x4_f32: fp32 operands, fp32 accumulation, so no operand
// splitting is needed). The contraction over D is split across NW wavefronts
// (D / NW coordinates each, KM = D / (4 NW) per lane group of 16 lanes); every
// lane loads its operands for the whole contraction with 16-byte loads in one
// round, and the NW partial tiles are summed through LDS. Lane l feeds query
// row l % 16 and W row l % 16 with the KM consecutive coordinates
// k0 + KM (l / 16) + m, and MFMA m contracts coordinate m of every lane group,
// so both operands take the same order. Queries are the MFMA rows and W rows
// the columns: each query's outputs are written as contiguous 64-byte runs.
// Small tiles keep the chain short: at 32 queries and D = 128 the grid has 32
// workgroups, each with 8 KiB of operands and 8 dependent MFMAs per wavefront.
//
// Query rows of a workgroup: problems that share a head use the same W, so a
// group of PG of them (problems h + H j, j = j0 .. j0 + PG - 1, for head h)
// forms one list of PG * B query rows, cut into 16-row tiles: a few queries per
// problem (GQA) still fill the MFMA rows. Row k of group g is query k % B of
// problem h + H (j0 + k / B), with h = g % H and j0 = (g / H) PG.
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void query_transform_mfma16_kernel(
    const float* __restrict__ q, const float* __restrict__ Pi,
    const float* __restrict__ S_mat, float* __restrict__ A, float* __restrict__ T,
    int H, int B, int PG) {
    constexpr int KM = D / (4 * NW);
    static_assert(D % (16 * NW) == 0, "KM must be a whole number of float4s");
    __shared__ float part[NW][64][5];             // partial tiles, padded against bank conflicts
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int r0 = blockIdx.x * 16;
    const int b0 = blockIdx.y * 16;
    const int grp = blockIdx.z;
    const int h = grp % H;
    const int64_t j0 = (int64_t)(grp / H) * PG;
    const int nrows = PG * B;
    const int i = lane & 15, g = lane >> 4;
    const int k0 = wave * (D / NW) + g * KM;
    auto qrow = [&](int k) -> int64_t {
        return PG == 1 ? (int64_t)grp * B + k : (h + (int64_t)H * (j0 + k / B)) * B + k % B;
    };

    const int wr = r0 + i;                        // always < 2D: the grid has 2D / 16 column tiles
    const float* wsrc = wr < D ? Pi + ((int64_t)h * D + wr) * D : S_mat + ((int64_t)h * D + wr - D) * D;
    const int b = b0 + i;
    const int bc = b < nrows ? b : nrows - 1;
    const float* qsrc = q + qrow(bc) * D;
    float wv[KM], qv[KM];
#pragma unroll
    for (int k = 0; k < KM; k += 4) {
        const float4 x = *reinterpret_cast<const float4*>(wsrc + k0 + k);
        const float4 y = *reinterpret_cast<const float4*>(qsrc + k0 + k);
        wv[k] = x.x; wv[k + 1] = x.y; wv[k + 2] = x.z; wv[k + 3] = x.w;
        qv[k] = y.x; qv[k + 1] = y.y; qv[k + 2] = y.z; qv[k + 3] = y.w;
    }
    if (b >= nrows) {
#pragma unroll
        for (int k = 0; k < KM; ++k) qv[k] = 0.f;
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KM; ++k) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qv[k], wv[k], acc, 0, 0, 0);
#pragma unroll
    for (int v = 0; v < 4; ++v) part[wave][lane][v] = acc[v];
    __syncthreads();
    // element e of the tile -> (lane l of the tile layout, accumulator slot v): row 4 (l / 16) + v, column l % 16
    const int l = tid & 63;
    const int wcol = r0 + (l & 15);
    float* out = wcol < D ? A : T;
    const int d = wcol < D ? wcol : wcol - D;
    for (int e = tid; e < 256; e += 64 * NW) {
        const int v = e >> 6;
        float y = part[0][l][v];
#pragma unroll
        for (int w = 1; w < NW; ++w) y += part[w][l][v];
        const int bb = b0 + 4 * (l >> 4) + v;
        if (bb < nrows) out[qrow(bb) * D + d] = y;
    }
}

// Randomized Hadamard query transform A = H (signs * q) with H the orthonormal
// Walsh-Hadamard matrix in Sylvester order ("TurboQuant: Rotate-then-Quantize
// KV Caches at 3 Bits", section 2: y = H D x, O(d log d)). One wavefront per
// query; lane l holds coordinates E*l .. E*l+E-1 (E = D/64, at least 1). The
// butterfly at distance h pairs coordinates i and i+h (bit h of i clear):
// (x_i + x_(i+h), x_i - x_(i+h)); distances below E stay inside a lane, larger
// ones pair lane l with lane l ^ (h/E). The 1/sqrt(D) normalisation comes last.
template <int D>
__global__ __launch_bounds__(256) void hadamard_query_kernel(const float* __restrict__ q,
                                                             const float* __restrict__ signs,
                                                             float* __restrict__ A, int H, int B, int NQ) {
    constexpr int E = D >= 64 ? D / 64 : 1;
    const int lane = threadIdx.x & 63;
    const int qi = blockIdx.x * 4 + (threadIdx.x >> 6);     // query index over all problems
    if (qi >= NQ) return;                                     // whole wavefronts leave together
    const int p = qi / B;
    const float* src = q + (int64_t)qi * D;
    const float* sg = signs + (int64_t)(p % H) * D;
    const bool active = lane * E < D;
    float x[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int i = min(lane * E + e, D - 1);
        x[e] = active ? src[i] * sg[i] : 0.f;
    }
#pragma unroll
    for (int h = 1; h < E; h <<= 1) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if ((e & h) == 0) {
                const float a = x[e], b = x[e + h];
                x[e] = a + b;
                x[e + h] = a - b;
            }
        }
    }
#pragma unroll
    for (int h = E; h < D; h <<= 1) {
        const int m = h / E;                                  // lane distance
        const bool upper = (lane & m) != 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float other = __shfl_xor(x[e], m);
            x[e] = upper ? other - x[e] : x[e] + other;
        }
    }
    const float norm = 1.0f / sqrtf((float)D);
    if (active) {
#pragma unroll
        for (int e = 0; e < E; ++e) A[(int64_t)qi * D + lane * E + e] = x[e] * norm;
    }
}

}  // namespace

bool hadamard_supported(int D) { return D >= 1 && D <= 1024 && (D & (D - 1)) == 0; }

hipError_t launch_query_transform_hadamard(const float* q, const float* signs, float* A, int P, int H, int B,
                                           int D, hipStream_t stream) {
    const int nq = P * B;
    const dim3 grid((unsigned)((nq + 3) / 4)), block(256);
    switch (D) {
#define TQ_HADAMARD(DV) \
    case DV: hipLaunchKernelGGL(hadamard_query_kernel<DV>, grid, block, 0, stream, q, signs, A, H, B, nq); break;
        TQ_HADAMARD(1) TQ_HADAMARD(2) TQ_HADAMARD(4) TQ_HADAMARD(8) TQ_HADAMARD(16) TQ_HADAMARD(32)
        TQ_HADAMARD(64) TQ_HADAMARD(128) TQ_HADAMARD(256) TQ_HADAMARD(512) TQ_HADAMARD(1024)
#undef TQ_HADAMARD
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_query_transform(const float* q, const float* Pi, const float* S_mat,
                                  float* A, float* T, int P, int H, int B, int D,
                                  hipStream_t stream) {
    if (D % 32 == 0 && D <= 256) {
        // all P / H problems of a head in one row list when the tile count fits the grid
        const int64_t per_head = (int64_t)(P / H) * B;
        const int PG = (per_head + 15) / 16 <= 65535 ? P / H : 1;
        dim3 grid(2 * D / 16, (unsigned)(((int64_t)PG * B + 15) / 16), (unsigned)(P / PG));
        // four wavefronts split the contraction where D / 4 is a whole number of
        // 16-coordinate steps, else two
        switch (D) {
            case 32: hipLaunchKernelGGL((query_transform_mfma16_kernel<32, 2>), grid, dim3(128), 0, stream,
                                   q, Pi, S_mat, A, T, H, B, PG); break;
            case 64: hipLaunchKernelGGL((query_transform_mfma16_kernel<64, 4>), grid, dim3(256), 0, stream,
                                   q, Pi, S_mat, A, T, H, B, PG); break;
            case 96: hipLaunchKernelGGL((query_transform_mfma16_kernel<96, 2>), grid, dim3(128), 0, stream,
                                   q, Pi, S_mat, A, T, H, B, PG); break;
            case 128: hipLaunchKernelGGL((query_transform_mfma16_kernel<128, 4>), grid, dim3(256), 0, stream,
                                   q, Pi, S_mat, A, T, H, B, PG); break;
            case 160: hipLaunchKernelGGL((query_transform_mfma16_kernel<160, 2>), grid, dim3(128), 0, stream,
                                   q, Pi, S_mat, A, T, H, B, PG); break;
            case 192: hipLaunchKernelGGL((query_transform_mfma16_kernel<192, 4>), grid, dim3(256), 0, stream,
                                   q, Pi, S_mat, A, T, H, B, PG); break;
            case 224: hipLaunchKernelGGL((query_transform_mfma16_kernel<224, 2>), grid, dim3(128), 0, stream,
                                   q, Pi, S_mat, A, T, H, B, PG); break;
            default: hipLaunchKernelGGL((query_transform_mfma16_kernel<256, 4>), grid, dim3(256), 0, stream,
                                   q, Pi, S_mat, A, T, H, B, PG); break;
        }
        return hipGetLastError();
    }
    const int kc = D < kChunk ? D : kChunk;
    const size_t lds = (size_t)(kRows + kQueries) * (((kc + 3) & ~3) + kPad) * sizeof(float);
    dim3 grid((2 * D + kRows - 1) / kRows, (B + kQueries - 1) / kQueries, P);
    hipLaunchKernelGGL(query_transform_kernel, grid, dim3(256), lds, stream,
                       q, Pi, S_mat, A, T, H, B, D);
    return hipGetLastError();
}

}  // namespace tq
