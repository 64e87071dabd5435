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
// The product is tiny (4 P B D^2 flops) and latency-bound, so the kernel is
// shaped for few dependent memory rounds: a 256-lane workgroup owns 16 rows of
// W and 32 queries of one problem; for D <= 256 all of its operands (16 W rows
// and the 32 query rows) are requested in a single round of 16-byte loads into
// LDS, then every lane forms two outputs from broadcast LDS reads with eight
// independent fp32 FMA chains. Larger D is staged in 256-column chunks.
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

}  // namespace

hipError_t launch_query_transform(const float* q, const float* Pi, const float* S_mat,
                                  float* A, float* T, int P, int H, int B, int D,
                                  hipStream_t stream) {
    const int kc = D < kChunk ? D : kChunk;
    const size_t lds = (size_t)(kRows + kQueries) * (((kc + 3) & ~3) + kPad) * sizeof(float);
    dim3 grid((2 * D + kRows - 1) / kRows, (B + kQueries - 1) / kQueries, P);
    hipLaunchKernelGGL(query_transform_kernel, grid, dim3(256), lds, stream,
                       q, Pi, S_mat, A, T, H, B, D);
    return hipGetLastError();
}

}  // namespace tq
