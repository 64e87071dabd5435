// Key compressor (TurboQuant_prod at b = log2(C) + 1 bits), the step that
// produces the scoring kernels' inputs: "TurboQuant: Rotate-then-Quantize KV
// Caches at 3 Bits", section 3 (rotate, nearest centroid by midpoint search,
// residual, QJL signs of the projected residual, residual norm), with the
// storage of "TurboQuant Attention in CUDA", section "The keys arrived in
// pieces", and the LSB-first packing of "Fitting 4.4x More Context on Jetson",
// section "v6".
//
// All arithmetic is float64, as in the reference compressor: the index and sign
// of each coordinate are decisions, and taking them in the same precision as the
// float64 reference makes them identical to it except for values that fall within
// rounding distance of a decision boundary (probability about 1e-15 per
// coordinate). On this part fp64 matrix and vector throughput are the same
// (78.6 TFLOP/s); the three D x D products per key run as v_mfma_f64_16x16x4_f64.
//
// One wavefront compresses 16 keys (the MFMA columns). Per tile:
//   0. u = k / ||k||            (the page's "normalize, then rotate"; a zero key
//                                stays the zero vector; ||k|| is stored if asked)
//   1. y = Pi u                 (A = Pi rows, B = the 16 unit keys)
//   2. idx = #{midpoints < y}, c = codebook[idx]
//   3. x = Pi^T c               (A = Pi columns, B = c)
//   4. r = u - x, gamma = ||r||
//   5. p = S_mat r              (A = S_mat rows, B = r)
//   6. sign = (p >= 0)          (a zero projection counts as +1)
//   7. pack and store           (through LDS, one lane per 32 coordinates of a key)
// Pi and S_mat of the workgroup's head are staged in LDS once (fp32, rows padded
// by 16 bytes so that rows read at the same column by different lanes fall in
// different banks: 132 KiB at D = 128), and the workgroup's wavefronts then walk
// 16-key tiles, reading every A operand from LDS: read from L2 instead (the
// former form), each wavefront fetched 192 KiB of matrix data per tile with 576
// load instructions. Every operand address is one per-lane base plus a constant.
// v_mfma_f64_16x16x4_f64 holds A[row][slot] in lane 16 slot + row, B[slot][col]
// in lane 16 slot + col, and output register v of lane 16 q + col at row 4 v + q
// (a layout checked on the device). So after a product, lane group q = lane / 16
// holds coordinates 16 rb + 4 v + q of its key, and the next product contracts
// in exactly that order (slot q of sub-step t = coordinate 16 kq + 4 t + q): c
// and r never leave the registers of the lane that computed them. The first
// product's contraction order is free; it takes j = 16 kq + 4 q + t, so a lane's
// four sub-steps read four consecutive elements of a row (one 16-byte load).
#include "tq_common.hpp"

namespace tq {
namespace {

typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr int kKeysPerWave = 16;
constexpr int kCompressWaves = 4;
constexpr int kMaxCodebook = 16;

// float64 -> binary16 with a single rounding (to nearest, ties to even):
// round to float32 with round-to-odd first (24 bits >= 11 + 2, so the final
// rounding sees the exact value's relation to its two fp16 neighbours).
__device__ __forceinline__ _Float16 half_of(double x) {
    float t = (float)x;
    const double td = (double)t;
    if (td != x) {
        uint32_t b = __builtin_bit_cast(uint32_t, t);
        // step toward zero if RNE rounded away from it, then mark inexact
        if (fabs(td) > fabs(x)) b -= 1;
        b |= 1u;
        t = __builtin_bit_cast(float, b);
    }
    return (_Float16)t;
}

template <int D>
struct CompressLds {
    static constexpr int BYTES = kKeysPerWave * D;          // idx or sign bytes of 16 keys
    static constexpr int PER_WAVE = 2 * BYTES;
    static constexpr int LD = D + 4;                         // staged row stride (floats)
    static constexpr int MAT = D * LD;                       // floats of one staged matrix
};

// LDS position of element (row, c) of a staged D x D matrix.
template <int D>
__device__ __forceinline__ int staged(int row, int c) {
    return row * CompressLds<D>::LD + c;
}

template <int D, int LAYOUT, int BITS, int NC>
__global__ __launch_bounds__(kCompressWaves * 64) void compress_kernel(
    const float* __restrict__ keys, const float* __restrict__ Pi, const float* __restrict__ Smat,
    const float* __restrict__ codebook, int C, uint8_t* __restrict__ idx_out, uint8_t* __restrict__ sign_out,
    void* __restrict__ gamma_out, void* __restrict__ norm_out, int H, int S) {
    constexpr int RB = D / 16;                 // 16-row output blocks
    constexpr int KQ = D / 16;                 // 16-wide contraction chunks (4 MFMAs each)
    using L = CompressLds<D>;
    __shared__ __attribute__((aligned(16))) float mats[2 * L::MAT];   // Pi_h, then S_mat_h (staged())
    __shared__ __attribute__((aligned(16))) uint8_t lds[kCompressWaves * L::PER_WAVE];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int p = blockIdx.y;
    const int h = p % H;
    const float* Pp = mats;
    const float* Sp = mats + L::MAT;
    {
        const float4* gp = reinterpret_cast<const float4*>(Pi + (int64_t)h * D * D);
        const float4* gs = reinterpret_cast<const float4*>(Smat + (int64_t)h * D * D);
        for (int i = threadIdx.x; i < D * D / 4; i += kCompressWaves * 64) {
            const int row = i / (D / 4), c = 4 * (i % (D / 4));
            const float4 a = gp[i], b = gs[i];
            *reinterpret_cast<float4*>(mats + staged<D>(row, c)) = a;
            *reinterpret_cast<float4*>(mats + L::MAT + staged<D>(row, c)) = b;
        }
    }
    __syncthreads();                           // the only barrier: the matrices are read-only below
    uint8_t* ibuf = lds + wave * L::PER_WAVE;                  // [16][D] indices
    uint8_t* sbuf = ibuf + L::BYTES;                            // [16][D] sign bits (0/1)
    const int q = lane >> 4;                   // contraction slot / output row group
    const int col = lane & 15;                 // key column

    for (int s0 = (blockIdx.x * kCompressWaves + wave) * kKeysPerWave; s0 < S;
         s0 += gridDim.x * kCompressWaves * kKeysPerWave) {
    const int key = min(s0 + col, S - 1);      // clamped: keys past S are computed, not stored
    const float* kp = keys + ((int64_t)p * S + key) * D;

    // ---- 0. the key's length: this lane holds coordinates j = 16 kq + 4 q + t
    //      (the order of the first product), the four lane groups the rest
    float4 kv[KQ];
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq) kv[kq] = *reinterpret_cast<const float4*>(kp + 16 * kq + 4 * q);
    double nn = 0.0;
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq) {
        nn = fma((double)kv[kq].x, (double)kv[kq].x, nn);
        nn = fma((double)kv[kq].y, (double)kv[kq].y, nn);
        nn = fma((double)kv[kq].z, (double)kv[kq].z, nn);
        nn = fma((double)kv[kq].w, (double)kv[kq].w, nn);
    }
    nn += __shfl_xor(nn, 16);
    nn += __shfl_xor(nn, 32);
    const double nrm = sqrt(nn);
    const double div = nrm > 0.0 ? nrm : 1.0;   // a zero key stays the zero vector

    // ---- 1. y = Pi u: B holds this lane's unit key at j = 16 kq + 4 q + t
    f64x4 acc[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[rb] = (f64x4){0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq) {
        const double u0 = (double)kv[kq].x / div, u1 = (double)kv[kq].y / div;
        const double u2 = (double)kv[kq].z / div, u3 = (double)kv[kq].w / div;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const float4 av = *reinterpret_cast<const float4*>(Pp + staged<D>(16 * rb + col, 16 * kq + 4 * q));
            acc[rb] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)av.x, u0, acc[rb], 0, 0, 0);
            acc[rb] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)av.y, u1, acc[rb], 0, 0, 0);
            acc[rb] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)av.z, u2, acc[rb], 0, 0, 0);
            acc[rb] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)av.w, u3, acc[rb], 0, 0, 0);
        }
    }
    // ---- 2. indices: acc[rb][v] = y[d = 16 rb + 4 v + q] of key col; the index
    //      is the number of midpoints strictly below y (a value on a midpoint
    //      takes the lower index)
    // codebook and its midpoints (sorted codebook, C <= NC), built here so they
    // are not live during the first product
    double cb[NC], edge[NC - 1];
#pragma unroll
    for (int i = 0; i < NC; ++i) cb[i] = i < C ? (double)codebook[i] : 0.0;
#pragma unroll
    for (int i = 0; i + 1 < NC; ++i) edge[i] = 0.5 * (cb[i] + cb[i + 1]);
    f64x4 cr[RB];                              // c = codebook[idx], later r
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            int n = 0;
#pragma unroll
            for (int i = 0; i + 1 < NC; ++i) n += (i + 1 < C && edge[i] < acc[rb][v]) ? 1 : 0;
            ibuf[col * D + 16 * rb + 4 * v + q] = (uint8_t)n;
            double c = cb[0];
#pragma unroll
            for (int i = 1; i < NC; ++i) c = n == i ? cb[i] : c;
            cr[rb][v] = c;
        }
    }

    // ---- 3. x = Pi^T c: A[row j = 16 rb + col][slot q] = Pi[d][j] and
    //      B[slot q][key] = c[d] = cr[kq][t] of this lane, d = 16 kq + 4 t + q
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[rb] = (f64x4){0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                acc[rb] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)Pp[staged<D>(16 * kq + 4 * t + q, 16 * rb + col)],
                                                             cr[kq][t], acc[rb], 0, 0, 0);
        }
    }
    // ---- 4. r = u - x (acc[rb][v] = x[j = 16 rb + 4 v + q] of key col), gamma;
    //      u is recomputed from the key in this order (the same division as above)
    double rr = 0.0;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            cr[rb][v] = (double)kp[16 * rb + 4 * v + q] / div - acc[rb][v];
            rr = fma(cr[rb][v], cr[rb][v], rr);
        }
    }
    rr += __shfl_xor(rr, 16);                  // the key's four lane groups
    rr += __shfl_xor(rr, 32);
    const double gam = sqrt(rr);

    // ---- 5. p = S_mat r: A[row d = 16 rb + col][slot q] = S_mat[d][j] and
    //      B[slot q][key] = r[j] = cr[kq][t] of this lane, j = 16 kq + 4 t + q
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[rb] = (f64x4){0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
                acc[rb] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)Sp[staged<D>(16 * rb + col, 16 * kq + q + 4 * t)],
                                                             cr[kq][t], acc[rb], 0, 0, 0);
        }
    }
    // ---- 6. sign bits (1 = +1, also for an exactly zero projection) of
    //      p[d = 16 rb + 4 v + q]
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int v = 0; v < 4; ++v) sbuf[col * D + 16 * rb + 4 * v + q] = acc[rb][v] >= 0.0 ? 1 : 0;
    }
    // the packing lanes read bytes other lanes wrote: LDS operations of one
    // wavefront complete in order, and this keeps the compiler from moving them
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- 7. pack: lane (key kk, 32-coordinate block blk) for kk < 16, blk < D/32
    constexpr int NB = D / 32;
#pragma unroll
    for (int pass = 0; pass < (16 * NB + 63) / 64; ++pass) {
        const int u = pass * 64 + lane;
        const int kk = u / NB, blk = u % NB;
        const int s = s0 + kk;
        const double gk = __shfl(gam, kk & 15);   // gamma and length of key kk sit in lane kk
        const double nk = __shfl(nrm, kk & 15);
        if (kk < 16 && s < S) {
            const uint8_t* ib = ibuf + kk * D + 32 * blk;
            const uint8_t* sb = sbuf + kk * D + 32 * blk;
            uint32_t iw[8], sw[8];
#pragma unroll
            for (int w = 0; w < 8; w += 4) {
                const uint4 a = *reinterpret_cast<const uint4*>(ib + 4 * w);
                const uint4 b = *reinterpret_cast<const uint4*>(sb + 4 * w);
                iw[w] = a.x; iw[w + 1] = a.y; iw[w + 2] = a.z; iw[w + 3] = a.w;
                sw[w] = b.x; sw[w + 1] = b.y; sw[w + 2] = b.z; sw[w + 3] = b.w;
            }
            const int64_t krow = (int64_t)p * S + s;
            if constexpr (LAYOUT == 0) {
                // indices as bytes; signs as int8 +-1 (bit b of byte -> 2 b - 1)
                uint4* io = reinterpret_cast<uint4*>(idx_out + krow * D + 32 * blk);
                io[0] = make_uint4(iw[0], iw[1], iw[2], iw[3]);
                io[1] = make_uint4(iw[4], iw[5], iw[6], iw[7]);
                uint32_t so[8];
#pragma unroll
                for (int w = 0; w < 8; ++w) so[w] = ~(sw[w] * 0xFEu);   // byte 1 -> 0x01, 0 -> 0xFF
                uint4* sp = reinterpret_cast<uint4*>(sign_out + krow * D + 32 * blk);
                sp[0] = make_uint4(so[0], so[1], so[2], so[3]);
                sp[1] = make_uint4(so[4], so[5], so[6], so[7]);
                if (blk == 0) {
                    reinterpret_cast<float*>(gamma_out)[krow] = (float)gk;
                    if (norm_out) reinterpret_cast<float*>(norm_out)[krow] = (float)nk;
                }
            } else {
                // LSB-first bitstream: coordinate c of the block at bits [BITS c, BITS c + BITS)
                uint32_t out[BITS] = {};
#pragma unroll
                for (int c = 0; c < 32; ++c) {
                    const uint32_t v = (iw[c / 4] >> (8 * (c % 4))) & 0xFFu;
                    const int bit = BITS * c;
                    out[bit / 32] |= v << (bit % 32);
                    if (bit % 32 > 32 - BITS) out[bit / 32 + 1] |= v >> (32 - bit % 32);
                }
                uint32_t* io = reinterpret_cast<uint32_t*>(idx_out + krow * (D * BITS / 8) + 4 * BITS * blk);
#pragma unroll
                for (int w = 0; w < BITS; ++w) io[w] = out[w];
                uint32_t sbits = 0;
#pragma unroll
                for (int c = 0; c < 32; ++c) sbits |= ((sw[c / 4] >> (8 * (c % 4))) & 1u) << c;
                reinterpret_cast<uint32_t*>(sign_out + krow * (D / 8))[blk] = sbits;
                if (blk == 0) {
                    reinterpret_cast<_Float16*>(gamma_out)[krow] = half_of(gk);
                    if (norm_out) reinterpret_cast<_Float16*>(norm_out)[krow] = half_of(nk);
                }
            }
        }
    }
    // the next tile's index and sign bytes go to the same LDS rows: every lane's
    // packing reads above come first
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

template <int D, int LAYOUT, int BITS>
hipError_t launch_compress_d(const float* keys, const float* Pi, const float* S_mat, const float* codebook,
                             int C, KeyOut out, int P, int H, int S, hipStream_t stream) {
    // about one workgroup per compute unit (each stages its head's two matrices,
    // 128 KiB at D = 128, once), its wavefronts walking 16-key tiles
    const int per_block = kCompressWaves * kKeysPerWave;
    int64_t gx = (S + per_block - 1) / per_block;
    const int64_t cap = 256 / P > 0 ? 256 / P : 1;
    if (gx > cap) gx = cap;
    const dim3 grid((unsigned)gx, (unsigned)P);
    // codebook registers sized to the codebook: 8 entries cover every packed format
    if (C <= 8)
        hipLaunchKernelGGL((compress_kernel<D, LAYOUT, BITS, 8>), grid, dim3(kCompressWaves * 64), 0, stream,
                           keys, Pi, S_mat, codebook, C, out.idx, out.sign, out.gamma, out.norm, H, S);
    else
        hipLaunchKernelGGL((compress_kernel<D, LAYOUT, BITS, kMaxCodebook>), grid, dim3(kCompressWaves * 64), 0,
                           stream, keys, Pi, S_mat, codebook, C, out.idx, out.sign, out.gamma, out.norm, H, S);
    return hipGetLastError();
}

template <int D>
hipError_t launch_compress_layout(const float* keys, const float* Pi, const float* S_mat, const float* codebook,
                                  int C, KeyOut out, int layout, int bits, int P, int H, int S, hipStream_t stream) {
    if (layout == 0) return launch_compress_d<D, 0, 0>(keys, Pi, S_mat, codebook, C, out, P, H, S, stream);
    if (bits == 2) return launch_compress_d<D, 1, 2>(keys, Pi, S_mat, codebook, C, out, P, H, S, stream);
    return launch_compress_d<D, 1, 3>(keys, Pi, S_mat, codebook, C, out, P, H, S, stream);
}

}  // namespace

bool compress_supported(int layout, int bits, int C, int D) {
    if (C < 2 || C > kMaxCodebook) return false;
    if (D != 64 && D != 128) return false;
    return layout == 0 || bits == 2 || bits == 3;
}

hipError_t launch_compress(const float* keys, const float* Pi, const float* S_mat, const float* codebook,
                           int C, KeyOut out, int layout, int bits, int P, int H, int S, int D,
                           hipStream_t stream) {
    if (!compress_supported(layout, bits, C, D)) return hipErrorInvalidValue;
    if (D == 64) return launch_compress_layout<64>(keys, Pi, S_mat, codebook, C, out, layout, bits, P, H, S, stream);
    return launch_compress_layout<128>(keys, Pi, S_mat, codebook, C, out, layout, bits, P, H, S, stream);
}

}  // namespace tq
