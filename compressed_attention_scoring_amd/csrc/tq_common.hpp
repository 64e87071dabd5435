// Shared host/device definitions for the compressed-key scoring kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

// sqrt(pi/2): the QJL de-biasing constant; the estimator divides it by the
// number of projection rows, D ("TurboQuant: Rotate-then-Quantize KV Caches at
// 3 Bits", section 3, the QJL bullet).
constexpr double kSqrtHalfPi = 1.2533141373155002512078826424055;

struct KeyStreams {
    const uint8_t* idx;    // unpacked: [P,S,D] bytes; packed: [P,S,D*bits/8]
    const uint8_t* sign;   // unpacked: [P,S,D] int8 +-1; packed: [P,S,D/8] bits
    const void* gamma;     // unpacked: float [P,S]; packed: _Float16 [P,S]
};

// Bytes of one key's index stream, sign stream and gamma for a layout.
__host__ __device__ inline int64_t idx_row_bytes(int layout, int bits, int D) {
    return layout == 0 ? (int64_t)D : (int64_t)D * bits / 8;
}
__host__ __device__ inline int64_t sign_row_bytes(int layout, int D) {
    return layout == 0 ? (int64_t)D : (int64_t)D / 8;
}

// Kernel launchers (defined in the .hip files; all return hipError_t of the launch).
hipError_t launch_query_transform(const float* q, const float* Pi, const float* S_mat,
                                  float* A, float* T, int P, int H, int B, int D,
                                  hipStream_t stream);

hipError_t launch_score_valu(const float* A, const float* T, KeyStreams keys,
                             int layout, int bits, const float* codebook, int C,
                             float* scores, int P, int B, int S, int D,
                             hipStream_t stream);

// Matrix-core kernels come in three variants: 32x32 tiles with the query-side
// operands staged once per workgroup in LDS, 32x32 tiles with them held in each
// wavefront's registers, and 16x16 tiles for a few queries per problem.
// kMfmaAuto picks by shape. kMfmaF16 is the single-pass f16 form of the
// automatic choice (one f16 product per contraction; the register variant's
// shapes take the LDS-staged kernel).
enum MfmaVariant { kMfmaAuto = 0, kMfmaLds = 1, kMfmaReg = 2, kMfmaSmall = 3, kMfmaShared = 4, kMfmaF16 = 5 };

// Returns false if the variant does not cover (layout, bits, C, B, D).
bool score_mfma_supported(int layout, int bits, int C, int B, int D, int variant);
const char* score_mfma_name(int layout, int bits, int C, int P, int B, int S, int D, int variant);
hipError_t launch_score_mfma(const float* A, const float* T, KeyStreams keys,
                             int layout, int bits, const float* codebook, int C,
                             float* scores, int P, int B, int S, int D, int variant,
                             hipStream_t stream);

// Compressor outputs (device pointers; layout and sizes as in KeyStreams).
struct KeyOut {
    uint8_t* idx;
    uint8_t* sign;
    void* gamma;
    void* norm;   // the keys' lengths in gamma's dtype, or null
};
bool compress_supported(int layout, int bits, int C, int D);
hipError_t launch_compress(const float* keys, const float* Pi, const float* S_mat, const float* codebook,
                           int C, KeyOut out, int layout, int bits, int P, int H, int S, int D,
                           hipStream_t stream);

// Compressed values: idx as for keys (unpacked bytes or packed bitstreams),
// norm float [P,S] (unpacked) or _Float16 [P,S] (packed).
struct ValueStreams {
    const uint8_t* idx;
    const void* norm;
};
// Upper bound on the key chunks the attention step splits each problem into
// (for any value layout); the workspace holds P * B * chunks * (D + 2) floats.
int attend_chunks(int P, int B, int S, int D);
bool attend_supported(int layout, int bits, int C, int D);
hipError_t launch_attend(const float* scores, ValueStreams v, int layout, int bits, const float* codebook, int C,
                         const float* Pi_v, float scale, float* out, float* ws, int P, int H, int B, int S, int D,
                         hipStream_t stream);

// MSE-only keys (indices as in KeyStreams, one norm per key, no signs):
// scores = norm_s * sum_d A[b,d] codebook[idx[s,d]], on the LDS-staged kernel.
bool score_mse_supported(int layout, int bits, int C, int D);
hipError_t launch_score_mse(const float* A, const uint8_t* idx, const void* norm, int layout, int bits,
                            const float* codebook, int C, float* scores, int P, int B, int S, int D,
                            hipStream_t stream);

// A = H (signs * q) / sqrt(D) for D a power of two up to 1024.
bool hadamard_supported(int D);
hipError_t launch_query_transform_hadamard(const float* q, const float* signs, float* A, int P, int H, int B,
                                           int D, hipStream_t stream);

// The outlier split: two MSE-only instances per head (hot channels, the rest).
struct SplitStreams {
    const uint8_t* idx_hi;
    const void* norm_hi;
    const uint8_t* idx_lo;
    const void* norm_lo;
};
hipError_t launch_query_transform_split(const float* q, const int32_t* perm, const float* Pi_hi, const float* Pi_lo,
                                        float* A_hi, float* A_lo, int P, int H, int B, int D, int D_hi,
                                        hipStream_t stream);
// The 2.5-bit setting (32 hot channels packed at 3 bits, 96 at 2) on the
// matrix cores; launch_score_split takes it when split_mfma_supported.
bool split_mfma_supported(int bits_hi, int C_hi, int bits_lo, int C_lo, int D_hi, int D_lo, int S);
hipError_t launch_score_split_mfma(const float* A_hi, const float* A_lo, SplitStreams k, const float* cb_hi, int C_hi,
                                   const float* cb_lo, int C_lo, float* scores, int P, int B, int S,
                                   hipStream_t stream);
// bits_hi, bits_lo: 0 for one byte per index, else 2 or 3 (packed)
hipError_t launch_score_split(const float* A_hi, const float* A_lo, SplitStreams k, int bits_hi, int bits_lo,
                              const float* cb_hi, int C_hi, const float* cb_lo, int C_lo, float* scores, int P,
                              int B, int S, int D_hi, int D_lo, hipStream_t stream);

// Fused decode step: scores, online softmax and values in one pass
// (score_fused.hip), writing the attend workspace records; then the attend
// combine (attend.hip).
void score_attend_plan(int P, int B, int S, int& chunk, int& nch);
bool score_attend_supported(int layout, int bits, int C, int vlayout, int vbits, int VC, int D);
hipError_t launch_score_attend_partial(const float* A, const float* T, KeyStreams keys, int layout, int bits,
                                       const float* codebook, int C, ValueStreams v, int vlayout, int vbits,
                                       const float* vcodebook, int VC, float scale, float* ws, int P, int B, int S,
                                       int chunk, int nch, hipStream_t stream);
hipError_t launch_attend_combine(const float* ws, const float* Pi_v, float* out, int P, int H, int B, int D, int nch,
                                 hipStream_t stream);

// Streaming probes (probe.hip): bytes must be multiples of 16.
hipError_t launch_probe_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream);
hipError_t launch_probe_write(void* dst, int64_t bytes, hipStream_t stream);
hipError_t launch_probe_read_write(const void* src, int64_t rbytes, void* dst, int64_t wbytes, hipStream_t stream);
// The unpacked 32 x 32 scorer's loads and stores without its arithmetic (B <= 32).
bool probe_tile_supported(int B, int S, int D);
hipError_t launch_probe_tile(const uint8_t* idx, const uint8_t* sign, const float* gamma, float* out, int B, int S,
                             int D, hipStream_t stream);

hipError_t launch_decode(KeyStreams keys, int layout, int bits,
                         uint8_t* idx_out, int8_t* sign_out, float* gamma_out,
                         int P, int S, int D, hipStream_t stream);

}  // namespace tq
