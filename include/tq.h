/*
 * tq.h -- C ABI of the compressed-key attention scoring library (MI355X, gfx950).
 *
 * The library scores queries against a TurboQuant-compressed key cache without
 * rebuilding any key. A compressed key s holds, per coordinate d, a codebook
 * index idx[s,d] and a QJL sign sigma[s,d] in {-1,+1}, plus one residual norm
 * gamma[s]. Its raw score against query q_b is
 *
 *   scores[b,s] = sum_d A[b,d] * codebook[idx[s,d]]
 *               + (sqrt(pi/2) / D) * gamma[s] * sum_d T[b,d] * sigma[s,d]
 *
 * with A = Pi q_b and T = S_mat q_b computed once per query. No softmax, no
 * 1/sqrt(D) scaling, no values. Source: "TurboQuant Attention in CUDA:
 * Transform the Query, Reuse the Work" (riteshyadav.xyz), sections "Move the
 * transforms to the query" and "Two kernels, two jobs"; the reconstruction
 * this equals is the inner-product quantizer of "TurboQuant: Rotate-then-
 * Quantize KV Caches at 3 Bits" (kanthi.in), section 3.
 *
 * Conventions for every entry point
 *  - All array arguments are DEVICE pointers (memory of the current HIP
 *    device), row-major, densely packed, with base addresses aligned to
 *    16 bytes. The caller allocates and owns every buffer; the library
 *    allocates nothing and keeps no state between calls, so calls are
 *    reentrant. Outputs must not alias inputs.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Work
 *    is enqueued asynchronously; results are visible after the stream
 *    synchronizes. Calls on one stream run in order.
 *  - Arguments are validated on the host before anything is launched. The
 *    return value is TQ_OK or a negative TQ_ERR_* code; nothing is thrown
 *    across the ABI. TQ_ERR_LAUNCH reports a HIP error from the launch.
 *  - Empty calls: if P, B or S is 0 (after the format checks pass) nothing is
 *    launched, TQ_OK is returned, and array pointers may be NULL. Negative
 *    sizes, and D <= 0 or H <= 0, are TQ_ERR_ARG.
 *  - Problems: P independent scoring problems are handled in one call. With H
 *    heads, problem p uses head p % H (its own Pi and S_mat); P % H must be 0.
 *  - Not checked (as in the page's challenge, where indices are guaranteed
 *    valid): unpacked indices must be < C and unpacked signs must be +-1.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define TQ_OK               0
#define TQ_ERR_ARG         -1  /* null pointer, negative size, D or H <= 0, P % H != 0, unknown layout/kernel */
#define TQ_ERR_UNSUPPORTED -2  /* shape or format outside what the kernels support (see tq_score) */
#define TQ_ERR_ALIGN       -3  /* a base pointer is not 16-byte aligned */
#define TQ_ERR_LAUNCH      -4  /* HIP reported an error launching a kernel */

/* key layouts */
#define TQ_UNPACKED 0
#define TQ_PACKED   1

/* largest supported coordinate count D */
#define TQ_MAX_D 1024

/*
 * Compressed keys of P problems, S keys each, D coordinates per key.
 *
 * layout == TQ_UNPACKED ("TurboQuant Attention in CUDA", section "Full CUDA
 * solution": one byte per index and per sign):
 *   idx   uint8  [P, S, D]   codebook index, < C
 *   sign  int8   [P, S, D]   +1 or -1
 *   gamma float32 [P, S]     residual norm
 *   bits  ignored
 *
 * layout == TQ_PACKED (bitstreams, one run of bytes per key):
 *   idx   uint8 [P, S, D*bits/8]  coordinate d occupies bits [bits*d, bits*d+bits)
 *                                 of the key's bytes read as one little-endian
 *                                 integer (LSB-first, as the 2-bit extraction of
 *                                 "Fitting 4.4x More Context on Jetson", section
 *                                 "v6: Fused Vectorized Hybrid"; a 128-dim 3-bit
 *                                 key is 48 bytes, "TurboQuant: Rotate-then-
 *                                 Quantize", section 8)
 *   sign  uint8 [P, S, D/8]       bit d (LSB-first) is 1 for sigma = +1, 0 for -1
 *   gamma float16 [P, S]          residual norm as IEEE binary16
 *   bits  2 or 3; C must equal 2^bits; D must be a multiple of 8
 */
typedef struct tq_keys {
    int32_t layout;
    int32_t bits;
    const void* idx;
    const void* sign;
    const void* gamma;
} tq_keys;

/*
 * tq_query_transform: A = Pi q and T = S_mat q for every query.
 * "TurboQuant Attention in CUDA", section "Move the transforms to the query";
 * indexing as the comment over its first kernel: A[b,d] = sum_j Pi[d,j] q[b,j].
 *
 *   q      float32 [P, B, D]   queries
 *   Pi     float32 [H, D, D]   rotation of each head, row-major
 *   S_mat  float32 [H, D, D]   QJL projection of each head, row-major
 *   A, T   float32 [P, B, D]   outputs (problem p uses head p % H)
 *
 * Arithmetic is fp32 with fp32 accumulation. D <= TQ_MAX_D.
 */
int tq_query_transform(const float* q, const float* Pi, const float* S_mat,
                       float* A, float* T,
                       int P, int H, int B, int D, void* stream);

/*
 * tq_score: raw scores of B transformed queries against S compressed keys,
 * for each of P problems (formula at the top of this file; "TurboQuant
 * Attention in CUDA", sections "Two kernels, two jobs" and "Full CUDA
 * solution", with the packed layouts above added).
 *
 *   A, T      float32 [P, B, D]   from tq_query_transform
 *   keys      compressed keys (struct above; host pointer to the struct,
 *             device pointers inside it)
 *   codebook  float32 [C]         centroids (C <= 256 unpacked, 2^bits packed)
 *   scores    float32 [P, B, S]   output
 *
 * Result: fp32, within 1e-4 * (1 + |exact|) of the exact (float64) value of
 * the formula for the given inputs. D <= TQ_MAX_D, B <= 262144, P <= 65535.
 */
int tq_score(const float* A, const float* T, const tq_keys* keys,
             const float* codebook, int C, float* scores,
             int P, int B, int S, int D, void* stream);

/* kernel families tq_score can use; TQ_KERNEL_AUTO picks by shape */
#define TQ_KERNEL_AUTO   0
#define TQ_KERNEL_VALU   1  /* any shape: one key per lane, fp32 FMAs */
#define TQ_KERNEL_MFMA   2  /* C <= 8 and D in {64, 128, 256} (also 32 when unpacked),
                               S < 2^24: split-f16 matrix-core contraction; picks one
                               of the variants below by shape */
#define TQ_KERNEL_MFMA_LDS 3  /* matrix cores, query operands staged once per
                                 workgroup in LDS (the MFMA shapes above) */
#define TQ_KERNEL_MFMA_REG 4  /* matrix cores, query operands held in each
                                 wavefront's registers (the MFMA shapes above
                                 with D <= 128) */
#define TQ_KERNEL_MFMA16   5  /* matrix cores, 16x16 tiles of four queries times
                                 their four operand rows (the MFMA shapes above
                                 with D in {128, 256}); the automatic choice for
                                 B <= 4 with P * S >= 2^20 keys. Packed keys run
                                 on the int8 matrix cores, A, T and the codebook
                                 split into three int8 limbs each (exact integer
                                 products, the same 1e-4 contract) */
#define TQ_KERNEL_MFMA_SHARED 6  /* matrix cores, four query tiles per workgroup in
                                    registers sharing one unpacking of each key
                                    tile through LDS (the MFMA shapes above with
                                    D in {64, 128}); the automatic choice for
                                    B > 96 */
#define TQ_KERNEL_MFMA_F16 7  /* NOT fp32-accurate: the single-pass f16 form of the
                                 automatic matrix-core choice (the MFMA shapes
                                 above; the LDS-staged kernel where the automatic
                                 choice is the register one). A and the codebook
                                 enter as one f16 product, T and the signs as one
                                 (the 16x16 form also keeps the query's lo rows,
                                 which share its instructions), after the same
                                 power-of-two scaling. Its contract is max over
                                 elements of |got - exact| / (1 + |exact|) <= 2e-2
                                 instead of tq_score's 1e-4: a reported comparison
                                 point, never chosen by TQ_KERNEL_AUTO. */

/*
 * tq_score_with_kernel: tq_score with an explicit kernel family, so that every
 * family can be checked on every shape it supports. TQ_ERR_UNSUPPORTED if the
 * family cannot run the shape. tq_score == tq_score_with_kernel(..., AUTO).
 */
int tq_score_with_kernel(const float* A, const float* T, const tq_keys* keys,
                         const float* codebook, int C, float* scores,
                         int P, int B, int S, int D, int kernel, void* stream);

/*
 * tq_score_kernel_name: name of the kernel tq_score_with_kernel would launch
 * for this shape and format, or NULL if unsupported (including sizes
 * tq_score_with_kernel refuses). Host-only, no GPU work.
 * The returned string is static.
 */
const char* tq_score_kernel_name(int layout, int bits, int C, int P, int B, int S, int D, int kernel);

/*
 * tq_decode_debug: expand keys of either layout into the unpacked layout,
 * bit-exactly (gamma is widened to float32, which is exact from fp16).
 *
 *   keys       compressed keys (struct above)
 *   idx_out    uint8  [P, S, D]
 *   sign_out   int8   [P, S, D]   +-1
 *   gamma_out  float32 [P, S]
 */
int tq_decode_debug(const tq_keys* keys, uint8_t* idx_out, int8_t* sign_out,
                    float* gamma_out, int P, int S, int D, void* stream);

/*
 * Output descriptor of tq_compress_keys: the same layouts as tq_keys, with
 * writable device pointers, and an optional output of the keys' lengths.
 */
typedef struct tq_keys_out {
    int32_t layout;   /* TQ_UNPACKED or TQ_PACKED */
    int32_t bits;     /* packed: 2 or 3 */
    void* idx;
    void* sign;
    void* gamma;
    void* norm;       /* NULL, or [P, S] lengths ||k|| in gamma's dtype (float32
                         unpacked, float16 packed) */
} tq_keys_out;

/*
 * tq_compress_keys: compress keys into either layout above (the inner-product
 * quantizer of "TurboQuant: Rotate-then-Quantize KV Caches at 3 Bits",
 * section 3, with the residual norm of "TurboQuant Attention in CUDA",
 * section "The keys arrived in pieces"), normalising first as that page's
 * section 3 orders it. For each key k of problem p, with head h = p % H:
 *   u = k / ||k|| (a zero key is compressed as the zero vector);
 *   y = Pi_h u;  idx_d = number of codebook midpoints strictly below y_d
 *   (a value on a midpoint takes the lower index);  r = u - Pi_h^T c[idx];
 *   gamma = ||r||;  sign_d = +1 if (S_h r)_d >= 0 else -1;
 *   norm = ||k|| if out->norm is not NULL.
 * tq_score's scores are against the unit key u; multiplying them by the
 * stored norm gives scores against k as given.
 *
 *   keys      float32 [P, S, D]
 *   Pi, S_mat float32 [H, D, D]   (the matrices tq_query_transform takes)
 *   codebook  float32 [C]         sorted ascending, 2 <= C <= 16; packed: C == 2^bits
 *   out       host pointer to the descriptor; its device buffers are written
 *
 * Arithmetic is float64, so indices and signs equal those of a float64
 * reference except for values within rounding distance of a midpoint or of a
 * zero projection; gamma is rounded once to float32 (unpacked) or binary16
 * (packed). D in {64, 128}. TQ_ERR_ARG for bad pointers or sizes (as above,
 * P % H != 0), TQ_ERR_UNSUPPORTED for other D or C, TQ_ERR_ALIGN for a buffer
 * that is not 16-byte aligned. Empty calls (P or S == 0) return TQ_OK.
 */
int tq_compress_keys(const float* keys, const float* Pi, const float* S_mat,
                     const float* codebook, int C, const tq_keys_out* out,
                     int P, int H, int S, int D, void* stream);

/*
 * MSE-only codes of P problems, S vectors each, D coordinates per vector: the
 * MSE quantizer of "TurboQuant: Rotate-then-Quantize KV Caches at 3 Bits"
 * (section 3, the norm kept separately as its value cache does in section 8):
 * x_s = norm[s] * Pi^T codebook[idx[s, :]]. The format of compressed values
 * (tq_attend) and of keys in the MSE-only scoring variant (tq_score_mse).
 *
 * layout == TQ_UNPACKED: idx uint8 [P, S, D] (< C), norm float32 [P, S]; bits ignored.
 * layout == TQ_PACKED:   idx uint8 [P, S, D*bits/8] as the packed key indices
 *                        above (LSB-first bitstream per vector), norm float16
 *                        [P, S]; bits 2 or 3, C == 2^bits.
 */
typedef struct tq_mse_codes {
    int32_t layout;
    int32_t bits;
    const void* idx;
    const void* norm;
} tq_mse_codes;

/* compressed values */
typedef tq_mse_codes tq_values;

/*
 * tq_attend_workspace_bytes: bytes of the workspace tq_attend needs for this
 * shape with either value layout (0 for an empty shape, invalid sizes or sizes
 * tq_attend refuses).
 * Host-only. The size depends only on (P, B, S, D).
 */
size_t tq_attend_workspace_bytes(int P, int B, int S, int D);

/*
 * tq_attend: decode attention output from raw scores and compressed values
 * ("TurboQuant: Rotate-then-Quantize KV Caches at 3 Bits", section 8, kernel
 * view; the online softmax and split over key ranges of "Fitting 4.4x More
 * Context on Jetson", FAQ). For each problem p (head h = p % H) and query b:
 *
 *   w_s    = exp(scale * scores[p,b,s] - max_t scale * scores[p,b,t])
 *   out[p,b,:] = Pi_v[h]^T ( sum_s w_s norm[s] codebook[idx[s,:]] ) / sum_s w_s
 *
 * which equals softmax(scale * scores) times the dequantized values; the sum is
 * accumulated in the rotated basis and un-rotated once per query.
 *
 *   scores     float32 [P, B, S]   e.g. from tq_score; must be finite
 *   values     compressed values (struct above; host pointer to the struct)
 *   codebook   float32 [C]         value centroids, 1 <= C <= 8
 *   Pi_v       float32 [H, D, D]   value rotation of each head, row-major
 *   scale      softmax temperature (1/sqrt(D) for standard attention)
 *   out        float32 [P, B, D]
 *   workspace  device buffer of at least tq_attend_workspace_bytes(P, B, S, D)
 *              bytes (per-range partial results; contents on return unspecified)
 *
 * D in {64, 128}, S >= 1 when B >= 1 (a softmax over no keys is undefined:
 * TQ_ERR_ARG). Result: fp32, within 1e-4 * (1 + |exact|) of the exact value.
 * TQ_ERR_ARG for bad pointers/sizes (as above) or a workspace that is too
 * small; TQ_ERR_UNSUPPORTED for other D, C or formats; TQ_ERR_ALIGN for a
 * buffer that is not 16-byte aligned. Calls that share a workspace must be
 * ordered (same stream).
 */
int tq_attend(const float* scores, const tq_values* values, const float* codebook, int C,
              const float* Pi_v, float scale, float* out, void* workspace, size_t workspace_bytes,
              int P, int H, int B, int S, int D, void* stream);

/*
 * tq_attend_no_alloc: tq_attend for callers that cannot allocate (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, result and errors as tq_attend, without the workspace: the
 * partial results go to a fixed scratch array in device memory that the
 * library holds per GPU for the life of the process (TQ_NO_ALLOC_SCRATCH_BYTES,
 * 48 MiB). It calls no allocating routine. Shapes whose workspace
 * (tq_attend_workspace_bytes) exceeds the scratch are TQ_ERR_UNSUPPORTED.
 * Every call on one GPU shares that GPU's scratch: calls that may overlap on
 * one GPU (different streams, or host threads without ordering) race and must
 * not be issued; calls ordered on one stream are fine. TQ_ERR_LAUNCH if the
 * scratch's device address cannot be obtained.
 */
#define TQ_NO_ALLOC_SCRATCH_BYTES (48u * 1024u * 1024u)
int tq_attend_no_alloc(const float* scores, const tq_values* values, const float* codebook, int C,
                       const float* Pi_v, float scale, float* out, int P, int H, int B, int S, int D,
                       void* stream);

/* forms of the fused decode step; TQ_ATTEND_AUTO picks by shape */
#define TQ_ATTEND_AUTO     0
#define TQ_ATTEND_FUSED    1  /* one pass: scores never written */
#define TQ_ATTEND_TWO_PASS 2  /* scores into the workspace, then softmax and values */

/*
 * tq_score_attend_workspace_bytes: workspace tq_score_attend_with_mode needs
 * for this shape and form (0 for an empty shape, invalid sizes, sizes
 * tq_score_attend_with_mode refuses or an unknown form). Host-only.
 */
size_t tq_score_attend_workspace_bytes(int P, int B, int S, int D, int mode);

/*
 * tq_score_attend: the fused decode step, tq_score then tq_attend without
 * writing the scores: each key tile is scored and immediately folded into an
 * online softmax and the value sum ("Fitting 4.4x More Context on Jetson",
 * section "v6: Fused Vectorized Hybrid" and its online-softmax FAQ;
 * "TurboQuant: Rotate-then-Quantize KV Caches at 3 Bits", section 8). For each
 * problem p (head h = p % H) and query b:
 *
 *   s_t    = the raw score of query b against key t (tq_score's formula)
 *   out[p,b,:] = Pi_v[h]^T sum_t softmax(scale * s)_t norm[t] codebook_v[idx_v[t,:]]
 *
 *   A, T, keys, codebook, C   as for tq_score (C <= 8)
 *   values, codebook_v, C_v   as for tq_attend (C_v <= 8)
 *   Pi_v, scale, out          as for tq_attend
 *   workspace                 at least tq_score_attend_workspace_bytes(P, B, S, D)
 *
 * The call runs fused (one pass over keys and values, scores never written)
 * when every wavefront of the fused kernel gets at least two 32-key tiles and
 * B > 8; otherwise, where the two-pass form measured faster (short key chunks,
 * a few queries per problem), it writes the scores into the workspace and runs
 * tq_score and tq_attend's kernels. tq_score_attend_with_mode forces a form.
 * The workspace is tq_score_attend_workspace_bytes(P, B, S, D, mode) bytes for
 * the form used (TQ_ATTEND_AUTO for tq_score_attend).
 *
 * D = 128, S < 2^24. Result within 1e-4 * (1 + |exact|) of the exact output
 * for the given inputs. Errors as for tq_score and tq_attend.
 */
int tq_score_attend(const float* A, const float* T, const tq_keys* keys, const float* codebook, int C,
                    const tq_values* values, const float* codebook_v, int C_v, const float* Pi_v, float scale,
                    float* out, void* workspace, size_t workspace_bytes, int P, int H, int B, int S, int D,
                    void* stream);

/* tq_score_attend with an explicit form (TQ_ATTEND_*), so that both forms can be checked on every shape. */
int tq_score_attend_with_mode(const float* A, const float* T, const tq_keys* keys, const float* codebook, int C,
                              const tq_values* values, const float* codebook_v, int C_v, const float* Pi_v,
                              float scale, float* out, void* workspace, size_t workspace_bytes, int P, int H, int B,
                              int S, int D, int mode, void* stream);

/*
 * tq_query_transform_hadamard: A = H D q for every query, the randomized
 * Hadamard rotation ("TurboQuant: Rotate-then-Quantize KV Caches at 3 Bits",
 * section 2): D = diag(signs) of the query's head, H the orthonormal
 * Walsh-Hadamard matrix in Sylvester order (H[i][j] = (-1)^popcount(i & j) /
 * sqrt(D)). O(D log D) per query instead of the dense product.
 *
 *   q      float32 [P, B, D]
 *   signs  float32 [H, D]      +1 or -1 (problem p uses head p % H)
 *   A      float32 [P, B, D]   output
 *
 * D a power of two, 1 <= D <= TQ_MAX_D (else TQ_ERR_UNSUPPORTED). fp32
 * arithmetic (log2(D) butterfly stages, then the 1/sqrt(D) scale).
 */
int tq_query_transform_hadamard(const float* q, const float* signs, float* A,
                                int P, int H, int B, int D, void* stream);

/*
 * tq_score_mse: raw scores against MSE-only keys, the variant that drops the
 * QJL term ("TurboQuant: Rotate-then-Quantize KV Caches at 3 Bits", sections 3
 * and 6: the MSE quantizer with a stored norm, used for attention with norm
 * correction):
 *
 *   scores[p,b,s] = norm[p,s] * sum_d A[p,b,d] * codebook[idx[p,s,d]]
 *
 * with A = Pi q (tq_query_transform's A, or tq_query_transform_hadamard). With
 * norm correction the stored norm is ||k|| / ||codebook[idx]||, so the same
 * formula serves both.
 *
 *   A         float32 [P, B, D]
 *   keys      MSE-only codes (struct above; host pointer, device pointers inside)
 *   codebook  float32 [C], 1 <= C <= 8 (packed: C == 2^bits)
 *   scores    float32 [P, B, S]   output
 *
 * D in {64, 128, 256} (also 32 unpacked), S < 2^24 (else TQ_ERR_UNSUPPORTED).
 * Result within 1e-4 * (1 + |exact|) of the exact value for the given inputs.
 */
int tq_score_mse(const float* A, const tq_mse_codes* keys, const float* codebook, int C,
                 float* scores, int P, int B, int S, int D, void* stream);

/*
 * The outlier split ("TurboQuant: Rotate-then-Quantize KV Caches at 3 Bits",
 * section 7): two MSE-only instances per head over disjoint channel sets, the
 * hot channels with more bits, each with its own rotation and its own norm.
 * A key stores one tq_mse_codes per instance, over D_hi and D_lo coordinates.
 */
typedef struct tq_split_codes {
    tq_mse_codes hi;   /* the hot channels' instance */
    tq_mse_codes lo;   /* the other channels' instance */
} tq_split_codes;

/*
 * tq_query_transform_split: A_hi = Pi_hi q[perm[0 .. D_hi)] and
 * A_lo = Pi_lo q[perm[D_hi .. D)] for every query (dense fp32 products).
 *
 *   q      float32 [P, B, D]
 *   perm   int32 [D]             a permutation of 0..D-1: the hot channels, then
 *                                the others (not checked)
 *   Pi_hi  float32 [H, D_hi, D_hi], Pi_lo float32 [H, D - D_hi, D - D_hi]
 *   A_hi   float32 [P, B, D_hi],  A_lo float32 [P, B, D - D_hi]   outputs
 *
 * 0 < D_hi < D <= TQ_MAX_D.
 */
int tq_query_transform_split(const float* q, const int32_t* perm, const float* Pi_hi, const float* Pi_lo,
                             float* A_hi, float* A_lo, int P, int H, int B, int D, int D_hi, void* stream);

/*
 * tq_score_split: raw scores against outlier-split keys, the sum of the two
 * instances' MSE scores:
 *
 *   scores[p,b,s] = norm_hi[p,s] * sum_i A_hi[p,b,i] * codebook_hi[idx_hi[p,s,i]]
 *                 + norm_lo[p,s] * sum_j A_lo[p,b,j] * codebook_lo[idx_lo[p,s,j]]
 *
 *   keys       host pointer to the two instances' codes (layouts as tq_mse_codes;
 *              each instance has its own layout and width)
 *   codebooks  float32 [C_hi], [C_lo]: unpacked C <= 256, packed C == 2^bits
 *   scores     float32 [P, B, S]   output
 *
 * D_hi and D_lo multiples of 8 in [8, TQ_MAX_D]. The 2.5-bit setting of the
 * section (D_hi = 32 packed at 3 bits with C_hi = 8, D_lo = 96 packed at 2 bits
 * with C_lo = 4, S < 2^24) runs on the matrix cores (f16 hi/lo parts of fp32
 * operands, fp32 accumulation); other formats in fp32 on the vector ALU. Either
 * way within 1e-4 * (1 + |exact|) of the exact value.
 */
int tq_score_split(const float* A_hi, const float* A_lo, const tq_split_codes* keys,
                   const float* codebook_hi, int C_hi, const float* codebook_lo, int C_lo,
                   float* scores, int P, int B, int S, int D_hi, int D_lo, void* stream);

/* tq_status_string: static description of a status code. */
const char* tq_status_string(int status);

/*
 * Measurement probes (not part of the method): kernels that only move bytes,
 * so a launch of tq_score can be compared with what a launch of the same size
 * can move on the same GPU. Buffers are device memory, 16-byte aligned; byte
 * counts are multiples of 16 and at most 2^36. Contents read are arbitrary.
 *
 * tq_probe_read: loads every 16-byte word of src once (one word per lane); the
 *   loaded words are folded into a value that is written to *sink (a 4-byte
 *   aligned device word) only if it equals an improbable constant.
 * tq_probe_write: stores every 16-byte word of dst once.
 * tq_probe_read_write: workgroup k loads its contiguous slice of src (512
 *   words), then stores its slice of dst (write_bytes spread evenly over the
 *   workgroups) with values that depend on the words it loaded: the
 *   codes-in, scores-out dependency of a scoring launch without its arithmetic.
 *
 * TQ_ERR_ARG for null pointers with nonzero sizes, sizes that are not
 * multiples of 16 or exceed 2^36 (and empty read_write calls); TQ_ERR_ALIGN
 * for misaligned buffers; empty read and write calls return TQ_OK.
 */
int tq_probe_read(const void* src, size_t bytes, void* sink, void* stream);
int tq_probe_write(void* dst, size_t bytes, void* stream);
int tq_probe_read_write(const void* src, size_t read_bytes, void* dst, size_t write_bytes, void* stream);

/*
 * tq_probe_tile: the memory traffic of tq_score's LDS-staged kernel on
 * unpacked keys with one 32-query tile (the decode shape), without its
 * arithmetic, in the same grid: every wavefront takes 32-key tiles; lane
 * (k, g), k = lane % 32, g = lane / 32, loads bytes [g D/2, (g+1) D/2) of key
 * k's index and sign rows (16 bytes per instruction) and gamma[k], folds them
 * into x = bits(gamma) ^ (xor of those 32-bit words), and stores x + v as the
 * bits of out[row, key] for v = 0..15, row = 8 (v / 4) + 4 g + v % 4 (rows
 * past B and keys past S are not written).
 *   keys  unpacked (idx uint8 [S, D], sign int8 [S, D], gamma fp32 [S])
 *   out   float32 [B, S]
 * B <= 32, S < 2^24, D in {64, 128, 256}. TQ_ERR_ARG for a null pointer or a
 * negative size, TQ_ERR_UNSUPPORTED for packed keys or other shapes,
 * TQ_ERR_ALIGN for a buffer that is not 16-byte aligned; B = 0 or S = 0 is a
 * no-op.
 */
int tq_probe_tile(const tq_keys* keys, float* out, int B, int S, int D, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
