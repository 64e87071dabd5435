// tq_score on the matrix cores for B > 96: four register-resident query tiles
// per workgroup share one unpacking of each key tile through LDS (CDNA4
// v_mfma_f32_32x32x16_f16). The scoring identity and the split-f16 products
// are those of score_lds.hip.
#include <type_traits>

#include "score_families.hpp"

namespace tq {
namespace {

using namespace ops;
using namespace layout;

// ---------------------------------------------------------------------------
// Shared-decode variant (B > 96): the four wavefronts of a workgroup hold four
// different 32-query tiles in registers (as in score_qs_kernel) and walk the
// same key tiles. Each key tile is unpacked once per workgroup: wavefront w
// builds the key-side operands of k-steps [w KS/4, (w+1) KS/4) into one of two
// LDS buffers while the MFMAs of the previous tile read the other, with one
// workgroup barrier per tile. This removes the fourfold key decoding of the
// register variant, whose main loop was bound by vector-ALU issue.
// ---------------------------------------------------------------------------
// Coalesced loading of one wavefront's 32 query rows into the register layout
// in which lane (col, g) holds row col's coordinates [g D/2, (g+1) D/2). Loading
// that half row directly makes each load instruction touch 64 different
// 128-byte lines, one per lane; with every workgroup re-reading all of A and T
// that prologue took about a fifth of the long launch (timeline stamps: operands
// ready ~8 us after the first wave starts). Here each instruction reads whole
// lines of consecutive rows, and a transpose through the wavefront's own LDS
// region hands every lane its half row. Chunk c holds the CW/2 columns from
// c CW/2 on of both halves of all 32 rows; 16-byte slots are XOR-swizzled by row
// so that neither the writes nor the reads conflict on banks.
template <int D, int CW>
struct RowStage {
    static constexpr int HALF = D / 2;
    static constexpr int NSL = CW / 4;            // 16-byte slots per staged row
    static constexpr int NCH = HALF / (CW / 2);   // chunks per matrix
    static constexpr int PER = CW / 8;            // 16-byte loads per lane per chunk
    static constexpr int BYTES = 32 * CW * 4;     // LDS region per wavefront
    static_assert(CW == 32 || CW == 64, "16 or 8 slots per staged row");
    static_assert(HALF % (CW / 2) == 0, "chunks tile each half row");

    // slot of (row r, slot q): rows that one 16-lane LDS pass touches land on
    // distinct 4-bank groups (two rows share the 64 banks when CW = 32)
    __device__ static __forceinline__ int swz(int r, int q) { return q ^ ((r / (16 / NSL)) % NSL); }

    // Requests this lane's part of chunk c of the matrix whose wavefront rows
    // start at `rows`; row r reads row min(r, last) (rows past the end re-read
    // a valid one and are never stored).
    __device__ static __forceinline__ void load(const float* rows, int last, int lane, int c, float (&v)[4 * PER]) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int f = i * 64 + lane;
            const int r = f / NSL, q = f % NSL;
            const int h = q / (NSL / 2), w = q % (NSL / 2);
            const float4 x = *reinterpret_cast<const float4*>(rows + (int64_t)min(r, last) * D + h * HALF + c * (CW / 2) + w * 4);
            v[4 * i] = x.x; v[4 * i + 1] = x.y; v[4 * i + 2] = x.z; v[4 * i + 3] = x.w;
        }
    }

    // Writes chunk c to the wavefront's region and reads back this lane's
    // columns of it into dst[c CW/2 ...]. The region is private to the
    // wavefront, so wavefront-scope ordering suffices; the second fence keeps
    // the next chunk's writes behind this chunk's reads.
    __device__ static __forceinline__ void transpose(uint8_t* region, int lane, int c, const float (&v)[4 * PER],
                                                     float (&dst)[HALF]) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int f = i * 64 + lane;
            const int r = f / NSL, q = f % NSL;
            *reinterpret_cast<float4*>(region + r * CW * 4 + swz(r, q) * 16) =
                make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int col = lane & 31, g = lane >> 5;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const float4 x = *reinterpret_cast<const float4*>(region + col * CW * 4 + swz(col, g * (NSL / 2) + i) * 16);
            dst[c * (CW / 2) + 4 * i] = x.x;
            dst[c * (CW / 2) + 4 * i + 1] = x.y;
            dst[c * (CW / 2) + 4 * i + 2] = x.z;
            dst[c * (CW / 2) + 4 * i + 3] = x.w;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
};

// Per k-step LDS blocks: the codebook's hi part, its lo part unless F16, and
// the signs with QJL.
template <int LAYOUT, int BITS, int D, bool QJL = true, bool F16 = false>
struct SharedLds {
    static constexpr int KS = D / 16;
    static constexpr int BLOCK = 64 * 16;                       // one operand: 64 lanes x 16 bytes
    static constexpr int CLO = 1;                               // block of the codebook lo part (not F16)
    static constexpr int SG = F16 ? 1 : 2;                      // block of the signs (QJL)
    static constexpr int NB = (F16 ? 1 : 2) + (QJL ? 1 : 0);    // operands per k-step
    static constexpr int BUF = KS * NB * BLOCK;
};

template <int LAYOUT, int BITS, int D, int W, bool QJL = true, bool F16 = false>
__device__ __forceinline__ void decode_share(const TileCodes<Fmt<LAYOUT, BITS>::template idx_dw<D>(),
                                                         Fmt<LAYOUT, BITS>::template sign_dw<D>()>& c,
                                             const uint32_t (&tab_hi)[4], const uint32_t (&tab_lo)[4],
                                             uint8_t* buf, int lane) {
    using F = Fmt<LAYOUT, BITS>;
    constexpr int NI = F::template idx_dw<D>(), NS = F::template sign_dw<D>();
    using L = SharedLds<LAYOUT, BITS, D, QJL, F16>;
    constexpr int KS = D / 16, JW = KS / kWaves, BLOCK = L::BLOCK;
#pragma unroll
    for (int jj = 0; jj < JW; ++jj) {
        const int j = W * JW + jj;
        Op8 chi, clo, sg;
        key_operands<LAYOUT, BITS, NI, NS, QJL, !F16>(c, j, tab_hi, tab_lo, chi, clo, sg);
        uint8_t* base = buf + (j * L::NB) * BLOCK + lane * 16;
        *reinterpret_cast<uint4*>(base + 0 * BLOCK) = *reinterpret_cast<const uint4*>(chi.u);
        if constexpr (!F16) *reinterpret_cast<uint4*>(base + L::CLO * BLOCK) = *reinterpret_cast<const uint4*>(clo.u);
        if constexpr (QJL) *reinterpret_cast<uint4*>(base + L::SG * BLOCK) = *reinterpret_cast<const uint4*>(sg.u);
    }
}

// QJL = false: MSE-only keys (no sign stream, no T, gamma = the key's norm).
// F16 = true (with QJL): the single-pass f16 form, two products per k-step
// (A_hi c_hi, T_hi sigma) and no lo halves in registers or LDS.
template <int LAYOUT, int BITS, int D, bool QJL = true, bool F16 = false>
__global__ __launch_bounds__(kThreads, 2) void score_shared_kernel(
    const float* __restrict__ A, const float* __restrict__ T,
    const uint8_t* __restrict__ idx, const uint8_t* __restrict__ sign,
    const void* __restrict__ gamma, const float* __restrict__ codebook, int C,
    float* __restrict__ scores, int B, int S, float coef) {
    using F = Fmt<LAYOUT, BITS>;
    using L = SharedLds<LAYOUT, BITS, D, QJL, F16>;
    constexpr int HALF = D / 2;
    constexpr int KS = D / 16;
    constexpr int NI = F::template idx_dw<D>();
    constexpr int NS = F::template sign_dw<D>();
    constexpr int QT = QJL ? KS : 1;            // T operands kept (none without QJL)
    constexpr int LT = F16 ? 1 : KS;            // lo halves kept (none in the f16 form)
    static_assert(KS % kWaves == 0, "each wavefront unpacks the same number of k-steps");

    __shared__ __attribute__((aligned(16))) uint8_t kops[2 * L::BUF];
    __shared__ float2 rowk[kWaves][32];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int p = blockIdx.z;
    const int b0 = (blockIdx.y * kWaves + wave) * 32;
    const bool has_q = b0 < B;                 // uniform per wavefront; others only unpack keys
    const int rows = has_q ? min(32, B - b0) : 0;
    const int col = lane & 31;
    const int g = lane >> 5;
    const int ntiles = (S + kTileKeys - 1) / kTileKeys;
    const int64_t key0 = (int64_t)p * S;
    int tile = blockIdx.x;                     // uniform per workgroup: every barrier is reached by all
    const int stride = gridDim.x;
    if (tile >= ntiles) return;

    // Query half rows (rows past B re-read row B - 1; wavefronts past B never
    // store). Both LDS buffers serve as the staging area of the coalesced load
    // when they hold a 4 KiB region per wavefront; one barrier then frees them
    // for the first tile.
    constexpr bool STAGED = 2 * L::BUF / kWaves >= RowStage<D, 32>::BYTES;
    using RS = RowStage<D, (2 * L::BUF / kWaves >= RowStage<D, 64>::BYTES) ? 64 : 32>;
    static_assert(!STAGED || kWaves * RS::BYTES <= 2 * L::BUF, "staging regions fit the LDS buffers");
    float a[HALF], t[HALF];
    float va[RS::NCH][4 * RS::PER], vt[RS::NCH][4 * RS::PER];
    const int last = B - 1 - b0;
    if constexpr (STAGED) {
#pragma unroll
        for (int c = 0; c < RS::NCH; ++c) RS::load(A + ((int64_t)p * B + b0) * D, last, lane, c, va[c]);
        if constexpr (QJL) {
#pragma unroll
            for (int c = 0; c < RS::NCH; ++c) RS::load(T + ((int64_t)p * B + b0) * D, last, lane, c, vt[c]);
        }
    } else {
        const int64_t roff = ((int64_t)p * B + min(b0 + col, B - 1)) * D + g * HALF;
#pragma unroll
        for (int k = 0; k < HALF; k += 4) {
            const float4 x = *reinterpret_cast<const float4*>(A + roff + k);
            a[k] = x.x; a[k + 1] = x.y; a[k + 2] = x.z; a[k + 3] = x.w;
            if constexpr (QJL) {
                const float4 y = *reinterpret_cast<const float4*>(T + roff + k);
                t[k] = y.x; t[k + 1] = y.y; t[k + 2] = y.z; t[k + 3] = y.w;
            }
        }
    }
    if constexpr (!QJL) {
#pragma unroll
        for (int k = 0; k < HALF; ++k) t[k] = 0.f;
    }
    TileCodes<NI, NS> c0, c1;
    asm volatile("" ::: "memory");
    load_tile_at<LAYOUT, BITS, D, QJL>(c0, idx, sign, gamma, key0, tile, S, col, g);
    load_tile_at<LAYOUT, BITS, D, QJL>(c1, idx, sign, gamma, key0, tile + stride, S, col, g);
    asm volatile("" ::: "memory");
    float sc;
    uint32_t tab_hi[4], tab_lo[4];
    codebook_tables(codebook, C, sc, tab_hi, tab_lo);
    if constexpr (STAGED) {
        uint8_t* region = kops + wave * RS::BYTES;
#pragma unroll
        for (int c = 0; c < RS::NCH; ++c) RS::transpose(region, lane, c, va[c], a);
        if constexpr (QJL) {
#pragma unroll
            for (int c = 0; c < RS::NCH; ++c) RS::transpose(region, lane, c, vt[c], t);
        }
        __syncthreads();
    }

    float ma = 0.f, mt = 0.f;
#pragma unroll
    for (int k = 0; k < HALF; ++k) {
        ma = fmaxf(ma, fabsf(a[k]));
        mt = fmaxf(mt, fabsf(t[k]));
    }
    ma = fmaxf(ma, __shfl_xor(ma, 32));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float sA = pow2_scale_for(ma);
    const float sT = pow2_scale_for(mt);
    if (g == 0) rowk[wave][col] = make_float2(inv_scales(sA, sc), coef / sT);
    Op8 ahi[KS], alo[LT], thi[QT], tlo[F16 ? 1 : QT];
#pragma unroll
    for (int j = 0; j < KS; ++j) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float xa = a[mse_dim<LAYOUT, BITS>(j, e)] * sA;
            const _Float16 ha = (_Float16)xa;
            ahi[j].h[e] = ha;
            if constexpr (!F16) alo[j].h[e] = (_Float16)(xa - (float)ha);
            if constexpr (QJL) {
                const float xt = t[qjl_dim<LAYOUT>(j, e)] * sT;
                const _Float16 ht = (_Float16)xt;
                thi[j].h[e] = ht;
                if constexpr (!F16) tlo[j].h[e] = (_Float16)(xt - (float)ht);
            }
        }
    }

    auto decode = [&](const TileCodes<NI, NS>& c, uint8_t* buf) __attribute__((always_inline)) {
        switch (wave) {
            case 0: decode_share<LAYOUT, BITS, D, 0, QJL, F16>(c, tab_hi, tab_lo, buf, lane); break;
            case 1: decode_share<LAYOUT, BITS, D, 1, QJL, F16>(c, tab_hi, tab_lo, buf, lane); break;
            case 2: decode_share<LAYOUT, BITS, D, 2, QJL, F16>(c, tab_hi, tab_lo, buf, lane); break;
            default: decode_share<LAYOUT, BITS, D, 3, QJL, F16>(c, tab_hi, tab_lo, buf, lane); break;
        }
    };
    decode(c0, kops);
    __syncthreads();
    // epilogue factors of the 16 rows this lane's accumulators hold, read once
    // (long workload 49.2 -> 48.0 us against an LDS read per row and tile)
    float2 rk[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) rk[v] = rowk[wave][8 * (v >> 2) + 4 * g + (v & 3)];

    // wavefronts past B compute too (no branch around the stores keeps the wait
    // counts exact); their descriptor covers no rows, so every store is dropped
    const __amdgpu_buffer_rsrc_t out_r = score_rows(scores + ((int64_t)p * B + (has_q ? b0 : 0)) * S, rows, S);
    float gam_cur = c0.gam;

    // One tile from LDS buffer `buf`: `cr` is refilled two tiles ahead, this
    // tile's MFMAs are issued, and then the next tile's codes `cn` are unpacked
    // into the other buffer (its gamma kept for the next step), so the wait for
    // those codes comes after this tile's matrix work rather than before it;
    // one barrier ends the step. Past the last tile `cn` holds zeros whose
    // unpacking nobody reads.
    auto step = [&](int t, uint8_t* buf, uint8_t* other, const TileCodes<NI, NS>& cn, TileCodes<NI, NS>& cr)
        __attribute__((always_inline)) {
        load_tile_at<LAYOUT, BITS, D, QJL>(cr, idx, sign, gamma, key0, t + 2 * stride, S, col, g);
        f32x16 accM, accR;
#pragma unroll
        for (int v = 0; v < 16; ++v) { accM[v] = 0.f; accR[v] = 0.f; }
        // key operands of k-step j + 1 are read from LDS while the MFMAs of k-step
        // j run (two register sets in turn), so LDS latency does not stall the chain
        const uint8_t* my = buf + lane * 16;
        Op8 kop[2][3];
        // o[0]: codebook hi, o[1]: codebook lo (not F16), o[2]: signs (QJL)
        auto read_ops = [&](int j, Op8 (&o)[3]) __attribute__((always_inline)) {
            *reinterpret_cast<uint4*>(o[0].u) = *reinterpret_cast<const uint4*>(my + (j * L::NB + 0) * L::BLOCK);
            if constexpr (!F16)
                *reinterpret_cast<uint4*>(o[1].u) =
                    *reinterpret_cast<const uint4*>(my + (j * L::NB + L::CLO) * L::BLOCK);
            if constexpr (QJL)
                *reinterpret_cast<uint4*>(o[2].u) =
                    *reinterpret_cast<const uint4*>(my + (j * L::NB + L::SG) * L::BLOCK);
        };
        read_ops(0, kop[0]);
#pragma unroll
        for (int j = 0; j < KS; ++j) {
            const Op8(&o)[3] = kop[j & 1];
            if (j + 1 < KS) read_ops(j + 1, kop[(j + 1) & 1]);
            accM = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[j].h, o[0].h, accM, 0, 0, 0);
            if constexpr (F16) {
                accR = __builtin_amdgcn_mfma_f32_32x32x16_f16(thi[j].h, o[2].h, accR, 0, 0, 0);
            } else if constexpr (QJL) {
                accR = __builtin_amdgcn_mfma_f32_32x32x16_f16(thi[j].h, o[2].h, accR, 0, 0, 0);
                accM = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo[j].h, o[0].h, accM, 0, 0, 0);
                accR = __builtin_amdgcn_mfma_f32_32x32x16_f16(tlo[j].h, o[2].h, accR, 0, 0, 0);
            } else {
                accM = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo[j].h, o[0].h, accM, 0, 0, 0);
            }
            if constexpr (!F16) accM = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[j].h, o[1].h, accM, 0, 0, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, L::NB, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, F16 ? 2 : QJL ? 5 : 3, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        decode(cn, other);
        const float gam_next = cn.gam;
        const uint32_t lo = lane_offset(t * kTileKeys + col, S, g);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float2 k = rk[v];
            if constexpr (QJL)
                store_score(out_r, lo + row_offset(v, S), fmaf(k.y * gam_cur, accR[v], accM[v] * k.x));
            else
                store_score(out_r, lo + row_offset(v, S), (k.x * gam_cur) * accM[v]);
        }
        gam_cur = gam_next;
        __syncthreads();
    };
    alternate_tiles(tile, stride, ntiles, [&](auto phase, int t) __attribute__((always_inline)) {
        if constexpr (decltype(phase)::value == 0)
            step(t, kops, kops + L::BUF, c1, c0);
        else
            step(t, kops + L::BUF, kops, c0, c1);
    });
}


// Shared-decode launch: workgroup rows are groups of four 32-query tiles; two
// workgroups per CU are resident (registers), so 512 workgroups fill the chip.
template <int LAYOUT, int BITS, int D, bool QJL = true, bool F16 = false>
hipError_t launch_shared_d(const float* A, const float* T, KeyStreams k, const float* codebook, int C,
                           float* scores, int P, int B, int S, hipStream_t stream) {
    const int groups_y = (B + 127) / 128;
    const int ntiles = (S + kTileKeys - 1) / kTileKeys;
    int64_t gx = ntiles;
    int64_t cap = 512 / ((int64_t)groups_y * P);
    if (cap < 1) cap = 1;
    if (gx > cap) gx = cap;
    const float coef = (float)(kSqrtHalfPi / (double)D);
    hipLaunchKernelGGL((score_shared_kernel<LAYOUT, BITS, D, QJL, F16>), dim3((unsigned)gx, groups_y, P),
                       dim3(kThreads), 0, stream, A, T, k.idx, k.sign, k.gamma, codebook, C,
                       scores, B, S, coef);
    return hipGetLastError();
}

template <int LAYOUT, int BITS, bool QJL = true, bool F16 = false>
hipError_t launch_shared_layout(const float* A, const float* T, KeyStreams k, const float* codebook,
                                int C, float* scores, int P, int B, int S, int D, hipStream_t stream) {
    if (D == 64) return launch_shared_d<LAYOUT, BITS, 64, QJL, F16>(A, T, k, codebook, C, scores, P, B, S, stream);
    if (D == 128) return launch_shared_d<LAYOUT, BITS, 128, QJL, F16>(A, T, k, codebook, C, scores, P, B, S, stream);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_family_shared(ScoreForm form, int layout, int bits, const float* A, const float* T, KeyStreams k,
                               const float* codebook, int C, float* scores, int P, int B, int S, int D,
                               hipStream_t stream) {
    auto by_layout = [&](auto qjl, auto f16) {
        constexpr bool QJL = decltype(qjl)::value, F16 = decltype(f16)::value;
        if (layout == 0) return launch_shared_layout<0, 0, QJL, F16>(A, T, k, codebook, C, scores, P, B, S, D, stream);
        if (bits == 2) return launch_shared_layout<1, 2, QJL, F16>(A, T, k, codebook, C, scores, P, B, S, D, stream);
        return launch_shared_layout<1, 3, QJL, F16>(A, T, k, codebook, C, scores, P, B, S, D, stream);
    };
    switch (form) {
        case ScoreForm::kF16: return by_layout(std::true_type{}, std::true_type{});
        case ScoreForm::kMse: return by_layout(std::false_type{}, std::false_type{});
        default: return by_layout(std::true_type{}, std::false_type{});
    }
}

}  // namespace tq
