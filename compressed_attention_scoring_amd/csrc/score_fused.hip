// The decode step fused on the matrix cores: scores, online softmax and the
// value sum in one pass (tq_score_attend's one-pass form).
#include "score_families.hpp"
#include "value_sel.hpp"

namespace tq {
namespace {

using namespace ops;
using namespace layout;

// ---------------------------------------------------------------------------
// Fused decode step: scores, online softmax and value aggregation in one pass,
// so no score reaches HBM ("Fitting 4.4x More Context on Jetson", section "v6:
// Fused Vectorized Hybrid" and its online-softmax FAQ; "TurboQuant:
// Rotate-then-Quantize KV Caches at 3 Bits", section 8, kernel view). One
// workgroup of four wavefronts per (key chunk, 32-query tile, problem); each
// wavefront takes every fourth 32-key tile of the chunk.
//
// Scores come from the same split-f16 products as score_mfma_kernel (query
// operands staged once per workgroup in LDS) with the operands swapped, so the
// accumulators hold keys as rows and queries as columns: lane (query n, half g)
// holds the scores of keys 8(v/4) + 4g + (v%4), v = 0..15, for query n. That is
// the layout the value product wants: with keys as the contraction, lane
// (n, g) supplies its 16 keys' weights in two 16-key steps (slot e of step s is
// its key v = 8s + e), and the value operand of lane (coordinate row, g) takes
// the same keys in the same slots. The online softmax, the norm scaling and the
// split-f16 value products follow attend_partial_kernel's wide mode (value
// coordinates NT*n + t of tile t in lane n). gamma and the value norms of a
// tile's keys are regrouped from the lanes that loaded them through a small
// per-wavefront LDS slot. The workgroup merges its four wavefronts and writes
// (m, l, acc) per query into the attend workspace layout; the attend combine
// kernel finishes.
// ---------------------------------------------------------------------------
constexpr float kFusedTau = 5.5f;   // rescale when a tile's maximum passes the reference by more
constexpr int kFusedNormBits = 4;   // scaled value norms stay below 2^(kFusedNormBits + 2)

template <int LAYOUT, int BITS, int D, int VLAYOUT, int VBITS>
__global__ __launch_bounds__(kThreads) void score_attend_kernel(
    const float* __restrict__ A, const float* __restrict__ T,
    const uint8_t* __restrict__ idx, const uint8_t* __restrict__ sign,
    const void* __restrict__ gamma, const float* __restrict__ codebook, int C,
    const uint8_t* __restrict__ vidx, const void* __restrict__ vnorm,
    const float* __restrict__ vcodebook, int VC, float scale, float* __restrict__ ws,
    int B, int S, int chunk, int nch, float coef) {
    using F = Fmt<LAYOUT, BITS>;
    constexpr int HALF = D / 2;
    constexpr int KS = D / 16;
    constexpr int NI = F::template idx_dw<D>();
    constexpr int NS = F::template sign_dw<D>();
    constexpr int BLOCK = 64 * 16;
    constexpr int OPS_BYTES = KS * 4 * BLOCK;
    constexpr int SEG = 16;
    constexpr int PER_ROW = D / SEG;
    constexpr int ROWS_PER_PASS = kThreads / PER_ROW;
    constexpr int NT = D / 32;                     // value coordinates per lane = tiles of the value product
    constexpr int VBW = VLAYOUT == 0 ? 8 : VBITS;  // value index bits per coordinate
    constexpr int VW = NT * VBW;                   // value bits per lane per key
    constexpr int VROWB = D * VBW / 8;             // bytes per value row
    constexpr int VCROSS = VW > 32 ? 2 : (32 % VW == 0 ? 0 : 1);
    constexpr int DP = D + 1;
    constexpr int MERGE_BYTES = kWaves * 32 * DP * 4;
    constexpr int LDS_BYTES = OPS_BYTES > MERGE_BYTES ? OPS_BYTES : MERGE_BYTES;
    static_assert(HALF % SEG == 0 && VW <= 64 && VROWB % 4 == 0, "fused tiling");

    // the query operands, then (after a barrier) the wavefronts' partial sums
    __shared__ __attribute__((aligned(16))) uint8_t lds_raw[LDS_BYTES];
    __shared__ float2 rowk[32];
    __shared__ __attribute__((aligned(16))) float kv[kWaves][2][32];   // gamma, value norm per tile key
    __shared__ float red_m[kWaves][32];
    __shared__ float red_l[kWaves][32];
    uint8_t* ops = lds_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int p = blockIdx.z;
    const int b0 = blockIdx.y * 32;
    const int rows = min(32, B - b0);
    const int c = blockIdx.x;
    const int col = lane & 31;
    const int g = lane >> 5;
    const int s_begin = c * chunk;
    const int s_end = min(S, s_begin + chunk);
    const int ntl = (s_end - s_begin + kTileKeys - 1) / kTileKeys;   // tiles in this chunk
    const int64_t key0 = (int64_t)p * S;
    const bool qvalid = col < rows;

    float sc = 1.f;
    uint32_t tab_hi[4] = {0u, 0u, 0u, 0u}, tab_lo[4] = {0u, 0u, 0u, 0u};
    TileCodes<NI, NS> codes[2];                  // key code buffers of the tile loop
    TileCodes<NI, NS>& cur = codes[0];
    int tl = wave;                                 // this wavefront's tiles: wave, wave + 4, ...
    auto tile_key = [&](int t) { return min(s_begin + min(t, ntl - 1) * kTileKeys + col, S - 1); };

    // ---- query operands into LDS (as score_mfma_kernel with one query tile)
    const float* Ap = A + ((int64_t)p * B + b0) * D;
    const float* Tp = T + ((int64_t)p * B + b0) * D;
    for (int r0 = 0; r0 < 32; r0 += ROWS_PER_PASS) {
        const int row = r0 + tid / PER_ROW;
        const int pl = tid % PER_ROW;
        float a[SEG], t[SEG];
        float ma = 0.f, mt = 0.f;
        const int rowc = min(row, rows - 1);
#pragma unroll
        for (int k = 0; k < SEG; k += 4) {
            const float4 va = *reinterpret_cast<const float4*>(Ap + (int64_t)rowc * D + pl * SEG + k);
            const float4 vt = *reinterpret_cast<const float4*>(Tp + (int64_t)rowc * D + pl * SEG + k);
            a[k] = va.x; a[k + 1] = va.y; a[k + 2] = va.z; a[k + 3] = va.w;
            t[k] = vt.x; t[k + 1] = vt.y; t[k + 2] = vt.z; t[k + 3] = vt.w;
        }
        if (r0 == 0) {
            asm volatile("" ::: "memory");
            load_tile<LAYOUT, BITS, D>(cur, idx, sign, gamma, key0 + tile_key(tl), g);
            asm volatile("" ::: "memory");
            codebook_tables(codebook, C, sc, tab_hi, tab_lo);
        }
        if (row >= rows) {
#pragma unroll
            for (int k = 0; k < SEG; ++k) a[k] = t[k] = 0.f;
        }
#pragma unroll
        for (int k = 0; k < SEG; ++k) {
            ma = fmaxf(ma, fabsf(a[k]));
            mt = fmaxf(mt, fabsf(t[k]));
        }
#pragma unroll
        for (int o = 1; o < PER_ROW; o <<= 1) {
            ma = fmaxf(ma, __shfl_xor(ma, o));
            mt = fmaxf(mt, __shfl_xor(mt, o));
        }
        const float sA = pow2_scale_for(ma);
        const float sT = pow2_scale_for(mt);
        if (row < 32 && pl == 0) rowk[row] = make_float2(inv_scales(sA, sc), coef / sT);
        {
            const int d0 = pl * SEG;
            const int gg = d0 / HALF;
            const int blk16 = (d0 % HALF) / SEG;
            prologue_store<LAYOUT, BITS, true, SEG>(ops, gg * 32 + row, blk16, a, t, sA, sT, row < 32);
        }
    }

    // value codebook tables (f16 hi and lo parts times a power of two)
    float vsc;
    uint32_t vtab_hi[4], vtab_lo[4];
    codebook_tables(vcodebook, VC, vsc, vtab_hi, vtab_lo);
    // value bits of coordinates NT*col .. NT*col+NT-1: dword k0 of the row, and
    // the next one when the field runs into it
    const int vbit = VBW * NT * col;
    const int vk0 = vbit >> 5;
    const int vsh = vbit & 31;
    const bool vtwo = VCROSS == 2 || (VCROSS == 1 && vsh + VW > 32);
    const uint8_t* vbase = vidx + key0 * VROWB + 4 * vk0;
    __syncthreads();
    const float2 kq = rowk[col];     // this lane's query's factors (M, R)

    // raw value loads of a tile: this lane's 16 keys 8(v/4) + 4g + (v%4)
    struct VRaw {
        uint32_t lo[16], hi[16];
        uint32_t nrm;                  // value norm bits of this lane's own key (col)
    };
    auto vkey = [&](int t, int v) {
        return min(s_begin + min(t, ntl - 1) * kTileKeys + 8 * (v >> 2) + 4 * g + (v & 3), S - 1);
    };
    auto load_values = [&](VRaw& r, int t) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const uint32_t* w = reinterpret_cast<const uint32_t*>(vbase + (int64_t)vkey(t, v) * VROWB);
            r.lo[v] = w[0];
            r.hi[v] = w[vtwo ? 1 : 0];
        }
        if constexpr (VLAYOUT == 0) r.nrm = reinterpret_cast<const uint32_t*>(vnorm)[key0 + tile_key(t)];
        else r.nrm = reinterpret_cast<const uint16_t*>(vnorm)[key0 + tile_key(t)];
    };

    f32x16 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[t][v] = 0.f;
    float M = -INFINITY;       // reference maximum of scale*score for query col
    float lsum = 0.f;          // sum of exp(scale*score - M) over this lane's keys
    float nexp = -1000.f;      // value norms are scaled by 2^-nexp ...
    float nlim = 0.f;          // ... and must stay below nlim

    auto tile_attend = [&](const TileCodes<NI, NS>& cd, const VRaw& vr, int t) __attribute__((always_inline)) {
        // ---- scores, keys as rows
        f32x16 accM, accR;
#pragma unroll
        for (int v = 0; v < 16; ++v) { accM[v] = 0.f; accR[v] = 0.f; }
        Op8 chi[2], clo[2], sg[2];
        key_operands<LAYOUT, BITS, NI, NS>(cd, 0, tab_hi, tab_lo, chi[0], clo[0], sg[0]);
#pragma unroll
        for (int j = 0; j < KS; ++j) {
            const int u = j & 1;
            Op8 ahi, alo, thi, tlo;
            const uint8_t* base = ops + (j * 4) * BLOCK + slot_pos(lane, j) * 16;
            *reinterpret_cast<uint4*>(ahi.u) = *reinterpret_cast<const uint4*>(base + 0 * BLOCK);
            *reinterpret_cast<uint4*>(alo.u) = *reinterpret_cast<const uint4*>(base + 1 * BLOCK);
            *reinterpret_cast<uint4*>(thi.u) = *reinterpret_cast<const uint4*>(base + 2 * BLOCK);
            *reinterpret_cast<uint4*>(tlo.u) = *reinterpret_cast<const uint4*>(base + 3 * BLOCK);
            if (j + 1 < KS) key_operands<LAYOUT, BITS, NI, NS>(cd, j + 1, tab_hi, tab_lo, chi[u ^ 1], clo[u ^ 1], sg[u ^ 1]);
            accM = __builtin_amdgcn_mfma_f32_32x32x16_f16(chi[u].h, ahi.h, accM, 0, 0, 0);
            accR = __builtin_amdgcn_mfma_f32_32x32x16_f16(sg[u].h, thi.h, accR, 0, 0, 0);
            accM = __builtin_amdgcn_mfma_f32_32x32x16_f16(chi[u].h, alo.h, accM, 0, 0, 0);
            accR = __builtin_amdgcn_mfma_f32_32x32x16_f16(sg[u].h, tlo.h, accR, 0, 0, 0);
            accM = __builtin_amdgcn_mfma_f32_32x32x16_f16(clo[u].h, ahi.h, accM, 0, 0, 0);
        }
        // ---- gamma and value norm of the keys this lane holds, regrouped
        if (g == 0) {
            kv[wave][0][col] = cd.gam;
            kv[wave][1][col] = VLAYOUT == 0 ? __builtin_bit_cast(float, vr.nrm)
                                            : (float)__builtin_bit_cast(_Float16, (uint16_t)vr.nrm);
        }
        __builtin_amdgcn_wave_barrier();
        float gm[16], vn[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const float4 a4 = *reinterpret_cast<const float4*>(&kv[wave][0][8 * q4 + 4 * g]);
            const float4 b4 = *reinterpret_cast<const float4*>(&kv[wave][1][8 * q4 + 4 * g]);
            gm[4 * q4 + 0] = a4.x; gm[4 * q4 + 1] = a4.y; gm[4 * q4 + 2] = a4.z; gm[4 * q4 + 3] = a4.w;
            vn[4 * q4 + 0] = b4.x; vn[4 * q4 + 1] = b4.y; vn[4 * q4 + 2] = b4.z; vn[4 * q4 + 3] = b4.w;
        }
        __builtin_amdgcn_wave_barrier();
        // ---- online softmax over this tile's keys for query col
        const int ts = s_begin + t * kTileKeys;
        float z[16];
        float ms = -INFINITY, nm = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int key = ts + 8 * (v >> 2) + 4 * g + (v & 3);
            const float sco = fmaf(kq.y * gm[v], accR[v], accM[v] * kq.x);
            z[v] = (qvalid && key < s_end) ? scale * sco : -INFINITY;
            ms = fmaxf(ms, z[v]);
            nm = fmaxf(nm, fabsf(vn[v]));
        }
        ms = fmaxf(ms, __shfl_xor(ms, 32));
        const bool need_m = ms > M + kFusedTau;
        if (__any(need_m || nm >= nlim)) {
            float nw = nm;
#pragma unroll
            for (int m = 1; m < 64; m <<= 1) nw = fmaxf(nw, __shfl_xor(nw, m));
            float fac = 1.f;
            if (nw >= nlim) {
                int e2;
                (void)frexpf(nw, &e2);
                const float ne = nw > 0.f ? (float)(e2 - kFusedNormBits) : 0.f;
                fac = exp2f(nexp - ne);
                nexp = ne;
                nlim = exp2f(ne + kFusedNormBits + 2);
            }
            const float Mn = need_m ? ms : M;
            const float fm = need_m ? __expf(M - Mn) : 1.f;
            M = Mn;
            lsum *= fm;
            fac *= fm;
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[tt][v] *= fac;
        }
        const float nscale = exp2f(-nexp);
        Op8 whi[2], wlo[2];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float w = z[v] == -INFINITY ? 0.f : __expf(z[v] - M);
            lsum += w;
            const float x = w * vn[v] * nscale;
            const _Float16 h = (_Float16)x;
            whi[v >> 3].h[v & 7] = h;
            wlo[v >> 3].h[v & 7] = (_Float16)(x - (float)h);
        }
        // ---- value products: step st takes keys v = 8 st + e in slot e
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            uint64_t vb[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int v = 8 * st + e;
                vb[e] = ((vtwo ? (uint64_t)vr.hi[v] << 32 : 0ull) | vr.lo[v]) >> vsh;
            }
            // packed fields (VW <= 32 bits per key): selectors from byte-transposed bits
            constexpr bool BYTES = VLAYOUT == 1 && VW <= 32;
            using VS = typename std::conditional<BYTES, ValueSelectors<VBW, VW>, NoValueSelectors>::type;
            const VS vs(vb);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                uint32_t sel0 = 0, sel1 = 0;
                if constexpr (BYTES) {
                    vs.tile(tt, sel0, sel1);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        sel0 |= ((uint32_t)(vb[e] >> (VBW * tt)) & ((1u << VBW) - 1u)) << (8 * e);
                        sel1 |= ((uint32_t)(vb[4 + e] >> (VBW * tt)) & ((1u << VBW) - 1u)) << (8 * e);
                    }
                }
                Op8 vhi, vlo;
                lut4(sel0, vtab_hi, vhi.u[0], vhi.u[1]);
                lut4(sel1, vtab_hi, vhi.u[2], vhi.u[3]);
                lut4(sel0, vtab_lo, vlo.u[0], vlo.u[1]);
                lut4(sel1, vtab_lo, vlo.u[2], vlo.u[3]);
                acc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vhi.h, whi[st].h, acc[tt], 0, 0, 0);
                acc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vlo.h, whi[st].h, acc[tt], 0, 0, 0);
                acc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vhi.h, wlo[st].h, acc[tt], 0, 0, 0);
            }
        }
    };

    if (tl < ntl) {
        VRaw vals[2];                                // the raw values travel with the key codes
        load_values(vals[0], tl);
        rotate_tiles<2>(
            tl, kWaves, ntl,
            [&](auto ph, int t) __attribute__((always_inline)) {
                load_tile<LAYOUT, BITS, D>(codes[decltype(ph)::value], idx, sign, gamma, key0 + tile_key(t), g);
                load_values(vals[decltype(ph)::value], t);
            },
            [&](auto ph, int t) __attribute__((always_inline)) {
                tile_attend(codes[decltype(ph)::value], vals[decltype(ph)::value], t);
            });
    }

    // ---- this wavefront's (m, l, acc) to LDS (true scale), then merge the four
    lsum += __shfl_xor(lsum, 32);
    const float unscale = exp2f(nexp) / vsc;
    __syncthreads();                                   // every wavefront is done with the query operands
    float* red_acc = reinterpret_cast<float*>(lds_raw);   // [kWaves][32][DP]
    if (g == 0) {
        red_m[wave][col] = M;
        red_l[wave][col] = lsum;
    }
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int row = 8 * (v >> 2) + 4 * g + (v & 3);
            red_acc[(wave * 32 + col) * DP + NT * row + tt] = acc[tt][v] * unscale;
        }
    __syncthreads();
    for (int i = tid; i < 32 * D; i += kThreads) {
        const int d = i % D;
        const int qi = i / D;
        if (qi >= rows) continue;
        float Mx = -INFINITY;
#pragma unroll
        for (int k = 0; k < kWaves; ++k) Mx = fmaxf(Mx, red_m[k][qi]);
        float a = 0.f, l = 0.f;
#pragma unroll
        for (int k = 0; k < kWaves; ++k) {
            const float f = red_m[k][qi] == -INFINITY ? 0.f : __expf(red_m[k][qi] - Mx);
            a = fmaf(red_acc[(k * 32 + qi) * DP + d], f, a);
            l = fmaf(red_l[k][qi], f, l);
        }
        float* rec = ws + (((int64_t)p * B + b0 + qi) * nch + c) * (D + 2);
        rec[2 + d] = a;
        if (d == 0) {
            rec[0] = Mx;
            rec[1] = l;
        }
    }
}

}  // namespace

namespace {

template <int LAYOUT, int BITS, int VLAYOUT, int VBITS>
hipError_t launch_fused(const float* A, const float* T, KeyStreams k, const float* codebook, int C,
                        ValueStreams v, const float* vcodebook, int VC, float scale, float* ws, int P, int B, int S,
                        int chunk, int nch, hipStream_t stream) {
    constexpr int D = 128;
    const float coef = (float)(kSqrtHalfPi / (double)D);
    hipLaunchKernelGGL((score_attend_kernel<LAYOUT, BITS, D, VLAYOUT, VBITS>), dim3((unsigned)nch, (B + 31) / 32, P),
                       dim3(kThreads), 0, stream, A, T, k.idx, k.sign, k.gamma, codebook, C, v.idx, v.norm,
                       vcodebook, VC, scale, ws, B, S, chunk, nch, coef);
    return hipGetLastError();
}

template <int LAYOUT, int BITS>
hipError_t launch_fused_v(int vlayout, int vbits, const float* A, const float* T, KeyStreams k, const float* codebook,
                          int C, ValueStreams v, const float* vcodebook, int VC, float scale, float* ws, int P, int B,
                          int S, int chunk, int nch, hipStream_t stream) {
    if (vlayout == 0)
        return launch_fused<LAYOUT, BITS, 0, 0>(A, T, k, codebook, C, v, vcodebook, VC, scale, ws, P, B, S, chunk, nch, stream);
    if (vbits == 2)
        return launch_fused<LAYOUT, BITS, 1, 2>(A, T, k, codebook, C, v, vcodebook, VC, scale, ws, P, B, S, chunk, nch, stream);
    return launch_fused<LAYOUT, BITS, 1, 3>(A, T, k, codebook, C, v, vcodebook, VC, scale, ws, P, B, S, chunk, nch, stream);
}

}  // namespace

// Chunks of the fused step: multiples of four 32-key tiles (one per wavefront),
// about 256 workgroups in all (one per compute unit: the kernel holds about
// 66 KB of LDS).
void score_attend_plan(int P, int B, int S, int& chunk, int& nch) {
    const int64_t blocks = (int64_t)P * ((B + 31) / 32);
    int64_t n = (256 + blocks - 1) / blocks;
    const int64_t most = ((int64_t)S + 4 * kTileKeys - 1) / (4 * kTileKeys);
    if (n > most) n = most;
    if (n < 1) n = 1;
    const int64_t per = ((int64_t)S + n - 1) / n;
    chunk = (int)((per + 4 * kTileKeys - 1) / (4 * kTileKeys) * (4 * kTileKeys));
    nch = (S + chunk - 1) / chunk;
}

bool score_attend_supported(int layout, int bits, int C, int vlayout, int vbits, int VC, int D) {
    return D == 128 && lds_supported(layout, bits, C, D) && VC >= 1 && VC <= 8 &&
           (vlayout == 0 || vbits == 2 || vbits == 3);
}

hipError_t launch_score_attend_partial(const float* A, const float* T, KeyStreams keys, int layout, int bits,
                                       const float* codebook, int C, ValueStreams v, int vlayout, int vbits,
                                       const float* vcodebook, int VC, float scale, float* ws, int P, int B, int S,
                                       int chunk, int nch, hipStream_t stream) {
    if (layout == 0)
        return launch_fused_v<0, 0>(vlayout, vbits, A, T, keys, codebook, C, v, vcodebook, VC, scale, ws, P, B, S, chunk, nch, stream);
    if (bits == 2)
        return launch_fused_v<1, 2>(vlayout, vbits, A, T, keys, codebook, C, v, vcodebook, VC, scale, ws, P, B, S, chunk, nch, stream);
    return launch_fused_v<1, 3>(vlayout, vbits, A, T, keys, codebook, C, v, vcodebook, VC, scale, ws, P, B, S, chunk, nch, stream);
}

}  // namespace tq
