// The matrix-core tq_score families (one source file each) and the shape rules
// the dispatch in score_mfma.hip uses to pick one.
#pragma once

#include "mfma_layout.hpp"

namespace tq {

// The products a family's kernels run: split-f16 with QJL signs (the fp32-
// accurate tq_score), its single-pass f16 form (2e-2, a reported comparison
// point), or MSE-only keys (split-f16, no signs, gamma holds the key norms).
enum class ScoreForm { kSplit, kF16, kMse };

// Shapes the families cover: codebooks of at most 8 entries (byte-table
// lookups), unpacked keys or 2/3-bit packed ones.
inline bool lds_supported(int layout, int bits, int C, int D) {
    if (C < 1 || C > 8) return false;          // byte-select lookup tables hold 8 entries
    if (layout == 0) return D == 32 || D == 64 || D == 128 || D == 256;
    if (bits != 2 && bits != 3) return false;
    return D == 64 || D == 128 || D == 256;
}
inline bool reg_supported(int layout, int bits, int C, int D) {
    return lds_supported(layout, bits, C, D) && D <= 128;   // D = 256 would need 256 operand registers
}
inline bool shared_supported(int layout, int bits, int C, int D) {
    return lds_supported(layout, bits, C, D) && (D == 64 || D == 128);   // k-steps split over 4 wavefronts
}
inline bool small_supported(int layout, int bits, int C, int D) {
    return lds_supported(layout, bits, C, D) && (D == 128 || D == 256);   // a lane owns D/4 >= 32 coordinates
}

// 32-query tiles per workgroup of the LDS-staged kernels: as many as B needs,
// up to four, within kMaxLdsBytes of query operands.
constexpr int kMaxLdsBytes = 128 * 1024;
inline int mt_for(int B, int D) {
    const int tiles = (B + 31) / 32;
    const int per_tile = (D / 16) * 4 * 1024;        // LDS bytes per 32-query tile
    int cap = kMaxLdsBytes / per_tile;
    if (cap > 4) cap = 4;
    if (cap < 1) cap = 1;
    if (tiles >= 4 && cap >= 4) return 4;
    if (tiles >= 2 && cap >= 2) return 2;
    return 1;
}

// scores [P, B, S] from A, T [P, B, D] (T unused for kMse) and the key streams.
// score_lds.hip: query operands staged once per workgroup in LDS.
hipError_t launch_family_lds(ScoreForm form, int layout, int bits, const float* A, const float* T, KeyStreams k,
                             const float* codebook, int C, float* scores, int P, int B, int S, int D,
                             hipStream_t stream);
// score_reg.hip: query operands in each wavefront's registers (split form only).
hipError_t launch_family_reg(int layout, int bits, const float* A, const float* T, KeyStreams k, const float* codebook,
                             int C, float* scores, int P, int B, int S, int D, hipStream_t stream);
// score_shared.hip: four query tiles per workgroup share each key tile's unpacking.
hipError_t launch_family_shared(ScoreForm form, int layout, int bits, const float* A, const float* T, KeyStreams k,
                                const float* codebook, int C, float* scores, int P, int B, int S, int D,
                                hipStream_t stream);
// score_small.hip: four queries per workgroup row over many keys.
hipError_t launch_family_small(ScoreForm form, int layout, int bits, const float* A, const float* T, KeyStreams k,
                               const float* codebook, int C, float* scores, int P, int B, int S, int D,
                               hipStream_t stream);

}  // namespace tq
