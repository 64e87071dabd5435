// Matrix-core tq_score: which family runs a shape, the kernels' names, and the
// dispatch. The families live one per file: score_lds.hip (LDS-staged query
// operands, B <= 32), score_reg.hip (register-resident, 32 < B <= 96),
// score_shared.hip (shared key unpacking, B > 96), score_small.hip (four
// queries over many keys), with the outlier split in score_split_mfma.hip and
// the fused decode step in score_fused.hip.
#include "score_families.hpp"

namespace tq {

namespace {

// Automatic choice, from measurements on the five workload shapes: with a single
// 32-query tile (B <= 32) the workgroup-shared LDS staging wins (its one-time
// operand build is split over 256 threads); with more query tiles the
// register-resident operands win (no LDS traffic in the main loop).
int pick_variant(int layout, int bits, int C, int B, int64_t keys, int D) {
    // One group of four queries: 12 16x16 MFMAs per 16 keys against 40 32x32
    // ones per 32 keys padded. Each wavefront builds its own query operands, so
    // this pays once wavefronts see many tiles (measured: GQA's 4.2 M keys run
    // 1.6x faster, one problem of 32 K keys runs slower). With two groups of
    // four the key decoding doubles and the padded 32x32 tile measured faster.
    if (B <= 4 && keys >= (int64_t(1) << 20) && small_supported(layout, bits, C, D)) return kMfmaSmall;
    // Four or more query tiles: the shared-decode variant unpacks each key tile
    // once for all four (long workload 51.3 -> 48.3 us against the register
    // variant); with three, one of its four wavefronts would idle.
    if (B > 96 && shared_supported(layout, bits, C, D)) return kMfmaShared;
    if (B > 32 && reg_supported(layout, bits, C, D)) return kMfmaReg;
    return kMfmaLds;
}

// The single-pass f16 form takes the automatic choice's family, with the
// LDS-staged kernel where that choice is the register-resident one.
int pick_f16_variant(int layout, int bits, int C, int B, int64_t keys, int D) {
    const int v = pick_variant(layout, bits, C, B, keys, D);
    return v == kMfmaReg ? kMfmaLds : v;
}

// The name of a kernel's single-pass f16 form (static strings).
const char* with_f16_suffix(const char* base) {
    if (!base) return nullptr;
    static const char* const names[][2] = {
        {"mfma32_unpacked_mt1", "mfma32_unpacked_mt1_f16"}, {"mfma32_unpacked_mt2", "mfma32_unpacked_mt2_f16"},
        {"mfma32_unpacked_mt4", "mfma32_unpacked_mt4_f16"}, {"mfma32_packed2_mt1", "mfma32_packed2_mt1_f16"},
        {"mfma32_packed2_mt2", "mfma32_packed2_mt2_f16"}, {"mfma32_packed2_mt4", "mfma32_packed2_mt4_f16"},
        {"mfma32_packed3_mt1", "mfma32_packed3_mt1_f16"}, {"mfma32_packed3_mt2", "mfma32_packed3_mt2_f16"},
        {"mfma32_packed3_mt4", "mfma32_packed3_mt4_f16"}, {"mfma16_unpacked", "mfma16_unpacked_f16"},
        {"mfma16i8_packed2", "mfma16_packed2_f16"}, {"mfma16i8_packed3", "mfma16_packed3_f16"},
        {"mfma32shared_unpacked", "mfma32shared_unpacked_f16"}, {"mfma32shared_packed2", "mfma32shared_packed2_f16"},
        {"mfma32shared_packed3", "mfma32shared_packed3_f16"},
    };
    for (const auto& n : names)
        if (__builtin_strcmp(n[0], base) == 0) return n[1];
    return nullptr;
}
}  // namespace

bool score_mfma_supported(int layout, int bits, int C, int B, int D, int variant) {
    (void)B;
    if (variant == kMfmaAuto || variant == kMfmaF16) return lds_supported(layout, bits, C, D);
    if (variant == kMfmaLds) return lds_supported(layout, bits, C, D);
    if (variant == kMfmaReg) return reg_supported(layout, bits, C, D);
    if (variant == kMfmaSmall) return small_supported(layout, bits, C, D);
    if (variant == kMfmaShared) return shared_supported(layout, bits, C, D);
    return false;
}

const char* score_mfma_name(int layout, int bits, int C, int P, int B, int S, int D, int variant) {
    if (!score_mfma_supported(layout, bits, C, B, D, variant)) return nullptr;
    if (variant == kMfmaF16)
        return with_f16_suffix(score_mfma_name(layout, bits, C, P, B, S, D,
                                               pick_f16_variant(layout, bits, C, B, (int64_t)P * S, D)));
    if (variant == kMfmaAuto) variant = pick_variant(layout, bits, C, B, (int64_t)P * S, D);
    if (variant == kMfmaReg) return layout == 0 ? "mfma32reg_unpacked" : bits == 2 ? "mfma32reg_packed2" : "mfma32reg_packed3";
    if (variant == kMfmaSmall) return layout == 0 ? "mfma16_unpacked" : bits == 2 ? "mfma16i8_packed2" : "mfma16i8_packed3";
    if (variant == kMfmaShared) return layout == 0 ? "mfma32shared_unpacked" : bits == 2 ? "mfma32shared_packed2" : "mfma32shared_packed3";
    const int mt = mt_for(B, D);
    if (layout == 0) return mt == 4 ? "mfma32_unpacked_mt4" : mt == 2 ? "mfma32_unpacked_mt2" : "mfma32_unpacked_mt1";
    if (bits == 2) return mt == 4 ? "mfma32_packed2_mt4" : mt == 2 ? "mfma32_packed2_mt2" : "mfma32_packed2_mt1";
    return mt == 4 ? "mfma32_packed3_mt4" : mt == 2 ? "mfma32_packed3_mt2" : "mfma32_packed3_mt1";
}

hipError_t launch_score_mfma(const float* A, const float* T, KeyStreams keys,
                             int layout, int bits, const float* codebook, int C,
                             float* scores, int P, int B, int S, int D, int variant,
                             hipStream_t stream) {
    if (!score_mfma_supported(layout, bits, C, B, D, variant)) return hipErrorInvalidValue;
    if (variant == kMfmaF16) {
        const int v = pick_f16_variant(layout, bits, C, B, (int64_t)P * S, D);
        if (v == kMfmaShared)
            return launch_family_shared(ScoreForm::kF16, layout, bits, A, T, keys, codebook, C, scores, P, B, S, D, stream);
        if (v == kMfmaSmall)
            return launch_family_small(ScoreForm::kF16, layout, bits, A, T, keys, codebook, C, scores, P, B, S, D, stream);
        return launch_family_lds(ScoreForm::kF16, layout, bits, A, T, keys, codebook, C, scores, P, B, S, D, stream);
    }
    if (variant == kMfmaAuto) variant = pick_variant(layout, bits, C, B, (int64_t)P * S, D);
    if (variant == kMfmaShared)
        return launch_family_shared(ScoreForm::kSplit, layout, bits, A, T, keys, codebook, C, scores, P, B, S, D, stream);
    if (variant == kMfmaSmall)
        return launch_family_small(ScoreForm::kSplit, layout, bits, A, T, keys, codebook, C, scores, P, B, S, D, stream);
    if (variant == kMfmaReg)
        return launch_family_reg(layout, bits, A, T, keys, codebook, C, scores, P, B, S, D, stream);
    return launch_family_lds(ScoreForm::kSplit, layout, bits, A, T, keys, codebook, C, scores, P, B, S, D, stream);
}

bool score_mse_supported(int layout, int bits, int C, int D) { return lds_supported(layout, bits, C, D); }

hipError_t launch_score_mse(const float* A, const uint8_t* idx, const void* norm, int layout, int bits,
                            const float* codebook, int C, float* scores, int P, int B, int S, int D,
                            hipStream_t stream) {
    if (!score_mse_supported(layout, bits, C, D)) return hipErrorInvalidValue;
    const KeyStreams k{idx, nullptr, norm};
    // as for tq_score: one group of four queries over many keys takes the 16x16
    // tiles, four or more query tiles the shared decode
    const int variant = pick_variant(layout, bits, C, B, (int64_t)P * S, D);
    if (variant == kMfmaSmall)
        return launch_family_small(ScoreForm::kMse, layout, bits, A, nullptr, k, codebook, C, scores, P, B, S, D, stream);
    if (variant == kMfmaShared)
        return launch_family_shared(ScoreForm::kMse, layout, bits, A, nullptr, k, codebook, C, scores, P, B, S, D, stream);
    return launch_family_lds(ScoreForm::kMse, layout, bits, A, nullptr, k, codebook, C, scores, P, B, S, D, stream);
}

}  // namespace tq
