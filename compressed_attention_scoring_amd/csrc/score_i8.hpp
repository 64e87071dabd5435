// Four-query scorer on the integer matrix cores (score_i8.hip): packed keys,
// QJL scores, fp32-level accuracy from three int8 limbs per operand.
#pragma once

#include <hip/hip_runtime.h>

#include "tq_common.hpp"

namespace tq {

// Shapes it covers: packed 2- or 3-bit keys with signs, C <= 8, D = 128 or 256.
bool score_i8_supported(int layout, int bits, int C, int D);

// scores[P,B,S] from A, T [P,B,D] and the packed key streams; B <= 4 per
// workgroup row, any B. Returns hipErrorInvalidValue for an unsupported shape.
hipError_t launch_score_i8(const float* A, const float* T, KeyStreams k, const float* codebook, int C,
                           float* scores, int P, int B, int S, int D, int bits, hipStream_t stream);

}  // namespace tq
