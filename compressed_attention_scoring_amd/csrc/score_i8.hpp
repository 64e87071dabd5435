// Four-query scorer on the integer matrix cores (score_i8.hip): packed keys,
// QJL or MSE-only scores, fp32-level accuracy from int8 limbs of each operand.
#pragma once

#include <hip/hip_runtime.h>

#include "tq_common.hpp"

namespace tq {

// Shapes it covers: packed 2- or 3-bit keys, C <= 8, D = 128 or 256.
bool score_i8_supported(int layout, int bits, int C, int D);

// scores[P,B,S] from A, T [P,B,D] and the packed key streams (four queries per
// workgroup row, any B). qjl = false: MSE-only keys (T and the sign stream are
// not read; gamma holds the key norms). Returns hipErrorInvalidValue for an
// unsupported shape.
hipError_t launch_score_i8(const float* A, const float* T, KeyStreams k, const float* codebook, int C,
                           float* scores, int P, int B, int S, int D, int bits, bool qjl, hipStream_t stream);

}  // namespace tq
