// C ABI of the scoring library: argument validation and kernel dispatch.
// Every check runs on the host before any launch; see include/tq.h for the
// contract of each entry point.
#include <stdint.h>

#include <mutex>

#include "tq.h"
#include "tq_common.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Products of sizes stay far below 2^62 for any input that fits in memory,
// but reject shapes whose element counts would not fit int64 arithmetic.
bool fits(int64_t a, int64_t b, int64_t c) {
    const int64_t lim = (int64_t)1 << 60;
    if (a > lim / b) return false;
    return a * b <= lim / c;
}

// Format checks that do not depend on the buffers.
int check_format(const tq_keys* keys, int C, int D, bool need_c) {
    if (!keys) return TQ_ERR_ARG;
    if (D <= 0) return TQ_ERR_ARG;
    if (keys->layout != TQ_UNPACKED && keys->layout != TQ_PACKED) return TQ_ERR_ARG;
    if (D > TQ_MAX_D) return TQ_ERR_UNSUPPORTED;
    if (keys->layout == TQ_PACKED) {
        if (keys->bits != 2 && keys->bits != 3) return TQ_ERR_UNSUPPORTED;
        if (D % 8 != 0) return TQ_ERR_UNSUPPORTED;
        if (need_c && C != (1 << keys->bits)) return TQ_ERR_UNSUPPORTED;
    } else if (need_c && (C < 1 || C > 256)) {
        return TQ_ERR_UNSUPPORTED;
    }
    return TQ_OK;
}

// Buffer checks for a non-empty call.
int check_buffers(const tq_keys* keys, int P, int S, int D) {
    if (!keys->idx || !keys->sign || !keys->gamma) return TQ_ERR_ARG;
    if (P > 65535) return TQ_ERR_UNSUPPORTED;
    if (!fits(P, S, D)) return TQ_ERR_UNSUPPORTED;
    if (!aligned16(keys->idx) || !aligned16(keys->sign) || !aligned16(keys->gamma)) return TQ_ERR_ALIGN;
    return TQ_OK;
}

tq::KeyStreams streams(const tq_keys* k) {
    return tq::KeyStreams{static_cast<const uint8_t*>(k->idx), static_cast<const uint8_t*>(k->sign),
                          k->gamma};
}

// The matrix-core kernels address one 32-query tile of scores with 32-bit
// byte offsets below 2^31, so they take S < 2^24 keys per problem.
constexpr int kMfmaMaxKeys = 1 << 24;

int mfma_variant(int kernel) {
    switch (kernel) {
        case TQ_KERNEL_MFMA_LDS: return tq::kMfmaLds;
        case TQ_KERNEL_MFMA_REG: return tq::kMfmaReg;
        case TQ_KERNEL_MFMA16: return tq::kMfmaSmall;
        case TQ_KERNEL_MFMA_SHARED: return tq::kMfmaShared;
        case TQ_KERNEL_MFMA_F16: return tq::kMfmaF16;
        default: return tq::kMfmaAuto;
    }
}

bool is_mfma(int kernel) {
    return kernel == TQ_KERNEL_MFMA || kernel == TQ_KERNEL_MFMA_LDS || kernel == TQ_KERNEL_MFMA_REG ||
           kernel == TQ_KERNEL_MFMA16 || kernel == TQ_KERNEL_MFMA_SHARED || kernel == TQ_KERNEL_MFMA_F16;
}

bool mfma_ok(int layout, int bits, int C, int B, int S, int D, int kernel = TQ_KERNEL_MFMA) {
    return S < kMfmaMaxKeys &&
           tq::score_mfma_supported(layout, layout == TQ_PACKED ? bits : 0, C, B, D, mfma_variant(kernel));
}

// Default choice: the matrix-core family wherever it applies, the vector
// family for everything else (odd D, codebooks over 8 entries).
int pick_kernel(int layout, int bits, int C, int B, int S, int D) {
    return mfma_ok(layout, bits, C, B, S, D) ? TQ_KERNEL_MFMA : TQ_KERNEL_VALU;
}

}  // namespace

namespace {
// Workspace of tq_attend_no_alloc: a file-scope device array, one copy per GPU
// (the code object's own storage, which lives as long as the process). Host
// code never passes `scratch` itself to a kernel -- in host code the name is a
// stand-in, not a device address -- but the address hipGetSymbolAddress
// returns for the current device, looked up once per device.
constexpr size_t kNoAllocScratchBytes = TQ_NO_ALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_ptr[kMaxDevices] = {};

// The current device's scratch address in *out; TQ_ERR_LAUNCH if HIP cannot
// name the device or the symbol.
int current_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TQ_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return TQ_ERR_LAUNCH;
        scratch_ptr[dev] = ptr;
    }
    *out = scratch_ptr[dev];
    return TQ_OK;
}
}  // namespace

extern "C" {

const char* tq_status_string(int status) {
    switch (status) {
        case TQ_OK: return "ok";
        case TQ_ERR_ARG: return "invalid argument (null pointer, negative size, D or H not positive, P % H != 0, unknown layout or kernel)";
        case TQ_ERR_UNSUPPORTED: return "unsupported shape or key format";
        case TQ_ERR_ALIGN: return "a buffer is not 16-byte aligned";
        case TQ_ERR_LAUNCH: return "HIP kernel launch failed";
        default: return "unknown status";
    }
}

int tq_query_transform(const float* q, const float* Pi, const float* S_mat, float* A, float* T,
                       int P, int H, int B, int D, void* stream) {
    if (P < 0 || H <= 0 || B < 0 || D <= 0 || P % H != 0) return TQ_ERR_ARG;
    if (D > TQ_MAX_D) return TQ_ERR_UNSUPPORTED;
    if (P == 0 || B == 0) return TQ_OK;   // empty call: nothing to launch
    if (!q || !Pi || !S_mat || !A || !T) return TQ_ERR_ARG;
    if (D > TQ_MAX_D || P > 65535 || !fits(P, B, D)) return TQ_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(Pi) || !aligned16(S_mat) || !aligned16(A) || !aligned16(T))
        return TQ_ERR_ALIGN;
    const hipError_t e = tq::launch_query_transform(q, Pi, S_mat, A, T, P, H, B, D,
                                                    static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TQ_OK : TQ_ERR_LAUNCH;
}

const char* tq_score_kernel_name(int layout, int bits, int C, int P, int B, int S, int D, int kernel) {
    if (layout != TQ_UNPACKED && layout != TQ_PACKED) return nullptr;
    if (P <= 0 || B <= 0 || S <= 0 || D <= 0 || D > TQ_MAX_D) return nullptr;
    // the sizes tq_score_with_kernel refuses
    if (P > 65535 || B > 262144 || !fits(P, B, S) || !fits(P, B, D) || !fits(P, S, D)) return nullptr;
    if (layout == TQ_PACKED && ((bits != 2 && bits != 3) || D % 8 || C != (1 << bits))) return nullptr;
    if (layout == TQ_UNPACKED && (C < 1 || C > 256)) return nullptr;
    const int b = layout == TQ_PACKED ? bits : 0;
    if (kernel == TQ_KERNEL_AUTO) kernel = pick_kernel(layout, bits, C, B, S, D);
    if (kernel == TQ_KERNEL_VALU)
        return layout == TQ_UNPACKED ? "valu_unpacked" : bits == 2 ? "valu_packed2" : "valu_packed3";
    if (is_mfma(kernel))
        return mfma_ok(layout, bits, C, B, S, D, kernel) ? tq::score_mfma_name(layout, b, C, P, B, S, D, mfma_variant(kernel))
                                                         : nullptr;
    return nullptr;
}

int tq_score_with_kernel(const float* A, const float* T, const tq_keys* keys, const float* codebook,
                         int C, float* scores, int P, int B, int S, int D, int kernel, void* stream) {
    if (P < 0 || B < 0 || S < 0) return TQ_ERR_ARG;
    int kc = check_format(keys, C, D, true);
    if (kc != TQ_OK) return kc;
    if (kernel != TQ_KERNEL_AUTO && kernel != TQ_KERNEL_VALU && !is_mfma(kernel)) return TQ_ERR_ARG;
    if (P == 0 || B == 0 || S == 0) return TQ_OK;   // empty call: nothing to launch
    if (!A || !T || !codebook || !scores) return TQ_ERR_ARG;
    kc = check_buffers(keys, P, S, D);
    if (kc != TQ_OK) return kc;
    if (B > 262144 || !fits(P, B, S) || !fits(P, B, D)) return TQ_ERR_UNSUPPORTED;
    if (!aligned16(A) || !aligned16(T) || !aligned16(codebook) || !aligned16(scores)) return TQ_ERR_ALIGN;
    const int bits = keys->layout == TQ_PACKED ? keys->bits : 0;
    if (kernel == TQ_KERNEL_AUTO) kernel = pick_kernel(keys->layout, bits, C, B, S, D);
    hipError_t e;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (is_mfma(kernel)) {
        if (!mfma_ok(keys->layout, bits, C, B, S, D, kernel)) return TQ_ERR_UNSUPPORTED;
        e = tq::launch_score_mfma(A, T, streams(keys), keys->layout, bits, codebook, C, scores, P, B, S, D,
                                  mfma_variant(kernel), st);
    } else if (kernel == TQ_KERNEL_VALU) {
        e = tq::launch_score_valu(A, T, streams(keys), keys->layout, bits, codebook, C, scores, P, B, S, D, st);
    } else {
        return TQ_ERR_ARG;
    }
    return e == hipSuccess ? TQ_OK : TQ_ERR_LAUNCH;
}

int tq_score(const float* A, const float* T, const tq_keys* keys, const float* codebook, int C,
             float* scores, int P, int B, int S, int D, void* stream) {
    return tq_score_with_kernel(A, T, keys, codebook, C, scores, P, B, S, D, TQ_KERNEL_AUTO, stream);
}

int tq_compress_keys(const float* keys, const float* Pi, const float* S_mat, const float* codebook, int C,
                     const tq_keys_out* out, int P, int H, int S, int D, void* stream) {
    if (!out || P < 0 || S < 0 || H <= 0 || D <= 0) return TQ_ERR_ARG;
    if (out->layout != TQ_UNPACKED && out->layout != TQ_PACKED) return TQ_ERR_ARG;
    if (P % H != 0) return TQ_ERR_ARG;
    const int bits = out->layout == TQ_PACKED ? out->bits : 0;
    if (out->layout == TQ_PACKED && ((bits != 2 && bits != 3) || C != (1 << bits))) return TQ_ERR_UNSUPPORTED;
    if (!tq::compress_supported(out->layout, bits, C, D)) return TQ_ERR_UNSUPPORTED;
    if (P == 0 || S == 0) return TQ_OK;   // empty call: nothing to launch
    if (!keys || !Pi || !S_mat || !codebook || !out->idx || !out->sign || !out->gamma) return TQ_ERR_ARG;
    if (P > 65535 || !fits(P, S, D)) return TQ_ERR_UNSUPPORTED;
    if (!aligned16(keys) || !aligned16(Pi) || !aligned16(S_mat) || !aligned16(codebook) || !aligned16(out->idx) ||
        !aligned16(out->sign) || !aligned16(out->gamma) || (out->norm && !aligned16(out->norm)))
        return TQ_ERR_ALIGN;
    const tq::KeyOut ko{static_cast<uint8_t*>(out->idx), static_cast<uint8_t*>(out->sign), out->gamma, out->norm};
    const hipError_t e = tq::launch_compress(keys, Pi, S_mat, codebook, C, ko, out->layout, bits, P, H, S, D,
                                             static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TQ_OK : TQ_ERR_LAUNCH;
}

size_t tq_attend_workspace_bytes(int P, int B, int S, int D) {
    if (P <= 0 || B <= 0 || S <= 0 || D <= 0 || D > TQ_MAX_D || P > 65535 || B > 262144) return 0;
    if (!fits(P, B, S) || !fits(P, S, D)) return 0;   // sizes tq_attend refuses
    const int64_t n = (int64_t)P * B * tq::attend_chunks(P, B, S, D) * (D + 2) * (int64_t)sizeof(float);
    return (size_t)n;
}

int tq_attend(const float* scores, const tq_values* values, const float* codebook, int C, const float* Pi_v,
              float scale, float* out, void* workspace, size_t workspace_bytes, int P, int H, int B, int S, int D,
              void* stream) {
    if (!values || P < 0 || B < 0 || S < 0 || H <= 0 || D <= 0 || P % H != 0) return TQ_ERR_ARG;
    if (values->layout != TQ_UNPACKED && values->layout != TQ_PACKED) return TQ_ERR_ARG;
    const int bits = values->layout == TQ_PACKED ? values->bits : 0;
    if (values->layout == TQ_PACKED && ((bits != 2 && bits != 3) || C != (1 << bits))) return TQ_ERR_UNSUPPORTED;
    if (!tq::attend_supported(values->layout, bits, C, D)) return TQ_ERR_UNSUPPORTED;
    if (P == 0 || B == 0) return TQ_OK;   // empty call: nothing to launch
    if (S == 0) return TQ_ERR_ARG;        // softmax over no keys
    if (!scores || !codebook || !Pi_v || !out || !workspace || !values->idx || !values->norm) return TQ_ERR_ARG;
    if (P > 65535 || B > 262144 || !fits(P, B, S) || !fits(P, S, D)) return TQ_ERR_UNSUPPORTED;
    if (workspace_bytes < tq_attend_workspace_bytes(P, B, S, D)) return TQ_ERR_ARG;
    if (!aligned16(scores) || !aligned16(codebook) || !aligned16(Pi_v) || !aligned16(out) || !aligned16(workspace) ||
        !aligned16(values->idx) || !aligned16(values->norm))
        return TQ_ERR_ALIGN;
    const tq::ValueStreams v{static_cast<const uint8_t*>(values->idx), values->norm};
    const hipError_t e = tq::launch_attend(scores, v, values->layout, bits, codebook, C, Pi_v, scale, out,
                                           static_cast<float*>(workspace), P, H, B, S, D,
                                           static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TQ_OK : TQ_ERR_LAUNCH;
}

int tq_attend_no_alloc(const float* scores, const tq_values* values, const float* codebook, int C,
                       const float* Pi_v, float scale, float* out, int P, int H, int B, int S, int D,
                       void* stream) {
    // the shape checks of tq_attend come first, so errors match it
    if (!values || P < 0 || B < 0 || S < 0 || H <= 0 || D <= 0 || P % H != 0) return TQ_ERR_ARG;
    if (values->layout != TQ_UNPACKED && values->layout != TQ_PACKED) return TQ_ERR_ARG;
    const int bits = values->layout == TQ_PACKED ? values->bits : 0;
    if (values->layout == TQ_PACKED && ((bits != 2 && bits != 3) || C != (1 << bits))) return TQ_ERR_UNSUPPORTED;
    if (!tq::attend_supported(values->layout, bits, C, D)) return TQ_ERR_UNSUPPORTED;
    if (P == 0 || B == 0) return TQ_OK;
    if (S == 0) return TQ_ERR_ARG;
    if (P > 65535 || B > 262144 || !fits(P, B, S) || !fits(P, S, D)) return TQ_ERR_UNSUPPORTED;
    const size_t need = tq_attend_workspace_bytes(P, B, S, D);
    if (need == 0 || need > kNoAllocScratchBytes) return TQ_ERR_UNSUPPORTED;
    void* ws = nullptr;
    const int rc = current_scratch(&ws);
    if (rc != TQ_OK) return rc;
    // every partial record the combine reads is written first by the partial
    // kernel, so nothing in the scratch has to start at zero
    return tq_attend(scores, values, codebook, C, Pi_v, scale, out, ws, kNoAllocScratchBytes, P, H, B, S, D, stream);
}

namespace {
// tq_score_attend runs fused when every wavefront of the fused kernel gets at
// least two 32-key tiles and the query tile is not mostly padding; otherwise as
// two passes with the scores in the workspace. Measured (us per call, fused /
// two passes): B=32 S=131072 31 / 41, B=128 S=262144 118 / 141, B=32 S=32768
// 22.5 / 20.5, P=128 B=4 404 / 255.
// Callers have checked S < 2^24, which keeps the plan's int arithmetic in range.
bool fused_step(int P, int B, int S, int& chunk, int& nch) {
    tq::score_attend_plan(P, B, S, chunk, nch);
    return B > 8 && chunk >= 8 * 32;
}

int64_t align256(int64_t n) { return (n + 255) / 256 * 256; }
}  // namespace

size_t tq_score_attend_workspace_bytes(int P, int B, int S, int D, int mode) {
    if (P <= 0 || B <= 0 || S <= 0 || D <= 0 || D > TQ_MAX_D || P > 65535 || B > 262144) return 0;
    // sizes tq_score_attend_with_mode refuses
    if (S >= kMfmaMaxKeys || !fits(P, B, S) || !fits(P, B, D) || !fits(P, S, D)) return 0;
    if (mode != TQ_ATTEND_AUTO && mode != TQ_ATTEND_FUSED && mode != TQ_ATTEND_TWO_PASS) return 0;
    int chunk = 0, nch = 0;
    const bool fused = fused_step(P, B, S, chunk, nch);
    if (mode == TQ_ATTEND_FUSED || (mode == TQ_ATTEND_AUTO && fused))
        return (size_t)((int64_t)P * B * nch * (D + 2) * (int64_t)sizeof(float));
    return (size_t)(align256((int64_t)P * B * S * (int64_t)sizeof(float)) +
                    (int64_t)tq_attend_workspace_bytes(P, B, S, D));
}

int tq_score_attend_with_mode(const float* A, const float* T, const tq_keys* keys, const float* codebook, int C,
                              const tq_values* values, const float* codebook_v, int C_v, const float* Pi_v,
                              float scale, float* out, void* workspace, size_t workspace_bytes, int P, int H, int B,
                              int S, int D, int mode, void* stream) {
    if (!values || P < 0 || B < 0 || S < 0 || H <= 0 || P % H != 0) return TQ_ERR_ARG;
    if (mode != TQ_ATTEND_AUTO && mode != TQ_ATTEND_FUSED && mode != TQ_ATTEND_TWO_PASS) return TQ_ERR_ARG;
    int kc = check_format(keys, C, D, true);
    if (kc != TQ_OK) return kc;
    if (values->layout != TQ_UNPACKED && values->layout != TQ_PACKED) return TQ_ERR_ARG;
    const int bits = keys->layout == TQ_PACKED ? keys->bits : 0;
    const int vbits = values->layout == TQ_PACKED ? values->bits : 0;
    if (values->layout == TQ_PACKED && ((vbits != 2 && vbits != 3) || C_v != (1 << vbits))) return TQ_ERR_UNSUPPORTED;
    if (!tq::score_attend_supported(keys->layout, bits, C, values->layout, vbits, C_v, D)) return TQ_ERR_UNSUPPORTED;
    if (P == 0 || B == 0) return TQ_OK;   // empty call: nothing to launch
    if (S == 0) return TQ_ERR_ARG;        // softmax over no keys
    if (!A || !T || !codebook || !codebook_v || !Pi_v || !out || !workspace || !values->idx || !values->norm)
        return TQ_ERR_ARG;
    kc = check_buffers(keys, P, S, D);
    if (kc != TQ_OK) return kc;
    if (S >= kMfmaMaxKeys || B > 262144 || !fits(P, B, S) || !fits(P, B, D)) return TQ_ERR_UNSUPPORTED;
    if (workspace_bytes < tq_score_attend_workspace_bytes(P, B, S, D, mode)) return TQ_ERR_ARG;
    if (!aligned16(A) || !aligned16(T) || !aligned16(codebook) || !aligned16(codebook_v) || !aligned16(Pi_v) ||
        !aligned16(out) || !aligned16(workspace) || !aligned16(values->idx) || !aligned16(values->norm))
        return TQ_ERR_ALIGN;
    int chunk = 0, nch = 0;
    const bool auto_fused = fused_step(P, B, S, chunk, nch);
    const bool fused = mode == TQ_ATTEND_FUSED || (mode == TQ_ATTEND_AUTO && auto_fused);
    hipStream_t st = static_cast<hipStream_t>(stream);
    float* ws = static_cast<float*>(workspace);
    const tq::ValueStreams v{static_cast<const uint8_t*>(values->idx), values->norm};
    hipError_t e;
    if (fused) {
        e = tq::launch_score_attend_partial(A, T, streams(keys), keys->layout, bits, codebook, C, v, values->layout,
                                            vbits, codebook_v, C_v, scale, ws, P, B, S, chunk, nch, st);
        if (e == hipSuccess) e = tq::launch_attend_combine(ws, Pi_v, out, P, H, B, D, nch, st);
    } else {
        float* scores = ws;
        float* aws = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(workspace) +
                                              align256((int64_t)P * B * S * (int64_t)sizeof(float)));
        e = tq::launch_score_mfma(A, T, streams(keys), keys->layout, bits, codebook, C, scores, P, B, S, D,
                                  tq::kMfmaAuto, st);
        if (e == hipSuccess)
            e = tq::launch_attend(scores, v, values->layout, vbits, codebook_v, C_v, Pi_v, scale, out, aws, P, H, B,
                                  S, D, st);
    }
    return e == hipSuccess ? TQ_OK : TQ_ERR_LAUNCH;
}

int tq_score_attend(const float* A, const float* T, const tq_keys* keys, const float* codebook, int C,
                    const tq_values* values, const float* codebook_v, int C_v, const float* Pi_v, float scale,
                    float* out, void* workspace, size_t workspace_bytes, int P, int H, int B, int S, int D,
                    void* stream) {
    return tq_score_attend_with_mode(A, T, keys, codebook, C, values, codebook_v, C_v, Pi_v, scale, out, workspace,
                                     workspace_bytes, P, H, B, S, D, TQ_ATTEND_AUTO, stream);
}

int tq_query_transform_hadamard(const float* q, const float* signs, float* A, int P, int H, int B, int D,
                                void* stream) {
    if (P < 0 || H <= 0 || B < 0 || D <= 0 || P % H != 0) return TQ_ERR_ARG;
    if (!tq::hadamard_supported(D)) return TQ_ERR_UNSUPPORTED;
    if (P == 0 || B == 0) return TQ_OK;   // empty call: nothing to launch
    if (!q || !signs || !A) return TQ_ERR_ARG;
    if (!fits(P, B, D) || (int64_t)P * B > (int64_t)1 << 30) return TQ_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(signs) || !aligned16(A)) return TQ_ERR_ALIGN;
    const hipError_t e = tq::launch_query_transform_hadamard(q, signs, A, P, H, B, D, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TQ_OK : TQ_ERR_LAUNCH;
}

int tq_score_mse(const float* A, const tq_mse_codes* keys, const float* codebook, int C, float* scores, int P,
                 int B, int S, int D, void* stream) {
    if (!keys || P < 0 || B < 0 || S < 0 || D <= 0) return TQ_ERR_ARG;
    if (keys->layout != TQ_UNPACKED && keys->layout != TQ_PACKED) return TQ_ERR_ARG;
    const int bits = keys->layout == TQ_PACKED ? keys->bits : 0;
    if (keys->layout == TQ_PACKED && ((bits != 2 && bits != 3) || C != (1 << bits))) return TQ_ERR_UNSUPPORTED;
    if (!tq::score_mse_supported(keys->layout, bits, C, D)) return TQ_ERR_UNSUPPORTED;
    if (P == 0 || B == 0 || S == 0) return TQ_OK;   // empty call: nothing to launch
    if (!A || !codebook || !scores || !keys->idx || !keys->norm) return TQ_ERR_ARG;
    if (S >= kMfmaMaxKeys || P > 65535 || B > 262144 || !fits(P, B, S) || !fits(P, S, D)) return TQ_ERR_UNSUPPORTED;
    if (!aligned16(A) || !aligned16(codebook) || !aligned16(scores) || !aligned16(keys->idx) || !aligned16(keys->norm))
        return TQ_ERR_ALIGN;
    const hipError_t e = tq::launch_score_mse(A, static_cast<const uint8_t*>(keys->idx), keys->norm, keys->layout,
                                              bits, codebook, C, scores, P, B, S, D, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TQ_OK : TQ_ERR_LAUNCH;
}

int tq_query_transform_split(const float* q, const int32_t* perm, const float* Pi_hi, const float* Pi_lo, float* A_hi,
                             float* A_lo, int P, int H, int B, int D, int D_hi, void* stream) {
    if (P < 0 || H <= 0 || B < 0 || D <= 0 || P % H != 0 || D_hi <= 0 || D_hi >= D) return TQ_ERR_ARG;
    if (D > TQ_MAX_D) return TQ_ERR_UNSUPPORTED;
    if (P == 0 || B == 0) return TQ_OK;   // empty call: nothing to launch
    if (!q || !perm || !Pi_hi || !Pi_lo || !A_hi || !A_lo) return TQ_ERR_ARG;
    if (P > 65535 || !fits(P, B, D)) return TQ_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(perm) || !aligned16(Pi_hi) || !aligned16(Pi_lo) || !aligned16(A_hi) ||
        !aligned16(A_lo))
        return TQ_ERR_ALIGN;
    const hipError_t e = tq::launch_query_transform_split(q, perm, Pi_hi, Pi_lo, A_hi, A_lo, P, H, B, D, D_hi,
                                                          static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TQ_OK : TQ_ERR_LAUNCH;
}

namespace {
// Format of one MSE instance for the split scorer: 0 unpacked, else the packed width.
int split_bits(const tq_mse_codes& c, int C, int D, int* bits) {
    if (c.layout != TQ_UNPACKED && c.layout != TQ_PACKED) return TQ_ERR_ARG;
    if (D < 8 || D > TQ_MAX_D || D % 8 != 0) return TQ_ERR_UNSUPPORTED;
    if (c.layout == TQ_UNPACKED) {
        if (C < 1 || C > 256) return TQ_ERR_UNSUPPORTED;
        *bits = 0;
    } else {
        if ((c.bits != 2 && c.bits != 3) || C != (1 << c.bits)) return TQ_ERR_UNSUPPORTED;
        *bits = c.bits;
    }
    return TQ_OK;
}
}  // namespace

int tq_score_split(const float* A_hi, const float* A_lo, const tq_split_codes* keys, const float* codebook_hi, int C_hi,
                   const float* codebook_lo, int C_lo, float* scores, int P, int B, int S, int D_hi, int D_lo,
                   void* stream) {
    if (!keys || P < 0 || B < 0 || S < 0 || D_hi <= 0 || D_lo <= 0) return TQ_ERR_ARG;
    int bh = 0, bl = 0;
    int kc = split_bits(keys->hi, C_hi, D_hi, &bh);
    if (kc != TQ_OK) return kc;
    kc = split_bits(keys->lo, C_lo, D_lo, &bl);
    if (kc != TQ_OK) return kc;
    if (P == 0 || B == 0 || S == 0) return TQ_OK;   // empty call: nothing to launch
    if (!A_hi || !A_lo || !codebook_hi || !codebook_lo || !scores || !keys->hi.idx || !keys->hi.norm ||
        !keys->lo.idx || !keys->lo.norm)
        return TQ_ERR_ARG;
    if (P > 65535 || B > 262144 || !fits(P, B, S) || !fits(P, S, D_hi + D_lo)) return TQ_ERR_UNSUPPORTED;
    if (!aligned16(A_hi) || !aligned16(A_lo) || !aligned16(codebook_hi) || !aligned16(codebook_lo) ||
        !aligned16(scores) || !aligned16(keys->hi.idx) || !aligned16(keys->hi.norm) || !aligned16(keys->lo.idx) ||
        !aligned16(keys->lo.norm))
        return TQ_ERR_ALIGN;
    const tq::SplitStreams k{static_cast<const uint8_t*>(keys->hi.idx), keys->hi.norm,
                             static_cast<const uint8_t*>(keys->lo.idx), keys->lo.norm};
    const hipError_t e = tq::launch_score_split(A_hi, A_lo, k, bh, bl, codebook_hi, C_hi, codebook_lo, C_lo, scores,
                                                P, B, S, D_hi, D_lo, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TQ_OK : TQ_ERR_LAUNCH;
}

int tq_decode_debug(const tq_keys* keys, uint8_t* idx_out, int8_t* sign_out, float* gamma_out,
                    int P, int S, int D, void* stream) {
    if (P < 0 || S < 0) return TQ_ERR_ARG;
    int kc = check_format(keys, 0, D, false);
    if (kc != TQ_OK) return kc;
    if (P == 0 || S == 0) return TQ_OK;   // empty call: nothing to launch
    if (!idx_out || !sign_out || !gamma_out) return TQ_ERR_ARG;
    kc = check_buffers(keys, P, S, D);
    if (kc != TQ_OK) return kc;
    if (!aligned16(idx_out) || !aligned16(sign_out) || !aligned16(gamma_out)) return TQ_ERR_ALIGN;
    const hipError_t e = tq::launch_decode(streams(keys), keys->layout, keys->bits, idx_out, sign_out,
                                           gamma_out, P, S, D, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TQ_OK : TQ_ERR_LAUNCH;
}

// ---- measurement probes
namespace {
constexpr size_t kProbeMaxBytes = (size_t)1 << 36;
int probe_buffer_ok(const void* p, size_t bytes) {
    if (bytes % 16 != 0 || bytes > kProbeMaxBytes) return TQ_ERR_ARG;
    if (bytes > 0 && !p) return TQ_ERR_ARG;
    if (bytes > 0 && !aligned16(p)) return TQ_ERR_ALIGN;
    return TQ_OK;
}
}  // namespace

int tq_probe_read(const void* src, size_t bytes, void* sink, void* stream) {
    int rc = probe_buffer_ok(src, bytes);
    if (rc != TQ_OK) return rc;
    if (bytes == 0) return TQ_OK;
    if (!sink) return TQ_ERR_ARG;
    if ((reinterpret_cast<uintptr_t>(sink) & 3u) != 0) return TQ_ERR_ALIGN;
    const hipError_t e = tq::launch_probe_read(src, (int64_t)bytes, static_cast<uint32_t*>(sink),
                                               static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TQ_OK : TQ_ERR_LAUNCH;
}

int tq_probe_write(void* dst, size_t bytes, void* stream) {
    int rc = probe_buffer_ok(dst, bytes);
    if (rc != TQ_OK) return rc;
    if (bytes == 0) return TQ_OK;
    const hipError_t e = tq::launch_probe_write(dst, (int64_t)bytes, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TQ_OK : TQ_ERR_LAUNCH;
}

int tq_probe_read_write(const void* src, size_t read_bytes, void* dst, size_t write_bytes, void* stream) {
    int rc = probe_buffer_ok(src, read_bytes);
    if (rc != TQ_OK) return rc;
    rc = probe_buffer_ok(dst, write_bytes);
    if (rc != TQ_OK) return rc;
    if (read_bytes == 0 || write_bytes == 0) return TQ_ERR_ARG;
    const hipError_t e = tq::launch_probe_read_write(src, (int64_t)read_bytes, dst, (int64_t)write_bytes,
                                                     static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TQ_OK : TQ_ERR_LAUNCH;
}

int tq_probe_tile(const tq_keys* keys, float* out, int B, int S, int D, void* stream) {
    if (!keys || B < 0 || S < 0 || D <= 0) return TQ_ERR_ARG;
    if (keys->layout != TQ_UNPACKED) return TQ_ERR_UNSUPPORTED;
    if (B == 0 || S == 0) return TQ_OK;
    if (!keys->idx || !keys->sign || !keys->gamma || !out) return TQ_ERR_ARG;
    if (!tq::probe_tile_supported(B, S, D)) return TQ_ERR_UNSUPPORTED;
    if (!aligned16(keys->idx) || !aligned16(keys->sign) || !aligned16(keys->gamma) || !aligned16(out))
        return TQ_ERR_ALIGN;
    const hipError_t e = tq::launch_probe_tile(static_cast<const uint8_t*>(keys->idx),
                                               static_cast<const uint8_t*>(keys->sign),
                                               static_cast<const float*>(keys->gamma), out, B, S, D,
                                               static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TQ_OK : TQ_ERR_LAUNCH;
}

}  // extern "C"
