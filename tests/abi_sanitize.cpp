// Host-only driver for the C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer (built and run by tests/test_abi_sanitize.py).
//
// Every call below is one the library must answer on the host: a bad
// argument, an unsupported shape, a misaligned pointer, an empty call, or a
// pure query (workspace sizes, kernel names, status strings), including sizes
// at the int32 and int64 extremes. No call reaches a kernel launch, so no GPU
// is needed and the device pointers are never dereferenced: they are fake
// addresses, 16-byte aligned or deliberately not.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "tq.h"

namespace {

int failures = 0, checks = 0;

void expect(int got, int want, const char* what, int line) {
    ++checks;
    if (got != want) {
        std::printf("FAIL line %d: %s returned %d, expected %d\n", line, what, got, want);
        ++failures;
    }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

float* const F = reinterpret_cast<float*>(uintptr_t(1) << 12);          // aligned fake device address
float* const M = reinterpret_cast<float*>((uintptr_t(1) << 12) + 4);    // misaligned
void* const V = F;
void* const VM = M;
const int32_t* const PERM = reinterpret_cast<const int32_t*>(F);

tq_keys keys(int layout, int bits, const void* p = V) { return tq_keys{layout, bits, p, p, p}; }
tq_mse_codes codes(int layout, int bits, const void* p = V) { return tq_mse_codes{layout, bits, p, p}; }

void transforms() {
    EXPECT(tq_query_transform(F, F, F, F, F, -1, 1, 1, 64, nullptr), TQ_ERR_ARG);
    EXPECT(tq_query_transform(F, F, F, F, F, 1, 0, 1, 64, nullptr), TQ_ERR_ARG);
    EXPECT(tq_query_transform(F, F, F, F, F, 1, 1, -1, 64, nullptr), TQ_ERR_ARG);
    EXPECT(tq_query_transform(F, F, F, F, F, 1, 1, 1, 0, nullptr), TQ_ERR_ARG);
    EXPECT(tq_query_transform(F, F, F, F, F, 3, 2, 1, 64, nullptr), TQ_ERR_ARG);
    EXPECT(tq_query_transform(F, F, F, F, F, 1, 1, 1, TQ_MAX_D + 1, nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_query_transform(F, F, F, F, F, 0, 1, 1, 64, nullptr), TQ_OK);
    EXPECT(tq_query_transform(F, F, F, F, F, 1, 1, 0, 64, nullptr), TQ_OK);
    EXPECT(tq_query_transform(nullptr, F, F, F, F, 1, 1, 1, 64, nullptr), TQ_ERR_ARG);
    EXPECT(tq_query_transform(F, F, F, F, F, 65536, 1, 1, 64, nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_query_transform(F, F, F, F, F, INT_MAX, 1, INT_MAX, TQ_MAX_D, nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_query_transform(M, F, F, F, F, 65535, 1, INT_MAX, TQ_MAX_D, nullptr), TQ_ERR_ALIGN);
    EXPECT(tq_query_transform(F, F, F, F, M, 1, 1, 1, 64, nullptr), TQ_ERR_ALIGN);

    EXPECT(tq_query_transform_hadamard(F, F, F, 1, 1, 1, 96, nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_query_transform_hadamard(F, F, F, 2, 3, 1, 64, nullptr), TQ_ERR_ARG);
    EXPECT(tq_query_transform_hadamard(F, F, F, 0, 1, 1, 64, nullptr), TQ_OK);
    EXPECT(tq_query_transform_hadamard(nullptr, F, F, 1, 1, 1, 64, nullptr), TQ_ERR_ARG);
    EXPECT(tq_query_transform_hadamard(F, F, F, INT_MAX, 1, INT_MAX, 1024, nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_query_transform_hadamard(F, M, F, 1, 1, 1, 64, nullptr), TQ_ERR_ALIGN);

    EXPECT(tq_query_transform_split(F, PERM, F, F, F, F, 1, 1, 1, 128, 0, nullptr), TQ_ERR_ARG);
    EXPECT(tq_query_transform_split(F, PERM, F, F, F, F, 1, 1, 1, 128, 128, nullptr), TQ_ERR_ARG);
    EXPECT(tq_query_transform_split(F, PERM, F, F, F, F, 1, 1, 1, TQ_MAX_D + 8, 8, nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_query_transform_split(F, PERM, F, F, F, F, 1, 1, 0, 128, 32, nullptr), TQ_OK);
    EXPECT(tq_query_transform_split(F, nullptr, F, F, F, F, 1, 1, 1, 128, 32, nullptr), TQ_ERR_ARG);
    EXPECT(tq_query_transform_split(F, PERM, F, F, F, F, INT_MAX, 1, INT_MAX, 128, 32, nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_query_transform_split(F, PERM, F, F, M, F, 1, 1, 1, 128, 32, nullptr), TQ_ERR_ALIGN);
}

void scoring() {
    tq_keys u = keys(TQ_UNPACKED, 0), p3 = keys(TQ_PACKED, 3);
    EXPECT(tq_score(F, F, nullptr, F, 4, F, 1, 1, 1, 64, nullptr), TQ_ERR_ARG);
    EXPECT(tq_score(F, F, &u, F, 4, F, -1, 1, 1, 64, nullptr), TQ_ERR_ARG);
    EXPECT(tq_score(F, F, &u, F, 4, F, 1, 1, 1, 0, nullptr), TQ_ERR_ARG);
    tq_keys bad = keys(7, 0);
    EXPECT(tq_score(F, F, &bad, F, 4, F, 1, 1, 1, 64, nullptr), TQ_ERR_ARG);
    tq_keys p4 = keys(TQ_PACKED, 4);
    EXPECT(tq_score(F, F, &p4, F, 16, F, 1, 1, 1, 64, nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_score(F, F, &p3, F, 8, F, 1, 1, 1, 12, nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_score(F, F, &p3, F, 4, F, 1, 1, 1, 64, nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_score(F, F, &u, F, 0, F, 1, 1, 1, 64, nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_score(F, F, &u, F, 257, F, 1, 1, 1, 64, nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_score(F, F, &u, F, 4, F, 1, 1, 0, 64, nullptr), TQ_OK);
    EXPECT(tq_score(nullptr, F, &u, F, 4, F, 1, 1, 1, 64, nullptr), TQ_ERR_ARG);
    tq_keys nullidx{TQ_UNPACKED, 0, nullptr, V, V};
    EXPECT(tq_score(F, F, &nullidx, F, 4, F, 1, 1, 1, 64, nullptr), TQ_ERR_ARG);
    EXPECT(tq_score(F, F, &u, F, 4, F, 65536, 1, 1, 64, nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_score(F, F, &u, F, 4, F, 1, 262145, 1, 64, nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_score(F, F, &u, F, 4, F, 65535, 262144, INT_MAX, TQ_MAX_D, nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_score(M, F, &u, F, 4, F, 1, 1, 1, 64, nullptr), TQ_ERR_ALIGN);
    tq_keys um = keys(TQ_UNPACKED, 0, VM);
    EXPECT(tq_score(F, F, &um, F, 4, F, 1, 1, 1, 64, nullptr), TQ_ERR_ALIGN);
    EXPECT(tq_score_with_kernel(F, F, &u, F, 4, F, 1, 1, 1, 64, 99, nullptr), TQ_ERR_ARG);
    EXPECT(tq_score_with_kernel(F, F, &u, F, 4, F, 1, 1, 1 << 24, 128, TQ_KERNEL_MFMA, nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_score_with_kernel(F, F, &p3, F, 8, F, 1, 1, 100, 48, TQ_KERNEL_MFMA, nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_score_with_kernel(F, F, &u, F, 16, F, 1, 1, 100, 128, TQ_KERNEL_MFMA_LDS, nullptr), TQ_ERR_UNSUPPORTED);

    // names are pure queries: any input, including the int32 extremes, gives a name or NULL
    const int ext[] = {INT_MIN, -1, 0, 1, 31, 32, 33, 65535, 65536, 262144, 262145, (1 << 24) - 1, 1 << 24, INT_MAX};
    const int kernels[] = {TQ_KERNEL_AUTO, TQ_KERNEL_VALU, TQ_KERNEL_MFMA, TQ_KERNEL_MFMA_LDS, TQ_KERNEL_MFMA_REG,
                           TQ_KERNEL_MFMA16, TQ_KERNEL_MFMA_SHARED, TQ_KERNEL_MFMA_F16, 99};
    for (int P : ext)
        for (int B : ext)
            for (int S : ext)
                for (int k : kernels) {
                    const char* n = tq_score_kernel_name(TQ_PACKED, 3, 8, P, B, S, 128, k);
                    if (n) checks += std::strlen(n) > 0;
                    n = tq_score_kernel_name(TQ_UNPACKED, 0, 4, P, B, S, 64, k);
                    if (n) checks += std::strlen(n) > 0;
                }

    tq_mse_codes mu = codes(TQ_UNPACKED, 0), m3 = codes(TQ_PACKED, 3);
    EXPECT(tq_score_mse(F, nullptr, F, 4, F, 1, 1, 1, 128, nullptr), TQ_ERR_ARG);
    EXPECT(tq_score_mse(F, &m3, F, 4, F, 1, 1, 1, 128, nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_score_mse(F, &mu, F, 4, F, 1, 0, 1, 128, nullptr), TQ_OK);
    EXPECT(tq_score_mse(nullptr, &mu, F, 4, F, 1, 1, 1, 128, nullptr), TQ_ERR_ARG);
    EXPECT(tq_score_mse(F, &mu, F, 4, F, 1, 1, 1 << 24, 128, nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_score_mse(F, &mu, F, 4, F, 65535, 262145, (1 << 24) - 1, 128, nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_score_mse(M, &mu, F, 4, F, 65535, 262144, (1 << 24) - 1, 128, nullptr), TQ_ERR_ALIGN);
    EXPECT(tq_score_mse(F, &mu, M, 4, F, 1, 1, 1, 128, nullptr), TQ_ERR_ALIGN);

    tq_split_codes sc{codes(TQ_PACKED, 3), codes(TQ_PACKED, 2)};
    EXPECT(tq_score_split(F, F, nullptr, F, 8, F, 4, F, 1, 1, 1, 32, 96, nullptr), TQ_ERR_ARG);
    EXPECT(tq_score_split(F, F, &sc, F, 8, F, 4, F, 1, 1, 1, 0, 96, nullptr), TQ_ERR_ARG);
    EXPECT(tq_score_split(F, F, &sc, F, 4, F, 4, F, 1, 1, 1, 32, 96, nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_score_split(F, F, &sc, F, 8, F, 4, F, 1, 1, 0, 32, 96, nullptr), TQ_OK);
    EXPECT(tq_score_split(F, F, &sc, F, 8, F, 4, F, 65536, 1, 1, 32, 96, nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_score_split(F, F, &sc, F, 8, F, 4, F, 1, 262145, INT_MAX, 32, 96, nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_score_split(M, F, &sc, F, 8, F, 4, F, 65535, 262144, 4096, 32, 96, nullptr), TQ_ERR_ALIGN);
    EXPECT(tq_score_split(F, M, &sc, F, 8, F, 4, F, 1, 1, 1, 32, 96, nullptr), TQ_ERR_ALIGN);
}

void compress_and_decode() {
    tq_keys_out o3{TQ_PACKED, 3, V, V, V}, o4{TQ_PACKED, 4, V, V, V}, ou{TQ_UNPACKED, 0, V, V, V};
    tq_keys_out om{TQ_PACKED, 3, V, VM, V};
    EXPECT(tq_compress_keys(F, F, F, F, 8, nullptr, 1, 1, 1, 128, nullptr), TQ_ERR_ARG);
    EXPECT(tq_compress_keys(F, F, F, F, 8, &o3, 1, 0, 1, 128, nullptr), TQ_ERR_ARG);
    EXPECT(tq_compress_keys(F, F, F, F, 8, &o3, 3, 2, 1, 128, nullptr), TQ_ERR_ARG);
    EXPECT(tq_compress_keys(F, F, F, F, 16, &o4, 1, 1, 1, 128, nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_compress_keys(F, F, F, F, 4, &o3, 1, 1, 1, 128, nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_compress_keys(F, F, F, F, 4, &ou, 1, 1, 1, 96, nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_compress_keys(F, F, F, F, 8, &o3, 1, 1, 0, 128, nullptr), TQ_OK);
    EXPECT(tq_compress_keys(nullptr, F, F, F, 8, &o3, 1, 1, 1, 128, nullptr), TQ_ERR_ARG);
    EXPECT(tq_compress_keys(F, F, F, F, 8, &o3, 65536, 1, 1, 128, nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_compress_keys(F, F, F, F, 8, &om, 65535, 1, INT_MAX, 128, nullptr), TQ_ERR_ALIGN);
    EXPECT(tq_compress_keys(F, F, F, F, 8, &om, 1, 1, 1, 128, nullptr), TQ_ERR_ALIGN);

    tq_keys u = keys(TQ_UNPACKED, 0);
    uint8_t* I = reinterpret_cast<uint8_t*>(F);
    int8_t* Sg = reinterpret_cast<int8_t*>(F);
    EXPECT(tq_decode_debug(nullptr, I, Sg, F, 1, 1, 64, nullptr), TQ_ERR_ARG);
    EXPECT(tq_decode_debug(&u, I, Sg, F, -1, 1, 64, nullptr), TQ_ERR_ARG);
    EXPECT(tq_decode_debug(&u, I, Sg, F, 1, 0, 64, nullptr), TQ_OK);
    EXPECT(tq_decode_debug(&u, nullptr, Sg, F, 1, 1, 64, nullptr), TQ_ERR_ARG);
    EXPECT(tq_decode_debug(&u, I, Sg, F, 65536, 1, 64, nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_decode_debug(&u, I, Sg, M, 1, 1, 64, nullptr), TQ_ERR_ALIGN);
}

void attention() {
    tq_values vu = codes(TQ_UNPACKED, 0), v2 = codes(TQ_PACKED, 2);
    tq_keys p3 = keys(TQ_PACKED, 3);
    // workspace sizes are pure queries: 0 for shapes the entry points refuse,
    // never an overflowed product
    const int ext[] = {INT_MIN, -1, 0, 1, 8, 9, 31, 33, 255, 65535, 65536, 262144, 262145, (1 << 24) - 1, INT_MAX};
    const int ds[] = {-1, 0, 1, 64, 128, TQ_MAX_D, TQ_MAX_D + 1, INT_MAX};
    for (int P : ext)
        for (int B : ext)
            for (int S : ext)
                for (int D : ds) {
                    const size_t a = tq_attend_workspace_bytes(P, B, S, D);
                    checks += a <= ((size_t)1 << 62);
                    for (int mode = -1; mode <= 3; ++mode) {
                        const size_t w = tq_score_attend_workspace_bytes(P, B, S, D, mode);
                        checks += w <= ((size_t)1 << 62);
                    }
                }

    EXPECT(tq_attend(F, nullptr, F, 4, F, 1.f, F, V, 1 << 20, 1, 1, 1, 1, 128, nullptr), TQ_ERR_ARG);
    EXPECT(tq_attend(F, &vu, F, 4, F, 1.f, F, V, 1 << 20, 1, 0, 1, 1, 128, nullptr), TQ_ERR_ARG);
    EXPECT(tq_attend(F, &v2, F, 8, F, 1.f, F, V, 1 << 20, 1, 1, 1, 1, 128, nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_attend(F, &vu, F, 4, F, 1.f, F, V, 1 << 20, 1, 1, 1, 1, 96, nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_attend(F, &vu, F, 4, F, 1.f, F, V, 0, 0, 1, 1, 1, 128, nullptr), TQ_OK);
    EXPECT(tq_attend(F, &vu, F, 4, F, 1.f, F, V, 1 << 20, 1, 1, 1, 0, 128, nullptr), TQ_ERR_ARG);
    EXPECT(tq_attend(F, &vu, F, 4, F, 1.f, F, nullptr, 1 << 20, 1, 1, 1, 1, 128, nullptr), TQ_ERR_ARG);
    EXPECT(tq_attend(F, &vu, F, 4, F, 1.f, F, V, 16, 1, 1, 32, 32768, 128, nullptr), TQ_ERR_ARG);
    EXPECT(tq_attend(F, &vu, F, 4, F, 1.f, F, V, SIZE_MAX, 65535, 1, 262144, INT_MAX, 128, nullptr),
           TQ_ERR_UNSUPPORTED);
    EXPECT(tq_attend(F, &vu, F, 4, F, 1.f, M, V, SIZE_MAX, 1, 1, 1, 1, 128, nullptr), TQ_ERR_ALIGN);
    // the allocation-free form: the same argument checks, then the scratch bound,
    // all before any device call
    EXPECT(tq_attend_no_alloc(F, nullptr, F, 4, F, 1.f, F, 1, 1, 1, 1, 128, nullptr), TQ_ERR_ARG);
    EXPECT(tq_attend_no_alloc(F, &vu, F, 4, F, 1.f, F, 1, 0, 1, 1, 128, nullptr), TQ_ERR_ARG);
    EXPECT(tq_attend_no_alloc(F, &v2, F, 8, F, 1.f, F, 1, 1, 1, 1, 128, nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_attend_no_alloc(F, &vu, F, 4, F, 1.f, F, 0, 1, 1, 1, 128, nullptr), TQ_OK);
    EXPECT(tq_attend_no_alloc(F, &vu, F, 4, F, 1.f, F, 1, 1, 1, 0, 128, nullptr), TQ_ERR_ARG);
    EXPECT(tq_attend_no_alloc(F, &vu, F, 4, F, 1.f, F, 1, 1, 262144, 1000, 128, nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_attend_no_alloc(F, &vu, F, 4, F, 1.f, F, 65535, 1, 262144, INT_MAX, 128, nullptr), TQ_ERR_UNSUPPORTED);

    EXPECT(tq_score_attend_with_mode(F, F, &p3, F, 8, &v2, F, 4, F, 1.f, F, V, SIZE_MAX, 1, 1, 32, 100, 128, 5,
                                     nullptr), TQ_ERR_ARG);
    EXPECT(tq_score_attend_with_mode(F, F, &p3, F, 8, &v2, F, 4, F, 1.f, F, V, SIZE_MAX, 1, 1, 32, 100, 64, 0,
                                     nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_score_attend_with_mode(F, F, &p3, F, 8, &v2, F, 4, F, 1.f, F, V, SIZE_MAX, 1, 1, 0, 100, 128, 0,
                                     nullptr), TQ_OK);
    EXPECT(tq_score_attend_with_mode(F, F, &p3, F, 8, &v2, F, 4, F, 1.f, F, V, SIZE_MAX, 1, 1, 32, 0, 128, 0,
                                     nullptr), TQ_ERR_ARG);
    EXPECT(tq_score_attend_with_mode(F, F, &p3, F, 8, &v2, F, 4, F, 1.f, F, V, SIZE_MAX, 1, 1, 32, 1 << 24, 128, 0,
                                     nullptr), TQ_ERR_UNSUPPORTED);
    EXPECT(tq_score_attend_with_mode(F, F, &p3, F, 8, &v2, F, 4, F, 1.f, F, V, 16, 1, 1, 32, 32768, 128, 1,
                                     nullptr), TQ_ERR_ARG);
    EXPECT(tq_score_attend(F, F, &p3, F, 8, &v2, F, 4, F, 1.f, M, V, SIZE_MAX, 1, 1, 32, 100, 128, nullptr),
           TQ_ERR_ALIGN);
}

void status_strings() {
    const int codes_[] = {INT_MIN, -5, TQ_ERR_LAUNCH, TQ_ERR_ALIGN, TQ_ERR_UNSUPPORTED, TQ_ERR_ARG, TQ_OK, 1, INT_MAX};
    for (int c : codes_) checks += tq_status_string(c) != nullptr && std::strlen(tq_status_string(c)) > 0;
}

}  // namespace

int main() {
    transforms();
    scoring();
    compress_and_decode();
    attention();
    status_strings();
    std::printf("%d checks, %d failures\n", checks, failures);
    return failures == 0 ? 0 : 1;
}
