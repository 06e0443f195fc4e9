// Host sanitizer run of the C ABI (test infrastructure): built by hipcc with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code together
// with the library source, it calls every entry point in ways that return
// before any kernel launch: argument errors, empty products, the variant
// table, and the launch plan over edge and extreme sizes.  No call here can
// enqueue GPU work, so the run is the same with or without a GPU.  A
// sanitizer finding aborts the run; a wrong result makes it exit 1.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gemm_nt_f16.h"

namespace {

int failures = 0;
#define CHECK(cond)                                                                   \
    do {                                                                              \
        if (!(cond)) {                                                                \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                               \
        }                                                                             \
    } while (0)

constexpr int kInvalid = 1;  // hipErrorInvalidValue
constexpr int64_t kMax = (int64_t(1) << 31) - 1;

void plan_is_consistent(int64_t M, int64_t N, int64_t K)
{
    int64_t rows = -7;
    int32_t rest = -7;
    const int32_t v = gemm_nt_f16_plan(M, N, K, &rows, &rest);
    const int32_t count = gemm_nt_f16_variant_count();
    if (M < 0 || N < 0 || K < 0 || M > kMax || N > kMax || K > kMax) {
        CHECK(v == -1);
        return;
    }
    CHECK(v >= 0 && v < count);
    CHECK(gemm_nt_f16_select(M, N, K) == v);
    const char* name = gemm_nt_f16_config_name(M, N, K);
    CHECK(name != nullptr && strcmp(name, gemm_nt_f16_variant_name(v)) == 0);
    CHECK(rows >= 0 && rows <= M);
    if (rows < M) CHECK(rest >= 0 && rest < count && rows > 0);
    else CHECK(rest == -1);
    CHECK(gemm_nt_f16_plan(M, N, K, nullptr, nullptr) == v);
}

}  // namespace

int main()
{
    CHECK(gemm_nt_f16_version() == GEMM_NT_F16_VERSION);
    const int32_t count = gemm_nt_f16_variant_count();
    CHECK(count > 1);
    for (int32_t i = 0; i < count; ++i) CHECK(gemm_nt_f16_variant_name(i) != nullptr);
    CHECK(gemm_nt_f16_variant_name(-1) == nullptr && gemm_nt_f16_variant_name(count) == nullptr);

    // the plan: edge sizes, the largest accepted, past the limits, and a
    // pseudo-random spread (64-bit LCG)
    const int64_t edge[] = {0, 1, 7, 8, 15, 16, 63, 64, 65, 255, 256, 257, 4095, 4096, 8192, 65536,
                            1 << 20, kMax - 1, kMax, kMax + 1, -1};
    for (int64_t M : edge)
        for (int64_t N : edge)
            for (int64_t K : edge) plan_is_consistent(M, N, K);
    uint64_t s = 12345;
    for (int i = 0; i < 20000; ++i) {
        int64_t d[3];
        for (int64_t& x : d) {
            s = s * 6364136223846793005ull + 1442695040888963407ull;
            const int bits = (int)((s >> 59) % 31) + 1;  // 1 .. 31 bits
            x = (int64_t)((s >> 20) & ((uint64_t(1) << bits) - 1));
        }
        plan_is_consistent(d[0], d[1], d[2]);
    }

    // argument errors come back before anything is launched; pointers here
    // are never dereferenced.  A, B and C (4 x 4 each, 32 bytes) lie apart.
    alignas(16) static char buf[256];
    void* A = buf;
    void* B = buf + 64;
    void* C = buf + 128;
    CHECK(gemm_nt_f16(A, B, C, -1, 4, 4, nullptr) == kInvalid);
    CHECK(gemm_nt_f16(A, B, C, 4, -1, 4, nullptr) == kInvalid);
    CHECK(gemm_nt_f16(A, B, C, 4, 4, -1, nullptr) == kInvalid);
    CHECK(gemm_nt_f16(A, B, C, kMax + 1, 4, 4, nullptr) == kInvalid);
    CHECK(gemm_nt_f16(A, B, C, 4, 4, kMax + 1, nullptr) == kInvalid);
    CHECK(gemm_nt_f16(A, B, nullptr, 4, 4, 4, nullptr) == kInvalid);
    CHECK(gemm_nt_f16(nullptr, B, C, 4, 4, 4, nullptr) == kInvalid);
    CHECK(gemm_nt_f16(A, nullptr, C, 4, 4, 4, nullptr) == kInvalid);
    CHECK(gemm_nt_f16(buf + 1, B, C, 4, 4, 4, nullptr) == kInvalid);       // odd A
    CHECK(gemm_nt_f16(A, B, buf + 129, 4, 4, 4, nullptr) == kInvalid);     // odd C
    CHECK(gemm_nt_f16(A, B, buf + 16, 4, 4, 4, nullptr) == kInvalid);      // C overlaps A
    CHECK(gemm_nt_f16(A, B, buf + 80, 4, 4, 4, nullptr) == kInvalid);      // C overlaps B
    CHECK(gemm_nt_f16(A, B, C, kMax, kMax, kMax, nullptr) == kInvalid);    // C's extent covers A and B
    CHECK(gemm_nt_f16_ex(A, B, C, 4, 4, 4, count, nullptr) == kInvalid);   // unknown variant
    // empty products succeed without touching anything, whatever the pointers
    CHECK(gemm_nt_f16(nullptr, nullptr, nullptr, 0, 5, 3, nullptr) == 0);
    CHECK(gemm_nt_f16(nullptr, nullptr, nullptr, 5, 0, 3, nullptr) == 0);
    CHECK(gemm_nt_f16_ex(nullptr, nullptr, nullptr, 0, 0, 0, count - 1, nullptr) == 0);

    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("ABI sanitizer run: all checks passed\n");
    return 0;
}
