/* Host sanitizer run of the CPU oracle (test infrastructure): built with
 * AddressSanitizer and UndefinedBehaviorSanitizer together with
 * oracle/gemm_oracle.c, it drives every entry point over edge shapes and bad
 * arguments.  A sanitizer finding aborts the run; a wrong result or return
 * code makes it exit 1. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_f16_decode(uint16_t h);
uint16_t oracle_f16_encode_rne(double x);
void oracle_f16_decode_array(const uint16_t* h, double* out, int64_t n);
void oracle_f16_encode_array(const double* x, uint16_t* out, int64_t n);
int oracle_gemm_nt_f16(const uint16_t* A, const uint16_t* B, int64_t M, int64_t N, int64_t K, double* C64,
                       uint16_t* C16, int threads);
int oracle_gemm_nt_f64(const double* a, const double* b, int64_t M, int64_t N, int64_t K, double* C64,
                       int threads);
int oracle_gemm_nt_f16_entries(const uint16_t* A, const uint16_t* B, int64_t M, int64_t N, int64_t K,
                               const int64_t* rows, const int64_t* cols, int64_t count, double* C64);

static int failures = 0;
#define CHECK(cond)                                                         \
    do {                                                                    \
        if (!(cond)) {                                                      \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                     \
        }                                                                   \
    } while (0)

static uint64_t state = 0x9e3779b97f4a7c15ull;
static uint16_t small_value(void) /* integers -3 .. 3 as binary16 bits */
{
    state = state * 6364136223846793005ull + 1442695040888963407ull;
    static const uint16_t v[7] = {0xC200, 0xC000, 0xBC00, 0x0000, 0x3C00, 0x4000, 0x4200};
    return v[(state >> 33) % 7];
}

static void product(int64_t M, int64_t N, int64_t K)
{
    uint16_t* A = malloc(sizeof(uint16_t) * (size_t)(M * K > 0 ? M * K : 1));
    uint16_t* B = malloc(sizeof(uint16_t) * (size_t)(N * K > 0 ? N * K : 1));
    double* c1 = malloc(sizeof(double) * (size_t)(M * N > 0 ? M * N : 1));
    double* c3 = malloc(sizeof(double) * (size_t)(M * N > 0 ? M * N : 1));
    uint16_t* h1 = malloc(sizeof(uint16_t) * (size_t)(M * N > 0 ? M * N : 1));
    uint16_t* h8 = malloc(sizeof(uint16_t) * (size_t)(M * N > 0 ? M * N : 1));
    for (int64_t i = 0; i < M * K; ++i) A[i] = small_value();
    for (int64_t i = 0; i < N * K; ++i) B[i] = small_value();
    CHECK(oracle_gemm_nt_f16(A, B, M, N, K, c1, h1, 1) == 0);
    CHECK(oracle_gemm_nt_f16(A, B, M, N, K, c3, NULL, 3) == 0);
    CHECK(oracle_gemm_nt_f16(A, B, M, N, K, c3, h8, 8) == 0);
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0; /* small integers: every order gives the same exact sum */
            for (int64_t k = 0; k < K; ++k) s += oracle_f16_decode(A[m * K + k]) * oracle_f16_decode(B[n * K + k]);
            CHECK(c1[m * N + n] == s && c3[m * N + n] == s);
            CHECK(h1[m * N + n] == h8[m * N + n] && h1[m * N + n] == oracle_f16_encode_rne(s));
        }
    if (M > 0 && N > 0) {
        int64_t rows[3] = {0, M - 1, M / 2}, cols[3] = {N - 1, 0, N / 2};
        double e[3];
        CHECK(oracle_gemm_nt_f16_entries(A, B, M, N, K, rows, cols, 3, e) == 0);
        for (int i = 0; i < 3; ++i) CHECK(e[i] == c1[rows[i] * N + cols[i]]);
        int64_t bad_row[1] = {M}, ok_col[1] = {0};
        CHECK(oracle_gemm_nt_f16_entries(A, B, M, N, K, bad_row, ok_col, 1, e) == -1);
        double* a = malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
        double* b = malloc(sizeof(double) * (size_t)(N * K > 0 ? N * K : 1));
        oracle_f16_decode_array(A, a, M * K);
        oracle_f16_decode_array(B, b, N * K);
        CHECK(oracle_gemm_nt_f64(a, b, M, N, K, c3, 5) == 0);
        for (int64_t i = 0; i < M * N; ++i) CHECK(c3[i] == c1[i]);
        free(a);
        free(b);
    }
    free(A); free(B); free(c1); free(c3); free(h1); free(h8);
}

int main(void)
{
    /* the codec: every pattern decodes, and every non-NaN one encodes back */
    static uint16_t all[65536], back[65536];
    static double dec[65536];
    for (int i = 0; i < 65536; ++i) all[i] = (uint16_t)i;
    oracle_f16_decode_array(all, dec, 65536);
    oracle_f16_encode_array(dec, back, 65536);
    for (int i = 0; i < 65536; ++i) {
        CHECK(dec[i] == oracle_f16_decode(all[i]) || (isnan(dec[i]) && isnan(oracle_f16_decode(all[i]))));
        if (!isnan(dec[i])) CHECK(back[i] == all[i]);
    }
    /* edge shapes: single elements, tails, more threads than row blocks, K = 0, empty */
    const int64_t shapes[][3] = {{1, 1, 1}, {7, 5, 3}, {33, 17, 65}, {17, 33, 8}, {40, 3, 0}, {0, 5, 4}, {5, 0, 4},
                                 {1, 64, 129}, {65, 1, 7}};
    for (size_t s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s) product(shapes[s][0], shapes[s][1], shapes[s][2]);
    /* bad arguments come back as -1 before anything is touched */
    double c = 0.0;
    uint16_t h = 0;
    CHECK(oracle_gemm_nt_f16(&h, &h, -1, 1, 1, &c, NULL, 1) == -1);
    CHECK(oracle_gemm_nt_f16(&h, &h, 1, 1, -1, &c, NULL, 1) == -1);
    CHECK(oracle_gemm_nt_f16(NULL, &h, 1, 1, 1, &c, NULL, 1) == -1);
    CHECK(oracle_gemm_nt_f16(&h, &h, 1, 1, 1, NULL, NULL, 1) == -1);
    CHECK(oracle_gemm_nt_f64(NULL, NULL, 1, 1, 1, &c, 1) == -1);
    CHECK(oracle_gemm_nt_f16_entries(&h, &h, 1, 1, 1, NULL, NULL, -1, &c) == -1);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer run: all checks passed\n");
    return 0;
}
