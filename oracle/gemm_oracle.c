/*
 * CPU oracle for the fp16 product C = A * B^T   (TEST INFRASTRUCTURE ONLY).
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * load this file's library.  The GPU library never links, includes or calls
 * it, and this file includes nothing from the GPU library: the two share no
 * code.
 *
 * What it computes is the plain definition of the operation, not an emulation
 * of any kernel:
 *
 *   C64[m][n] = sum_{k=0}^{K-1} dec(A[m][k]) * dec(B[n][k])      (binary64)
 *   C16[m][n] = rne_fp16(C64[m][n])
 *
 * "0. A Minimal Hopper Matmul", section "Block Tiling": C = A x B^T with A of
 * shape (M, K) and B of shape (N, K), so C is (M, N); the K-major note of the
 * same section stores both operands with K contiguous, which is the layout
 * taken here (A[m*K + k], B[n*K + k], C[m*N + n]).
 * Same page, section "Data Flow" (steps 3 and 4) and "Walkthrough",
 * subsection "Epilogue": the products accumulate into a wider (fp32)
 * accumulator and the result is converted to fp16 once, after the K loop.
 * The oracle widens further, to binary64, and rounds once (round to nearest,
 * ties to even) to fp16.
 *
 * Products of two fp16 values are exact in binary64 (11 + 11 significand
 * bits); the only rounding in C64 is the binary64 running sum, taken in the
 * plain sequential order k = 0, 1, ..., K-1.  Build with -ffp-contract=off so
 * no fused multiply-add changes that order of rounding.
 *
 * The fp16 codec below works on the bit fields of IEEE 754 binary16 (1 sign
 * bit, 5 exponent bits with bias 15, 10 fraction bits); it uses no compiler
 * half type and no vendor header.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- codec -- */

/* binary16 bits -> exact binary64 value (subnormals kept, never flushed). */
double oracle_f16_decode(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int expo = (h >> 10) & 0x1f;
    const int frac = h & 0x3ff;
    double v;
    if (expo == 0) {
        v = ldexp((double)frac, -24);              /* 0.frac * 2^-14 */
    } else if (expo == 31) {
        v = frac ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + frac), expo - 25); /* 1.frac * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* Round a non-negative binary64 value q (q < 2^52) to the nearest integer,
 * ties to the even integer.  q - floor(q) is exact in this range. */
static double round_half_even(double q)
{
    double f = floor(q);
    double r = q - f;
    if (r > 0.5 || (r == 0.5 && fmod(f, 2.0) != 0.0)) f += 1.0;
    return f;
}

/* binary64 -> binary16 bits, round to nearest, ties to even.
 * Magnitudes at or beyond 65520 (the midpoint between the largest finite
 * value 65504 and the next step 65536) become infinity; results below the
 * normal range become subnormals; NaN maps to the canonical quiet NaN with
 * the input's sign. */
uint16_t oracle_f16_encode_rne(double x)
{
    const uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x)) return sign | 0x7e00;
    double a = fabs(x);
    if (a >= 65520.0) return sign | 0x7c00;
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: count of 2^-24 steps; 1024 steps is exactly the
         * smallest normal and encodes as such (exponent field 1, fraction 0) */
        double q = round_half_even(ldexp(a, 24));
        return sign | (uint16_t)q;
    }
    int e2;
    (void)frexp(a, &e2);          /* a in [2^(e2-1), 2^e2) */
    int e = e2 - 1;               /* unbiased fp16 exponent, -14 .. 15 */
    double q = round_half_even(ldexp(a, 10 - e));  /* in [1024, 2048] */
    if (q == 2048.0) { q = 1024.0; e += 1; }
    if (e > 15) return sign | 0x7c00;
    return sign | (uint16_t)((e + 15) << 10) | (uint16_t)((int)q - 1024);
}

void oracle_f16_decode_array(const uint16_t* h, double* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_decode(h[i]);
}

void oracle_f16_encode_array(const double* x, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_encode_rne(x[i]);
}

/* ---------------------------------------------------------------- GEMM -- */

typedef struct {
    const double* a;   /* decoded A, [M][K] */
    const double* b;   /* decoded B, [N][K] */
    double* c64;       /* [M][N] */
    uint16_t* c16;     /* [M][N] or NULL */
    int64_t M, N, K;
    int64_t row_block; /* rows of A per work item */
    int64_t next;      /* shared work counter (guarded by lock) */
    pthread_mutex_t lock;
} gemm_job;

/* One block of rows: for every column n, the plain sequential k-sum of each
 * row in the block.  Rows are grouped only so that each row of B is reused
 * from cache; every output is still its own sequential sum over k. */
static void gemm_rows(gemm_job* j, int64_t m0, int64_t m1)
{
    const int64_t K = j->K, N = j->N;
    for (int64_t n = 0; n < N; ++n) {
        const double* bn = j->b + n * K;
        for (int64_t m = m0; m < m1; ++m) {
            const double* am = j->a + m * K;
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k) s += am[k] * bn[k];
            j->c64[m * N + n] = s;
            if (j->c16) j->c16[m * N + n] = oracle_f16_encode_rne(s);
        }
    }
}

static void* gemm_worker(void* arg)
{
    gemm_job* j = (gemm_job*)arg;
    for (;;) {
        pthread_mutex_lock(&j->lock);
        int64_t m0 = j->next;
        j->next += j->row_block;
        pthread_mutex_unlock(&j->lock);
        if (m0 >= j->M) break;
        int64_t m1 = m0 + j->row_block < j->M ? m0 + j->row_block : j->M;
        gemm_rows(j, m0, m1);
    }
    return NULL;
}

static int run_threads(gemm_job* job, int threads)
{
    if (threads < 1) threads = 1;
    if (threads > 256) threads = 256;
    pthread_t tid[256];
    int started = 0;
    for (int t = 0; t < threads; ++t) {
        if (pthread_create(&tid[t], NULL, gemm_worker, job) != 0) break;
        ++started;
    }
    if (started == 0) gemm_worker(job);
    for (int t = 0; t < started; ++t) pthread_join(tid[t], NULL);
    return 0;
}

/* C64 (and C16 if non-NULL) for fp16 inputs given as raw binary16 bits.
 * Returns 0 on success, -1 on bad arguments, -2 if memory is short. */
int oracle_gemm_nt_f16(const uint16_t* A, const uint16_t* B, int64_t M, int64_t N,
                       int64_t K, double* C64, uint16_t* C16, int threads)
{
    if (M < 0 || N < 0 || K < 0) return -1;
    if (M == 0 || N == 0) return 0;
    if (!C64) return -1;
    if (K > 0 && (!A || !B)) return -1;
    double* a = (double*)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
    double* b = (double*)malloc(sizeof(double) * (size_t)(N * K > 0 ? N * K : 1));
    if (!a || !b) { free(a); free(b); return -2; }
    oracle_f16_decode_array(A, a, M * K);
    oracle_f16_decode_array(B, b, N * K);
    gemm_job job;
    memset(&job, 0, sizeof(job));
    job.a = a; job.b = b; job.c64 = C64; job.c16 = C16;
    job.M = M; job.N = N; job.K = K;
    job.row_block = 16;
    pthread_mutex_init(&job.lock, NULL);
    run_threads(&job, threads);
    pthread_mutex_destroy(&job.lock);
    free(a); free(b);
    return 0;
}

/* Same definition on binary64 inputs that are already decoded (used by the
 * tests to evaluate the oracle on values that are not fp16, e.g. sums). */
int oracle_gemm_nt_f64(const double* a, const double* b, int64_t M, int64_t N,
                       int64_t K, double* C64, int threads)
{
    if (M < 0 || N < 0 || K < 0) return -1;
    if (M == 0 || N == 0) return 0;
    if (!C64 || (K > 0 && (!a || !b))) return -1;
    gemm_job job;
    memset(&job, 0, sizeof(job));
    job.a = a; job.b = b; job.c64 = C64; job.c16 = NULL;
    job.M = M; job.N = N; job.K = K;
    job.row_block = 16;
    pthread_mutex_init(&job.lock, NULL);
    run_threads(&job, threads);
    pthread_mutex_destroy(&job.lock);
    return 0;
}

/* Selected outputs only: for i < count, C64[i] = sum_k A[rows[i]][k]*B[cols[i]][k].
 * Lets a test check sampled outputs of a product too large to evaluate in full. */
int oracle_gemm_nt_f16_entries(const uint16_t* A, const uint16_t* B, int64_t M, int64_t N,
                               int64_t K, const int64_t* rows, const int64_t* cols,
                               int64_t count, double* C64)
{
    if (M < 0 || N < 0 || K < 0 || count < 0) return -1;
    for (int64_t i = 0; i < count; ++i) {
        int64_t m = rows[i], n = cols[i];
        if (m < 0 || m >= M || n < 0 || n >= N) return -1;
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k)
            s += oracle_f16_decode(A[m * K + k]) * oracle_f16_decode(B[n * K + k]);
        C64[i] = s;
    }
    return 0;
}
