/*
 * gemm_nt_f16 -- fp16 matrix product C = A * B^T on AMD Instinct MI355X (gfx950).
 *
 * The operation is the one of "0. A Minimal Hopper Matmul", section "Block
 * Tiling": C = A x B^T with A of shape (M, K) and B of shape (N, K), so C is
 * (M, N).  The K-major note of that section fixes the layout used here: both
 * operands are stored with K contiguous, B^T is only a view.  Products
 * accumulate in fp32 ("Data Flow", step 3) and the accumulator is converted
 * to fp16 once, after the K loop ("Walkthrough", subsection "Epilogue"); the
 * conversion rounds to nearest, ties to even.
 *
 * Layout (all three matrices row-major and dense, no leading-dimension
 * arguments):
 *   A[m * K + k]   IEEE binary16, M x K
 *   B[n * K + k]   IEEE binary16, N x K
 *   C[m * N + n]   IEEE binary16, M x N, written; never read
 *
 *   C[m][n] = fp16_rne( sum_{k<K} A[m][k] * B[n][k] )   with an fp32 sum
 *
 * The order of the fp32 additions is not specified (it is the kernel's tile
 * order), so results may differ from a sequential sum by fp32 rounding.
 *
 * Ownership and concurrency: A, B and C are device pointers owned by the
 * caller.  The library allocates no memory, keeps no per-call state and never
 * synchronizes the host; every call only enqueues kernels on `stream` (0 is
 * the null stream) and returns.  C is valid once that stream has reached the
 * point of the call.  Calls from several host threads are safe.  Because a
 * call is nothing but kernel launches (no allocation, no memset, no
 * synchronization), it may be captured into a HIP graph; each replay then
 * reads A and B and writes C at the addresses given at capture.
 *
 * Errors: every entry point returns a hipError_t value as int: 0
 * (hipSuccess) or an error.  Argument errors return 1 (hipErrorInvalidValue)
 * before anything is enqueued: a negative dimension, a null pointer with a
 * non-zero extent, C overlapping A or B, a dimension beyond the supported
 * range (M, N, K < 2^31, tile count < 2^31), or an unknown variant.
 * A failed launch returns the runtime's error code.  M == 0 or N == 0 writes
 * nothing and succeeds; K == 0 writes +0 to every element of C.
 *
 * Alignment and size: any 2-byte aligned pointers are accepted.  The MFMA
 * kernels need 16-byte aligned A and B, K % 8 == 0 (so every row starts on
 * 16 bytes) and K < 2^22 (a 256-row operand tile then spans less than 2^31
 * bytes, the reach of their 32-bit buffer offsets); other inputs run a plain
 * per-element kernel that gives the same results within fp32 rounding, only
 * slower.  gemm_nt_f16_ex refuses an MFMA variant for such inputs.
 */
#ifndef GEMM_NT_F16_H
#define GEMM_NT_F16_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The HIP runtime's stream handle (identical to the typedef in
 * hip/hip_runtime_api.h, so both headers may be included together). */
typedef struct ihipStream_t* hipStream_t;

#define GEMM_NT_F16_VERSION 1

/* C = A * B^T as described above, with the kernel variant chosen from
 * (M, N, K) and the pointers' alignment.  When 256 x 256 tiles would leave
 * a small last wave, the rows of C are split in two blocks, each enqueued
 * as its own kernel on `stream` (see gemm_nt_f16_plan). */
int gemm_nt_f16(const void* A, const void* B, void* C,
                int64_t M, int64_t N, int64_t K, hipStream_t stream);

/* Same operation with an explicit kernel variant (0 <= variant <
 * gemm_nt_f16_variant_count()), run on all of C, or the automatic choice
 * (the plan of gemm_nt_f16) if variant < 0.
 * For benchmarks and ablations.  A variant whose requirements (alignment,
 * K % 8, K < 2^22) the arguments do not meet returns hipErrorInvalidValue. */
int gemm_nt_f16_ex(const void* A, const void* B, void* C,
                   int64_t M, int64_t N, int64_t K, int32_t variant,
                   hipStream_t stream);

/* Number of kernel variants compiled into the library. */
int32_t gemm_nt_f16_variant_count(void);

/* Static, NUL-terminated name of a variant (tile shape, waves, stages), or
 * NULL for an unknown index.  The string is owned by the library. */
const char* gemm_nt_f16_variant_name(int32_t variant);

/* Index of the variant gemm_nt_f16 uses for these sizes (for the first
 * block of rows if it splits them) when A and B are 16-byte aligned, or -1
 * for invalid sizes.  Host-only; enqueues nothing. */
int32_t gemm_nt_f16_select(int64_t M, int64_t N, int64_t K);

/* The whole launch plan of gemm_nt_f16 for these sizes (A and B 16-byte
 * aligned): returns the variant for rows [0, *rows) of C, as
 * gemm_nt_f16_select does; *rows (if rows is not NULL) receives the number
 * of rows it covers (M when nothing is split, else a multiple of 256) and
 * *rest (if not NULL) the variant for rows [*rows, M), or -1.  Host-only;
 * enqueues nothing.  -1 for invalid sizes. */
int32_t gemm_nt_f16_plan(int64_t M, int64_t N, int64_t K, int64_t* rows,
                         int32_t* rest);

/* Name of the variant gemm_nt_f16_select returns (NULL for invalid sizes). */
const char* gemm_nt_f16_config_name(int64_t M, int64_t N, int64_t K);

/* GEMM_NT_F16_VERSION of the built library. */
int gemm_nt_f16_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_NT_F16_H */
