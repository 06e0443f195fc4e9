// fp16 C = A * B^T for gfx950 (CDNA4): MFMA kernels and the C ABI.
//
// The operation and layout are those of "0. A Minimal Hopper Matmul",
// section "Block Tiling" (A is M x K, B is N x K, both K-major, C is M x N)
// with fp32 accumulation ("Data Flow") and one fp16 cast after the K loop
// ("Walkthrough" / "Epilogue").  The pages build this for Hopper out of TMA,
// mbarriers and warp-group MMA; none of those exist on CDNA4, so the kernel
// keeps only the ideas that still hold and re-derives the rest for gfx950:
//
//  * one workgroup per BM x BN output tile, K walked in BK = 64 steps
//    ("0. A Minimal Hopper Matmul", "Block Tiling");
//  * a multi-stage shared-memory ring so loads of step k+1 overlap the
//    matrix-core work of step k ("3. Warp Specialization", introduction and
//    "Draining the Pipeline").  On CDNA4 every wave issues its own loads, so
//    there is no producer warp; loads go straight from global memory to LDS
//    (buffer_load ... lds), completion is tracked with the vmcnt counter and
//    made visible to the other waves with one s_barrier per K step;
//  * several waves per workgroup, each owning a sub-tile of C and sharing the
//    B tile in LDS ("6. Four Consumers, FP16 Accumulation, and a TMA
//    Epilogue", introduction);
//  * a grouped raster of tiles for cache reuse ("6. Four Consumers ...",
//    "What Changed from V5", raster group width), here additionally made
//    aware of the 8 XCDs, each with its own L2;
//  * an fp32 accumulator sized to the register file ("6. Four Consumers ...",
//    "The Register Budget Problem"): on CDNA4 the MFMA accumulates in fp32 in
//    the 256 accumulation registers (AGPRs) per lane, so a 4-wave 256 x 256
//    tile gives each wave a 128 x 128 fp32 accumulator = 256 AGPRs.
//
// LDS layout of one stage: the A tile (BM rows) then the B tile (BN rows);
// each row is BK = 64 fp16 = 128 bytes = 8 chunks of 16 bytes.  Chunk c of
// row r is stored at chunk position c ^ (r & 7), so the 16-byte fragment
// reads of 8 consecutive rows at the same logical chunk land in 8 different
// positions of the row (different LDS banks).
//
// Matrix-core step: v_mfma_f32_32x32x16_f16.  Operand lane l holds 8
// consecutive-k fp16 values of row (l % 32), k offset 8 * (l / 32); the same
// k mapping is used for both operands, so the contraction is over matching k
// whatever order the hardware multiplies them in.  The B fragment is passed
// as the first operand and the A fragment as the second, which makes the
// 32 x 32 result C^T: lane l then holds row m = l % 32 of C and, in
// accumulator register r, column n = 8 * (r / 4) + 4 * (l / 32) + r % 4, i.e.
// four consecutive columns per group of four registers, stored as one 8-byte
// write.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "gemm_nt_f16.h"

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));

typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kWave = 64;
constexpr int kXcds = 8;          // MI355X: 8 accelerator complex dies
constexpr uint32_t kOob = 0x80000000u;  // buffer offset past any tile: loads 0

// Buffer resource word 3 for gfx9-family (data format 32, no swizzle).
constexpr int kRsrcWord3 = 0x00020000;

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] + vmcnt[5:4] at bits 15:14,
// expcnt[6:4], lgkmcnt[11:8]); the counters not waited on are left at max.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// Tile order.  Workgroups are dispatched round-robin over the XCDs (workgroup
// id modulo 8), so consecutive ids land on different L2 caches.  First
// renumber ids so each XCD owns one contiguous range of the linear order, then
// sweep that order in groups of `group_m` tile rows, column by column, so the
// tiles that run at the same time on one XCD share rows of A and of B.
__device__ __forceinline__ void tile_coords(int pid, int tiles_m, int tiles_n, int group_m,
                                            int& tm, int& tn)
{
    const int total = tiles_m * tiles_n;
    const int per = total / kXcds, extra = total % kXcds;
    const int x = pid % kXcds, local = pid / kXcds;
    const int lin = x * per + (x < extra ? x : extra) + local;
    const int width = group_m * tiles_n;
    const int g = lin / width;
    const int first = g * group_m;
    const int rows = min(tiles_m - first, group_m);
    const int r = lin - g * width;
    tm = first + r % rows;
    tn = r / rows;
}

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int STAGES_>
struct TileShape {
    static constexpr int BM = BM_, BN = BN_, BK = 64;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int WAVES = WAVES_M * WAVES_N, THREADS = WAVES * kWave;
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;  // wave sub-tile
    static constexpr int FM = WTM / 32, FN = WTN / 32;            // 32x32 blocks per wave
    static constexpr int STAGES = STAGES_;
    static constexpr int ROW_BYTES = BK * 2;                       // 128
    static constexpr int A_BYTES = BM * ROW_BYTES, B_BYTES = BN * ROW_BYTES;
    // LDS: all A stages, then all B stages (keeps every offset inside the
    // 16-bit immediate of ds_read for each operand's own base register)
    static constexpr int B_BASE = STAGES * A_BYTES;
    static constexpr int LDS_BYTES = STAGES * (A_BYTES + B_BYTES);
    static constexpr int A_LOADS = A_BYTES / (kWave * 16) / WAVES;  // 1 KiB per wave load
    static constexpr int B_LOADS = B_BYTES / (kWave * 16) / WAVES;
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(A_LOADS * WAVES * kWave * 16 == A_BYTES, "A tile must split evenly over waves");
    static_assert(B_LOADS * WAVES * kWave * 16 == B_BYTES, "B tile must split evenly over waves");
    static_assert(LDS_BYTES <= 160 * 1024, "gfx950 has 160 KiB of LDS per workgroup");
    static_assert(A_BYTES <= 65536 && B_BYTES * STAGES <= 65536, "ds_read offsets");
};

// Main MFMA kernel.  Requirements checked on the host: A and B 16-byte
// aligned, K % 8 == 0, K < 2^22, M, N < 2^31.  `c_vec` says whether C rows
// allow aligned 8-byte stores (N % 4 == 0 and C 8-byte aligned).
template <class T>
__global__ void __launch_bounds__(T::THREADS, 1)
gemm_nt_f16_mfma(const _Float16* __restrict__ A, const _Float16* __restrict__ B,
                 _Float16* __restrict__ C, int M, int N, int K, int tiles_m, int tiles_n,
                 int group_m, int c_vec)
{
    __shared__ __attribute__((aligned(1024))) unsigned char smem[T::LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wave / T::WAVES_N, wn = wave % T::WAVES_N;

    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * T::BM, n0 = tn * T::BN;
    const int rows_a = min(T::BM, M - m0), rows_b = min(T::BN, N - n0);
    const uint32_t row_bytes = (uint32_t)K * 2u;

    // One buffer per operand tile: base at the tile's first row, size up to
    // its last valid row, so rows past M (or N) read as zero.
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + (size_t)m0 * K, (uint32_t)rows_a * row_bytes);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + (size_t)n0 * K, (uint32_t)rows_b * row_bytes);

    // Global->LDS copy assignment.  Load j of this wave fills LDS bytes
    // [g * 1024, g * 1024 + 1024) of the operand tile, g = wave * LOADS + j:
    // rows 8g .. 8g+7; lane l writes position (l & 7) of row 8g + l / 8, so it
    // fetches logical chunk (l & 7) ^ (row & 7) = (l & 7) ^ (l / 8).
    const int ld_row = lane >> 3;
    const int ld_chunk = (lane & 7) ^ ld_row;
    const uint32_t ld_voff = (uint32_t)ld_row * row_bytes + (uint32_t)ld_chunk * 16u;
    const int ld_k = ld_chunk * 8;  // first k of this lane's chunk within the step

    auto issue_loads = [&](int stage, int kstep) {
        const int k0 = kstep * T::BK;
        // K tail: chunks at or past K read as zero (both operands), so the
        // padded products add nothing.
        const uint32_t voff = (k0 + ld_k < K) ? ld_voff : kOob;
        const uint32_t soff = (uint32_t)k0 * 2u;
#pragma unroll
        for (int j = 0; j < T::A_LOADS; ++j) {
            const int g = wave * T::A_LOADS + j;
            const uint32_t v = voff == kOob ? kOob : voff + (uint32_t)(g * 8) * row_bytes;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ra, (lds_void_t*)(smem + stage * T::A_BYTES + g * 1024), 16, v, soff, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < T::B_LOADS; ++j) {
            const int g = wave * T::B_LOADS + j;
            const uint32_t v = voff == kOob ? kOob : voff + (uint32_t)(g * 8) * row_bytes;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rb, (lds_void_t*)(smem + T::B_BASE + stage * T::B_BYTES + g * 1024), 16, v, soff,
                0, 0);
        }
    };

    // Fragment reads: row (l % 32) of each 32-row block, logical chunk
    // 2 * kk + l / 32 for k sub-step kk (16 k values per MFMA).
    const int fr_row = lane & 31;
    const int fr_hi = lane >> 5;
    const unsigned char* a_lds = smem + (wm * T::WTM + fr_row) * T::ROW_BYTES;
    const unsigned char* b_lds = smem + T::B_BASE + (wn * T::WTN + fr_row) * T::ROW_BYTES;

    half8_t fa[2][T::FM], fb[2][T::FN];
    float16_t acc[T::FM][T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    auto read_frags = [&](int buf, int stage, int kk) {
        const int pos = ((2 * kk + fr_hi) ^ (fr_row & 7)) * 16;
#pragma unroll
        for (int i = 0; i < T::FM; ++i)
            fa[buf][i] = *(const half8_t*)(a_lds + stage * T::A_BYTES + i * 32 * T::ROW_BYTES + pos);
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
            fb[buf][j] = *(const half8_t*)(b_lds + stage * T::B_BYTES + j * 32 * T::ROW_BYTES + pos);
    };

    auto mma = [&](int buf) {
#pragma unroll
        for (int i = 0; i < T::FM; ++i)
#pragma unroll
            for (int j = 0; j < T::FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[buf][j], fa[buf][i], acc[i][j],
                                                                   0, 0, 0);
    };

    const int nk = (K + T::BK - 1) / T::BK;

    // Two-stage ring.  Invariant at the top of step ks: stage ks & 1 holds
    // step ks and is visible to all waves; the loads of step ks + 1 are in
    // flight into the other stage; fa/fb[0] hold sub-step 0 of step ks.
    // Sub-step 3's MFMAs run after the barrier, overlapping the first
    // fragment reads of the next stage.
    static_assert(T::STAGES == 2, "ring below is written for two stages");
    if (nk > 0) {
        issue_loads(0, 0);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        __syncthreads();
        if (nk > 1) issue_loads(1, 1);
        read_frags(0, 0, 0);

        auto step = [&](int ks, int cur) {
            read_frags(1, cur, 1);
            mma(0);
            read_frags(0, cur, 2);
            mma(1);
            read_frags(1, cur, 3);
            mma(0);
            if (ks + 1 < nk) {
                // own loads of step ks+1 landed; the barrier makes everyone's
                // visible and (its fence drains LDS reads) frees stage `cur`
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
                __syncthreads();
                if (ks + 2 < nk) issue_loads(cur, ks + 2);
                read_frags(0, cur ^ 1, 0);
            }
            mma(1);
        };

        int ks = 0;
        for (; ks + 1 < nk; ks += 2) {
            step(ks, 0);
            step(ks + 1, 1);
        }
        if (ks < nk) step(ks, 0);
    }

    // Epilogue: fp32 -> fp16 (round to nearest even), 4 consecutive columns
    // per 8-byte store; rows past M and columns past N are not written.
    const int cm_base = m0 + wm * T::WTM + fr_row;
    const int cn_base = n0 + wn * T::WTN + 4 * fr_hi;
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
        const int m = cm_base + i * 32;
        if (m >= M) continue;
        _Float16* crow = C + (size_t)m * N;
#pragma unroll
        for (int j = 0; j < T::FN; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = cn_base + j * 32 + 8 * q;
                half4_t h;
                h[0] = (_Float16)acc[i][j][4 * q + 0];
                h[1] = (_Float16)acc[i][j][4 * q + 1];
                h[2] = (_Float16)acc[i][j][4 * q + 2];
                h[3] = (_Float16)acc[i][j][4 * q + 3];
                if (c_vec && n + 3 < N) {
                    *(half4_t*)(crow + n) = h;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < N) crow[n + e] = h[e];
                }
            }
        }
    }
}

// Plain per-element kernel for inputs the MFMA kernels do not take
// (unaligned pointers, K % 8 != 0, very long K).  One thread per output,
// fp32 accumulation in k order, one fp16 rounding at the end.
__global__ void __launch_bounds__(256)
gemm_nt_f16_simple(const _Float16* __restrict__ A, const _Float16* __restrict__ B,
                   _Float16* __restrict__ C, int64_t M, int64_t N, int64_t K)
{
    const int64_t n = (int64_t)blockIdx.x * 16 + (threadIdx.x & 15);
    const int64_t m = (int64_t)blockIdx.y * 16 + (threadIdx.x >> 4);
    if (m >= M || n >= N) return;
    const _Float16* a = A + m * K;
    const _Float16* b = B + n * K;
    float s = 0.0f;
    for (int64_t k = 0; k < K; ++k) s += (float)a[k] * (float)b[k];
    C[m * N + n] = (_Float16)s;
}

// ------------------------------------------------------------------ host --

typedef TileShape<256, 256, 2, 2, 2> Tile256;
typedef TileShape<128, 128, 2, 2, 2> Tile128;
typedef TileShape<64, 64, 2, 2, 2> Tile64;

constexpr int64_t kMaxK = (int64_t)1 << 22;
constexpr int64_t kMaxMN = ((int64_t)1 << 31) - 1;

struct Variant {
    const char* name;
    int bm, bn;    // 0 for the per-element kernel
    int group_m;
    int (*launch)(const void*, const void*, void*, int64_t, int64_t, int64_t, int, hipStream_t);
};

template <class T>
int launch_mfma(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int group_m,
                hipStream_t stream)
{
    const int64_t tiles_m = (M + T::BM - 1) / T::BM, tiles_n = (N + T::BN - 1) / T::BN;
    if (tiles_m * tiles_n > kMaxMN) return hipErrorInvalidValue;
    const int c_vec = (N % 4 == 0) && ((uintptr_t)C % 8 == 0);
    hipLaunchKernelGGL((gemm_nt_f16_mfma<T>), dim3((unsigned)(tiles_m * tiles_n)), dim3(T::THREADS),
                       0, stream, (const _Float16*)A, (const _Float16*)B, (_Float16*)C, (int)M,
                       (int)N, (int)K, (int)tiles_m, (int)tiles_n, group_m, c_vec);
    return (int)hipGetLastError();
}

int launch_simple(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int,
                  hipStream_t stream)
{
    const int64_t gx = (N + 15) / 16, gy = (M + 15) / 16;
    if (gx > kMaxMN || gy > 65535) return hipErrorInvalidValue;
    hipLaunchKernelGGL(gemm_nt_f16_simple, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, stream,
                       (const _Float16*)A, (const _Float16*)B, (_Float16*)C, M, N, K);
    return (int)hipGetLastError();
}

const Variant kVariants[] = {
    {"mfma32_256x256x64_w2x2_s2_g8", 256, 256, 8, launch_mfma<Tile256>},
    {"mfma32_128x128x64_w2x2_s2_g8", 128, 128, 8, launch_mfma<Tile128>},
    {"mfma32_64x64x64_w2x2_s2_g8", 64, 64, 8, launch_mfma<Tile64>},
    {"simple_f32_per_element", 0, 0, 0, launch_simple},
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);
constexpr int kSimple = kNumVariants - 1;

bool overlaps(const void* p, int64_t pbytes, const void* q, int64_t qbytes)
{
    const uintptr_t a0 = (uintptr_t)p, a1 = a0 + (uintptr_t)pbytes;
    const uintptr_t b0 = (uintptr_t)q, b1 = b0 + (uintptr_t)qbytes;
    return a0 < b1 && b0 < a1;
}

// Host-side argument check; touches no HIP state.
int validate(const void* A, const void* B, const void* C, int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || N < 0 || K < 0) return hipErrorInvalidValue;
    if (M > kMaxMN || N > kMaxMN || K > kMaxMN) return hipErrorInvalidValue;
    if (M == 0 || N == 0) return hipSuccess;
    if (!C) return hipErrorInvalidValue;
    if (K > 0 && (!A || !B)) return hipErrorInvalidValue;
    if (((uintptr_t)A | (uintptr_t)B | (uintptr_t)C) & 1) return hipErrorInvalidValue;
    const int64_t cbytes = M * N * 2;
    if (K > 0 && (overlaps(C, cbytes, A, M * K * 2) || overlaps(C, cbytes, B, N * K * 2)))
        return hipErrorInvalidValue;
    return hipSuccess;
}

bool mfma_eligible(const void* A, const void* B, int64_t K)
{
    return K % 8 == 0 && K < kMaxK && ((uintptr_t)A % 16 == 0) && ((uintptr_t)B % 16 == 0);
}

// Shape -> variant.  Prefer the largest tile that still gives the chip (256
// CUs) about one tile per CU; smaller tiles only when the large one would
// leave most CUs idle.
int select_mfma(int64_t M, int64_t N)
{
    const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
    const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
    if (t256 >= 192) return 0;
    if (t128 >= 128) return 1;
    return 2;
}

}  // namespace

extern "C" {

int gemm_nt_f16_version(void) { return GEMM_NT_F16_VERSION; }

int32_t gemm_nt_f16_variant_count(void) { return kNumVariants; }

const char* gemm_nt_f16_variant_name(int32_t variant)
{
    if (variant < 0 || variant >= kNumVariants) return nullptr;
    return kVariants[variant].name;
}

int32_t gemm_nt_f16_select(int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || N < 0 || K < 0 || M > kMaxMN || N > kMaxMN || K > kMaxMN) return -1;
    if (K % 8 != 0 || K >= kMaxK) return kSimple;
    return select_mfma(M, N);
}

const char* gemm_nt_f16_config_name(int64_t M, int64_t N, int64_t K)
{
    const int32_t v = gemm_nt_f16_select(M, N, K);
    return v < 0 ? nullptr : kVariants[v].name;
}

int gemm_nt_f16_ex(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                   int32_t variant, hipStream_t stream)
{
    int rc = validate(A, B, C, M, N, K);
    if (rc != hipSuccess) return rc;
    if (variant >= kNumVariants) return hipErrorInvalidValue;
    if (M == 0 || N == 0) return hipSuccess;
    const bool fast = mfma_eligible(A, B, K);
    if (variant < 0) variant = fast ? select_mfma(M, N) : kSimple;
    else if (variant != kSimple && !fast) return hipErrorInvalidValue;
    const Variant& v = kVariants[variant];
    return v.launch(A, B, C, M, N, K, v.group_m, stream);
}

int gemm_nt_f16(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                hipStream_t stream)
{
    return gemm_nt_f16_ex(A, B, C, M, N, K, -1, stream);
}

}  // extern "C"
