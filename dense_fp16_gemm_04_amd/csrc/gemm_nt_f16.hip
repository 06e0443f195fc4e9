// fp16 C = A * B^T for gfx950 (CDNA4): MFMA kernels and the C ABI.
//
// The operation and layout are those of "0. A Minimal Hopper Matmul",
// section "Block Tiling" (A is M x K, B is N x K, both K-major, C is M x N)
// with fp32 accumulation ("Data Flow") and one fp16 cast after the K loop
// ("Walkthrough" / "Epilogue").  The pages build this for Hopper out of TMA,
// mbarriers and warp-group MMA; none of those exist on CDNA4, so the kernels
// keep only the ideas that still hold and re-derive the rest for gfx950:
//
//  * a BM x BN output tile per workgroup at a time, K walked in BK-deep
//    steps ("0. A Minimal Hopper Matmul", "Block Tiling"); the default
//    256 x 256 kernel keeps one workgroup per CU walking its tiles, and the
//    host may split the rows of C over two kernels (plan_mfma);
//  * a multi-stage shared-memory ring so loads of later steps overlap the
//    matrix-core work of the current one ("3. Warp Specialization",
//    introduction and "Draining the Pipeline").  On CDNA4 every wave issues
//    its own loads, so there is no producer warp: loads go straight from
//    global memory to LDS (buffer_load ... lds), completion is tracked with
//    the vmcnt counter and made visible to the other waves with one
//    s_barrier per K step;
//  * several waves per workgroup, each owning a sub-tile of C and sharing the
//    operand tiles in LDS ("6. Four Consumers, FP16 Accumulation, and a TMA
//    Epilogue", introduction);
//  * a grouped raster of tiles for cache reuse ("6. Four Consumers ...",
//    "What Changed from V5", raster group width), here additionally made
//    aware of the 8 XCDs, each with its own L2;
//  * an fp32 accumulator sized to the register file ("6. Four Consumers ...",
//    "The Register Budget Problem"): the MFMA accumulates in fp32, and a
//    256 x 256 tile needs 256 KiB of accumulators: 4 waves x 256 AGPRs per
//    lane (one wave per SIMD), or 8 waves x 128 (two per SIMD).
//
// LDS layout of one stage: the A tile (BM rows) then the B tile (BN rows);
// the 5-slot kernels keep one operand tile per 32 KiB slot instead.  Each
// row holds BK fp16 (64 or 128 bytes) as 16-byte chunks.  gfx950's LDS
// serves 64 banks x 4 bytes per cycle; a 16-byte read (ds_read_b128) takes
// four passes of 16 lanes, and the lanes of one pass must hit 16 different
// 16-byte bank groups.  The passes are lanes {0-3, 12-15, 20-23, 24-27},
// {4-11, 16-19, 28-31} and the same plus 32 (measured with a probe that
// puts two lanes on one bank and reads SQ_LDS_BANK_CONFLICT).  Chunk c of
// row r is stored at position c ^ ((r / ROWS_PER_LINE) % CHUNKS),
// ROWS_PER_LINE being the rows that share one 256-byte line, which makes
// every fragment read conflict-free except 64-byte rows under 16x16x32
// MFMAs, which get their own XOR term (swz).
//
// Matrix-core step: v_mfma_f32_16x16x32_f16 (the kernels the library
// selects) or v_mfma_f32_32x32x16_f16 (ablations).  Operand lane l holds 8
// consecutive-k fp16 values of row (l % MI), k offset 8 * (l / MI), MI = 16
// or 32; the same k mapping is used for both operands, so the contraction is
// over matching k whatever order the hardware multiplies them in.  The B
// fragment is passed as the first operand and the A fragment as the second,
// which makes the result block C^T: lane l then holds row m = l % MI of C
// and, in accumulator register r, column n = 8 * (r / 4) + 4 * (l / MI) +
// r % 4 (16x16: the four columns 4 * (l / 16) .. +3), i.e. four consecutive
// columns per group of four registers, stored as one 8-byte piece.
//
// Kernels: gemm_nt_f16_mfma (compiler-scheduled, any TileShape),
// gemm_nt_f16_ordered (four or eight waves, K loop in a fixed hand-placed
// order, one tile per workgroup), gemm_nt_f16_ordered_persist (its
// persistent 5-slot form: the default for large shapes),
// gemm_nt_f16_simple (one output per thread, for K % 8 != 0 and unaligned
// operands).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <algorithm>

#include "gemm_nt_f16.h"

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// Accumulator block of one lane: 16 floats for a 32x32 MFMA block, 4 for a
// 16x16 one.
template <int MI>
struct AccBlock;
template <>
struct AccBlock<32> {
    using type = float16_t;
};
template <>
struct AccBlock<16> {
    using type = float4_t;
};

typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kWave = 64;
constexpr int kXcds = 8;          // MI355X: 8 accelerator complex dies
constexpr uint32_t kOob = 0x80000000u;  // buffer offset past any tile: loads 0

// Buffer resource word 3 for gfx9-family (data format 32, no swizzle).
constexpr int kRsrcWord3 = 0x00020000;
// Cache-policy operand of a buffer access: the nontemporal (nt) bit.
constexpr int kPolicyNt = 2;

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] + vmcnt[5:4] at bits 15:14,
// expcnt[6:4], lgkmcnt[11:8]); the counters not waited on are left at max.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Wait until at most VM of this wave's global->LDS loads are still in flight
// and all of its LDS reads have returned, then meet the other waves at the
// barrier.  Written as one asm statement with a memory clobber so no LDS
// access moves across it.  (__syncthreads() would add a workgroup fence,
// which waits for every outstanding load, vmcnt(0), and so would cap the
// ring at two stages whatever its depth.)
template <int VM>
__device__ __forceinline__ void lds_barrier()
{
    static_assert(VM >= 0 && VM <= 63, "vmcnt holds 0 .. 63");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"i"(VM) : "memory");
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// Tile order.  Workgroups are dispatched round-robin over the XCDs (workgroup
// id modulo 8), so consecutive ids land on different L2 caches.  First
// renumber ids so each XCD owns one contiguous range of the linear order, then
// sweep that order in groups of `group_m` tile rows, column by column, so the
// tiles that run at the same time on one XCD share rows of A and of B.
// Two other orders exist for comparison: group_m < 0 groups |group_m| tile
// rows without the XCD renumbering (the pages' grouped raster, made for one
// L2), and group_m == 0 walks the tiles row by row.
__device__ __forceinline__ void tile_coords(int pid, int tiles_m, int tiles_n, int group_m,
                                            int& tm, int& tn)
{
    if (group_m == 0) {
        tm = pid / tiles_n;
        tn = pid - tm * tiles_n;
        return;
    }
    const int total = tiles_m * tiles_n;
    int lin = pid;
    if (group_m > 0) {
        const int per = total / kXcds, extra = total % kXcds;
        const int x = pid % kXcds, local = pid / kXcds;
        lin = x * per + (x < extra ? x : extra) + local;
    } else {
        group_m = -group_m;
    }
    const int width = group_m * tiles_n;
    const int g = lin / width;
    const int first = g * group_m;
    const int rows = min(tiles_m - first, group_m);
    const int r = lin - g * width;
    tm = first + r % rows;
    tn = r / rows;
}

// Compile-time tile configuration.
//   BM x BN   output tile of one workgroup
//   BK        K depth of one pipeline step (32 or 64 fp16 = 64 or 128 bytes
//             per LDS row)
//   WAVES_M x WAVES_N waves, each owning a (BM / WAVES_M) x (BN / WAVES_N)
//             sub-tile of C, i.e. FM x FN blocks of 32 x 32
//   STAGES    depth of the LDS ring: loads run STAGES - 1 steps ahead
//   MIN_WAVES_PER_SIMD  occupancy hint (1: up to 512 registers per lane, the
//             256 AGPRs holding the accumulator; 2: up to 256)
//   LOADERS   how many waves issue the global->LDS loads (0: all of them);
//             with half of the waves loading, each SIMD runs one wave that
//             never waits on the vector memory queue and keeps the matrix
//             core busy while its partner issues loads
//   MI        MFMA block: 32 (v_mfma_f32_32x32x16_f16) or 16
//             (v_mfma_f32_16x16x32_f16: half the work per instruction, the
//             same bytes of operands per flop from LDS)
template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int STAGES_, int OCC_, int LOADERS_ = 0,
          int MI_ = 32>
struct TileShape {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int WAVES = WAVES_M * WAVES_N, THREADS = WAVES * kWave;
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;  // wave sub-tile
    static constexpr int MI = MI_;                                 // MFMA block edge
    static constexpr int KPI = MI == 32 ? 16 : 32;                 // k per MFMA
    static constexpr int CPS = KPI / 8;                            // 16-byte k chunks per MFMA
    static constexpr int ACC = MI * MI / kWave;                    // accumulator floats per lane per block
    static constexpr int NG = ACC / 4;                             // groups of 4 consecutive columns
    using acc_t = typename AccBlock<MI>::type;
    static constexpr int FM = WTM / MI, FN = WTN / MI;            // MFMA blocks per wave
    static constexpr int KK = BK / KPI;                            // MFMA k sub-steps per step
    static constexpr int STAGES = STAGES_;
    static constexpr int OCC = OCC_;
    static constexpr int ROW_BYTES = BK * 2;
    static constexpr int CHUNKS = ROW_BYTES / 16;                  // 16-byte chunks per row
    // LDS serves 64 banks x 4 bytes = 256 bytes per cycle; a 16-byte read of
    // 16 lanes covers it exactly.  Rows that share a 256-byte line
    // (ROWS_PER_LINE of them) already sit on different banks, so the chunk
    // position is XOR-ed with the row's line index: the 16 rows read by 16
    // consecutive lanes at one logical chunk then hit 16 distinct bank groups.
    static constexpr int ROWS_PER_LINE = 256 / ROW_BYTES;
    static constexpr int SWZ_SHIFT = ROWS_PER_LINE == 2 ? 1 : 2;
    static constexpr int ROWS_PER_LOAD = 1024 / ROW_BYTES;         // rows per 1 KiB wave load
    static constexpr int A_BYTES = BM * ROW_BYTES, B_BYTES = BN * ROW_BYTES;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
    static constexpr int LOADERS = LOADERS_ == 0 ? WAVES : LOADERS_;
    static constexpr int A_LOADS = A_BYTES / 1024 / LOADERS;       // 1 KiB per wave load
    static constexpr int B_LOADS = B_BYTES / 1024 / LOADERS;
    static constexpr int LOADS = A_LOADS + B_LOADS;                // per loading wave per step
    static_assert(BK == 32 || BK == 64, "BK is 32 or 64");
    static_assert(ROWS_PER_LINE * CHUNKS == 16, "swizzle covers 16 lanes");
    static_assert(MI == 32 || MI == 16, "MFMA block is 32x32 or 16x16");
    static_assert(WTM % MI == 0 && WTN % MI == 0, "wave tile must be whole MFMA blocks");
    static_assert(LOADERS >= 1 && LOADERS <= WAVES, "loading waves are a subset of the waves");
    static_assert(A_LOADS * LOADERS * 1024 == A_BYTES, "A tile must split evenly over loading waves");
    static_assert(B_LOADS * LOADERS * 1024 == B_BYTES, "B tile must split evenly over loading waves");
    static_assert(LDS_BYTES <= 160 * 1024, "gfx950 has 160 KiB of LDS per workgroup");
    static_assert(STAGES >= 1 && LOADS * (STAGES - 2) <= 63, "vmcnt holds at most 63");
    static_assert(KK % 2 == 0, "two fragment sets alternate by k sub-step");
    static_assert(LOADS <= 4 * FM * FN, "at most 4 loads per MFMA");
};

// Scheduling group of n (0 .. 4, known after unrolling) vector memory
// instructions in sync group G.
template <int G>
__device__ __forceinline__ void sched_vmem(int n)
{
    if (n == 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, G);
    else if (n == 2) __builtin_amdgcn_sched_group_barrier(0x020, 2, G);
    else if (n == 3) __builtin_amdgcn_sched_group_barrier(0x020, 3, G);
    else if (n == 4) __builtin_amdgcn_sched_group_barrier(0x020, 4, G);
}

template <bool B>
struct Flag {
    static constexpr bool value = B;
};

template <int V>
struct Int {
    static constexpr int value = V;
};

template <class T>
__device__ __forceinline__ int swz(int row, int chunk)
{
    // 64-byte rows read by 16x16x32 MFMAs (lane l: row l % 16, chunk
    // l / 16): one LDS pass serves lanes {0-3, 12-15, 20-23, 24-27}, i.e.
    // rows 0-3 and 12-15 at chunk 0 with rows 4-11 at chunk 1 (and likewise
    // for the other passes), so the row-quad term must split quads {0, 3}
    // from {1, 2}: XOR with 2 * ((row / 8) % 2) does, the default XOR with
    // (row / 4) % 4 puts half of each pass on the same banks.
    if constexpr (T::CHUNKS == 4 && T::MI == 16) return chunk ^ (((row >> 3) & 1) << 1);
    return chunk ^ ((row >> T::SWZ_SHIFT) & (T::CHUNKS - 1));
}

// acc += b * a (v_mfma_f32_16x16x32_f16) with the accumulator held in AGPRs.
// The memory clobber keeps every LDS and global access on its side of the
// MFMA, so the source order of a loop built from these is its issue order.
__device__ __forceinline__ void mfma16_agpr(float4_t& acc, const half8_t& b, const half8_t& a)
{
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(b), "v"(a) : "memory");
}

// acc += b * a with the accumulator held in VGPRs instead (a ladder
// option of the persistent kernel: the epilogue then converts it without
// moving it out of AGPRs first).
__device__ __forceinline__ void mfma16_vgpr(float4_t& acc, const half8_t& b, const half8_t& a)
{
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(acc) : "v"(b), "v"(a) : "memory");
}

// Store mode of C, passed to the kernels as `c_vec`: which stores the rows
// allow (2: aligned 16-byte, 1: aligned 8-byte, 0: single elements).

// Epilogue: fp32 -> fp16 (round to nearest even) and store.  In each MFMA
// block lane l holds row cm (its row in the first block) and, in accumulator
// registers 4q .. 4q+3, the four consecutive columns cn + 8q .. cn + 8q + 3,
// written with one 8-byte store.  Rows past M and columns past N are not
// written.
template <class T>
__device__ __forceinline__ void epilogue(const typename T::acc_t (&acc)[T::FM][T::FN], _Float16* __restrict__ C,
                                         int M, int N, int cm, int cn, int c_vec)
{
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
        const int m = cm + i * T::MI;
        if (m >= M) continue;
        _Float16* crow = C + (size_t)m * N;
#pragma unroll
        for (int j = 0; j < T::FN; ++j) {
#pragma unroll
            for (int q = 0; q < T::NG; ++q) {
                const int n = cn + j * T::MI + 8 * q;
                half4_t h;
                h[0] = (_Float16)acc[i][j][4 * q + 0];
                h[1] = (_Float16)acc[i][j][4 * q + 1];
                h[2] = (_Float16)acc[i][j][4 * q + 2];
                h[3] = (_Float16)acc[i][j][4 * q + 3];
                if ((c_vec & 3) && n + 3 < N) {
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

// Epilogue through LDS, for C rows that take aligned 16-byte stores (N % 8
// == 0, C 16-byte aligned).  The ring is dead once the K loop has ended, and
// the whole BM x BN fp16 tile fits in it.  Each wave writes its accumulators
// (fp32 -> fp16, round to nearest even) into a row-major copy of the tile,
// then every wave reads back whole rows, 16 bytes per lane, and stores them:
// each store instruction covers complete rows of the tile, so C is written
// in full cache lines instead of the scattered 8-byte pieces each lane holds.
// In LDS, 16-byte chunk c of row r sits at position c ^ (r % SW), so the
// 8-byte writes of 32 rows at one column touch 16 bank groups (2-way at
// most) and the 16-byte row reads are conflict-free.
template <class T>
__device__ __forceinline__ void epilogue_lds(const typename T::acc_t (&acc)[T::FM][T::FN], _Float16* __restrict__ C,
                                             int M, int N, int m0, int n0, int wm, int wn, int lane, int wave,
                                             unsigned char* smem)
{
    constexpr int PITCH = T::BN * 2;              // bytes per tile row
    constexpr int CH = T::BN / 8;                  // 16-byte chunks per row
    constexpr int SW = CH >= 16 ? 15 : CH - 1;
    constexpr int RPL = 1024 / PITCH;              // rows per wave-wide 1 KiB read
    constexpr int ITERS = T::BM / RPL / T::WAVES;  // reads per wave
    static_assert(T::BM * PITCH <= T::LDS_BYTES, "the C tile fits in the ring");
    static_assert(RPL >= 1 && ITERS * RPL * T::WAVES == T::BM, "rows split evenly over waves");
    // the lane index recomputed and laundered: the offsets derived from it
    // are computed here, not early and kept (or spilled) through the K loop
    int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    asm volatile("" : "+v"(ln));
    (void)lane;
    const int fr_row = ln % T::MI, fr_hi = ln / T::MI;
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
        const int r = wm * T::WTM + i * T::MI + fr_row;
        unsigned char* lrow = smem + r * PITCH;
#pragma unroll
        for (int j = 0; j < T::FN; ++j) {
#pragma unroll
            for (int q = 0; q < T::NG; ++q) {
                const int col = wn * T::WTN + j * T::MI + 8 * q + 4 * fr_hi;
                half4_t h;
                h[0] = (_Float16)acc[i][j][4 * q + 0];
                h[1] = (_Float16)acc[i][j][4 * q + 1];
                h[2] = (_Float16)acc[i][j][4 * q + 2];
                h[3] = (_Float16)acc[i][j][4 * q + 3];
                *(half4_t*)(lrow + (((col >> 3) ^ (r & SW)) << 4) + (col & 4) * 2) = h;
            }
        }
    }
    __syncthreads();
    const int lr = ln / CH, lc = ln % CH;
    const int n = n0 + lc * 8;
    if (N <= (1 << 22)) {
        // Buffer stores with one 32-bit offset per store: rows past M fall
        // outside the buffer, columns past N get an offset outside it.  C is
        // never read back, so it goes out with the nontemporal hint (0.5-3%
        // faster on every shape measured, one wave of tiles or several).
        // The hint is an immediate of the buffer store; as a pointer store
        // under a runtime condition it was lost (the compiler merged it with
        // the plain store of the other branch).
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(C + (size_t)m0 * N, (uint32_t)min(T::BM, M - m0) * (uint32_t)N * 2u);
        const uint32_t vbase = n < N ? ((uint32_t)lr * (uint32_t)N + (uint32_t)n) * 2u : kOob;
#pragma unroll
        for (int it = 0; it < ITERS; ++it) {
            const int r = (wave * ITERS + it) * RPL + lr;
            const u32x4_t v = *(const u32x4_t*)(smem + r * PITCH + ((lc ^ (r & SW)) << 4));
            const uint32_t off = vbase + (uint32_t)((wave * ITERS + it) * RPL) * (uint32_t)N * 2u;
            __builtin_amdgcn_raw_buffer_store_b128(v, rc, off, 0, kPolicyNt);
        }
    } else {
#pragma unroll
        for (int it = 0; it < ITERS; ++it) {
            const int r = (wave * ITERS + it) * RPL + lr;
            const half8_t v = *(const half8_t*)(smem + r * PITCH + ((lc ^ (r & SW)) << 4));
            const int m = m0 + r;
            if (m < M && n < N) *(half8_t*)(C + (size_t)m * N + n) = v;
        }
    }
}

// Main MFMA kernel.  Requirements checked on the host: A and B 16-byte
// aligned, K % 8 == 0, K < 2^22, M, N < 2^31.  `c_vec` is the store mode:
// bits 0-1 say which stores C rows allow, 2 for aligned 16-byte stores (N %
// 8 == 0, C 16-byte aligned; the tile then leaves through LDS), 1 for
// aligned 8-byte stores (N % 4 == 0, C 8-byte aligned), 0 for single
// elements.
template <class T>
__global__ void __launch_bounds__(T::THREADS, T::OCC)
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

    // Global->LDS copy assignment.  Load j of loading wave w fills bytes
    // [g * 1024, g * 1024 + 1024) of the operand's tile in the stage,
    // g = w * LOADS + j, i.e. ROWS_PER_LOAD whole rows; lane l writes
    // position l % CHUNKS of row g * ROWS_PER_LOAD + l / CHUNKS, so it
    // fetches the logical chunk that the swizzle puts at that position.
    // Waves 0 .. LOADERS-1 load (waves are dealt to the four SIMDs in turn,
    // so with LOADERS = WAVES / 2 every SIMD hosts one loading wave).
    const bool loader = wave < T::LOADERS;
    const int lw = loader ? wave : 0;
    const int ld_r = lane / T::CHUNKS, ld_p = lane % T::CHUNKS;
    uint32_t a_voff[T::A_LOADS], b_voff[T::B_LOADS];
    int a_kc[T::A_LOADS], b_kc[T::B_LOADS];  // first k of the fetched chunk
#pragma unroll
    for (int j = 0; j < T::A_LOADS; ++j) {
        const int row = (lw * T::A_LOADS + j) * T::ROWS_PER_LOAD + ld_r;
        const int c = swz<T>(row, ld_p);
        a_voff[j] = (uint32_t)row * row_bytes + (uint32_t)c * 16u;
        a_kc[j] = c * 8;
    }
#pragma unroll
    for (int j = 0; j < T::B_LOADS; ++j) {
        const int row = (lw * T::B_LOADS + j) * T::ROWS_PER_LOAD + ld_r;
        const int c = swz<T>(row, ld_p);
        b_voff[j] = (uint32_t)row * row_bytes + (uint32_t)c * 16u;
        b_kc[j] = c * 8;
    }

    // Issues loads [first, first + count) of step `kstep` into `stage`
    // (A's loads first, then B's).  Steps past the end of K load zeros (every
    // chunk is out of range), so the ring can run without branches; those
    // stages are never read.
    auto issue_load_range = [&](int stage, int kstep, int first, int count) {
        const int k0 = kstep * T::BK;
        const int krem = K - k0;  // chunks starting at or past K read as zero
        const uint32_t soff = (uint32_t)k0 * 2u;
        unsigned char* a_dst = smem + stage * T::STAGE_BYTES + lw * T::A_LOADS * 1024;
        unsigned char* b_dst = smem + stage * T::STAGE_BYTES + T::A_BYTES + lw * T::B_LOADS * 1024;
#pragma unroll
        for (int l = first; l < first + count; ++l) {
            if (l < T::A_LOADS) {
                const uint32_t v = a_kc[l] < krem ? a_voff[l] : kOob;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t*)(a_dst + l * 1024), 16, v, soff,
                                                         0, 0);
            } else {
                const int j = l - T::A_LOADS;
                const uint32_t v = b_kc[j] < krem ? b_voff[j] : kOob;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_t*)(b_dst + j * 1024), 16, v, soff,
                                                         0, 0);
            }
        }
    };
    auto issue_loads = [&](int stage, int kstep) { issue_load_range(stage, kstep, 0, T::LOADS); };

    // Fragment reads: row (l % 32) of each 32-row block, logical chunk
    // 2 * kk + l / 32 for k sub-step kk (16 k values per MFMA).  Row offsets
    // within a block are multiples of 32, so the swizzle term depends only on
    // l % 32 and is the same for every block.
    const int fr_row = lane % T::MI;
    const int fr_hi = lane / T::MI;
    const int a_row0 = wm * T::WTM + fr_row;
    const int b_row0 = wn * T::WTN + fr_row;
    int fr_pos[T::KK];
#pragma unroll
    for (int kk = 0; kk < T::KK; ++kk) fr_pos[kk] = swz<T>(fr_row, T::CPS * kk + fr_hi) * 16;

    // Fragment registers: two sets alternate by k sub-step (sub-step kk
    // uses set kk % 2; KK is even), each read one sub-step before its MFMAs.
    half8_t fa[2][T::FM], fb[2][T::FN];
    typename T::acc_t acc[T::FM][T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
#pragma unroll
            for (int r = 0; r < T::ACC; ++r) acc[i][j][r] = 0.0f;

    auto read_frags = [&](const unsigned char* stage_base, int kk) {
        const unsigned char* pa = stage_base + a_row0 * T::ROW_BYTES + fr_pos[kk];
        const unsigned char* pb = stage_base + T::A_BYTES + b_row0 * T::ROW_BYTES + fr_pos[kk];
#pragma unroll
        for (int i = 0; i < T::FM; ++i) fa[kk & 1][i] = *(const half8_t*)(pa + i * T::MI * T::ROW_BYTES);
#pragma unroll
        for (int j = 0; j < T::FN; ++j) fb[kk & 1][j] = *(const half8_t*)(pb + j * T::MI * T::ROW_BYTES);
    };

    // When the accumulators fill all 256 AGPRs (one wave per SIMD, 16x16
    // blocks), MFMAs compiled from the builtin get their accumulators moved
    // between AGPRs and VGPRs inside the loop; asm MFMAs keep them in place.
    constexpr bool kAgprAcc = T::MI == 16 && T::OCC == 1 && T::FM * T::FN * T::ACC == 256;
    auto mma = [&](int kk) {
#pragma unroll
        for (int i = 0; i < T::FM; ++i)
#pragma unroll
            for (int j = 0; j < T::FN; ++j)
                if constexpr (T::MI == 32)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[kk & 1][j], fa[kk & 1][i], acc[i][j], 0, 0, 0);
                else if constexpr (kAgprAcc)
                    mfma16_agpr(acc[i][j], fb[kk & 1][j], fa[kk & 1][i]);
                else
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fb[kk & 1][j], fa[kk & 1][i], acc[i][j], 0, 0, 0);
    };

    const int nk = (K + T::BK - 1) / T::BK;

    // STAGES-deep ring.  Step ks lives in stage ks % STAGES; its loads are
    // issued STAGES - 1 steps earlier.  Before step ks + 1 is read, each wave
    // waits until its own loads of that step have landed (vmcnt: only the
    // loads of the STAGES - 2 later steps may still be outstanding) and a
    // barrier makes all waves' loads visible; since every wave has also
    // finished its LDS reads of step ks by then (lgkmcnt(0) before the
    // barrier), step ks's stage is free after it and is refilled with step
    // ks + STAGES.
    //
    // Fragments of sub-step kk are read one sub-step before its MFMAs, so a
    // step splits at the barrier (pinned with scheduling-group barriers, so
    // the matrix core always has independent work queued):
    //   before:  sub-steps 0 .. KK-2: fragment reads of sub-step kk+1, then
    //            the FM*FN MFMAs of sub-step kk;
    //   after:   sub-step KK-1: fragment reads of the next step's sub-step
    //            0, then its MFMAs, with the step's loads spread between them.
    //
    // The loop is compiled twice: for loading waves and, when only some
    // waves load, for the others (no loads, and nothing in flight at the
    // barriers).
    auto main_loop = [&](auto tag) {
        constexpr bool LD = decltype(tag)::value;
        if constexpr (T::STAGES == 1) {
            // One stage, nothing overlaps: load a step, wait until every
            // wave's loads have landed, compute it, and wait until every wave
            // is done reading before the next step's loads overwrite it (the
            // first kernel of "0. A Minimal Hopper Matmul": the copy runs,
            // then everyone waits).  A ladder rung only.
            for (int ks = 0; ks < nk; ++ks) {
                if constexpr (LD) issue_loads(0, ks);
                lds_barrier<0>();
#pragma unroll
                for (int kk = 0; kk < T::KK; ++kk) {
                    read_frags(smem, kk);
                    mma(kk);
                }
                lds_barrier<0>();
            }
        } else {
            // every stage is free at the start: fill them all, then wait for
            // step 0 only
#pragma unroll
            for (int s = 0; s < T::STAGES; ++s)
                if constexpr (LD) issue_loads(s, s);
            lds_barrier<T::LOADS * (T::STAGES - 1)>();
            read_frags(smem, 0);

            int cur = 0;  // stage of step ks
            auto step = [&](int ks) {
                constexpr int G = T::FM * T::FN;  // MFMAs per sub-step
                const unsigned char* base = smem + cur * T::STAGE_BYTES;
                const int nxt = cur + 1 == T::STAGES ? 0 : cur + 1;
                // Each sub-step is its own scheduling region (fenced with
                // sched_barrier), so MFMAs of different sub-steps never
                // interleave into back-to-back dependent pairs.
#pragma unroll
                for (int kk = 0; kk < T::KK - 1; ++kk) {
                    read_frags(base, kk + 1);
                    mma(kk);
                    __builtin_amdgcn_sched_group_barrier(0x100, T::FM + T::FN, 0);  // DS reads
#pragma unroll
                    for (int i = 0; i < G; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                    __builtin_amdgcn_sched_barrier(0);
                }
                lds_barrier<T::LOADS * (T::STAGES - 2)>();
                __builtin_amdgcn_sched_barrier(0);
                constexpr int L = LD ? T::LOADS : 0;
                read_frags(smem + nxt * T::STAGE_BYTES, 0);
                mma(T::KK - 1);
                if constexpr (L > 0) issue_load_range(cur, ks + T::STAGES, 0, L);
                __builtin_amdgcn_sched_group_barrier(0x100, T::FM + T::FN, 1);  // DS reads
#pragma unroll
                for (int i = 0; i < G; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);  // one MFMA
                    sched_vmem<1>(L * (i + 1) / G - L * i / G);        // loads
                }
                __builtin_amdgcn_sched_barrier(0);
                cur = nxt;
            };
            for (int ks = 0; ks < nk; ++ks) step(ks);
        }
    };
    if (nk > 0) {
        if (T::LOADERS == T::WAVES || loader)
            main_loop(Flag<true>{});
        else
            main_loop(Flag<false>{});
        // no global->LDS load may still be writing when the workgroup ends
        // (nor when the ring is reused for the epilogue below)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        // asm MFMAs are opaque to the compiler's hazard checks: let the last
        // ones write their accumulators before they are read
        if constexpr (kAgprAcc) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    }

    // Small tiles (64 x 64) keep the direct stores: their epilogue is short
    // and the two extra barriers cost more than the wider stores save.
    if (T::BM * T::BN >= 128 * 128 && (c_vec & 3) == 2) {
        __syncthreads();  // every wave is done with the ring
        epilogue_lds<T>(acc, C, M, N, m0, n0, wm, wn, lane, wave, smem);
    } else {
        epilogue<T>(acc, C, M, N, m0 + wm * T::WTM + fr_row, n0 + wn * T::WTN + 4 * fr_hi, c_vec);
    }
}

// Every instruction of the K loop in a fixed order.
//
// Four or eight waves (one or two per SIMD) each own a sub-tile of C (for
// 256 x 256 with 8 waves: 128 x 64, i.e. 8 x 4 blocks of 16 x 16 and 128
// accumulator floats per lane in AGPRs); waves 0 .. LOADERS-1 issue the
// global->LDS loads.  Nothing is bunched, so no wave stalls for long.  A
// BK = 64 step is two sub-steps of 32 k (FM x FN MFMAs each):
//   sub-step 0: its MFMAs, and after every RS-th of them one fragment read
//               of sub-step 1;
//   barrier:    this wave's loads of step ks + 1 have landed (vmcnt), its
//               reads of sub-step 1 have returned; every wave is done with
//               this step's operand tiles;
//   sub-step 1: its MFMAs, with one fragment read of the next step's
//               sub-step 0 after every RS-th, and this wave's loads after
//               every LS-th, starting half-way into the first.
// LDS is either a ring of STAGES stages (A and B tiles of one step each;
// sub-step 1 loads step ks + STAGES into the stage step ks leaves) or, with
// SLOTS5, five slots of one operand tile each (A_j in slot 2j mod 5, B_j in
// slot 2j + 1 mod 5, 160 KiB for 256 x 256): then sub-step 0 loads A_{j+2}
// into the slot B_{j-1} left and sub-step 1 loads B_{j+2} into the slot A_j
// leaves, so the loads are spread over the whole step and the A tiles get
// half a step more time to land (8192^3: +2%, 5000 x 3000 x 6000: +8%
// over the 2-stage ring).
// The MFMAs are asm statements (mfma16_agpr), which keeps the accumulators
// in place: compiled from the builtin, a kernel whose accumulators fill all
// 256 AGPRs moves them between AGPRs and VGPRs inside the loop (1.3 copies
// per MFMA).  The fragments are read in the order the MFMAs first need them
// (A block 0, B blocks 0 .. FN-1, A blocks 1 .. FM-1), so the compiler's
// lgkmcnt waits before each MFMA only cover reads issued long before.  Loads
// of steps that lie wholly inside K skip the per-lane K check.
template <class T, int RS, int LS, bool SLOTS5 = false>
__global__ void __launch_bounds__(T::THREADS, 1)
gemm_nt_f16_ordered(const _Float16* __restrict__ A, const _Float16* __restrict__ B,
                    _Float16* __restrict__ C, int M, int N, int K, int tiles_m, int tiles_n,
                    int group_m, int c_vec)
{
    static_assert(T::MI == 16 && T::KK == 2 && (T::WAVES == 4 || T::WAVES == 8),
                  "16x16x32 MFMAs, two sub-steps per step, one or two waves per SIMD");
    constexpr int S = T::STAGES;
    constexpr int G = T::FM * T::FN;  // MFMAs per sub-step
    constexpr int R = T::FM + T::FN;  // fragment reads per sub-step
    constexpr int LOADS_SUB = SLOTS5 ? T::A_LOADS : T::LOADS;  // loads per loading sub-step
    static_assert(RS * (R - 1) < G && LS * (LOADS_SUB - 1) + LS / 2 < G, "reads and loads fit in a sub-step");
    constexpr int SLOT = T::A_BYTES;  // SLOTS5: one operand tile of one step
    static_assert(!SLOTS5 || (T::A_BYTES == T::B_BYTES && 5 * SLOT <= 160 * 1024 && 5 * SLOT >= T::LDS_BYTES),
                  "five equal slots, at least as much LDS as the ring");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[SLOTS5 ? 5 * SLOT : T::LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wave / T::WAVES_N, wn = wave % T::WAVES_N;

    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * T::BM, n0 = tn * T::BN;
    const int rows_a = min(T::BM, M - m0), rows_b = min(T::BN, N - n0);
    const uint32_t row_bytes = (uint32_t)K * 2u;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + (size_t)m0 * K, (uint32_t)rows_a * row_bytes);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + (size_t)n0 * K, (uint32_t)rows_b * row_bytes);

    // Waves 0 .. LOADERS-1 load.  Load l < A_LOADS of loading wave lw fills
    // KiB (lw * A_LOADS + l) of the stage's A tile, the others KiB (lw *
    // B_LOADS + l - A_LOADS) of its B tile; lane placement and swizzle as in
    // gemm_nt_f16_mfma.
    const int lw = wave < T::LOADERS ? wave : 0;
    const int ld_r = lane / T::CHUNKS, ld_p = lane % T::CHUNKS;
    uint32_t voff[T::LOADS];
    int kc[T::LOADS];  // first k of the fetched chunk
#pragma unroll
    for (int l = 0; l < T::LOADS; ++l) {
        const bool is_a = l < T::A_LOADS;
        const int row = (lw * (is_a ? T::A_LOADS : T::B_LOADS) + (is_a ? l : l - T::A_LOADS)) * T::ROWS_PER_LOAD +
                        ld_r;
        const int c = swz<T>(row, ld_p);
        voff[l] = (uint32_t)row * row_bytes + (uint32_t)c * 16u;
        kc[l] = c * 8;
    }
    // Load l of step kstep into stage `where` (SLOTS5: into slot `where`,
    // which holds the load's operand tile).  MASKED: the step may reach
    // past K (chunks at or past K read as zero).
    auto issue_load = [&](int where, int kstep, int l, auto masked) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked)::value;
        const int k0 = kstep * T::BK;
        const uint32_t v = (!MASKED || kc[l] < K - k0) ? voff[l] : kOob;
        const uint32_t soff = (uint32_t)k0 * 2u;
        unsigned char* a_tile = smem + where * (SLOTS5 ? SLOT : T::STAGE_BYTES);
        unsigned char* b_tile = SLOTS5 ? a_tile : a_tile + T::A_BYTES;
        if (l < T::A_LOADS)  // (a buffer resource cannot be the result of ?:)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t*)(a_tile + (lw * T::A_LOADS + l) * 1024), 16,
                                                     v, soff, 0, 0);
        else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rb, (lds_void_t*)(b_tile + (lw * T::B_LOADS + l - T::A_LOADS) * 1024), 16, v, soff, 0, 0);
    };

    const int fr_row = lane % T::MI;
    const int fr_hi = lane / T::MI;
    const int a_row0 = wm * T::WTM + fr_row;
    const int b_row0 = wn * T::WTN + fr_row;
    int fr_pos[T::KK];
#pragma unroll
    for (int kk = 0; kk < T::KK; ++kk) fr_pos[kk] = swz<T>(fr_row, T::CPS * kk + fr_hi) * 16;

    // Fragment set kk holds sub-step kk of the current step.
    half8_t fa[2][T::FM], fb[2][T::FN];
    typename T::acc_t acc[T::FM][T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
#pragma unroll
            for (int r = 0; r < T::ACC; ++r) acc[i][j][r] = 0.0f;

    // fragment read `idx` of sub-step `set` from A tile at abase, B tile at bbase
    auto read_one = [&](int set, const unsigned char* abase, const unsigned char* bbase, int idx)
                        __attribute__((always_inline)) {
        const unsigned char* pa = abase + a_row0 * T::ROW_BYTES + fr_pos[set];
        const unsigned char* pb = bbase + b_row0 * T::ROW_BYTES + fr_pos[set];
        if (idx == 0)
            fa[set][0] = *(const half8_t*)pa;
        else if (idx <= T::FN)
            fb[set][idx - 1] = *(const half8_t*)(pb + (idx - 1) * T::MI * T::ROW_BYTES);
        else
            fa[set][idx - T::FN] = *(const half8_t*)(pa + (idx - T::FN) * T::MI * T::ROW_BYTES);
    };
    // MFMAs of sub-step `cs`, along the rows of blocks and back (block row
    // i = t / FN; column j = t % FN on even rows, FN - 1 - t % FN on odd
    // ones), so consecutive MFMAs always share a fragment: 0.1-0.7% faster
    // than starting every row at column 0, in alternating replays on six
    // shapes (the clock is power-limited, and an operand that does not
    // change costs less), with the reads of sub-step 1 - cs from (ra_base,
    // rb_base) and, if LD, loads [l0, l0 + LOADS_SUB) of step `lstep` into
    // `where` interleaved.
    auto substep = [&](int cs, const unsigned char* ra_base, const unsigned char* rb_base, auto ld, int where,
                       int lstep, int l0, auto masked) __attribute__((always_inline)) {
        constexpr bool LD = decltype(ld)::value;
#pragma unroll
        for (int t = 0; t < G; ++t) {
            const int i = t / T::FN, j = (i & 1) ? T::FN - 1 - t % T::FN : t % T::FN;
            mfma16_agpr(acc[i][j], fb[cs][j], fa[cs][i]);
            if (t % RS == 0 && t / RS < R) read_one(1 - cs, ra_base, rb_base, t / RS);
            if constexpr (LD)
                if (t % LS == LS / 2 && t / LS < LOADS_SUB) issue_load(where, lstep, l0 + t / LS, masked);
        }
    };

    const int nk = (K + T::BK - 1) / T::BK;
    // The K loop, compiled once for loading waves and, when only some waves
    // load, once for the others.
    auto run = [&](auto ldtag) __attribute__((always_inline)) {
        constexpr bool LD = decltype(ldtag)::value;
        const int nfull = K / T::BK;  // steps that lie wholly inside K
        if constexpr (SLOTS5) {
            // steps 0 and 1 into slots 0 .. 3, then wait for step 0 only
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int l = 0; l < T::LOADS; ++l)
                    if constexpr (LD) issue_load(l < T::A_LOADS ? 2 * s : 2 * s + 1, s, l, Flag<true>{});
            lds_barrier<T::LOADS>();
#pragma unroll
            for (int idx = 0; idx < R; ++idx) read_one(0, smem, smem + SLOT, idx);
            int sa = 0;  // slot of A_j; B_j, A_{j+1}, B_{j+1}, A_{j+2} follow
            auto slot = [&](int i) __attribute__((always_inline)) {
                return smem + (sa + i >= 5 ? sa + i - 5 : sa + i) * SLOT;
            };
            auto step = [&](int ks, auto masked) __attribute__((always_inline)) {
                const int a2 = sa + 4 >= 5 ? sa - 1 : sa + 4;
                substep(0, slot(0), slot(1), Flag<LD>{}, a2, ks + 2, 0, masked);
                // A_{j+1} and B_{j+1} have landed; only A_{j+2} may be in flight
                lds_barrier<T::A_LOADS>();
                // steps past the end of K load zeros into slots never read
                substep(1, slot(2), slot(3), Flag<LD>{}, sa, ks + 2, T::A_LOADS, masked);
                sa = sa + 2 >= 5 ? sa - 3 : sa + 2;
            };
            int ks = 0;
            for (; ks < nk && ks + 2 < nfull; ++ks) step(ks, Flag<false>{});
            for (; ks < nk; ++ks) step(ks, Flag<true>{});
        } else {
            // every stage is free at the start: fill them all, then wait for
            // step 0 only
#pragma unroll
            for (int s = 0; s < S; ++s)
#pragma unroll
                for (int l = 0; l < T::LOADS; ++l)
                    if constexpr (LD) issue_load(s, s, l, Flag<true>{});
            lds_barrier<T::LOADS * (S - 1)>();
#pragma unroll
            for (int idx = 0; idx < R; ++idx) read_one(0, smem, smem + T::A_BYTES, idx);
            int cur = 0;  // stage of step ks
            auto step = [&](int ks, auto masked) __attribute__((always_inline)) {
                const int nxt = cur + 1 == S ? 0 : cur + 1;
                unsigned char* base = smem + cur * T::STAGE_BYTES;
                unsigned char* next = smem + nxt * T::STAGE_BYTES;
                substep(0, base, base + T::A_BYTES, Flag<false>{}, 0, 0, 0, masked);
                lds_barrier<T::LOADS * (S - 2)>();
                // steps past the end of K load zeros into stages never read
                substep(1, next, next + T::A_BYTES, Flag<LD>{}, cur, ks + S, 0, masked);
                cur = nxt;
            };
            int ks = 0;
            for (; ks < nk && ks + S < nfull; ++ks) step(ks, Flag<false>{});
            for (; ks < nk; ++ks) step(ks, Flag<true>{});
        }
    };
    if (nk > 0) {
        if (T::LOADERS == T::WAVES || wave < T::LOADERS)
            run(Flag<true>{});
        else
            run(Flag<false>{});
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        // The compiler cannot see that the asm statements are MFMAs: give
        // the last ones time to write their accumulators before they are
        // read (the longest MFMA-write to read hazard is under 24 wait
        // states).
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    }

    if ((c_vec & 3) == 2) {
        __syncthreads();  // every wave is done with the ring
        epilogue_lds<T>(acc, C, M, N, m0, n0, wm, wn, lane, wave, smem);
    } else {
        epilogue<T>(acc, C, M, N, m0 + wm * T::WTM + fr_row, n0 + wn * T::WTN + 4 * fr_hi, c_vec);
    }
}

// Persistent form of the 5-slot kernel above.  One workgroup per compute
// unit runs tiles b, b + G, b + 2G, ... (G = grid size, in the tile order of
// tile_coords).  What a tile costs beyond its K loop is the pipeline's fill
// and drain and the epilogue ("6. Four Consumers, FP16 Accumulation, and a
// TMA Epilogue", opening paragraph); here the load stream runs on across
// tiles: the last two steps of a tile load the first two steps of the next,
// so only the epilogue and one round of fragment reads stand between two
// tiles.  It stages C through the two slots the last
// step leaves free, in two rounds of 128 rows (the pages stage a 256 x 256
// tile through a quarter-sized buffer in turns, section "Serialized
// Shared-Memory Epilogue").  All waves write their rows; only the four
// waves that never load read them back and store them.  A loading wave's
// barrier waits on its vmcnt, which would also wait for any store it had
// issued; the non-loading waves never wait on theirs, so the stores drain
// while the next tile computes.  Host side: K > 64 (two steps at least),
// C rows allow aligned 16-byte stores.  With DIRECT (a ladder rung only) the
// LDS staging is skipped: every wave stores its own accumulators as 8-byte
// pieces, four consecutive columns of one row per lane, the way "6. Four
// Consumers, FP16 Accumulation, and a TMA Epilogue" ("Serialized
// Shared-Memory Epilogue") describes stores straight from registers.
// Two more options, FLAGS bits for the ladder: kVgprAcc keeps the
// accumulators in VGPRs, kColumns walks every column of MFMA blocks top to
// bottom instead of every second one bottom to top.  kSharedM0: groups of
// four global->LDS loads share one LDS base (M0), the pieces placed by the
// instruction offset; every load that needs a new M0 value costs the wave
// several issue cycles.
// kLean (four waves only) strips the scalar and vector arithmetic out of the
// steps that load whole K ranges.  With one wave per SIMD nothing hides that
// arithmetic: between two MFMAs (16 cycles of the matrix core) a lone wave
// issues one scalar or two vector instructions for free, and each further
// one delays the next MFMA by about 8 cycles (scalar) or 5 (vector), as
// measured with a probe loop of independent MFMAs.  Such steps run as a
// cycle of five, one per position of the slot ring, so every slot offset is
// a constant; the fragment reads use per-lane base addresses kept in
// registers (three copies 64 KiB apart, so that every offset fits the read's
// 16-bit immediate), the loads keep their per-lane offsets in registers and
// share M0 in groups of four, and the K position advances in one scalar
// register.  Steps past the end of K, the two steps that start the next
// tile, and up to four steps before a tile's first cycle and after its last
// keep the general form (the ring position in a register).
constexpr int kDirect = 1, kVgprAcc = 2, kColumns = 4, kSharedM0 = 8, kLean = 16;
template <class T, int RS, int LS, int FLAGS = 0>
__global__ void __launch_bounds__(T::THREADS, 1)
gemm_nt_f16_ordered_persist(const _Float16* __restrict__ A, const _Float16* __restrict__ B,
                            _Float16* __restrict__ C, int M, int N, int K, int tiles_m, int tiles_n,
                            int group_m)
{
    static_assert(T::MI == 16 && T::KK == 2 && T::LOADERS == 4 &&
                      (T::WAVES == 8 || T::WAVES == 4) && T::WAVES_M == 2 && T::NG == 1,
                  "16x16x32 MFMAs, two sub-steps per step, 2 x 4 waves of which 4 load, or 2 x 2 "
                  "waves that all load");
    // with eight waves the four that never load store C; with four, all do
    constexpr bool ALL_STORE = T::WAVES == T::LOADERS;
    constexpr bool DIRECT = FLAGS & kDirect, VACC = FLAGS & kVgprAcc, SNAKE = !(FLAGS & kColumns),
                   SHARED_M0 = FLAGS & kSharedM0, LEAN = FLAGS & kLean;
    static_assert(!LEAN || (ALL_STORE && !DIRECT && !VACC && T::A_LOADS == 8 && T::B_LOADS == 8 &&
                            T::A_BYTES == 32768 && T::KK == 2),
                  "the lean steps: four waves, 32 KiB slots, 8 + 8 loads per wave and step");
    static_assert(!SHARED_M0 || (T::A_LOADS % 4 == 0 && T::B_LOADS % 4 == 0),
                  "loads come in groups of four pieces");
    constexpr int G = T::FM * T::FN;  // MFMAs per sub-step
    constexpr int R = T::FM + T::FN;  // fragment reads per sub-step
    constexpr int SLOT = T::A_BYTES;  // one operand tile of one step
    static_assert(T::A_BYTES == T::B_BYTES && 5 * SLOT <= 160 * 1024, "five equal slots");
    static_assert(RS * (R - 1) < G && LS * (T::A_LOADS - 1) + LS / 2 < G, "reads and loads fit in a sub-step");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[5 * SLOT];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wave / T::WAVES_N, wn = wave % T::WAVES_N;
    const int total = tiles_m * tiles_n;
    const uint32_t row_bytes = (uint32_t)K * 2u;
    const int nk = (K + T::BK - 1) / T::BK;
    const int nfull = K / T::BK;  // steps that lie wholly inside K

    // Load assignment as in gemm_nt_f16_ordered: load l of loading wave lw
    // fills rows g * ROWS_PER_LOAD .. + ROWS_PER_LOAD - 1 of its operand tile
    // (g = lw * A_LOADS + l for A, lw * B_LOADS + l - A_LOADS for B).  The
    // swizzle repeats every two such row groups and g has the parity of l,
    // so a lane's offset within its group and the chunk it fetches take two
    // values, by the parity of l (two registers each instead of one per load).
    static_assert((T::CHUNKS << T::SWZ_SHIFT) == 2 * T::ROWS_PER_LOAD && T::A_LOADS % 2 == 0 &&
                      T::B_LOADS % 2 == 0,
                  "the swizzle repeats every two row groups of a load");
    const int lw = wave < T::LOADERS ? wave : 0;
    const int ld_r = lane / T::CHUNKS, ld_p = lane % T::CHUNKS;
    uint32_t vpar[2];
    int kpar[2];  // first k of the fetched chunk
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int c = swz<T>(p * T::ROWS_PER_LOAD + ld_r, ld_p);
        vpar[p] = (uint32_t)ld_r * row_bytes + (uint32_t)c * 16u;
        kpar[p] = c * 8;
    }

    // The tile being loaded (la, lb: its operand buffers, rows past M or N
    // read as zero) runs up to one tile ahead of the tile being computed.
    int tile = blockIdx.x;
    if (tile >= total) return;  // (the host launches at most one workgroup per tile)
    int tm, tn;
    tile_coords(tile, tiles_m, tiles_n, group_m, tm, tn);
    int m0 = tm * T::BM, n0 = tn * T::BN;
    __amdgpu_buffer_rsrc_t la = make_rsrc(A + (size_t)m0 * K, (uint32_t)min(T::BM, M - m0) * row_bytes);
    __amdgpu_buffer_rsrc_t lb = make_rsrc(B + (size_t)n0 * K, (uint32_t)min(T::BN, N - n0) * row_bytes);

    // Load l of step kstep of the loading tile into slot `where`.
    // (rbytes: row_bytes, laundered by the caller so that the 16 offsets
    // are computed where they are used, not kept in registers)
    auto issue_load = [&](int where, int kstep, int l, auto masked, uint32_t rbytes) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked)::value;
        const int k0 = kstep * T::BK;
        const int g = l < T::A_LOADS ? lw * T::A_LOADS + l : lw * T::B_LOADS + l - T::A_LOADS;
        const uint32_t off = (uint32_t)(g * T::ROWS_PER_LOAD) * rbytes + vpar[l & 1];
        const uint32_t v = (!MASKED || kpar[l & 1] < K - k0) ? off : kOob;
        const uint32_t soff = (uint32_t)k0 * 2u;
        if constexpr (SHARED_M0) {
            // Load r = g % 4 of a group of four consecutive 1 KiB pieces: the
            // LDS destination is the group's first piece (one M0 value for all
            // four) plus the instruction offset r KiB, which the hardware also
            // adds to the global offset, so the VGPR offset gives it back.
            // No wrap: the row offset of piece g >= r is at least g * 8 rows
            // * 2K bytes >= r KiB for K >= 64 (this kernel runs K > 64), and
            // the out-of-range sentinel stays past every tile's buffer.
            const int r = g & 3;
            lds_void_t* dst = (lds_void_t*)(smem + where * SLOT + (g - r) * 1024);
            const uint32_t vr = v - (uint32_t)r * 1024u;
            auto load = [&](__amdgpu_buffer_rsrc_t rs) __attribute__((always_inline)) {
                switch (r) {  // (the instruction offset must be a constant)
                    case 0: __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, vr, soff, 0, 0); break;
                    case 1: __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, vr, soff, 1024, 0); break;
                    case 2: __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, vr, soff, 2048, 0); break;
                    default: __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, vr, soff, 3072, 0); break;
                }
            };
            if (l < T::A_LOADS)  // (a buffer resource cannot be the result of ?:)
                load(la);
            else
                load(lb);
        } else {
            unsigned char* dst = smem + where * SLOT + g * 1024;
            if (l < T::A_LOADS)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(la, (lds_void_t*)dst, 16, v, soff, 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(lb, (lds_void_t*)dst, 16, v, soff, 0, 0);
        }
    };

    const int fr_row = lane % T::MI;
    const int fr_hi = lane / T::MI;
    const int a_row0 = wm * T::WTM + fr_row;
    const int b_row0 = wn * T::WTN + fr_row;
    int fr_pos[T::KK];
#pragma unroll
    for (int kk = 0; kk < T::KK; ++kk) fr_pos[kk] = swz<T>(fr_row, T::CPS * kk + fr_hi) * 16;

    // LEAN: rdb[c][x][kk] is this lane's LDS address of operand x's (A, B)
    // fragment rows at k-half kk, plus c * 64 KiB (slots 2c and 2c + 1 are
    // reached with an immediate of 0 or 32 KiB); lvo[l] the VGPR offset of
    // load l of this wave (A and B loads l and l + 8 fill the same rows of
    // their tiles), less the instruction offset that places it within its
    // group of four (see issue_load).
    uint32_t rdb[LEAN ? 3 : 1][2][T::KK];
    uint32_t lvo[LEAN ? 8 : 1];
    if constexpr (LEAN) {
#pragma unroll
        for (int c = 0; c < 3; ++c)
#pragma unroll
            for (int kk = 0; kk < T::KK; ++kk) {
                rdb[c][0][kk] = (uint32_t)(c * 65536 + a_row0 * T::ROW_BYTES + fr_pos[kk]);
                rdb[c][1][kk] = (uint32_t)(c * 65536 + b_row0 * T::ROW_BYTES + fr_pos[kk]);
                asm volatile("" : "+v"(rdb[c][0][kk]), "+v"(rdb[c][1][kk]));
            }
#pragma unroll
        for (int l = 0; l < 8; ++l) {
            lvo[l] = (uint32_t)((lw * 8 + l) * T::ROWS_PER_LOAD) * row_bytes + vpar[l & 1] - (uint32_t)(l & 3) * 1024u;
            asm volatile("" : "+v"(lvo[l]));
        }
    }

    half8_t fa[2][T::FM], fb[2][T::FN];
    typename T::acc_t acc[T::FM][T::FN];
    // Accumulators are cleared in place by an MFMA of zero fragments with an
    // inline zero as its C input: once at the start, and then block by block
    // in each epilogue, right after the block has been read out, so the
    // clearing MFMAs run on the matrix core while the wave converts and
    // stores the rest of the tile.  (Plain writes could be moved next to the
    // first accumulating MFMA, whose asm hides the VALU-to-MFMA hazard from
    // the compiler; pinning them in AGPRs with asm operands makes the
    // register allocator spill.)  The zero fragment is written by VALU moves,
    // which an MFMA may read only a few wait states later; the asm statement
    // it passes through waits that long, once.
    auto zero_frag = [&]() __attribute__((always_inline)) {
        half8_t z = {};
        asm volatile("s_nop 4" : "+v"(z));
        return z;
    };
    auto clear = [&](int i, int j, const half8_t& z) __attribute__((always_inline)) {
        if constexpr (VACC)
            asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %1, 0" : "=v"(acc[i][j]) : "v"(z) : "memory");
        else
            asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %1, 0" : "=a"(acc[i][j]) : "v"(z) : "memory");
    };

    // fragment read `idx` of set `set`, in the order the MFMAs below first
    // need them: B block 0, A blocks 0 .. FM-1, B blocks 1 .. FN-1
    auto read_one = [&](int set, const unsigned char* abase, const unsigned char* bbase, int idx)
                        __attribute__((always_inline)) {
        const unsigned char* pa = abase + a_row0 * T::ROW_BYTES + fr_pos[set];
        const unsigned char* pb = bbase + b_row0 * T::ROW_BYTES + fr_pos[set];
        if (idx == 0)
            fb[set][0] = *(const half8_t*)pb;
        else if (idx <= T::FM)
            fa[set][idx - 1] = *(const half8_t*)(pa + (idx - 1) * T::MI * T::ROW_BYTES);
        else
            fb[set][idx - T::FM] = *(const half8_t*)(pb + (idx - T::FM) * T::MI * T::ROW_BYTES);
    };
    // MFMAs of sub-step cs, with (if RD) the fragment reads of sub-step 1 -
    // cs and (if LD) loads l0 .. l0 + A_LOADS - 1 of step lstep interleaved.
    // The MFMAs go down the columns of blocks (column j = t / FM) and, unless
    // kColumns, back up every second one (block row i = t % FM, or FM - 1 -
    // t % FM on odd columns): each run of FM shares one B fragment, and the
    // turn at the end of a column keeps the A fragment.  Columns ran 0.3-1.1%
    // faster than rows (runs of FN sharing an A fragment), and the turns
    // another 0.4-0.5%, in alternating replays at 8192^3, 4096^3 and 4096 x
    // 4096 x 16384: the clock is power-limited, and an operand that does not
    // change between MFMAs costs less.
    auto substep = [&](int cs, const unsigned char* ra_base, const unsigned char* rb_base, auto ld, int where,
                       int lstep, int l0, auto masked, auto rd) __attribute__((always_inline)) {
        constexpr bool LD = decltype(ld)::value, RD = decltype(rd)::value;
        uint32_t rbytes = row_bytes;
        asm volatile("" : "+s"(rbytes));
#pragma unroll
        for (int t = 0; t < G; ++t) {
            const int j = t / T::FM, i = SNAKE && (j & 1) ? T::FM - 1 - t % T::FM : t % T::FM;
            if constexpr (VACC)
                mfma16_vgpr(acc[i][j], fb[cs][j], fa[cs][i]);
            else
                mfma16_agpr(acc[i][j], fb[cs][j], fa[cs][i]);
            if constexpr (RD)
                if (t % RS == 0 && t / RS < R) read_one(1 - cs, ra_base, rb_base, t / RS);
            if constexpr (LD)
                if (t % LS == LS / 2 && t / LS < T::A_LOADS) issue_load(where, lstep, l0 + t / LS, masked, rbytes);
        }
    };

    // LEAN steps.  Fragment read idx of set `set` from the A tile in slot SA
    // and the B tile in slot SB: B fragments 0 .. FN - 1, then A fragments
    // FM - 1 .. 0, the order in which the other set's MFMAs (down the
    // columns, the last column bottom to top) last used their registers.
    // (All of them are read in the first part of the sub-step and used in
    // the next one, so the order does not delay any MFMA; it was 0.1-0.3%
    // faster than read_one's order.)
    auto read_fast = [&](auto sa_c, auto sb_c, int set, int idx) __attribute__((always_inline)) {
        constexpr int SA = decltype(sa_c)::value, SB = decltype(sb_c)::value;
        if (idx < T::FN)
            fb[set][idx] = *(const half8_t*)(smem + rdb[SB / 2][1][set] + (SB % 2) * SLOT +
                                             idx * T::MI * T::ROW_BYTES);
        else
            fa[set][R - 1 - idx] = *(const half8_t*)(smem + rdb[SA / 2][0][set] + (SA % 2) * SLOT +
                                                     (R - 1 - idx) * T::MI * T::ROW_BYTES);
    };
    // Load l (0-7: A, 8-15: B) of the step whose K range starts soff bytes
    // into each row, into slot WHERE: piece lw * 8 + (l & 7) of the tile, in
    // groups of four sharing M0 (base of the group) with the instruction
    // offset (l & 3) KiB.
    int lw_bytes = __builtin_amdgcn_readfirstlane(lw * 8 * 1024);
    auto load_fast = [&](auto where_c, int l, uint32_t soff) __attribute__((always_inline)) {
        constexpr int WHERE = decltype(where_c)::value;
        lds_void_t* dst = (lds_void_t*)(smem + WHERE * SLOT + lw_bytes + (l & 4) * 1024);
        const uint32_t vo = lvo[l & 7];
        auto load = [&](__amdgpu_buffer_rsrc_t rs) __attribute__((always_inline)) {
            switch (l & 3) {  // (the instruction offset must be a constant)
                case 0: __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, vo, soff, 0, 0); break;
                case 1: __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, vo, soff, 1024, 0); break;
                case 2: __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, vo, soff, 2048, 0); break;
                default: __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, vo, soff, 3072, 0); break;
            }
        };
        if (l < 8)  // (a buffer resource cannot be the result of ?:)
            load(la);
        else
            load(lb);
    };
    // Sub-step cs of a lean step: its MFMAs, the other set's fragment reads
    // from slots RA and RB, and loads l0 .. l0 + 7 into slot WHERE, placed as
    // in substep.
    auto substep_fast = [&](int cs, auto ra, auto rb, auto where_c, int l0, uint32_t soff)
                            __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < G; ++t) {
            const int j = t / T::FM, i = SNAKE && (j & 1) ? T::FM - 1 - t % T::FM : t % T::FM;
            mfma16_agpr(acc[i][j], fb[cs][j], fa[cs][i]);
            if (t % RS == 0 && t / RS < R) read_fast(ra, rb, 1 - cs, t / RS);
            if (t % LS == LS / 2 && t / LS < T::A_LOADS) load_fast(where_c, l0 + t / LS, soff);
        }
    };
    // A lean step with the computed step's A tile in slot S (what step()
    // does with sa == S and a whole K range to load).
    auto step_fast = [&](auto s_c, uint32_t soff) __attribute__((always_inline)) {
        constexpr int S = decltype(s_c)::value;
        // The base registers are redefined (in place, by no instruction) at
        // every step, so the compiler cannot hoist base + offset sums out of
        // the loop into registers of their own; each stays a read's immediate.
#pragma unroll
        for (int c = 0; c < 3; ++c)
#pragma unroll
            for (int kk = 0; kk < T::KK; ++kk) asm volatile("" : "+v"(rdb[c][0][kk]), "+v"(rdb[c][1][kk]));
        asm volatile("" : "+s"(lw_bytes));
        substep_fast(0, Int<S>{}, Int<(S + 1) % 5>{}, Int<(S + 4) % 5>{}, 0, soff);
        lds_barrier<T::A_LOADS>();
        substep_fast(1, Int<(S + 2) % 5>{}, Int<(S + 3) % 5>{}, Int<S>{}, T::A_LOADS, soff);
    };

    // Epilogue of the tile at (cm0, cn0) through slots s0 and s1: round h
    // stages rows h * 64 .. h * 64 + 63 of each wave row (wave row wm into
    // slot s<wm>), then the non-loading waves store them with nontemporal
    // buffer stores (as in epilogue_lds: one 32-bit offset per store; rows
    // past M fall outside the buffer and columns past N get an offset outside
    // it, so neither is written).
    // Epilogue without staging: every wave converts its accumulators and
    // stores them itself, lane l writing columns 4 * (l / 16) .. + 3 of row
    // l % 16 of each 16 x 16 block as one 8-byte nontemporal buffer store
    // (rows past M outside the buffer, columns past N sent outside it).
    auto epilogue_direct = [&](int cm0, int cn0) __attribute__((always_inline)) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int e_row = ln % T::MI, e_hi = ln / T::MI;
        const __amdgpu_buffer_rsrc_t rc =
            make_rsrc(C + (size_t)cm0 * N, (uint32_t)min(T::BM, M - cm0) * (uint32_t)N * 2u);
        uint32_t pitch_c = (uint32_t)N * 2u;
        asm volatile("" : "+s"(pitch_c)::"memory");
        const half8_t z = zero_frag();
#pragma unroll
        for (int j = 0; j < T::FN; ++j) {
            const int n = cn0 + wn * T::WTN + j * T::MI + 4 * e_hi;
            const uint32_t vcol = n < N ? (uint32_t)n * 2u : kOob;
#pragma unroll
            for (int i = 0; i < T::FM; ++i) {
                const uint32_t r = (uint32_t)(wm * T::WTM + i * T::MI + e_row);
                half4_t v;
                v[0] = (_Float16)acc[i][j][0];
                v[1] = (_Float16)acc[i][j][1];
                v[2] = (_Float16)acc[i][j][2];
                v[3] = (_Float16)acc[i][j][3];
                clear(i, j, z);
                const uint32_t off = vcol == kOob ? kOob : vcol + r * pitch_c;
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, v), rc, off, 0, kPolicyNt);
            }
        }
    };

    auto epilogue = [&](unsigned char* s0, unsigned char* s1, int cm0, int cn0, bool storer)
                        __attribute__((always_inline)) {
        constexpr int PITCH = T::BN * 2;           // bytes per staged row
        constexpr int CH = T::BN / 8;              // 16-byte chunks per row
        constexpr int SW = CH >= 16 ? 15 : CH - 1;
        constexpr int HALF = T::FM / 2;            // MFMA block rows per round
        constexpr int SROWS = SLOT / PITCH;        // staged rows per slot
        constexpr int RPL = 1024 / PITCH;          // rows per wave-wide 1 KiB read
        constexpr int STORERS = ALL_STORE ? T::WAVES : T::WAVES - T::LOADERS;
        constexpr int ITERS = 2 * SROWS / RPL / STORERS;  // reads per storing wave per round
        static_assert(HALF * T::MI == SROWS && ITERS * RPL * STORERS == 2 * SROWS && ITERS % 4 == 0 &&
                          ITERS * RPL * 2 == SROWS,
                      "a round fills both slots, each storing wave reads half a slot");
        unsigned char* mine = wm == 0 ? s0 : s1;
        const int sw = ALL_STORE ? wave : wave - T::LOADERS;
        // the lane index laundered: offsets derived from it are computed
        // here rather than kept (or spilled) through the K loop
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int e_row = ln % T::MI, e_hi = ln / T::MI;
        const int lr = ln / CH, lc = ln % CH;
        const __amdgpu_buffer_rsrc_t rc =
            make_rsrc(C + (size_t)cm0 * N, (uint32_t)min(T::BM, M - cm0) * (uint32_t)N * 2u);
        // storing wave sw reads rows (sw % 2) * SROWS / 2 + RPL * it + lr of
        // slot sw / 2, i.e. tile row (sw / 2) * WTM + h * SROWS + that; this
        // lane's byte offset is vbase plus a wave-uniform part
        const int n = cn0 + lc * 8;
        const uint32_t vbase = n < N ? ((uint32_t)lr * (uint32_t)N + (uint32_t)n) * 2u : kOob;
        const unsigned char* rd = (sw < STORERS / 2 ? s0 : s1) + (sw % 2) * (SROWS / 2) * PITCH;
        const half8_t z = zero_frag();
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int i = 0; i < HALF; ++i) {
                const int x = i * T::MI + e_row;
                unsigned char* lrow = mine + x * PITCH;
#pragma unroll
                for (int j = 0; j < T::FN; ++j) {
                    const int col = wn * T::WTN + j * T::MI + 4 * e_hi;
                    half4_t v;
                    v[0] = (_Float16)acc[h * HALF + i][j][0];
                    v[1] = (_Float16)acc[h * HALF + i][j][1];
                    v[2] = (_Float16)acc[h * HALF + i][j][2];
                    v[3] = (_Float16)acc[h * HALF + i][j][3];
                    clear(h * HALF + i, j, z);
                    *(half4_t*)(lrow + (((col >> 3) ^ (x & SW)) << 4) + (col & 4) * 2) = v;
                }
            }
            lds_barrier<63>();  // staged; loads and stores may still be in flight
            if (storer) {
#pragma unroll
                for (int b4 = 0; b4 < ITERS; b4 += 4) {
                    // bytes per C row, laundered so that the offsets below
                    // are computed here and not hoisted out of the tile loop
                    uint32_t pitch_c = (uint32_t)N * 2u;
                    asm volatile("" : "+s"(pitch_c)::"memory");
#pragma unroll
                    for (int it = b4; it < b4 + 4; ++it) {
                        const int x = (sw % 2) * (SROWS / 2) + RPL * it + lr;  // row in the slot
                        const u32x4_t v = *(const u32x4_t*)(rd + (RPL * it + lr) * PITCH + ((lc ^ (x & SW)) << 4));
                        const uint32_t r0 = (uint32_t)((sw / 2) * T::WTM + h * SROWS + (sw % 2) * (SROWS / 2) + RPL * it);
                        const uint32_t off = vbase + r0 * pitch_c;
                        __builtin_amdgcn_raw_buffer_store_b128(v, rc, off, 0, kPolicyNt);
                    }
                }
            }
            lds_barrier<63>();  // both slots free again
        }
    };

    // The whole run, compiled once for the loading waves and once for the
    // others.
    auto run = [&](auto ldtag) __attribute__((always_inline)) {
        constexpr bool LD = decltype(ldtag)::value;
        // a step's barrier: this wave's loads but the last A tile have landed
        constexpr int VMW = LD ? T::A_LOADS : 63;
        {
            const half8_t z = zero_frag();
#pragma unroll
            for (int i = 0; i < T::FM; ++i)
#pragma unroll
                for (int j = 0; j < T::FN; ++j) clear(i, j, z);
        }
        // steps 0 and 1 of the first tile into slots 0 .. 3, then wait for step 0
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int l = 0; l < T::LOADS; ++l)
                if constexpr (LD) issue_load(l < T::A_LOADS ? 2 * s : 2 * s + 1, s, l, Flag<true>{}, row_bytes);
        lds_barrier<LD ? T::LOADS : 63>();
#pragma unroll
        for (int idx = 0; idx < R; ++idx) read_one(0, smem, smem + SLOT, idx);
        int sa = 0;  // slot of the computed step's A tile; its B, then A, B, A of the next two follow
        auto slot = [&](int i) __attribute__((always_inline)) {
            return smem + (sa + i >= 5 ? sa + i - 5 : sa + i) * SLOT;
        };
        // One step: sub-step 0 loads A of step lstep into the slot after
        // the next step's; sub-step 1 reads the next step's first fragments
        // and loads its B into the slot this step's A leaves, unless LAST
        // (the last step of a tile, whose epilogue needs both slots first).
        auto step = [&](int lstep, auto masked, auto last) __attribute__((always_inline)) {
            constexpr bool LAST = decltype(last)::value;
            const int a2 = sa + 4 >= 5 ? sa - 1 : sa + 4;
            substep(0, slot(0), slot(1), Flag<LD>{}, a2, lstep, 0, masked, Flag<true>{});
            lds_barrier<VMW>();
            substep(1, slot(2), slot(3), Flag<LD && !LAST>{}, sa, lstep, T::A_LOADS, masked, Flag<!LAST>{});
        };
        auto advance = [&]() __attribute__((always_inline)) { sa = sa + 2 >= 5 ? sa - 3 : sa + 2; };
        for (;;) {
            int ks = 0;
            if constexpr (LEAN) {
                // general steps until the ring is back at slot 0 (at most
                // four), then lean cycles of five steps from slot 0 (a loop
                // with one entry: entering a cycle at any of its five steps
                // makes the control flow irreducible, which the compiler
                // handles badly)
                for (; ks + 2 < nfull && sa != 0; ++ks) {
                    step(ks + 2, Flag<false>{}, Flag<false>{});
                    advance();
                }
                uint32_t soff = (uint32_t)(ks + 2) * T::ROW_BYTES;  // K range of the step loaded, in bytes
                for (; ks + 2 + 5 <= nfull; ks += 5) {
                    step_fast(Int<0>{}, soff);
                    step_fast(Int<2>{}, soff + T::ROW_BYTES);
                    step_fast(Int<4>{}, soff + 2 * T::ROW_BYTES);
                    step_fast(Int<1>{}, soff + 3 * T::ROW_BYTES);
                    step_fast(Int<3>{}, soff + 4 * T::ROW_BYTES);
                    soff += 5 * T::ROW_BYTES;
                }
            }
            for (; ks + 2 < nfull; ++ks) {
                step(ks + 2, Flag<false>{}, Flag<false>{});
                advance();
            }
            for (; ks + 2 < nk; ++ks) {
                step(ks + 2, Flag<true>{}, Flag<false>{});
                advance();
            }
            // The last two steps load steps 0 and 1 of the next tile (after
            // the last tile: zeros from past the end of K, into slots never
            // read).
            const int cm0 = m0, cn0 = n0;
            const int next = tile + (int)gridDim.x;
            int lbase = nk;
            if (next < total) {
                tile_coords(next, tiles_m, tiles_n, group_m, tm, tn);
                m0 = tm * T::BM;
                n0 = tn * T::BN;
                la = make_rsrc(A + (size_t)m0 * K, (uint32_t)min(T::BM, M - m0) * row_bytes);
                lb = make_rsrc(B + (size_t)n0 * K, (uint32_t)min(T::BN, N - n0) * row_bytes);
                lbase = 0;
            }
            step(lbase, Flag<true>{}, Flag<false>{});
            advance();
            step(lbase + 1, Flag<true>{}, Flag<true>{});
            // asm MFMAs are opaque to the compiler's hazard checks: let the
            // last ones write their accumulators before they are read
            asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
            // (and keep the scheduler from moving their reads above the wait)
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (DIRECT)
                epilogue_direct(cm0, cn0);
            else
                epilogue(slot(0), slot(1), cm0, cn0, ALL_STORE || !LD);
            if (next >= total) break;
            // B of the next tile's step 1 where the last step's A was
#pragma unroll
            for (int l = T::A_LOADS; l < T::LOADS; ++l)
                if constexpr (LD) issue_load(sa, lbase + 1, l, Flag<true>{}, row_bytes);
            advance();
#pragma unroll
            for (int idx = 0; idx < R; ++idx) read_one(0, slot(0), slot(1), idx);
            tile = next;
        }
    };
    if (wave < T::LOADERS)
        run(Flag<true>{});
    else
        run(Flag<false>{});
    // no global->LDS load may still be writing when the workgroup ends
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
}

// Plain per-element kernel for inputs the MFMA kernels do not take
// (unaligned pointers, K % 8 != 0, very long K).  One thread per output,
// fp32 accumulation in k order, one fp16 rounding at the end.  The grid is
// one-dimensional and at most kSimpleGrid workgroups of 16 x 16 outputs;
// workgroup g covers blocks g, g + gridDim.x, ... of the row-major order of
// 16 x 16 blocks of C, so every M, N < 2^31 runs.
__global__ void __launch_bounds__(256)
gemm_nt_f16_simple(const _Float16* __restrict__ A, const _Float16* __restrict__ B,
                   _Float16* __restrict__ C, int64_t M, int64_t N, int64_t K)
{
    const int64_t blocks_n = (N + 15) / 16;
    const int64_t blocks = ((M + 15) / 16) * blocks_n;
    for (int64_t blk = blockIdx.x; blk < blocks; blk += gridDim.x) {
        const int64_t m = (blk / blocks_n) * 16 + (threadIdx.x >> 4);
        const int64_t n = (blk % blocks_n) * 16 + (threadIdx.x & 15);
        if (m >= M || n >= N) continue;
        const _Float16* a = A + m * K;
        const _Float16* b = B + n * K;
        float s = 0.0f;
        for (int64_t k = 0; k < K; ++k) s += (float)a[k] * (float)b[k];
        C[m * N + n] = (_Float16)s;
    }
}

// ------------------------------------------------------------------ host --

//                  BM   BN   BK  WM  WN  S  OCC LOADERS MI
typedef TileShape<256, 256, 64, 2, 4, 2, 2> T256_k64_s2_w8;
typedef TileShape<256, 256, 64, 2, 2, 2, 1, 0, 16> T256_k64_s2_w4_mi16;
typedef TileShape<256, 256, 64, 2, 4, 2, 2, 0, 16> T256_k64_s2_w8_mi16;
typedef TileShape<256, 256, 64, 2, 4, 2, 2, 4, 16> T256_k64_s2_w8_l4_mi16;
typedef TileShape<128, 128, 64, 2, 2, 3, 1, 0, 16> T128_k64_s3_w4_mi16;
typedef TileShape<64, 64, 64, 2, 2, 3, 2, 0, 16> T64_k64_s3_w4_mi16;

constexpr int64_t kMaxK = (int64_t)1 << 22;
constexpr int64_t kMaxMN = ((int64_t)1 << 31) - 1;

struct Variant {
    const char* name;
    int bm, bn;    // 0 for the per-element kernel
    int group_m;
    int (*launch)(const void*, const void*, void*, int64_t, int64_t, int64_t, int, hipStream_t);
};

int num_cus(int device);

// Store mode of C (see c_vec above).
int c_store_mode(int64_t N, const void* C)
{
    return (N % 8 == 0 && (uintptr_t)C % 16 == 0) ? 2 : ((N % 4 == 0 && (uintptr_t)C % 8 == 0) ? 1 : 0);
}

template <class T>
int launch_mfma(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int group_m,
                hipStream_t stream)
{
    const int64_t tiles_m = (M + T::BM - 1) / T::BM, tiles_n = (N + T::BN - 1) / T::BN;
    if (tiles_m * tiles_n > kMaxMN) return hipErrorInvalidValue;
    const int c_vec = c_store_mode(N, C);
    hipLaunchKernelGGL((gemm_nt_f16_mfma<T>), dim3((unsigned)(tiles_m * tiles_n)), dim3(T::THREADS),
                       0, stream, (const _Float16*)A, (const _Float16*)B, (_Float16*)C, (int)M,
                       (int)N, (int)K, (int)tiles_m, (int)tiles_n, group_m, c_vec);
    return (int)hipGetLastError();
}

// The same with dynamic LDS padding the workgroup to a whole CU's 160 KiB,
// so only one workgroup runs per CU (a ladder rung: the single-stage kernel
// without other workgroups to overlap its copies).
template <class T>
int launch_mfma_one_per_cu(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int group_m,
                           hipStream_t stream)
{
    const int64_t tiles_m = (M + T::BM - 1) / T::BM, tiles_n = (N + T::BN - 1) / T::BN;
    if (tiles_m * tiles_n > kMaxMN) return hipErrorInvalidValue;
    const int c_vec = c_store_mode(N, C);
    hipLaunchKernelGGL((gemm_nt_f16_mfma<T>), dim3((unsigned)(tiles_m * tiles_n)), dim3(T::THREADS),
                       160 * 1024 - T::LDS_BYTES, stream, (const _Float16*)A, (const _Float16*)B, (_Float16*)C,
                       (int)M, (int)N, (int)K, (int)tiles_m, (int)tiles_n, group_m, c_vec);
    return (int)hipGetLastError();
}

template <class T, int RS, int LS, bool SLOTS5 = false>
int launch_ordered(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int group_m,
                   hipStream_t stream)
{
    const int64_t tiles_m = (M + T::BM - 1) / T::BM, tiles_n = (N + T::BN - 1) / T::BN;
    if (tiles_m * tiles_n > kMaxMN) return hipErrorInvalidValue;
    const int c_vec = c_store_mode(N, C);
    hipLaunchKernelGGL((gemm_nt_f16_ordered<T, RS, LS, SLOTS5>), dim3((unsigned)(tiles_m * tiles_n)),
                       dim3(T::THREADS), 0,
                       stream, (const _Float16*)A, (const _Float16*)B, (_Float16*)C, (int)M, (int)N, (int)K,
                       (int)tiles_m, (int)tiles_n, group_m, c_vec);
    return (int)hipGetLastError();
}

// The persistent 5-slot kernel (at most one workgroup per compute unit)
// where its conditions hold, else the one-tile-per-workgroup 5-slot kernel.
// Its epilogue is faster than the other's even with one tile per workgroup
// (4096^3: +1%).
template <class T, int RS, int LS, int FLAGS = 0>
int launch_ordered_persist(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int group_m,
                           hipStream_t stream)
{
    const int64_t tiles_m = (M + T::BM - 1) / T::BM, tiles_n = (N + T::BN - 1) / T::BN;
    if (tiles_m * tiles_n > kMaxMN) return hipErrorInvalidValue;
    const int c_vec = c_store_mode(N, C);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    const int64_t grid = std::min<int64_t>(num_cus(dev), tiles_m * tiles_n);
    // (C offsets are 32-bit and columns past N are sent to kOob: N <= 2^22)
    if ((c_vec & 3) != 2 || K <= T::BK || N > (int64_t(1) << 22))
        return launch_ordered<T, RS, LS, true>(A, B, C, M, N, K, group_m, stream);
    hipLaunchKernelGGL((gemm_nt_f16_ordered_persist<T, RS, LS, FLAGS>), dim3((unsigned)grid), dim3(T::THREADS), 0,
                       stream, (const _Float16*)A, (const _Float16*)B, (_Float16*)C, (int)M, (int)N, (int)K,
                       (int)tiles_m, (int)tiles_n, group_m);
    return (int)hipGetLastError();
}

int num_cus(int device)
{
    static int cache[64];
    if (device < 0 || device >= 64) return 256;
    int n = __atomic_load_n(&cache[device], __ATOMIC_RELAXED);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
            n <= 0)
            n = 256;
        __atomic_store_n(&cache[device], n, __ATOMIC_RELAXED);
    }
    return n;
}

constexpr int64_t kSimpleGrid = int64_t(1) << 20;  // workgroups of the per-element kernel at most

int launch_simple(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int,
                  hipStream_t stream)
{
    const int64_t blocks = ((M + 15) / 16) * ((N + 15) / 16);  // < 2^54 for M, N < 2^31
    const int64_t grid = std::min(blocks, kSimpleGrid);
    hipLaunchKernelGGL(gemm_nt_f16_simple, dim3((unsigned)grid), dim3(256), 0, stream,
                       (const _Float16*)A, (const _Float16*)B, (_Float16*)C, M, N, K);
    return (int)hipGetLastError();
}

// The variants select_mfma chooses from (kCandidates) are the defaults; the
// others are the rungs and side rows of the ablation ladder (tile shape,
// ring depth, persistence, hand-scheduled issue order, one wave per SIMD).
constexpr Variant kVariants[] = {
    {"mfma32_256x256x64_w8_s2", 256, 256, 8, launch_mfma<T256_k64_s2_w8>},
    {"mfma16_256x256x64_w8_s2", 256, 256, 8, launch_mfma<T256_k64_s2_w8_mi16>},
    {"mfma16_256x256x64_w8_s2_l4_ordered", 256, 256, 8, launch_ordered<T256_k64_s2_w8_l4_mi16, 2, 2>},
    {"mfma16_256x256x64_w8_r5_l4_ordered", 256, 256, 8, launch_ordered<T256_k64_s2_w8_l4_mi16, 2, 2, true>},
    {"mfma16_256x256x64_w8_r5_l4_persistent", 256, 256, 8, launch_ordered_persist<T256_k64_s2_w8_l4_mi16, 2, 2>},
    {"mfma16_256x256x64_w8_r5_l4_persistent_group4", 256, 256, 4, launch_ordered_persist<T256_k64_s2_w8_l4_mi16, 2, 2>},
    {"mfma16_256x256x64_w8_r5_l4_persistent_noxcd", 256, 256, -8, launch_ordered_persist<T256_k64_s2_w8_l4_mi16, 2, 2>},
    {"mfma16_256x256x64_w8_r5_l4_persistent_linear", 256, 256, 0, launch_ordered_persist<T256_k64_s2_w8_l4_mi16, 2, 2>},
    {"mfma16_256x256x64_w8_r5_l4_persistent_direct", 256, 256, 8,
     launch_ordered_persist<T256_k64_s2_w8_l4_mi16, 2, 2, kDirect>},
    {"mfma16_256x256x64_w8_r5_l4_persistent_vacc", 256, 256, 8,
     launch_ordered_persist<T256_k64_s2_w8_l4_mi16, 2, 2, kVgprAcc>},
    {"mfma16_256x256x64_w8_r5_l4_persistent_columns", 256, 256, 8,
     launch_ordered_persist<T256_k64_s2_w8_l4_mi16, 2, 2, kColumns>},
    {"mfma16_256x256x64_w4_r5_persistent_rs2_m0", 256, 256, 8,
     launch_ordered_persist<T256_k64_s2_w4_mi16, 2, 8, kSharedM0>},
    {"mfma16_256x256x64_w4_r5_persistent_rs2", 256, 256, 8, launch_ordered_persist<T256_k64_s2_w4_mi16, 2, 8>},
    {"mfma16_256x256x64_w4_r5_persistent_lean", 256, 256, 8, launch_ordered_persist<T256_k64_s2_w4_mi16, 3, 8, kLean>},
    {"mfma16_256x128x64_w8x_s3_l4_ordered", 256, 128, 8, launch_ordered<TileShape<256, 128, 64, 4, 2, 3, 2, 4, 16>, 1, 1>},
    {"mfma16_128x128x64_w8_s3_l4_ordered", 128, 128, 8, launch_ordered<TileShape<128, 128, 64, 2, 4, 3, 2, 4, 16>, 1, 1>},
    {"mfma16_128x128x64_w4_s1", 128, 128, 8, launch_mfma<TileShape<128, 128, 64, 2, 2, 1, 2, 0, 16>>},
    {"mfma16_128x128x64_w4_s1_one_per_cu", 128, 128, 8,
     launch_mfma_one_per_cu<TileShape<128, 128, 64, 2, 2, 1, 2, 0, 16>>},
    {"mfma16_128x128x64_w4_s3", 128, 128, 8, launch_mfma<T128_k64_s3_w4_mi16>},
    {"mfma16_64x64x64_w4_s3", 64, 64, 8, launch_mfma<T64_k64_s3_w4_mi16>},
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

constexpr bool same_name(const char* a, const char* b)
{
    return *a == *b && (*a == 0 || same_name(a + 1, b + 1));
}

constexpr int variant_index(const char* name)
{
    for (int i = 0; i < kNumVariants; ++i)
        if (same_name(kVariants[i].name, name)) return i;
    return -1;
}

// Shape -> variant.  Four kernels (four tile sizes) compete; each is priced
// as
//   ceil(tiles / 256 CUs) x (tile flops / per-CU rate + fixed cost),
// i.e. whole waves of tiles over the chip (one workgroup per CU), with the
// per-CU rate each kernel sustains on a full chip (measured on MI355X at
// 4096^3 .. 8192^3, fp16 random data) and a fixed per-wave cost for launch,
// pipeline fill and epilogue.  Small problems then take small tiles (more
// CUs busy), large ones the 256 x 256 kernel (most reuse per byte loaded).
struct Candidate {
    int variant;
    int bm, bn;
    double tflops_chip;  // sustained on a full chip
    double wave_us;      // fixed cost per wave of tiles
};

constexpr Candidate kCandidates[] = {
    {variant_index("mfma16_256x256x64_w4_r5_persistent_lean"), 256, 256, 1545.0, 3.0},
    {variant_index("mfma16_256x128x64_w8x_s3_l4_ordered"), 256, 128, 1330.0, 3.0},
    {variant_index("mfma16_128x128x64_w8_s3_l4_ordered"), 128, 128, 1150.0, 3.0},
    {variant_index("mfma16_64x64x64_w4_s3"), 64, 64, 730.0, 3.0},
};
static_assert(variant_index("mfma16_256x256x64_w4_r5_persistent_lean") >= 0 &&
                  variant_index("mfma16_256x128x64_w8x_s3_l4_ordered") >= 0 &&
                  variant_index("mfma16_128x128x64_w8_s3_l4_ordered") >= 0 &&
                  variant_index("mfma16_64x64x64_w4_s3") >= 0,
              "selected variants are in the table");

// Modelled time of one kernel on an M x N x K product: whole waves of
// tiles over the CUs at the kernel's sustained per-CU rate, plus a fixed
// cost per wave.  A wave that leaves CUs idle (a grid smaller than the
// chip, or the last wave of a larger one) runs its busy CUs faster (clock
// and L2 headroom): measured 1.25x per CU with half of them idle.
// The rates are for MI355X's 256 CUs; `cus` is the device's count (fewer
// in a partition mode), and the per-CU rate is kept.
constexpr int kRateCUs = 256;

double model_us(const Candidate& c, int64_t M, int64_t N, int64_t K, int cus)
{
    const int64_t tiles = ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
    const int64_t full = tiles / cus, rest = tiles % cus;
    const double tile_us = 2.0 * c.bm * c.bn * (double)K / (c.tflops_chip * 1e12 / kRateCUs) * 1e6;
    double us = (double)full * (tile_us + c.wave_us);
    if (rest > 0) us += tile_us / (1.0 + 0.5 * (1.0 - (double)rest / cus)) + c.wave_us;
    return us;
}

int select_mfma(int64_t M, int64_t N, int64_t K, int cus, double* us_out = nullptr)
{
    int best = kCandidates[0].variant;
    double best_us = 0;
    bool first = true;
    for (const Candidate& c : kCandidates) {
        const double us = model_us(c, M, N, K, cus);
        if (first || us < best_us) {
            best = c.variant;
            best_us = us;
            first = false;
        }
    }
    if (us_out) *us_out = best_us;
    return best;
}

// A launch plan: `variant` on rows [0, rows) of C and, if rows < M,
// `rest` on rows [rows, M).  When the 256 x 256 tiles of a product fill the
// chip except for a small last wave, running whole waves of them over the
// first rows and the remaining rows with the tile the model picks for them
// beats any single kernel (6144^3: 1376 TFLOP/s against 1260; 4352 x 4352 x
// 2048: 1138 against 978).  Only rows are split: C has no leading
// dimension, so a block of whole rows is the only sub-product that is
// itself a contiguous problem.
struct Plan {
    int variant;
    int64_t rows;
    int rest;
};
constexpr double kSplitUs = 4.0;  // the second launch (measured gap 2-4 us)

Plan plan_mfma(int64_t M, int64_t N, int64_t K)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    const int cus = num_cus(dev);
    double best_us = 0;
    Plan plan{select_mfma(M, N, K, cus, &best_us), M, -1};
    const Candidate& big = kCandidates[0];
    const int64_t tiles_m = (M + big.bm - 1) / big.bm, tiles_n = (N + big.bn - 1) / big.bn;
    const int64_t waves = (tiles_m * tiles_n + cus - 1) / cus;
    // main part: the most tile rows that fit in w whole waves, w = 1, 2, ...
    for (int64_t w = 1; w < waves && w <= 4096; ++w) {
        const int64_t r = w * cus / tiles_n;
        if (r < 1 || r >= tiles_m) continue;
        const int64_t rows = r * big.bm;
        double rest_us = 0;
        const int rest = select_mfma(M - rows, N, K, cus, &rest_us);
        const double us = model_us(big, rows, N, K, cus) + rest_us + kSplitUs;
        if (us < best_us) {
            best_us = us;
            plan = Plan{big.variant, rows, rest};
        }
    }
    return plan;
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
    return gemm_nt_f16_plan(M, N, K, nullptr, nullptr);
}

int32_t gemm_nt_f16_plan(int64_t M, int64_t N, int64_t K, int64_t* rows, int32_t* rest)
{
    if (rows) *rows = M;
    if (rest) *rest = -1;
    if (M < 0 || N < 0 || K < 0 || M > kMaxMN || N > kMaxMN || K > kMaxMN) return -1;
    if (K % 8 != 0 || K >= kMaxK) return kSimple;
    const Plan p = plan_mfma(M, N, K);
    if (rows) *rows = p.rows;
    if (rest) *rest = p.rest;
    return p.variant;
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
    if (variant < 0 && fast) {
        const Plan p = plan_mfma(M, N, K);
        const Variant& v = kVariants[p.variant];
        rc = v.launch(A, B, C, p.rows, N, K, v.group_m, stream);
        if (rc != hipSuccess || p.rows == M) return rc;
        const Variant& r = kVariants[p.rest];
        return r.launch((const _Float16*)A + p.rows * K, B, (_Float16*)C + p.rows * N, M - p.rows, N, K,
                        r.group_m, stream);
    }
    if (variant < 0) variant = kSimple;
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
