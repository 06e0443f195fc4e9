// What the board sustains, under its power limit, for each part of the
// default GEMM kernel's K loop taken alone: a measuring instrument for the
// hardware, built into its own library (libpower_probe.so), never called by
// the GEMM path and computing no product.
//
// The engine clock of an MI355X is power-managed, so the rate a kernel
// reaches depends on the energy of every instruction it issues, not only on
// how densely it issues MFMAs.  These kernels replay the default kernel's K
// loop piece by piece on every CU: four waves per workgroup (one per SIMD),
// one workgroup per CU (160 KiB of LDS), 8 x 8 blocks of 16 x 16 fp32
// accumulators in the 256 AGPRs of each lane, v_mfma_f32_16x16x32_f16 down
// the columns of blocks with a turn at each column's end, two fragment sets
// of 8 + 8 sixteen-byte registers, two sub-steps of 64 MFMAs per step.  The
// pieces, switched on one at a time (mode flags):
//   kReads: the other set's 16 fragments read from LDS with ds_read_b128, one
//           after every third MFMA (1 KiB contiguous per read: no bank
//           conflicts), from LDS bytes [0, 64 KiB) filled once with the
//           Gaussian data;
//   kLoads: 8 direct-to-LDS buffer loads (16 bytes per lane) per sub-step,
//           one after every eighth MFMA, from a 1 MiB window of the data that
//           stays resident in every L2, into LDS bytes [64 KiB, 128 KiB);
//   kBarrier: once per step, between its two sub-steps, the wait for all but
//           the last 8 loads and the LDS reads, then s_barrier;
//   kVgprLoads: the other set's 8 B fragments of each sub-step loaded from
//           the same L2-resident window straight into VGPRs (16-byte buffer
//           loads, the same bytes per step as kLoads), no LDS;
//   kZero: fragments of zeros instead of the Gaussian data;
//   kMfma32: MFMAs alone as v_mfma_f32_32x32x16_f16 on 4 x 4 blocks of
//           32 x 32 (the same 256 accumulators, the same 128 fragment
//           registers as four K slices of 4 + 4, the same flops per step in
//           64 MFMAs of twice the work).
// With every piece but kZero on, the loop issues per 128 MFMAs what the
// default kernel's K loop issues: 32 fragment reads, 16 loads, one barrier.
// The reads never depend on the loads (the DMA writes a region the reads do
// not touch), so each piece costs what its issue and its energy cost, not a
// wait.
//
// Bounds: LDS reads in [0, 65536) (lane * 16 + 32 KiB * (step & 1) + 1 KiB *
// read + 16 KiB * sub-step, plus 16 bytes), LDS writes in [0, 65536) before
// the loop and [65536, 131072) by the loads (64 KiB + 16 KiB * wave + 1 KiB
// * load); global reads within src_bytes (a power of two, 64 MiB to 1 GiB:
// the start-up reads are masked to it, and a load's offset, at most 4 KiB *
// 3 + 1008 + 256 KiB * 3 + 64 KiB * 3 + 3 KiB (kLoads) or 4 KiB * 3 + 1008 +
// 256 KiB * 3 + 16 KiB * 15 (kVgprLoads), plus 16 bytes, stays below 1 MiB);
// global writes: one float per thread of sink[grid * 256].
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kReads = 1, kLoads = 2, kBarrier = 4, kZero = 8, kMfma32 = 16, kVgprLoads = 32;
// buffer resource word 3 for gfx950 raw buffer accesses (32-bit data format)
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ void mfma(float4_t& acc, const half8_t& b, const half8_t& a)
{
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(b), "v"(a) : "memory");
}

typedef float float16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ void mfma32(float16_t& acc, const half8_t& b, const half8_t& a)
{
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(b), "v"(a) : "memory");
}

// kMfma32: 4 x 4 blocks of 32 x 32 per wave, K slices of 16, fragments
// fa[s][i], fb[s][j] (s = 0 .. 3); MFMAs down the columns with turns.
__global__ void __launch_bounds__(256, 1)
power_probe_mfma32(const _Float16* __restrict__ src, uint32_t src_bytes, float* __restrict__ sink, int steps)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const unsigned char* s8 = (const unsigned char*)src;
    const uint32_t mask = src_bytes - 1u;
    half8_t fa[4][4], fb[4][4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t piece = (blockIdx.x * 4u + (uint32_t)wave) * 32u + (uint32_t)(s * 8 + i);
            fa[s][i] = *(const half8_t*)(s8 + ((piece * 1024u + lane * 16u) & mask));
            fb[s][i] = *(const half8_t*)(s8 + (((piece + 4u) * 1024u + lane * 16u) & mask));
        }
    float16_t acc[4][4];
    {
        half8_t z = {};
        asm volatile("s_nop 4" : "+v"(z));
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %1, 0" : "=a"(acc[i][j]) : "v"(z) : "memory");
    }
    for (int st = 0; st < steps; ++st) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const int j = t / 4, i = (j & 1) ? 3 - t % 4 : t % 4;
                mfma32(acc[i][j], fb[s][j], fa[s][i]);
            }
    }
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    sink[blockIdx.x * 256 + threadIdx.x] = acc[0][0][0] + acc[3][3][15];
}

template <int MODE>
__global__ void __launch_bounds__(256, 1)
power_probe_kernel(const _Float16* __restrict__ src, uint32_t src_bytes, float* __restrict__ sink, int steps)
{
    constexpr bool RD = MODE & kReads, LD = MODE & kLoads, BAR = MODE & kBarrier, ZERO = MODE & kZero,
                   VL = MODE & kVgprLoads;
    static_assert(!(VL && (RD || LD)), "register loads replace the LDS path");
    __shared__ __attribute__((aligned(1024))) unsigned char lds[160 * 1024];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const unsigned char* s8 = (const unsigned char*)src;
    const uint32_t mask = src_bytes - 1u;
    // LDS [0, 64 KiB): 64 KiB of the data, a different range per workgroup
    for (int i = threadIdx.x; i < 4096; i += 256)
        *(half8_t*)(lds + i * 16) = *(const half8_t*)(s8 + ((blockIdx.x * 65536u + (uint32_t)i * 16u) & mask));
    // both fragment sets: 32 KiB of the data per wave, a different range per wave
    half8_t fa[2][8], fb[2][8];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t piece = (blockIdx.x * 4u + (uint32_t)wave) * 32u + (uint32_t)(s * 16 + i);
            fa[s][i] = ZERO ? half8_t{} : *(const half8_t*)(s8 + ((piece * 1024u + lane * 16u) & mask));
            fb[s][i] = ZERO ? half8_t{} : *(const half8_t*)(s8 + (((piece + 8u) * 1024u + lane * 16u) & mask));
        }
    // accumulators cleared by an MFMA of zero fragments with an inline zero C
    float4_t acc[8][8];
    {
        half8_t z = {};
        asm volatile("s_nop 4" : "+v"(z));  // VALU writes, then an MFMA reads them
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %1, 0" : "=a"(acc[i][j]) : "v"(z) : "memory");
    }
    __syncthreads();

    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16*>(src), (short)0, (int)src_bytes, kRsrcWord3);
    const uint32_t rbase = (uint32_t)lane * 16u;
    const uint32_t vo = (uint32_t)lane * 16u + (uint32_t)wave * 4096u;
    unsigned char* const ld_base = lds + 65536 + wave * 16384;

    for (int st = 0; st < steps; ++st) {
        const uint32_t rot = (uint32_t)(st & 1) * 32768u;
        // load 4 * grp + r of this step reads 1 KiB at soff + 64 KiB * grp + r KiB + this wave's 4 KiB
        const uint32_t soff = (uint32_t)(st & 3) * 262144u;
#pragma unroll
        for (int cs = 0; cs < 2; ++cs) {
#pragma unroll
            for (int t = 0; t < 64; ++t) {
                const int j = t / 8, i = (j & 1) ? 7 - t % 8 : t % 8;
                mfma(acc[i][j], fb[cs][j], fa[cs][i]);
                if constexpr (RD) {
                    if (t % 3 == 0 && t / 3 < 16) {
                        const int idx = t / 3;
                        const unsigned char* p = lds + rbase + rot + (uint32_t)idx * 1024u + (uint32_t)cs * 16384u;
                        if (idx < 8)
                            fb[1 - cs][idx] = *(const half8_t*)p;
                        else
                            fa[1 - cs][15 - idx] = *(const half8_t*)p;
                    }
                }
                if constexpr (VL) {
                    if (t % 8 == 4) {
                        const int l = cs * 8 + t / 8;
                        fb[1 - cs][t / 8] = __builtin_bit_cast(
                            half8_t, __builtin_amdgcn_raw_buffer_load_b128(rs, vo, soff + (uint32_t)l * 16384u, 0));
                    }
                }
                if constexpr (LD) {
                    if (t % 8 == 4) {
                        // load l = 4 * grp + r: LDS base (M0) and global offset
                        // shared by a group of four, the instruction offset r
                        // KiB added to both, as in the default kernel
                        const int l = cs * 8 + t / 8, grp = l / 4;
                        lds_void_t* dst = (lds_void_t*)(ld_base + grp * 4096);
                        const uint32_t so = soff + (uint32_t)grp * 65536u;
                        switch (l % 4) {  // (the instruction offset must be a constant)
                            case 0: __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, vo, so, 0, 0); break;
                            case 1: __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, vo, so, 1024, 0); break;
                            case 2: __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, vo, so, 2048, 0); break;
                            default: __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, vo, so, 3072, 0); break;
                        }
                    }
                }
            }
            if constexpr (BAR)
                if (cs == 0) asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        }
    }
    __builtin_amdgcn_s_waitcnt(0);  // no load may still be writing LDS when the workgroup ends
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");  // the last MFMAs' results
    // (the MFMAs are volatile asm and are all issued; two results are kept)
    sink[blockIdx.x * 256 + threadIdx.x] = acc[0][0][0] + acc[7][7][3];
}

struct Mode {
    const char* name;
    int flags;
    void (*kernel)(const _Float16*, uint32_t, float*, int);
};

const Mode kModes[] = {
    {"mfma_zero_data", kZero, power_probe_kernel<kZero>},
    {"mfma", 0, power_probe_kernel<0>},
    {"mfma_lds_reads", kReads, power_probe_kernel<kReads>},
    {"mfma_loads", kLoads, power_probe_kernel<kLoads>},
    {"mfma_lds_reads_loads", kReads | kLoads, power_probe_kernel<kReads | kLoads>},
    {"k_loop_mix", kReads | kLoads | kBarrier, power_probe_kernel<kReads | kLoads | kBarrier>},
    {"mfma32", kMfma32, power_probe_mfma32},
    {"mfma_vgpr_loads", kVgprLoads, power_probe_kernel<kVgprLoads>},
};
constexpr int kNumModes = sizeof(kModes) / sizeof(kModes[0]);

}  // namespace

extern "C" {

int32_t power_probe_mode_count(void) { return kNumModes; }

const char* power_probe_mode_name(int32_t mode)
{
    return mode >= 0 && mode < kNumModes ? kModes[mode].name : nullptr;
}

// Launch mode `mode` on `grid` workgroups (one per CU), `steps` steps of 128
// MFMAs per wave: grid * 4 * steps * 128 MFMAs of 16384 flop.  src: device
// fp16 data, src_bytes a power of two from 64 MiB to 1 GiB; sink: device floats, grid *
// 256 of them.  Returns a hipError_t code; hipErrorInvalidValue for
// arguments outside these ranges.
int power_probe_launch(int32_t mode, const void* src, uint64_t src_bytes, float* sink, int32_t grid, int32_t steps,
                       hipStream_t stream)
{
    if (mode < 0 || mode >= kNumModes || src == nullptr || sink == nullptr || src_bytes < (uint64_t(64) << 20) ||
        src_bytes > (uint64_t(1) << 30) || (src_bytes & (src_bytes - 1)) || grid <= 0 || grid > 4096 || steps <= 0)
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(kModes[mode].kernel, dim3((unsigned)grid), dim3(256), 0, stream, (const _Float16*)src,
                       (uint32_t)src_bytes, sink, (int)steps);
    return (int)hipGetLastError();
}

}  // extern "C"
