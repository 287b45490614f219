// The prefill GEMM's inner-loop instruction mix with no global memory: the
// MFMA-rate ceiling that mix allows on this GPU, reported by the benchmark
// beside the prefill rows (measurement only; not part of libfqm's interface).
//
// One "slice" repeats what a wave of the LUT6 GEMM issues per 16-wide k slice:
// 8 MFMAs v_mfma_f32_32x32x16_bf16 (eight 32-row blocks of X against one
// gathered 32-row B operand), 8 ds_read_b128 operand reads (the next slice's
// A, one after each MFMA), 8 ds_read_u16 table gathers at code-dependent
// addresses (the slice after next), 16 VALU ops computing those addresses and
// 4 v_perm_b32 packing the gathered entries; a workgroup barrier every 4
// slices.  The same LDS layouts and scheduling groups as the GEMM, 8 waves
// per workgroup, one workgroup per compute unit.  The codes are rotated in
// registers instead of being loaded, and X is never refreshed, so the kernel
// measures the issue and LDS cost of the mix, not memory.  The accumulators
// feed a store that runs only if the sum equals a value the caller passes and
// the data never produce.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds8_t;
typedef __attribute__((address_space(3))) const uint16_t lds16c_t;
typedef __attribute__((address_space(3))) const u32x4_t lds128c_t;

constexpr int kWaves = 8, kThreads = 64 * kWaves, kBlocks = 8;  // 8 x 32 rows of X per wave
constexpr int kX = 32768, kTab = 32768;                        // one X tile, the row tables

__global__ __launch_bounds__(kThreads) void gemm_mix_kernel(float* __restrict__ sink, uint64_t* __restrict__ clk,
                                                            int slices, uint32_t seed, float never) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[kX + kTab];
    lds8_t* const X = (lds8_t*)lds;
    lds8_t* const TAB = (lds8_t*)lds + kX;
    for (int i = threadIdx.x; i < (kX + kTab) / 4; i += kThreads)
        reinterpret_cast<uint32_t*>(lds)[i] = 0x3F803F80u + ((uint32_t)i & 0x7Fu) * 0x10001u;  // bf16 pairs in [1, 2)
    __syncthreads();
    // shader-clock and constant-rate counters around the loop (the clock the
    // matrix cores run at under this load)
    const uint64_t sc0 = __builtin_amdgcn_s_memtime(), rt0 = __builtin_amdgcn_s_memrealtime();
    const int lane = threadIdx.x & 63, j = lane & 31, g = lane >> 5;
    const int wave = threadIdx.x >> 6;
    // the GEMM's gather base (row j of the wave's 32, plane and half of the wave)
    const uint32_t base = 8192u * (uint32_t)(wave >> 1) + 4u * j + 2u * (wave & 1);
    uint32_t mask = 63u << 7;
    asm volatile("" : "+v"(mask));
    uint32_t cw[6];
    for (int q = 0; q < 6; ++q) cw[q] = seed * (uint32_t)(lane + 17 * q + 1);
    // A read: row 32 i + j, swizzled 16-byte chunk of the slice
    const int aoff = 128 * j + 16 * ((4 * g) ^ ((j >> 1) & 7));
    f32x16_t acc[kBlocks];
    for (int i = 0; i < kBlocks; ++i)
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
    bf16x8_t a[kBlocks];
    for (int i = 0; i < kBlocks; ++i) a[i] = __builtin_bit_cast(bf16x8_t, *(lds128c_t*)(X + aoff + 4096 * i));
    uint32_t wv[8];
    for (int e = 0; e < 8; ++e) wv[e] = (uint32_t)e;
    bf16x8_t bop = __builtin_bit_cast(bf16x8_t, u32x4_t{1u, 2u, 3u, 4u});
    constexpr int kHalf = kBlocks / 2, kGpm = 8 / kHalf;
    for (int it = 0; it < slices; ++it) {
        __builtin_amdgcn_sched_barrier(0);
        u32x4_t bw;
        for (int e = 0; e < 4; ++e) bw[e] = __builtin_amdgcn_perm(wv[2 * e + 1], wv[2 * e], 0x05040100u);
        const bf16x8_t bnext = __builtin_bit_cast(bf16x8_t, bw);
        uint32_t ad[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) ad[e] = ((cw[e % 6] >> (e + 1)) & mask) | base;
        const int so = 16 * (it & 3);
#pragma unroll
        for (int i = 0; i < kBlocks; ++i) {
            acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bop, acc[i], 0, 0, 0);
            a[i] = __builtin_bit_cast(bf16x8_t, *(lds128c_t*)(X + ((aoff + so) & 4095) + 4096 * i));
            if (i < kHalf) {
#pragma unroll
                for (int e = kGpm * i; e < kGpm * (i + 1); ++e) wv[e] = *(lds16c_t*)(TAB + ad[e]);
            }
        }
        bop = bnext;
        for (int q = 0; q < 6; ++q) cw[q] = __builtin_amdgcn_alignbit(cw[q], cw[(q + 1) % 6], 5);
        __builtin_amdgcn_sched_group_barrier(0x0002, 4 + 2 * kGpm, 0);
#pragma unroll
        for (int i = 0; i < kHalf; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x0100, 1 + kGpm, 0);
            __builtin_amdgcn_sched_group_barrier(0x0002, 2 * kGpm, 0);
        }
#pragma unroll
        for (int i = kHalf; i < kBlocks; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        if ((it & 3) == 3) __syncthreads();
    }
    if (clk && threadIdx.x == 0) {
        const uint64_t sc1 = __builtin_amdgcn_s_memtime(), rt1 = __builtin_amdgcn_s_memrealtime();
        clk[2 * blockIdx.x] = sc1 - sc0;
        clk[2 * blockIdx.x + 1] = rt1 - rt0;
    }
    float s = 0.f;
    for (int i = 0; i < kBlocks; ++i)
        for (int r = 0; r < 16; ++r) s += acc[i][r];
    if (s == never) sink[0] = s;
}

}  // namespace

// Launch one compute unit's worth of the mix per workgroup on `cus`
// workgroups, `slices` slices each.  Flops per launch:
// cus * 8 waves * slices * 8 MFMAs * 32768.  clk (nullable, 2 * cus values):
// per workgroup, the shader-clock ticks and the constant-rate ticks of its
// loop (fqm_bench_wall_clock_khz gives the rate of the latter).
extern "C" int fqm_bench_gemm_mix(float* sink, uint64_t* clk, int cus, int slices, float never, void* stream) {
    if (!sink || cus <= 0 || slices <= 0) return 1;
    hipLaunchKernelGGL(gemm_mix_kernel, dim3((unsigned)cus), dim3(kThreads), 0, reinterpret_cast<hipStream_t>(stream),
                       sink, clk, slices, 3u, never);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Rate of the constant-rate counter (s_memrealtime) of the current device, kHz.
extern "C" int fqm_bench_wall_clock_khz(void) {
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
    return khz;
}
