// Plain streaming read of a device buffer: the achievable-bandwidth reference
// the benchmark reports beside the GEMV rows (measurement only; not part of
// libfqm's interface).  Every lane reads 16-byte pieces, consecutive lanes
// consecutive pieces (one 1 KB coalesced request per wave instruction), eight
// per lane, with non-temporal loads like the GEMV's code stream; the XOR of
// what was read is stored only if it equals a value the caller passes and the
// data never holds, so the loads cannot be dropped and nothing is written
// except, when the caller passes a clock buffer, each workgroup's shader-clock
// and constant-rate ticks (the clock the GPU holds while it streams).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

namespace {

constexpr int kThreads = 256, kPer = 8;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4_t* __restrict__ src, int64_t n,
                                                               uint32_t* __restrict__ sink,
                                                               uint64_t* __restrict__ clk, uint32_t never) {
    const uint64_t sc0 = __builtin_amdgcn_s_memtime(), rt0 = __builtin_amdgcn_s_memrealtime();
    const int64_t base = (int64_t)blockIdx.x * kThreads * kPer + threadIdx.x;
    u32x4_t v[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int64_t i = min(base + (int64_t)u * kThreads, n - 1);
        v[u] = __builtin_nontemporal_load(src + i);
    }
    uint32_t acc = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    if (acc == never) sink[0] = acc;
    if (clk && threadIdx.x == 0) {  // shader-clock and constant-rate ticks of this workgroup
        const uint64_t sc1 = __builtin_amdgcn_s_memtime(), rt1 = __builtin_amdgcn_s_memrealtime();
        clk[2 * blockIdx.x] = sc1 - sc0;
        clk[2 * blockIdx.x + 1] = rt1 - rt0;
    }
}

}  // namespace

// clk (nullable): two values per workgroup, ceil(bytes / 32768) workgroups.
extern "C" int fqm_bench_stream_read(const void* src, int64_t bytes, uint32_t* sink, uint64_t* clk, uint32_t never,
                                     void* stream) {
    const int64_t n = bytes / 16;
    if (n <= 0 || !src || !sink || (reinterpret_cast<uintptr_t>(src) & 15)) return 1;
    const int64_t per_block = (int64_t)kThreads * kPer;
    const unsigned grid = (unsigned)((n + per_block - 1) / per_block);
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), static_cast<const u32x4_t*>(src), n, sink,
                       clk, never);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
