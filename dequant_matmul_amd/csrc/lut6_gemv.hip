// Per-row LUT 6-bit GEMV: y[b][r] = sum_k lut[r][code[r][k]] * x[b][k].
//
// Source: "Qwen3.8-27B - BenQ 6-bit", "What BenQ stores": a weight is its
// row's table entry selected by the 6-bit code, and the product gathers from
// the table inside the matmul instead of writing the decoded matrix out.
//
// Layout: a row's packed codes are 12-byte pieces of 16 codes; lane i of a
// wavefront takes pieces i, i+64, ... so each load instruction of the wave
// covers 768 contiguous bytes.  Each wavefront owns whole rows, stages the
// row's 128-byte table in LDS (one table per wave: the 64 lanes gather from
// the same 32 banks without conflicts), and reduces its per-lane partial sums
// across the wave at the end of the row.
#include "fqm_internal.h"

namespace fqm {
namespace {

constexpr int kWaves = 4;

template <int B>
__global__ __launch_bounds__(256) void lut6_gemv_generic(const uint8_t* __restrict__ packed,
                                                         int64_t ld,
                                                         const uint16_t* __restrict__ lut,
                                                         const uint16_t* __restrict__ x,
                                                         void* __restrict__ y, int y_f32,
                                                         int64_t rows, int64_t cols) {
    __shared__ uint32_t s_lut[kWaves][32];
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kWaves + wave;
    if (row < rows && lane < 32)
        s_lut[wave][lane] = reinterpret_cast<const uint32_t*>(lut + row * 64)[lane];
    __syncthreads();
    if (row >= rows) return;
    const uint16_t* tab = reinterpret_cast<const uint16_t*>(s_lut[wave]);

    float acc[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = 0.f;

    const int64_t npieces = cols / 16;
    const uint8_t* prow = packed + row * ld;
    for (int64_t p = lane; p < npieces; p += 64) {
        const uint32_t* q = reinterpret_cast<const uint32_t*>(prow + 12 * p);
        uint32_t c[16];
        codes16(q[0], q[1], q[2], c);
        float w[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) w[j] = bf16_to_f32(tab[c[j]]);
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const uint4* xp = reinterpret_cast<const uint4*>(x + (int64_t)b * cols + 16 * p);
            const uint4 x0 = xp[0], x1 = xp[1];
            const uint32_t xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            float a = acc[b];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                a = fmaf(w[2 * j], bf16lo(xv[j]), a);
                a = fmaf(w[2 * j + 1], bf16hi(xv[j]), a);
            }
            acc[b] = a;
        }
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const float v = wave_sum(acc[b]);
        if (lane == 0) {
            if (y_f32)
                reinterpret_cast<float*>(y)[(int64_t)b * rows + row] = v;
            else
                reinterpret_cast<uint16_t*>(y)[(int64_t)b * rows + row] = f32_to_bf16(v);
        }
    }
}

template <int B>
hipError_t launch_b(const fqm_weights& w, const uint16_t* x, void* y, int y_f32, hipStream_t s) {
    const unsigned grid = (unsigned)((w.rows + kWaves - 1) / kWaves);
    hipLaunchKernelGGL(lut6_gemv_generic<B>, dim3(grid), dim3(64 * kWaves), 0, s, w.lut6.packed,
                       w.lut6.ld, w.lut6.lut, x, y, y_f32, w.rows, w.cols);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_lut6_gemv(const fqm_weights& w, const uint16_t* x, void* y, int y_f32,
                            int batch, hipStream_t s) {
    switch (batch) {
        case 1: return launch_b<1>(w, x, y, y_f32, s);
        case 2: return launch_b<2>(w, x, y, y_f32, s);
        case 3: return launch_b<3>(w, x, y, y_f32, s);
        case 4: return launch_b<4>(w, x, y, y_f32, s);
        case 5: return launch_b<5>(w, x, y, y_f32, s);
        case 6: return launch_b<6>(w, x, y, y_f32, s);
        case 7: return launch_b<7>(w, x, y, y_f32, s);
        case 8: return launch_b<8>(w, x, y, y_f32, s);
        case 9: return launch_b<9>(w, x, y, y_f32, s);
        case 10: return launch_b<10>(w, x, y, y_f32, s);
        case 11: return launch_b<11>(w, x, y, y_f32, s);
        case 12: return launch_b<12>(w, x, y, y_f32, s);
        case 13: return launch_b<13>(w, x, y, y_f32, s);
        case 14: return launch_b<14>(w, x, y, y_f32, s);
        case 15: return launch_b<15>(w, x, y, y_f32, s);
        case 16: return launch_b<16>(w, x, y, y_f32, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fqm
