// Per-row LUT 6-bit GEMM (prefill): Y[m][n] = sum_k X[m][k] * lut[n][code[n][k]].
//
// Source: "Qwen3.8-27B - BenQ 6-bit", "What BenQ stores": decode is the
// row-wise gather of codes into the row's table, fused into the matrix
// product so the decoded matrix is never written out.  Here each workgroup
// decodes one BN x BK tile of W at a time into LDS as bf16 (exact: the table
// entries are bf16) and contracts it with the matching X tile on the bf16
// matrix cores (v_mfma_f32_16x16x32_bf16), accumulating in fp32.
#include "fqm_internal.h"

namespace fqm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDT = BK + 8;  // LDS row stride (bf16 elements) of the X and W tiles

__global__ __launch_bounds__(256) void lut6_gemm_kernel(const uint16_t* __restrict__ X,
                                                        const uint8_t* __restrict__ packed,
                                                        int64_t ld,
                                                        const uint16_t* __restrict__ lut,
                                                        uint16_t* __restrict__ Y, int64_t M,
                                                        int64_t N, int64_t K) {
    __shared__ __attribute__((aligned(16))) uint16_t sX[BM * LDT];
    __shared__ __attribute__((aligned(16))) uint16_t sW[BN * LDT];
    __shared__ __attribute__((aligned(16))) uint16_t sL[BN * 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;

    // The BN row tables stay resident for the whole K loop.
    for (int i = tid; i < BN * 8; i += 256) {
        const int r = i >> 3, part = i & 7;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (n0 + r < N) v = *reinterpret_cast<const u32x4*>(lut + (n0 + r) * 64 + part * 8);
        *reinterpret_cast<u32x4*>(sL + r * 64 + part * 8) = v;
    }

    const int wm = wave >> 1, wn = wave & 1;  // 2 x 2 waves, 64 x 64 outputs each
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int lr = tid >> 1, lh = tid & 1;  // loader: tile row 0..127, 32-element half

    for (int64_t k0 = 0; k0 < K; k0 += BK) {
        __syncthreads();
        {   // X tile, 32 bf16 per thread
            const int64_t m = m0 + lr;
            u32x4 v[4];
            if (m < M) {
                const u32x4* src = reinterpret_cast<const u32x4*>(X + m * K + k0 + 32 * lh);
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = src[i];
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = u32x4{0u, 0u, 0u, 0u};
            }
            u32x4* dst = reinterpret_cast<u32x4*>(sX + lr * LDT + 32 * lh);
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[i] = v[i];
        }
        {   // W tile: 32 codes (24 bytes) per thread, gathered from the row's table
            const int64_t n = n0 + lr;
            uint32_t out[16];
            if (n < N) {
                const uint32_t* src =
                    reinterpret_cast<const uint32_t*>(packed + n * ld + (k0 * 3) / 4 + 24 * lh);
                uint32_t d[6];
#pragma unroll
                for (int i = 0; i < 6; ++i) d[i] = src[i];
                uint32_t c[32];
                codes16(d[0], d[1], d[2], c);
                codes16(d[3], d[4], d[5], c + 16);
                const uint16_t* tab = sL + lr * 64;
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    out[j] = (uint32_t)tab[c[2 * j]] | ((uint32_t)tab[c[2 * j + 1]] << 16);
            } else {
#pragma unroll
                for (int j = 0; j < 16; ++j) out[j] = 0u;
            }
            u32x4* dst = reinterpret_cast<u32x4*>(sW + lr * LDT + 32 * lh);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dst[i] = u32x4{out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]};
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; kk += 32) {
            bf16x8 a[4], b[4];
            const int koff = kk + 8 * (lane >> 4);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a[i] = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(sX + (wm * 64 + 16 * i + (lane & 15)) * LDT + koff));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                b[j] = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(sW + (wn * 64 + 16 * j + (lane & 15)) * LDT + koff));
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    }

    // D layout of a 16x16 MFMA block: lane l, element r -> row 4*(l/16) + r, column l%16.
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t m = m0 + wm * 64 + 16 * i + 4 * (lane >> 4) + r;
                const int64_t n = n0 + wn * 64 + 16 * j + (lane & 15);
                if (m < M && n < N) Y[m * N + n] = f32_to_bf16(acc[i][j][r]);
            }
}

}  // namespace

hipError_t launch_lut6_gemm(const fqm_weights& w, const uint16_t* X, uint16_t* Y, int64_t M,
                            hipStream_t s) {
    const dim3 grid((unsigned)((w.rows + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
    hipLaunchKernelGGL(lut6_gemm_kernel, grid, dim3(256), 0, s, X, w.lut6.packed, w.lut6.ld,
                       w.lut6.lut, Y, M, w.rows, w.cols);
    return hipGetLastError();
}

}  // namespace fqm
