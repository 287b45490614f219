// MDBF double-binary GEMV in two passes over the packed sign matrices.
//
// Source: OneCompression "MDBF (Multi-Envelope Double Binary
// Factorization)", "Algorithm": W = sum_p F_p G_p, F = S_A (.) (A_amp Q_U^T),
// G = S_B (.) (Q_V B_amp^T), signs stored one bit each and unpacked on the fly
// ("Save and Load").  Distributing the Hadamard products over the rank-l
// envelopes gives, per path,
//   pass 1:  z[j] = sum_k Q_V[j][k] * sum_i S_B[j][i] * (B_amp[i][k] x[i])   (j < r)
//   pass 2:  y[i] = sum_k A_amp[i][k] * sum_j S_A[i][j] * (Q_U[j][k] z[j])   (i < n)
// so neither F, G nor W is formed.  z stays fp32 in the caller's workspace;
// stream order makes pass 2 see all of pass 1.
#include "fqm_internal.h"

namespace fqm {
namespace {

constexpr int kWaves = 4;

__device__ __forceinline__ float flip_if_zero(float v, uint32_t d, int bit) {
    return __uint_as_float(__float_as_uint(v) ^ (((~d >> bit) & 1u) << 31));
}

// One wavefront per (path, row of S_B); batch rows [b0, b0 + BC) per grid row y.
template <int LMAX, int BC>
__global__ __launch_bounds__(256) void mdbf_pass1(fqm_mdbf md, const uint16_t* __restrict__ x,
                                                  float* __restrict__ z, int64_t m, int batch) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t gid = (int64_t)blockIdx.x * kWaves + wave;
    const int64_t r = md.r;
    if (gid >= (int64_t)md.P * r) return;
    const int p = (int)(gid / r);
    const int64_t j = gid - (int64_t)p * r;
    const fqm_mdbf_path path = p == 0 ? md.path[0] : md.path[1];
    const int l = md.l;
    const int b0 = blockIdx.y * BC;

    float t[BC][LMAX];
#pragma unroll
    for (int bb = 0; bb < BC; ++bb)
#pragma unroll
        for (int k = 0; k < LMAX; ++k) t[bb][k] = 0.f;

    const uint32_t* row = reinterpret_cast<const uint32_t*>(path.S_B + j * path.ld_B);
    const int64_t words = m / 32;
    for (int64_t q = lane; q < words; q += 64) {
        const uint32_t d = row[q];
        for (int bit = 0; bit < 32; ++bit) {
            const int64_t i = 32 * q + bit;
            float bk[LMAX];
#pragma unroll
            for (int k = 0; k < LMAX; ++k) bk[k] = k < l ? fp16_to_f32(path.B_amp[i * l + k]) : 0.f;
#pragma unroll
            for (int bb = 0; bb < BC; ++bb) {
                const int b = b0 + bb;
                const float xv = b < batch ? bf16_to_f32(x[(int64_t)b * m + i]) : 0.f;
#pragma unroll
                for (int k = 0; k < LMAX; ++k) t[bb][k] += flip_if_zero(bk[k] * xv, d, bit);
            }
        }
    }
#pragma unroll
    for (int bb = 0; bb < BC; ++bb) {
        float zj = 0.f;
#pragma unroll
        for (int k = 0; k < LMAX; ++k) {
            const float s = wave_sum(t[bb][k]);
            if (k < l) zj = fmaf(fp16_to_f32(path.Q_V[j * l + k]), s, zj);
        }
        const int b = b0 + bb;
        if (lane == 0 && b < batch) z[((int64_t)p * batch + b) * r + j] = zj;
    }
}

// One wavefront per output row i; sums over all paths.
template <int LMAX, int BC>
__global__ __launch_bounds__(256) void mdbf_pass2(fqm_mdbf md, const float* __restrict__ z,
                                                  void* __restrict__ y, int y_f32, int64_t n,
                                                  int batch) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t i = (int64_t)blockIdx.x * kWaves + wave;
    if (i >= n) return;
    const int64_t r = md.r;
    const int l = md.l;
    const int b0 = blockIdx.y * BC;
    float out[BC];
#pragma unroll
    for (int bb = 0; bb < BC; ++bb) out[bb] = 0.f;

    for (int p = 0; p < md.P; ++p) {
        const fqm_mdbf_path path = p == 0 ? md.path[0] : md.path[1];
        float acc[BC][LMAX];
#pragma unroll
        for (int bb = 0; bb < BC; ++bb)
#pragma unroll
            for (int k = 0; k < LMAX; ++k) acc[bb][k] = 0.f;
        const uint32_t* row = reinterpret_cast<const uint32_t*>(path.S_A + i * path.ld_A);
        const int64_t words = (r + 31) / 32;
        for (int64_t q = lane; q < words; q += 64) {
            const uint32_t d = row[q];
            for (int bit = 0; bit < 32; ++bit) {
                const int64_t j = 32 * q + bit;
                if (j >= r) break;
                float qu[LMAX];
#pragma unroll
                for (int k = 0; k < LMAX; ++k) qu[k] = k < l ? fp16_to_f32(path.Q_U[j * l + k]) : 0.f;
#pragma unroll
                for (int bb = 0; bb < BC; ++bb) {
                    const int b = b0 + bb;
                    const float zv = b < batch ? z[((int64_t)p * batch + b) * r + j] : 0.f;
#pragma unroll
                    for (int k = 0; k < LMAX; ++k) acc[bb][k] += flip_if_zero(qu[k] * zv, d, bit);
                }
            }
        }
#pragma unroll
        for (int bb = 0; bb < BC; ++bb)
#pragma unroll
            for (int k = 0; k < LMAX; ++k) {
                const float s = wave_sum(acc[bb][k]);
                if (k < l) out[bb] = fmaf(fp16_to_f32(path.A_amp[i * l + k]), s, out[bb]);
            }
    }
#pragma unroll
    for (int bb = 0; bb < BC; ++bb) {
        const int b = b0 + bb;
        if (lane == 0 && b < batch) {
            if (y_f32)
                reinterpret_cast<float*>(y)[(int64_t)b * n + i] = out[bb];
            else
                reinterpret_cast<uint16_t*>(y)[(int64_t)b * n + i] = f32_to_bf16(out[bb]);
        }
    }
}

template <int LMAX>
hipError_t launch_l(const fqm_weights& w, const uint16_t* x, void* y, int y_f32, int batch,
                    float* z, hipStream_t s) {
    constexpr int BC = 32 / LMAX < 16 ? 32 / LMAX : 16;
    const unsigned gy = (unsigned)((batch + BC - 1) / BC);
    const int64_t rows1 = (int64_t)w.mdbf.P * w.mdbf.r;
    hipLaunchKernelGGL((mdbf_pass1<LMAX, BC>), dim3((unsigned)((rows1 + kWaves - 1) / kWaves), gy),
                       dim3(64 * kWaves), 0, s, w.mdbf, x, z, w.cols, batch);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((mdbf_pass2<LMAX, BC>), dim3((unsigned)((w.rows + kWaves - 1) / kWaves), gy),
                       dim3(64 * kWaves), 0, s, w.mdbf, z, y, y_f32, w.rows, batch);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mdbf_gemv(const fqm_weights& w, const uint16_t* x, void* y, int y_f32,
                            int batch, float* z, hipStream_t s) {
    const int l = w.mdbf.l;
    if (l <= 2) return launch_l<2>(w, x, y, y_f32, batch, z, s);
    if (l <= 4) return launch_l<4>(w, x, y, y_f32, batch, z, s);
    if (l <= 8) return launch_l<8>(w, x, y, y_f32, batch, z, s);
    return launch_l<16>(w, x, y, y_f32, batch, z, s);
}

}  // namespace fqm
