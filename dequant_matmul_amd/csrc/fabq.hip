// FABQ-RC-style binary-core GEMV.
//
// Sources: "FABQ-RC" README, "Key Ideas" (top channels at higher precision,
// the rest binary +-1, a k-means residual codebook whose centroid is added
// back at inference) and the FABQ-RC model card, "How It Works" and
// "Quantization Details" (int4 top 5 %, binary +-1 with per-block scaling,
// 4-bit indices into 16 centroids).
//
//   int4 row i:    y[row_of[i]]        = s_hi[i] * sum_k q[i][k] x[k]
//   binary row j:  y[row_of[n_hi + j]] = sum_b ( s_b * sum_{k in b} (+-x[k])
//                                               + c[idx_b] * sum_{k in b} x[k] )
// The second form is the per-weight decode s_b*(+-1) + c[idx_b] summed block
// by block; the decoded weights are never rounded to bf16.
#include "fqm_internal.h"

namespace fqm {
namespace {

constexpr int kWaves = 4;

template <int B>
__global__ __launch_bounds__(256) void fabq_gemv_kernel(fqm_fabq f, const uint16_t* __restrict__ x,
                                                        void* __restrict__ y, int y_f32,
                                                        int64_t rows, int64_t cols) {
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t i = (int64_t)blockIdx.x * kWaves + wave;  // stored row
    if (i >= rows) return;

    float acc[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = 0.f;

    if (i < f.n_hi) {
        // int4 row: one dword = 8 nibbles = 8 columns per lane step.
        const uint32_t* q = reinterpret_cast<const uint32_t*>(f.q4 + i * f.ld_q4);
        const int64_t nw = cols / 8;
        for (int64_t p = lane; p < nw; p += 64) {
            const uint32_t d = q[p];
            float wq[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) wq[j] = (float)((int32_t)(d << (28 - 4 * j)) >> 28);
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const uint4 xv = *reinterpret_cast<const uint4*>(x + (int64_t)b * cols + 8 * p);
                const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w};
                float a = acc[b];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    a = fmaf(wq[2 * j], bf16lo(xs[j]), a);
                    a = fmaf(wq[2 * j + 1], bf16hi(xs[j]), a);
                }
                acc[b] = a;
            }
        }
        const float s = fp16_to_f32(f.s_hi[i]);
#pragma unroll
        for (int b = 0; b < B; ++b) acc[b] *= s;
    } else {
        // binary row: one dword = 32 sign bits; a block (>= 64 columns) holds whole dwords.
        const int64_t j = i - f.n_hi;
        const uint32_t* sg = reinterpret_cast<const uint32_t*>(f.signs + j * f.ld_signs);
        const int64_t nb = cols / f.blocksize;
        const uint16_t* sb = f.s_blk + j * nb;
        const uint8_t* ib = f.idx + j * f.ld_idx;
        const int words_per_block = f.blocksize / 32;
        const int64_t nw = cols / 32;
        for (int64_t p = lane; p < nw; p += 64) {
            const uint32_t d = sg[p];
            const int64_t blk = p / words_per_block;
            const float s = fp16_to_f32(sb[blk]);
            const uint32_t id = (ib[blk >> 1] >> ((blk & 1) * 4)) & 15u;
            const float c = fp16_to_f32(f.codebook[id]);
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const uint4* xp = reinterpret_cast<const uint4*>(x + (int64_t)b * cols + 32 * p);
                float ps = 0.f, xsum = 0.f;
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const uint4 xv = xp[h];
                    const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const int bit = 8 * h + 2 * t;
                        const float x0 = bf16lo(xs[t]), x1 = bf16hi(xs[t]);
                        // +-x by flipping the sign bit where the sign bit of W is 0
                        ps += __uint_as_float(__float_as_uint(x0) ^ ((~d >> bit) & 1u) << 31);
                        ps += __uint_as_float(__float_as_uint(x1) ^ ((~d >> (bit + 1)) & 1u) << 31);
                        xsum += x0 + x1;
                    }
                }
                acc[b] = fmaf(s, ps, fmaf(c, xsum, acc[b]));
            }
        }
    }
    const int64_t out_row = f.row_of[i];
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const float v = wave_sum(acc[b]);
        if (lane == 0) {
            if (y_f32)
                reinterpret_cast<float*>(y)[(int64_t)b * rows + out_row] = v;
            else
                reinterpret_cast<uint16_t*>(y)[(int64_t)b * rows + out_row] = f32_to_bf16(v);
        }
    }
}

template <int B>
hipError_t launch_b(const fqm_weights& w, const uint16_t* x, void* y, int y_f32, hipStream_t s) {
    const unsigned grid = (unsigned)((w.rows + kWaves - 1) / kWaves);
    hipLaunchKernelGGL(fabq_gemv_kernel<B>, dim3(grid), dim3(64 * kWaves), 0, s, w.fabq, x, y,
                       y_f32, w.rows, w.cols);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fabq_gemv(const fqm_weights& w, const uint16_t* x, void* y, int y_f32,
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
