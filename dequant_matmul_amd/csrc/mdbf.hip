// MDBF double-binary GEMV: two sign-matrix products on the matrix cores.
//
// Source: OneCompression "MDBF (Multi-Envelope Double Binary
// Factorization)", "Algorithm": W = sum_p F_p G_p, F = S_A (.) (A_amp Q_U^T),
// G = S_B (.) (Q_V B_amp^T), signs stored one bit each and unpacked on the fly
// ("Save and Load").  Distributing the Hadamard products over the rank-l
// envelopes gives, per path and batch row,
//   pass 1:  z[j] = sum_k Q_V[j][k] * sum_i S_B[j][i] * u_k[i],  u_k[i] = B_amp[i][k] x[i]   (j < r)
//   pass 2:  y[i] = sum_k A_amp[i][k] * sum_j S_A[i][j] * v_k[j],  v_k[j] = Q_U[j][k] z[j]   (i < n)
// so neither F, G nor W is formed.
//
// Both inner sums are a +-1 matrix times a few dense columns (one per
// envelope k and batch row b).  They run on the bf16 matrix cores
// (v_mfma_f32_32x32x16_bf16, fp32 accumulate): a sign byte expands in
// registers to eight exact bf16 +-1.0, and each dense fp32 column v enters
// as three bf16 columns, h0 = bf16(v), h1 = bf16(v - h0), h2 = bf16(v - h0 -
// h1), whose sum carries the fp32 value (u is an exact fp32 product, v a
// rounded one).  Three launches:
//   prep:   D1[p][c][i] = part t of u_k[i] for column c = 3 (b l + k) + t;
//   pass 1: sign products over S_B, then z and D2[p][c][j] = parts of v_k[j];
//   pass 2: sign products over S_A for every path, then y.
// A workgroup owns 32 rows and a batch slice; its 8 waves split K and their
// partial sums are added in a fixed order in LDS, so results do not depend
// on timing.  Columns past the logical width hold zeros in D1/D2, so the sign
// bits read there (padding, or a clamped re-read) contribute nothing.
#include <algorithm>

#include "fqm_internal.h"

namespace fqm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int NW = 8;        // waves per workgroup (K split)
constexpr int KB = 256;      // columns per K block

__host__ __device__ inline int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// batch rows per workgroup so that its 3 l bs dense columns fit two MFMA blocks
__host__ __device__ inline int batch_slice(int l) { return 3 * l >= 64 ? 1 : 64 / (3 * l); }

struct MdbfDims {
    int64_t m_pad, r_pad;     // padded widths of D1 and D2 rows
    int64_t cp;               // dense columns per path: 3 l batch
    size_t d1_elems, d2_elems;
};

__host__ __device__ inline MdbfDims mdbf_dims(int64_t m, int64_t r, int l, int P, int batch) {
    MdbfDims d;
    d.m_pad = round_up(m, KB);
    d.r_pad = round_up(r, KB);
    d.cp = 3LL * l * batch;
    d.d1_elems = (size_t)P * d.cp * d.m_pad;
    d.d2_elems = (size_t)P * d.cp * d.r_pad;
    return d;
}

// v = h0 + h1 + h2 (bf16 parts; each remainder is exact in fp32)
__device__ __forceinline__ void split3_bf16(float v, uint16_t (&h)[3]) {
    h[0] = f32_to_bf16(v);
    const float r1 = v - bf16_to_f32(h[0]);
    h[1] = f32_to_bf16(r1);
    h[2] = f32_to_bf16(r1 - bf16_to_f32(h[1]));
}

// Eight bf16 +-1.0 from one sign byte: bit e set -> +1, clear -> -1 (element e
// of the fragment).  Dword d holds elements 2d (low half) and 2d + 1.
__device__ __forceinline__ bf16x8 expand_signs(uint32_t byte) {
    const uint32_t nb = ~byte;
    u32x4 v;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t t = (nb >> (2 * d)) & 3u;
        v[d] = 0x3F803F80u | (((t | (t << 15)) & 0x10001u) << 15);
    }
    return __builtin_bit_cast(bf16x8, v);
}

// D1[p][c][i]: c = 3 (b l + k) + t; zero for i >= m.
__global__ __launch_bounds__(256) void mdbf_prep(fqm_mdbf md, const uint16_t* __restrict__ x,
                                                 uint16_t* __restrict__ D1, int64_t m, int batch,
                                                 int64_t m_pad) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (p, b, k, i)
    const int l = md.l;
    const int64_t per_p = (int64_t)batch * l * m_pad;
    if (t >= per_p * md.P) return;
    const int p = (int)(t / per_p);
    int64_t rem = t - p * per_p;
    const int b = (int)(rem / ((int64_t)l * m_pad));
    rem -= (int64_t)b * l * m_pad;
    const int k = (int)(rem / m_pad);
    const int64_t i = rem - (int64_t)k * m_pad;
    const fqm_mdbf_path path = p == 0 ? md.path[0] : md.path[1];
    uint16_t h[3] = {0, 0, 0};
    if (i < m) split3_bf16(fp16_to_f32(path.B_amp[i * l + k]) * bf16_to_f32(x[(int64_t)b * m + i]), h);
    const int64_t c = 3 * ((int64_t)b * l + k);
    uint16_t* dp = D1 + (int64_t)p * 3 * batch * l * m_pad;
#pragma unroll
    for (int t3 = 0; t3 < 3; ++t3) dp[(c + t3) * m_pad + i] = h[t3];
}

// Sign products for one path: acc[nb] = S[row0 .. row0 + 31][:] * D[c0 + 32 nb + (0..31)][:]^T over
// this wave's K blocks.  k order inside a 256-column block: slice s, lane half g, element e
// -> column 128 g + 8 s + e (the same order for both operands).
template <int NB>
__device__ __forceinline__ void sign_products(const uint8_t* __restrict__ S, int64_t ldS, int64_t rows,
                                              const uint16_t* __restrict__ D, int64_t ldD, int64_t row0, int64_t c0, int64_t cend, int blk0, int blk1,
                                              f32x16 (&acc)[NB]) {
    const int lane = threadIdx.x & 63, g = lane >> 5, j = lane & 31;
    const uint8_t* srow = S + min(row0 + j, rows - 1) * ldS;
    const int64_t last16 = ldS - 16;  // the last 16-byte piece inside a row
    // dense column c0 + 32 nb + j (columns past cend read as zeros)
    const uint16_t* dcol[NB];
    bool dvalid[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int64_t c = c0 + 32 * nb + j;
        dvalid[nb] = c < cend;
        dcol[nb] = D + (dvalid[nb] ? c : c0) * ldD + 128 * g;
    }
    for (int blk = blk0; blk < blk1; ++blk) {
        const u32x4 sb = *reinterpret_cast<const u32x4*>(srow + min((int64_t)(32 * blk + 16 * g), last16));
        // a clamped re-read only happens where the dense columns are zero
        bf16x8 bf[NB][16];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(dcol[nb] + (int64_t)KB * blk + 8 * s);
                bf[nb][s] = __builtin_bit_cast(bf16x8, dvalid[nb] ? v : u32x4{0u, 0u, 0u, 0u});
            }
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const bf16x8 a = expand_signs((sb[s >> 2] >> (8 * (s & 3))) & 255u);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bf[nb][s], acc[nb], 0, 0, 0);
        }
    }
}

// Sum of the NW waves' partial blocks in a fixed tree order (waves w and
// w + h for h = 4, 2, 1) into red[nb][row][col] (LDS).  D layout of a 32x32
// block: lane l, item q -> row (q % 4) + 8 (q / 4) + 4 (l / 32), column l % 32.
template <int NB>
__device__ __forceinline__ void reduce_waves(f32x16 (&acc)[NB], float* buf, float* red) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int h = NW / 2; h >= 1; h >>= 1) {
        if (wave >= h && wave < 2 * h) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int q = 0; q < 16; ++q) buf[(((wave - h) * NB + nb) * 16 + q) * 64 + lane] = acc[nb][q];
        }
        __syncthreads();
        if (wave < h) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[nb][q] += buf[((wave * NB + nb) * 16 + q) * 64 + lane];
        }
        __syncthreads();
    }
    if (wave == 0) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int row = (q & 3) + 8 * (q >> 2) + 4 * (lane >> 5), col = lane & 31;
                red[(nb * 32 + row) * 32 + col] = acc[nb][q];
            }
    }
    __syncthreads();
}

// Pass 1: rows j of S_B; D1 columns of batch slice [b0, b0 + bs).  Writes
// D2[p][c][j] = parts of Q_U[j][k] z[j] (zero for j >= r, which the grid
// covers up to r_pad).
template <int NB>
__global__ __launch_bounds__(64 * NW) void mdbf_pass1(fqm_mdbf md, const uint16_t* __restrict__ D1,
                                                      uint16_t* __restrict__ D2, int64_t m, int batch,
                                                      int64_t m_pad, int64_t r_pad) {
    __shared__ float red_buf[NW / 2 * NB * 1024];
    __shared__ float red[NB * 1024];
    const int p = blockIdx.z;
    const fqm_mdbf_path path = p == 0 ? md.path[0] : md.path[1];
    const int l = md.l;
    const int64_t r = md.r;
    const int bs = batch_slice(l);
    const int b0 = blockIdx.y * bs, nb_rows = min(bs, batch - b0);
    const int64_t j0 = (int64_t)blockIdx.x * 32;
    const int64_t cp = 3LL * l * batch;
    const uint16_t* Dp = D1 + (int64_t)p * cp * m_pad;
    const int wave = threadIdx.x >> 6;
    const int nblk = (int)(m_pad / KB);
    const int per = (nblk + NW - 1) / NW;
    const int blk0 = min(wave * per, nblk), blk1 = min(blk0 + per, nblk);

    f32x16 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[nb][q] = 0.f;
    const int64_t c0 = 3LL * l * b0, cend = c0 + 3LL * l * nb_rows;
    sign_products<NB>(path.S_B, path.ld_B, r, Dp, m_pad, j0, c0, cend, blk0, blk1, acc);
    reduce_waves<NB>(acc, red_buf, red);

    // one thread per (row, batch row of the slice)
    uint16_t* D2p = D2 + (int64_t)p * cp * r_pad;
    for (int e = threadIdx.x; e < 32 * bs; e += 64 * NW) {
        const int jr = e & 31, bl = e >> 5;
        const int64_t jj = j0 + jr;
        if (bl >= nb_rows) continue;
        float z = 0.f;
        if (jj < r) {
            for (int k = 0; k < l; ++k) {
                const int cl = 3 * (bl * l + k);
                float t = 0.f;
#pragma unroll
                for (int t3 = 0; t3 < 3; ++t3) t += red[((cl + t3) >> 5) * 1024 + jr * 32 + ((cl + t3) & 31)];
                z = fmaf(fp16_to_f32(path.Q_V[jj * l + k]), t, z);
            }
        }
        for (int k = 0; k < l; ++k) {
            uint16_t h[3] = {0, 0, 0};
            if (jj < r) split3_bf16(fp16_to_f32(path.Q_U[jj * l + k]) * z, h);
            const int64_t c = 3 * ((int64_t)(b0 + bl) * l + k);
#pragma unroll
            for (int t3 = 0; t3 < 3; ++t3) D2p[(c + t3) * r_pad + jj] = h[t3];
        }
    }
}

// Pass 2: rows i of S_A, summed over the paths; D2 columns of batch slice [b0, b0 + bs).
template <int NB>
__global__ __launch_bounds__(64 * NW) void mdbf_pass2(fqm_mdbf md, const uint16_t* __restrict__ D2,
                                                      void* __restrict__ y, int y_f32, int64_t n, int batch,
                                                      int64_t r_pad) {
    __shared__ float red_buf[NW / 2 * NB * 1024];
    __shared__ float red[NB * 1024];
    const int l = md.l;
    const int64_t r = md.r;
    const int bs = batch_slice(l);
    const int b0 = blockIdx.y * bs, nb_rows = min(bs, batch - b0);
    const int64_t i0 = (int64_t)blockIdx.x * 32;
    const int64_t cp = 3LL * l * batch;
    const int wave = threadIdx.x >> 6;
    const int nblk = (int)(r_pad / KB);
    const int per = (nblk + NW - 1) / NW;
    const int blk0 = min(wave * per, nblk), blk1 = min(blk0 + per, nblk);
    const int64_t c0 = 3LL * l * b0, cend = c0 + 3LL * l * nb_rows;

    float out[2] = {0.f, 0.f};  // (row, batch row) pairs e = tid, tid + 512 of this thread
    for (int p = 0; p < md.P; ++p) {
        const fqm_mdbf_path path = p == 0 ? md.path[0] : md.path[1];
        f32x16 acc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[nb][q] = 0.f;
        sign_products<NB>(path.S_A, path.ld_A, n, D2 + (int64_t)p * cp * r_pad, r_pad, i0, c0, cend, blk0, blk1,
                          acc);
        reduce_waves<NB>(acc, red_buf, red);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int e = threadIdx.x + 64 * NW * h;
            const int ir = e & 31, bl = e >> 5;
            const int64_t ii = i0 + ir;
            if (bl >= nb_rows || ii >= n) continue;
            float v = out[h];
            for (int k = 0; k < l; ++k) {
                const int cl = 3 * (bl * l + k);
                float t = 0.f;
#pragma unroll
                for (int t3 = 0; t3 < 3; ++t3) t += red[((cl + t3) >> 5) * 1024 + ir * 32 + ((cl + t3) & 31)];
                v = fmaf(fp16_to_f32(path.A_amp[ii * l + k]), t, v);
            }
            out[h] = v;
        }
        __syncthreads();  // red is rewritten by the next path
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int e = threadIdx.x + 64 * NW * h;
        const int ir = e & 31, bl = e >> 5;
        const int64_t ii = i0 + ir;
        if (bl >= nb_rows || ii >= n) continue;
        const int64_t o = (int64_t)(b0 + bl) * n + ii;
        if (y_f32)
            reinterpret_cast<float*>(y)[o] = out[h];
        else
            reinterpret_cast<uint16_t*>(y)[o] = f32_to_bf16(out[h]);
    }
}

template <int NB>
hipError_t launch_nb(const fqm_weights& w, const uint16_t* x, void* y, int y_f32, int batch, uint16_t* D1,
                     uint16_t* D2, const MdbfDims& d, hipStream_t s) {
    const fqm_mdbf& md = w.mdbf;
    const int bs = batch_slice(md.l);
    const unsigned gy = (unsigned)((batch + bs - 1) / bs);
    hipLaunchKernelGGL((mdbf_pass1<NB>), dim3((unsigned)(d.r_pad / 32), gy, (unsigned)md.P), dim3(64 * NW), 0, s,
                       md, D1, D2, w.cols, batch, d.m_pad, d.r_pad);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((mdbf_pass2<NB>), dim3((unsigned)((w.rows + 31) / 32), gy), dim3(64 * NW), 0, s, md, D2, y,
                       y_f32, w.rows, batch, d.r_pad);
    return hipGetLastError();
}

}  // namespace

size_t mdbf_workspace_bytes(const fqm_weights& w, int batch) {
    const MdbfDims d = mdbf_dims(w.cols, w.mdbf.r, w.mdbf.l, w.mdbf.P, batch);
    return (d.d1_elems + d.d2_elems) * sizeof(uint16_t);
}

hipError_t launch_mdbf_gemv(const fqm_weights& w, const uint16_t* x, void* y, int y_f32, int batch, void* ws,
                            hipStream_t s) {
    const fqm_mdbf& md = w.mdbf;
    const MdbfDims d = mdbf_dims(w.cols, md.r, md.l, md.P, batch);
    uint16_t* D1 = static_cast<uint16_t*>(ws);
    uint16_t* D2 = D1 + d.d1_elems;
    const int64_t nprep = (int64_t)md.P * batch * md.l * d.m_pad;
    hipLaunchKernelGGL(mdbf_prep, dim3((unsigned)((nprep + 255) / 256)), dim3(256), 0, s, md, x, D1, w.cols, batch,
                       d.m_pad);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int bs = batch_slice(md.l);
    const int cols_per_wg = 3 * md.l * std::min(bs, batch);
    return cols_per_wg <= 32 ? launch_nb<1>(w, x, y, y_f32, batch, D1, D2, d, s)
                             : launch_nb<2>(w, x, y, y_f32, batch, D1, D2, d, s);
}

}  // namespace fqm
