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
//   prep:   D1 = parts of u_k[i], column 3 (b l + k) + t of batch slice b / bs;
//   pass 1: sign products over S_B, then z and D2 = parts of v_k[j];
//   pass 2: sign products over S_A for every path, then y.
// D1 and D2 are stored fragment-major: for each batch slice, 32-column
// block, 256-wide K block and 16-wide k slice, the 64 lanes' 16-byte MFMA
// operand pieces are contiguous, so every operand load is one coalesced 1 KB
// wave read.
// A workgroup owns 32 rows and a batch slice; its waves (16 in pass 1, 8 in
// pass 2) split K and their partial sums are added in a fixed order in LDS,
// so results do not depend on timing.  Columns past the logical width hold zeros in D1/D2, so the sign
// bits read there (padding, or a clamped re-read) contribute nothing.
#include <algorithm>

#include "fqm_internal.h"

namespace fqm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int NW1 = 16;      // waves per pass-1 workgroup (K split)
constexpr int NW2 = 8;       // waves per pass-2 workgroup
constexpr int KB = 256;      // columns per K block

__host__ __device__ inline int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// batch rows per workgroup so that its 3 l bs dense columns fit two MFMA blocks
__host__ __device__ inline int batch_slice(int l) { return 3 * l >= 64 ? 1 : 64 / (3 * l); }

struct MdbfDims {
    int64_t m_pad, r_pad;     // padded K widths of D1 and D2
    int64_t nsg;              // batch slices
    int64_t d1_path, d2_path; // elements of one path's D1 / D2
    size_t d1_elems, d2_elems;
};

__host__ __device__ inline MdbfDims mdbf_dims(int64_t m, int64_t r, int l, int P, int batch) {
    MdbfDims d;
    d.m_pad = round_up(m, KB);
    d.r_pad = round_up(r, KB);
    d.nsg = (batch + batch_slice(l) - 1) / batch_slice(l);
    d.d1_path = d.nsg * (d.m_pad / KB) * 16384;
    d.d2_path = d.nsg * (d.r_pad / KB) * 16384;
    d.d1_elems = (size_t)P * d.d1_path;
    d.d2_elems = (size_t)P * d.d2_path;
    return d;
}

// Element index of column lc (0..63) of batch slice sg at k in a fragment-major
// operand with nkb 256-wide K blocks: slice s, lane half g, element e of k
// within its K block follow the MFMA k order (k = 128 g + 8 s + e).
__host__ __device__ inline int64_t dfrag_index(int64_t sg, int lc, int64_t k, int64_t nkb) {
    const int nb = lc >> 5;
    const int64_t kb = k >> 8;
    const int rem = (int)(k & 255);
    const int g = rem >> 7, s = (rem & 127) >> 3, e = rem & 7;
    const int lane = (lc & 31) + 32 * g;
    return ((((sg * 2 + nb) * nkb + kb) * 16 + s) * 64 + lane) * 8 + e;
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

// D1 of path p: parts of u_k[i] at column 3 (b l + k) + t of batch slice
// b / bs; zero for i >= m.
__global__ __launch_bounds__(256) void mdbf_prep(fqm_mdbf md, const uint16_t* __restrict__ x,
                                                 uint16_t* __restrict__ D1, int64_t m, int batch,
                                                 int64_t m_pad, int64_t d1_path) {
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
    // the two paths' pointers are selected as values (p varies per thread)
    const uint16_t* bamp = p == 0 ? md.path[0].B_amp : md.path[1].B_amp;
    uint16_t h[3] = {0, 0, 0};
    if (i < m) split3_bf16(fp16_to_f32(bamp[i * l + k]) * bf16_to_f32(x[(int64_t)b * m + i]), h);
    const int bs = batch_slice(l);
    const int sg = b / bs, bl = b - sg * bs;
    uint16_t* dp = D1 + (int64_t)p * d1_path;
#pragma unroll
    for (int t3 = 0; t3 < 3; ++t3) dp[dfrag_index(sg, 3 * (bl * l + k) + t3, i, m_pad / KB)] = h[t3];
}

// Sign products for one path: acc[nb] = S[row0 .. row0 + 31][:] * (dense columns 32 nb + (0..31) of
// batch slice sg)^T over this wave's K blocks.  k order inside a 256-column block: slice s, lane
// half g, element e -> column 128 g + 8 s + e (the same order for both operands).
template <int NB>
__device__ __forceinline__ void sign_products(const uint8_t* __restrict__ S, int64_t ldS, int64_t rows,
                                              const uint16_t* __restrict__ D, int64_t nkb, int64_t sg,
                                              int64_t row0, int cend, int blk0, int blk1, f32x16 (&acc)[NB]) {
    const int lane = threadIdx.x & 63, g = lane >> 5, j = lane & 31;
    const uint8_t* srow = S + min(row0 + j, rows - 1) * ldS;
    const int64_t last16 = ldS - 16;  // the last 16-byte piece inside a row
    // this lane's 16-byte pieces of column block nb (columns past cend read as zeros)
    const uint16_t* dcol[NB];
    bool dvalid[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        dvalid[nb] = 32 * nb + j < cend;
        dcol[nb] = D + (sg * 2 + nb) * nkb * 8192 + 8 * lane;
    }
    for (int blk = blk0; blk < blk1; ++blk) {
        const u32x4 sb = *reinterpret_cast<const u32x4*>(srow + min((int64_t)(32 * blk + 16 * g), last16));
        // a clamped re-read only happens where the dense columns are zero;
        // lanes of columns past cend fetch nothing; the 16 k slices go in
        // groups of 8 / NB to bound the live operands
        constexpr int SG = 8 / NB;
#pragma unroll
        for (int s0 = 0; s0 < 16; s0 += SG) {
            bf16x8 bf[NB][SG];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int s = 0; s < SG; ++s) {
                    u32x4 v = {0u, 0u, 0u, 0u};
                    if (dvalid[nb]) v = *reinterpret_cast<const u32x4*>(dcol[nb] + (int64_t)8192 * blk + 512 * (s0 + s));
                    bf[nb][s] = __builtin_bit_cast(bf16x8, v);
                }
#pragma unroll
            for (int s = 0; s < SG; ++s) {
                const int ss = s0 + s;
                const bf16x8 a = expand_signs((sb[ss >> 2] >> (8 * (ss & 3))) & 255u);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bf[nb][s], acc[nb], 0, 0, 0);
            }
        }
    }
}

// Sum of the NW waves' partial blocks in a fixed tree order (waves w and
// w + h for h = NW / 2, ..., 2, 1) into red[nb][row][col] (LDS).  D layout of a 32x32
// block: lane l, item q -> row (q % 4) + 8 (q / 4) + 4 (l / 32), column l % 32.
template <int NB, int NW>
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
__global__ __launch_bounds__(64 * NW1) void mdbf_pass1(fqm_mdbf md, const uint16_t* __restrict__ D1,
                                                      uint16_t* __restrict__ D2, int64_t m, int batch,
                                                      int64_t m_pad, int64_t r_pad, int64_t d1_path,
                                                      int64_t d2_path) {
    __shared__ float red_buf[NW1 / 2 * NB * 1024];
    __shared__ float red[NB * 1024];
    __shared__ float qv_s[32 * 16], qu_s[32 * 16];  // Q_V, Q_U rows j0 .. j0 + 31
    const int p = blockIdx.z;
    const fqm_mdbf_path path = p == 0 ? md.path[0] : md.path[1];
    const int l = md.l;
    const int64_t r = md.r;
    const int bs = batch_slice(l);
    const int b0 = blockIdx.y * bs, nb_rows = min(bs, batch - b0);
    const int64_t j0 = (int64_t)blockIdx.x * 32;
    // the epilogue's envelope values, fetched before the long sign products
    // (rows j0 .. j0 + 31 of the [r][l] arrays are one contiguous run)
    // (unconditional loads at a clamped index, so that no wait lands here)
    const int64_t qo = j0 * l + threadIdx.x;
    const bool qin = threadIdx.x < 32 * l && qo < r * l;
    const int64_t qoc = min(qo, r * l - 1);
    const uint16_t qv_l = path.Q_V[qoc], qu_l = path.Q_U[qoc];
    const uint16_t qv_h = qin ? qv_l : 0, qu_h = qin ? qu_l : 0;
    const uint16_t* Dp = D1 + (int64_t)p * d1_path;
    const int wave = threadIdx.x >> 6;
    const int nblk = (int)(m_pad / KB);
    const int per = (nblk + NW1 - 1) / NW1;
    const int blk0 = min(wave * per, nblk), blk1 = min(blk0 + per, nblk);

    f32x16 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[nb][q] = 0.f;
    sign_products<NB>(path.S_B, path.ld_B, r, Dp, nblk, blockIdx.y, j0, 3 * l * nb_rows, blk0, blk1, acc);
    if (threadIdx.x < 32 * l) {
        qv_s[threadIdx.x] = fp16_to_f32(qv_h);
        qu_s[threadIdx.x] = fp16_to_f32(qu_h);
    }
    reduce_waves<NB, NW1>(acc, red_buf, red);  // ends with a barrier

    // one thread per (row, batch row of the slice)
    uint16_t* D2p = D2 + (int64_t)p * d2_path;
    for (int e = threadIdx.x; e < 32 * bs; e += 64 * NW1) {
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
                z = fmaf(qv_s[jr * l + k], t, z);
            }
        }
        for (int k = 0; k < l; ++k) {
            uint16_t h[3] = {0, 0, 0};
            if (jj < r) split3_bf16(qu_s[jr * l + k] * z, h);
#pragma unroll
            for (int t3 = 0; t3 < 3; ++t3) D2p[dfrag_index(blockIdx.y, 3 * (bl * l + k) + t3, jj, r_pad / KB)] = h[t3];
        }
    }
}

// Pass 2: rows i of S_A, summed over the paths; D2 columns of batch slice [b0, b0 + bs).
template <int NB>
__global__ __launch_bounds__(64 * NW2) void mdbf_pass2(fqm_mdbf md, const uint16_t* __restrict__ D2,
                                                      void* __restrict__ y, int y_f32, int64_t n, int batch,
                                                      int64_t r_pad, int64_t d2_path) {
    __shared__ float red_buf[NW2 / 2 * NB * 1024];
    __shared__ float red[NB * 1024];
    __shared__ float amp_s[2][32 * 16];  // A_amp rows i0 .. i0 + 31 of each path
    const int l = md.l;
    const int64_t r = md.r;
    const int bs = batch_slice(l);
    const int b0 = blockIdx.y * bs, nb_rows = min(bs, batch - b0);
    const int64_t i0 = (int64_t)blockIdx.x * 32;
    // the epilogue's envelope values, fetched before the long sign products
    // (unconditional loads at a clamped index, path 0 standing in for a
    // missing path 1, so that no wait lands here)
    uint16_t amp_h[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int64_t ao = i0 * l + threadIdx.x;
        const bool ain = p < md.P && threadIdx.x < 32 * l && ao < n * l;
        const uint16_t* ap = p < md.P ? md.path[p].A_amp : md.path[0].A_amp;
        const uint16_t a_l = ap[min(ao, n * l - 1)];
        amp_h[p] = ain ? a_l : 0;
    }
    const int wave = threadIdx.x >> 6;
    const int nblk = (int)(r_pad / KB);
    const int per = (nblk + NW2 - 1) / NW2;
    const int blk0 = min(wave * per, nblk), blk1 = min(blk0 + per, nblk);

    float out[2] = {0.f, 0.f};  // (row, batch row) pairs e = tid, tid + 512 of this thread
    for (int p = 0; p < md.P; ++p) {
        const fqm_mdbf_path path = p == 0 ? md.path[0] : md.path[1];
        f32x16 acc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[nb][q] = 0.f;
        sign_products<NB>(path.S_A, path.ld_A, n, D2 + (int64_t)p * d2_path, nblk, blockIdx.y, i0, 3 * l * nb_rows,
                          blk0, blk1, acc);
        if (p == 0 && threadIdx.x < 32 * l) {
            amp_s[0][threadIdx.x] = fp16_to_f32(amp_h[0]);
            amp_s[1][threadIdx.x] = fp16_to_f32(amp_h[1]);
        }
        reduce_waves<NB, NW2>(acc, red_buf, red);  // ends with a barrier
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int e = threadIdx.x + 64 * NW2 * h;
            const int ir = e & 31, bl = e >> 5;
            const int64_t ii = i0 + ir;
            if (bl >= nb_rows || ii >= n) continue;
            float v = out[h];
            for (int k = 0; k < l; ++k) {
                const int cl = 3 * (bl * l + k);
                float t = 0.f;
#pragma unroll
                for (int t3 = 0; t3 < 3; ++t3) t += red[((cl + t3) >> 5) * 1024 + ir * 32 + ((cl + t3) & 31)];
                v = fmaf(amp_s[p][ir * l + k], t, v);
            }
            out[h] = v;
        }
        __syncthreads();  // red is rewritten by the next path
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int e = threadIdx.x + 64 * NW2 * h;
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
    hipLaunchKernelGGL((mdbf_pass1<NB>), dim3((unsigned)(d.r_pad / 32), gy, (unsigned)md.P), dim3(64 * NW1), 0, s,
                       md, D1, D2, w.cols, batch, d.m_pad, d.r_pad, d.d1_path, d.d2_path);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((mdbf_pass2<NB>), dim3((unsigned)((w.rows + 31) / 32), gy), dim3(64 * NW2), 0, s, md, D2, y,
                       y_f32, w.rows, batch, d.r_pad, d.d2_path);
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
                       d.m_pad, d.d1_path);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int bs = batch_slice(md.l);
    const int cols_per_wg = 3 * md.l * std::min(bs, batch);
    return cols_per_wg <= 32 ? launch_nb<1>(w, x, y, y_f32, batch, D1, D2, d, s)
                             : launch_nb<2>(w, x, y, y_f32, batch, D1, D2, d, s);
}

}  // namespace fqm
