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
// envelope k and batch row b).  They run on v_mfma_f32_16x16x32_bf16 (fp32
// accumulate): the +-1 matrix is the 16-row A operand, one sign byte per lane
// and k step, and the dense columns are the B operand, 16 per column block.
// Each dense fp32 column v enters as three bf16 columns, h0 = bf16(v),
// h1 = bf16(v - h0), h2 = bf16(v - h0 - h1), whose sum carries the fp32 value
// (u is an exact fp32 product, v a rounded one).
//
// A sign byte becomes eight bf16 +-1.0 with one byte permute and, per pair of
// elements, one packed 16-bit shift and one v_and_or_b32.  The expansion maps
// a set bit to -1.0 (the bf16 sign bit is the stored bit itself); the sums
// are negated once in the epilogue, which is exact.
//
// Three launches:
//   prep:   D1 = parts of u_k[i], column 3 (b l + k) + t of batch slice b / bs;
//   pass 1: sign products over S_B, then z and D2 = parts of v_k[j];
//   pass 2: sign products over S_A for every path, then y.
// D1 and D2 are stored fragment-major: for each batch slice, 16-column block,
// 512-wide K block and 32-wide k step s (0..15), the 64 lanes' 16-byte B
// operand pieces are contiguous.  Lane (c, q) = (lane % 16, lane / 16) holds
// column c at k = 128 q + 8 s + e (e = 0..7) of the block, and the A operand
// of the same lane holds sign byte 16 q + s of its row's 64 bytes for the
// block, so one 16-byte load gives a lane its signs for the whole block.
// Both operands use one k order, so only the order of the fp32 sums differs
// from plain k order.
// A workgroup owns 16 rows and a batch slice; its waves take the K blocks in
// turn (wave w: blocks w, w + nw, ...), loading the next half block while
// the current one issues its MFMAs.  The waves' partial sums are added in
// wave order in LDS, so results do not depend on timing.  Columns past the
// logical width hold zeros in D1/D2, so sign bits read there (the padding of
// the last byte, or a clamped row) contribute nothing.
#include <algorithm>

#include "fqm_internal.h"

namespace fqm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) uint8_t lds8;
typedef __attribute__((address_space(3))) const u32x4 lds128c;
typedef __attribute__((address_space(3))) uint32_t lds32;

constexpr int KB = 512;      // columns per K block (16 MFMA k steps of 32)
constexpr int BLK = 8192;    // elements of one (column block, K block) operand piece: 16 steps x 64 lanes x 8

__host__ __device__ inline int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// batch rows per workgroup: their 3 l bs dense columns fit four 16-column blocks
__host__ __device__ inline int batch_slice(int l) { return 3 * l >= 64 ? 1 : 64 / (3 * l); }

struct MdbfDims {
    int64_t m_pad, r_pad;     // padded K widths of D1 and D2
    int nsg, ncb, bs;         // batch slices, 16-column blocks per slice, batch rows per slice
    int64_t d1_path, d2_path; // elements of one path's D1 / D2
    size_t d1_elems, d2_elems;
};

__host__ __device__ inline MdbfDims mdbf_dims(int64_t m, int64_t r, int l, int P, int batch) {
    MdbfDims d;
    d.bs = batch_slice(l);
    d.m_pad = round_up(m, KB);
    d.r_pad = round_up(r, KB);
    d.nsg = (batch + d.bs - 1) / d.bs;
    d.ncb = (3 * l * std::min(d.bs, batch) + 15) / 16;
    d.d1_path = (int64_t)d.nsg * d.ncb * d.m_pad * 16;
    d.d2_path = (int64_t)d.nsg * d.ncb * d.r_pad * 16;
    d.d1_elems = (size_t)P * d.d1_path;
    d.d2_elems = (size_t)P * d.d2_path;
    return d;
}

// Element index of column col of batch slice sg at k in a fragment-major
// operand (ncb column blocks, nkb K blocks).
__device__ __forceinline__ int64_t dfrag_index(int sg, int ncb, int col, int64_t k, int64_t nkb) {
    const int cb = col >> 4, c = col & 15;
    const int64_t kb = k >> 9;
    const int rem = (int)(k & 511);
    const int q = rem >> 7, s = (rem >> 3) & 15, e = rem & 7;
    return (((int64_t)(sg * ncb + cb) * nkb + kb) * 16 + s) * 512 + (c + 16 * q) * 8 + e;
}

// v = h0 + h1 + h2 (bf16 parts; each remainder is exact in fp32)
__device__ __forceinline__ void split3_bf16(float v, uint16_t (&h)[3]) {
    h[0] = f32_to_bf16(v);
    const float r1 = v - bf16_to_f32(h[0]);
    h[1] = f32_to_bf16(r1);
    h[2] = f32_to_bf16(r1 - bf16_to_f32(h[1]));
}

// Eight bf16 +-1.0 from byte S of the dword w: element e is -1.0 where bit e
// is set, +1.0 where it is clear.  The byte goes to both 16-bit halves; for
// the dword of elements 2d (low half) and 2d + 1 (high half) a packed shift
// by (15 - 2d, 14 - 2d) puts those two bits at bits 15 and 31, the bf16 sign
// bits, and v_and_or_b32 keeps them (mask = 0x80008000) and adds the
// exponent of 1.0 (ones = 0x3F803F80).  With mask = ones = 0 the operand is
// all zeros.  ones is held in a VGPR so that the mask can be the
// instruction's one scalar operand.
template <int S>
__device__ __forceinline__ bf16x8 expand_signs_neg(uint32_t w, uint32_t mask, uint32_t ones) {
    constexpr uint32_t sel = 0x0C000C00u | (uint32_t)(S << 16) | (uint32_t)S;
    const u16x2 p = __builtin_bit_cast(u16x2, __builtin_amdgcn_perm(w, w, sel));
    u32x4 v;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const u16x2 t = p << (u16x2){(unsigned short)(15 - 2 * d), (unsigned short)(14 - 2 * d)};
        v[d] = (__builtin_bit_cast(uint32_t, t) & mask) | ones;
    }
    return __builtin_bit_cast(bf16x8, v);
}

// D1 of path p: parts of u_k[i] at column 3 (b l + k) + t of batch slice
// b / bs; zero for i >= m.  One thread writes one lane's 16-byte piece of one
// k step: grid (4 nkb, nsg ncb, P), 256 threads = 4 k steps x 64 lanes.
__global__ __launch_bounds__(256) void mdbf_prep(fqm_mdbf md, const uint16_t* __restrict__ x,
                                                 uint16_t* __restrict__ D1, int64_t m, int batch, int nsg,
                                                 int ncb, int64_t nkb, int64_t d1_path) {
    const int lane = threadIdx.x & 63;
    const int64_t kb = blockIdx.x >> 2;
    const int s = 4 * (blockIdx.x & 3) + (threadIdx.x >> 6);
    const int sg = blockIdx.y / ncb, cb = blockIdx.y - sg * ncb;
    const int p = blockIdx.z;
    const int l = md.l, bs = batch_slice(l);
    const int c = lane & 15, q = lane >> 4;
    const int col = 16 * cb + c;
    const int nrows = min(bs, batch - sg * bs);
    if (col >= 3 * l * nrows) return;  // never read
    const int bl = col / (3 * l), rem = col - bl * 3 * l, k = rem / 3, t3 = rem - 3 * k;
    const int64_t b = (int64_t)sg * bs + bl;
    const int64_t i0 = kb * KB + 128 * q + 8 * s;
    const uint16_t* bamp = p == 0 ? md.path[0].B_amp : md.path[1].B_amp;
    u32x4 out;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        uint16_t h0[3] = {0, 0, 0}, h1[3] = {0, 0, 0};
        const int64_t i = i0 + e;
        if (i < m) {  // m is a multiple of 32, so i + 1 < m as well
            split3_bf16(fp16_to_f32(bamp[i * l + k]) * bf16_to_f32(x[b * m + i]), h0);
            split3_bf16(fp16_to_f32(bamp[(i + 1) * l + k]) * bf16_to_f32(x[b * m + i + 1]), h1);
        }
        const uint16_t lo = t3 == 0 ? h0[0] : t3 == 1 ? h0[1] : h0[2];
        const uint16_t hi = t3 == 0 ? h1[0] : t3 == 1 ? h1[1] : h1[2];
        out[e >> 1] = (uint32_t)lo | ((uint32_t)hi << 16);
    }
    uint16_t* dp = D1 + (int64_t)p * d1_path + (((int64_t)(sg * ncb + cb) * nkb + kb) * 16 + s) * 512 + 8 * lane;
    *reinterpret_cast<u32x4*>(dp) = out;
}

// The dense pieces of one quarter block (4 k steps) of NB column blocks.
template <int NB>
struct Half {
    u32x4 d[NB][4];
};

// Sign products for one path: acc[nb] = -(S[row0 .. row0 + 15][:] * (dense
// columns 16 nb + (0..15) of batch slice sg)^T) over this wave's K blocks,
// wave, wave + nw, ..., in chunks of BPW blocks.  A chunk is straight-line
// code with no branch between a load and its use, so the loads stay where
// they are written and the waits before the MFMAs are exact:
// - the signs of the whole chunk (the stream from HBM, 16 bytes per lane and
//   block) go out first, the next chunk's after this one's MFMAs;
// - the dense pieces run AHEAD quarter blocks ahead of their MFMAs;
// - a block past nkb re-reads block nkb - 1 and its A operand is all zeros
//   (the launch picks BPW so that such blocks are rare).
// The dense pieces come from D (global, fragment-major) or, with LDSD, from
// the compact copy at LDS byte address dl: for each K block and k step, the
// four lane quarters q of ce live columns, 16 bytes each.
// pre() runs once in every wave, after its first chunk's sign loads are
// issued and before any dense piece is read.
// Reads stay inside the operands:
// - a row's signs are its first kbytes = ceil(K / 8) bytes; a 16-byte piece
//   that starts at or past them is read at the last 16-byte piece that
//   starts inside them, so a row is read up to kbytes rounded up to 16 (at
//   most 15 bytes past kbytes, inside the row's ld), and the dense operand is
//   zero for every k >= K, so whatever those bits hold adds nothing;
// - a lane whose column is at or past cend reads the piece of column
//   cend - 1 (the same bytes as a live lane of the instruction) and only
//   feeds result columns that are never read.
template <int NB, int BPW, bool LDSD = false, typename Pre>
__device__ __forceinline__ void sign_products(const uint8_t* __restrict__ S, int64_t ldS, int64_t rows,
                                              int64_t kbytes, const uint16_t* __restrict__ D, uint32_t dl,
                                              int64_t nkb, int sg, int ncb, int64_t row0, int cend, int wave,
                                              int nw, f32x4 (&acc)[NB], Pre pre) {
    static_assert(!LDSD || NB == 1, "the LDS copy holds one column block");
    constexpr int T = 4 * BPW;                     // quarter blocks per chunk
    constexpr int AHEAD = NB > 1 ? 1 : BPW >= 4 ? 3 : 2;  // dense quarter blocks in flight ahead (fits the VGPRs)
    constexpr int NBUF = AHEAD + 1;
    const int lane = threadIdx.x & 63, c = lane & 15, q = lane >> 4;
    const uint8_t* srow = S + min(row0 + c, rows - 1) * ldS;
    const int64_t klast = (kbytes - 1) & ~(int64_t)15;
    const uint16_t* dcol[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int col = min(16 * nb + c, cend - 1);
        dcol[nb] = D + (int64_t)(sg * ncb + (col >> 4)) * nkb * BLK + 8 * ((col & 15) + 16 * q);
    }
    const uint32_t dlane = dl + 16u * (uint32_t)(q * cend + min(c, cend - 1));
    uint32_t ones;
    asm("v_mov_b32 %0, 0x3f803f80" : "=v"(ones));
    int64_t blk[BPW];
    u32x4 sgn[BPW];
    auto load_signs = [&](int64_t base) {
#pragma unroll
        for (int j = 0; j < BPW; ++j) {
            blk[j] = min(base + (int64_t)j * nw, nkb - 1);
            sgn[j] = *reinterpret_cast<const u32x4*>(srow + min(64 * blk[j] + 16 * q, klast));
        }
    };
    load_signs(wave);
    pre();
    for (int64_t base = wave; base < nkb; base += (int64_t)BPW * nw) {
        Half<NB> hb[NBUF];
        auto load_d = [&](int t) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int ks = 4 * (t % 4) + s;  // k step within the block
                    if constexpr (LDSD)
                        hb[t % NBUF].d[nb][s] =
                            *(lds128c*)(uintptr_t)(dlane + 64u * (uint32_t)cend * (uint32_t)(blk[t / 4] * 16 + ks));
                    else
                        hb[t % NBUF].d[nb][s] = *reinterpret_cast<const u32x4*>(dcol[nb] + blk[t / 4] * BLK + 512 * ks);
                }
        };
#pragma unroll
        for (int t = 0; t < AHEAD; ++t) load_d(t);
#pragma unroll
        for (int t = 0; t < T; ++t) {
            if (t + AHEAD < T) load_d(t + AHEAD);
            // the machine scheduler would otherwise move each load down to
            // its first use (to lower register pressure), so that every MFMA
            // waited for its own load
            __builtin_amdgcn_sched_barrier(0);
            const bool live = base + (int64_t)(t / 4) * nw < nkb;  // uniform over the wave
            const uint32_t mask = live ? 0x80008000u : 0u, one = live ? ones : 0u;
            bf16x8 a[4];
            const uint32_t sw = sgn[t / 4][t % 4];
            a[0] = expand_signs_neg<0>(sw, mask, one);
            a[1] = expand_signs_neg<1>(sw, mask, one);
            a[2] = expand_signs_neg<2>(sw, mask, one);
            a[3] = expand_signs_neg<3>(sw, mask, one);
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        a[s], __builtin_bit_cast(bf16x8, hb[t % NBUF].d[nb][s]), acc[nb], 0, 0, 0);
        }
        if (base + (int64_t)BPW * nw < nkb) load_signs(base + (int64_t)BPW * nw);
    }
}

// Sum of the nw waves' 16 x 16NB partial blocks in wave order into tot
// (LDS), negated: D layout of a 16x16 block is lane l, item i -> row
// 4 (l / 16) + i, column l % 16.  red holds nw x NB x 64 float4.
template <int NB>
__device__ __forceinline__ void reduce_waves(const f32x4 (&acc)[NB], f32x4* red, float* tot, int nw) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) red[(wave * NB + nb) * 64 + lane] = acc[nb];
    __syncthreads();
    for (int e = tid; e < NB * 256; e += 64 * nw) {
        const int nb = e >> 8, ln = (e >> 2) & 63, i = e & 3;
        float v = 0.f;
        for (int w = 0; w < nw; ++w) v += red[(w * NB + nb) * 64 + ln][i];
        tot[e] = -v;
    }
    __syncthreads();
}

// Column col, row (0..15) of the reduced tile.
__device__ __forceinline__ float tot_at(const float* tot, int col, int row) {
    return tot[(col >> 4) * 256 + ((col & 15) + 16 * (row >> 2)) * 4 + (row & 3)];
}

// Most waves per workgroup (a 512-thread group may use 256 VGPRs).  The
// launch keeps every floor on the wave count (at most 6) under this.
constexpr int NWM = 8;

// Pass 1: rows j of S_B; D1 columns of batch slice blockIdx.y.  Writes
// D2[p][.][j] = parts of Q_U[j][k] z[j] (zero for j >= r, which the grid
// covers up to r_pad).
// FUSE (one column block, ce m_pad 2 bytes <= FUSE_LDS): the workgroup forms
// the parts of u_k itself, from x and B_amp, in a compact LDS copy (the ce =
// 3 l rows live columns of its slice in the fragment order), and reads its
// dense operand there; D1 and the prep launch are not used.
constexpr int FUSE_LDS = 65536;
constexpr int FILL_PAIRS = 8;  // pairs of k per thread whose loads go out together in the fill

template <int NB, int BPW, bool FUSE>
__global__ __launch_bounds__(64 * NWM) void mdbf_pass1(fqm_mdbf md, const uint16_t* __restrict__ x,
                                                        const uint16_t* __restrict__ D1,
                                                        uint16_t* __restrict__ D2, int64_t m, int batch, int ncb,
                                                        int64_t m_pad, int64_t r_pad, int64_t d1_path,
                                                        int64_t d2_path) {
    __shared__ uint32_t dlds[FUSE ? FUSE_LDS / 4 : 1];
    __shared__ f32x4 red[NWM * NB * 64];
    __shared__ float tot[NB * 256];
    __shared__ float qv_s[16 * 16], qu_s[16 * 16];  // Q_V, Q_U rows j0 .. j0 + 15
    const int p = blockIdx.z;
    const fqm_mdbf_path path = p == 0 ? md.path[0] : md.path[1];
    const int l = md.l;
    const int64_t r = md.r;
    const int bs = batch_slice(l);
    const int sg = blockIdx.y;
    const int b0 = sg * bs, nb_rows = min(bs, batch - b0);
    const int64_t j0 = (int64_t)blockIdx.x * 16;
    const int nw = blockDim.x >> 6, wave = threadIdx.x >> 6;
    // the epilogue's envelope values, fetched before the sign products
    // (unconditional loads at a clamped index, so that no wait lands here)
    const int64_t qo = j0 * l + threadIdx.x;
    const bool qin = threadIdx.x < 16 * l && qo < r * l;
    const int64_t qoc = min(qo, r * l - 1);
    const uint16_t qv_l = path.Q_V[qoc], qu_l = path.Q_U[qoc];
    const uint16_t qv_h = qin ? qv_l : 0, qu_h = qin ? qu_l : 0;

    f32x4 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
    const int ce = 3 * l * nb_rows;
    if (j0 < r) {
        const uint32_t dl = (uint32_t)(uintptr_t)(lds8*)dlds;
        // the parts of u_k[i] = B_amp[i][k] x[b][i] for this slice: item
        // (bk = bl l + k, pair of i), written as two bf16 per dword at column
        // 3 bk + t of k step (i % 512) / 8 of K block i / 512; zero for i >= m
        auto fill = [&]() {
            if constexpr (FUSE) {
                const uint16_t* bamp = p == 0 ? md.path[0].B_amp : md.path[1].B_amp;
                const int64_t npair = m_pad / 2;
                constexpr int FP = FILL_PAIRS;
                for (int bk = 0; bk < l * nb_rows; ++bk) {
                    const int bl = bk / l, k = bk - bl * l;
                    const uint16_t* xr = x + (int64_t)(b0 + bl) * m;
                    for (int64_t p0 = threadIdx.x; p0 < npair; p0 += (int64_t)FP * blockDim.x) {
                        uint16_t xv[FP][2], bv[FP][2];
#pragma unroll
                        for (int j = 0; j < FP; ++j) {
                            const int64_t i = 2 * (p0 + (int64_t)j * blockDim.x);
                            const int64_t ic = i < m ? i : 0;  // m is a multiple of 32: i < m means i + 1 < m
                            xv[j][0] = xr[ic];
                            xv[j][1] = xr[ic + 1];
                            bv[j][0] = bamp[ic * l + k];
                            bv[j][1] = bamp[(ic + 1) * l + k];
                        }
#pragma unroll
                        for (int j = 0; j < FP; ++j) {
                            const int64_t i = 2 * (p0 + (int64_t)j * blockDim.x);
                            if (i >= m_pad) break;
                            uint16_t h0[3] = {0, 0, 0}, h1[3] = {0, 0, 0};
                            if (i < m) {
                                split3_bf16(fp16_to_f32(bv[j][0]) * bf16_to_f32(xv[j][0]), h0);
                                split3_bf16(fp16_to_f32(bv[j][1]) * bf16_to_f32(xv[j][1]), h1);
                            }
                            const int rem = (int)(i & 511), qq = rem >> 7, ks = (rem >> 3) & 15, e = rem & 7;
                            const uint32_t at =
                                dl + 16u * (uint32_t)((((i >> 9) * 16 + ks) * 4 + qq) * ce) + 2u * e;
#pragma unroll
                            for (int t3 = 0; t3 < 3; ++t3)
                                *(lds32*)(uintptr_t)(at + 16u * (uint32_t)(3 * bk + t3)) =
                                    (uint32_t)h0[t3] | ((uint32_t)h1[t3] << 16);
                        }
                    }
                }
                __syncthreads();
            }
        };
        sign_products<NB, BPW, FUSE>(path.S_B, path.ld_B, r, m / 8, D1 + (int64_t)p * d1_path, dl, m_pad / KB, sg,
                                     ncb, j0, ce, wave, nw, acc, fill);
    }
    if (threadIdx.x < 16 * l) {
        qv_s[threadIdx.x] = fp16_to_f32(qv_h);
        qu_s[threadIdx.x] = fp16_to_f32(qu_h);
    }
    reduce_waves<NB>(acc, red, tot, nw);  // ends with a barrier

    // one thread per (row, batch row of the slice)
    uint16_t* D2p = D2 + (int64_t)p * d2_path;
    const int64_t nkb2 = r_pad / KB;
    for (int e = threadIdx.x; e < 16 * nb_rows; e += blockDim.x) {
        const int jr = e & 15, bl = e >> 4;
        const int64_t jj = j0 + jr;
        float z = 0.f;
        if (jj < r) {
            for (int k = 0; k < l; ++k) {
                const int cl = 3 * (bl * l + k);
                const float t = tot_at(tot, cl, jr) + tot_at(tot, cl + 1, jr) + tot_at(tot, cl + 2, jr);
                z = fmaf(qv_s[jr * l + k], t, z);
            }
        }
        for (int k = 0; k < l; ++k) {
            uint16_t h[3] = {0, 0, 0};
            if (jj < r) split3_bf16(qu_s[jr * l + k] * z, h);
#pragma unroll
            for (int t3 = 0; t3 < 3; ++t3) D2p[dfrag_index(sg, ncb, 3 * (bl * l + k) + t3, jj, nkb2)] = h[t3];
        }
    }
}

// Pass 2: rows i of S_A, summed over the paths; D2 columns of batch slice blockIdx.y.
template <int NB, int BPW>
__global__ __launch_bounds__(64 * NWM) void mdbf_pass2(fqm_mdbf md, const uint16_t* __restrict__ D2,
                                                        void* __restrict__ y, int y_f32, int64_t n, int batch,
                                                        int ncb, int64_t r_pad, int64_t d2_path) {
    __shared__ f32x4 red[NWM * NB * 64];
    __shared__ float tot[NB * 256];
    __shared__ float amp_s[2][16 * 16];  // A_amp rows i0 .. i0 + 15 of each path
    const int l = md.l;
    const int64_t r = md.r;
    const int bs = batch_slice(l);
    const int sg = blockIdx.y;
    const int b0 = sg * bs, nb_rows = min(bs, batch - b0);
    const int64_t i0 = (int64_t)blockIdx.x * 16;
    const int nw = blockDim.x >> 6, wave = threadIdx.x >> 6;
    // the epilogue's envelope values, fetched before the sign products
    // (unconditional loads at a clamped index, path 0 standing in for a
    // missing path 1, so that no wait lands here)
    uint16_t amp_h[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int64_t ao = i0 * l + threadIdx.x;
        const bool ain = p < md.P && threadIdx.x < 16 * l && ao < n * l;
        const uint16_t* ap = p < md.P ? md.path[p].A_amp : md.path[0].A_amp;
        const uint16_t a_l = ap[min(ao, n * l - 1)];
        amp_h[p] = ain ? a_l : 0;
    }
    const int64_t nkb = r_pad / KB;

    float out = 0.f;  // (row, batch row) pair e = tid of this thread (the launch gives 64 nw >= 16 bs)
    const int ir = threadIdx.x & 15, bl = threadIdx.x >> 4;
    for (int p = 0; p < md.P; ++p) {
        const fqm_mdbf_path path = p == 0 ? md.path[0] : md.path[1];
        f32x4 acc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
        sign_products<NB, BPW>(path.S_A, path.ld_A, n, (r + 7) / 8, D2 + (int64_t)p * d2_path, 0u, nkb, sg, ncb, i0,
                          3 * l * nb_rows, wave, nw, acc, [] {});
        if (p == 0 && threadIdx.x < 16 * l) {
            amp_s[0][threadIdx.x] = fp16_to_f32(amp_h[0]);
            amp_s[1][threadIdx.x] = fp16_to_f32(amp_h[1]);
        }
        reduce_waves<NB>(acc, red, tot, nw);  // ends with a barrier
        if (bl < nb_rows && i0 + ir < n) {
            float v = out;
            for (int k = 0; k < l; ++k) {
                const int cl = 3 * (bl * l + k);
                const float t = tot_at(tot, cl, ir) + tot_at(tot, cl + 1, ir) + tot_at(tot, cl + 2, ir);
                v = fmaf(amp_s[p][ir * l + k], t, v);
            }
            out = v;
        }
        __syncthreads();  // red and tot are rewritten by the next path
    }
    if (bl < nb_rows && i0 + ir < n) {
        const int64_t o = (int64_t)(b0 + bl) * n + i0 + ir;
        if (y_f32)
            reinterpret_cast<float*>(y)[o] = out;
        else
            reinterpret_cast<uint16_t*>(y)[o] = f32_to_bf16(out);
    }
}

// Blocks per wave and chunk (bpw <= maxb) and waves per workgroup for nkb K
// blocks with at most cap waves: bpw = ceil(nkb / cap) blocks each, then as
// few waves as hold nkb blocks (at least floor); past maxb blocks per wave
// the waves go over their blocks in chunks of maxb.
struct Split {
    int bpw, nw;
};
inline Split split_k(int64_t nkb, int cap, int floor, int maxb) {
    const int bpw = (int)std::min<int64_t>(maxb, (nkb + cap - 1) / cap);
    const int64_t nw = std::min<int64_t>(cap, (nkb + bpw - 1) / bpw);
    return {bpw, (int)std::max<int64_t>(floor, nw)};
}

template <int NB, int BPW, bool FUSE>
hipError_t launch_pass1(const fqm_weights& w, const uint16_t* x, int batch, uint16_t* D1, uint16_t* D2,
                        const MdbfDims& d, int nw, hipStream_t s) {
    hipLaunchKernelGGL((mdbf_pass1<NB, BPW, FUSE>),
                       dim3((unsigned)(d.r_pad / 16), (unsigned)d.nsg, (unsigned)w.mdbf.P), dim3(64 * nw), 0, s,
                       w.mdbf, x, D1, D2, w.cols, batch, d.ncb, d.m_pad, d.r_pad, d.d1_path, d.d2_path);
    return hipGetLastError();
}

template <int NB, int BPW>
hipError_t launch_pass2(const fqm_weights& w, void* y, int y_f32, int batch, uint16_t* D2, const MdbfDims& d,
                        int nw, hipStream_t s) {
    hipLaunchKernelGGL((mdbf_pass2<NB, BPW>), dim3((unsigned)((w.rows + 15) / 16), (unsigned)d.nsg), dim3(64 * nw),
                       0, s, w.mdbf, D2, y, y_f32, w.rows, batch, d.ncb, d.r_pad, d.d2_path);
    return hipGetLastError();
}

// Whether pass 1 forms its dense operand in LDS (no prep launch): one column
// block whose live columns over the padded K fit FUSE_LDS, and few enough
// products that every thread of a nw-wave group fills its share with one
// batch of loads (as a separate launch, prep costs less than a longer fill).
inline bool fuse_prep(const MdbfDims& d, int l, int batch, int nw) {
    const int64_t cols = (int64_t)3 * l * std::min(d.bs, batch);
    return d.ncb == 1 && cols * d.m_pad * 2 <= FUSE_LDS &&
           (int64_t)l * std::min(d.bs, batch) * (d.m_pad / 2) <= (int64_t)FILL_PAIRS * 64 * nw;
}

// Waves per workgroup (pass 1, pass 2) and blocks per wave chunk.
struct Plan {
    Split k1, k2;
};

template <int NB>
Plan plan_passes(const fqm_weights& w, int batch, const MdbfDims& d) {
    const fqm_mdbf& md = w.mdbf;
    // At least one thread per envelope value of the tile's 16 rows (16 l <=
    // 256), and in pass 2 one per (row, batch row) of the slice (16 bs <=
    // 16 * 21).  At most enough waves per tile that tiles x waves is about
    // 4096 (16 waves per CU, all resident at once), and NWM.  Four column
    // blocks take chunks of at most 4 K blocks (their operands fill the VGPRs).
    constexpr int MAXB = NB == 1 ? 8 : 4;
    const int env = (16 * md.l + 63) / 64;
    const int64_t t1 = d.r_pad / 16 * d.nsg * md.P, t2 = (w.rows + 15) / 16 * d.nsg;
    const int f2 = std::max(env, (16 * std::min(d.bs, batch) + 63) / 64);
    const int c1 = (int)std::min<int64_t>(NWM, std::max<int64_t>(env, (4096 + t1 - 1) / t1));
    const int c2 = (int)std::min<int64_t>(NWM, std::max<int64_t>(f2, (4096 + t2 - 1) / t2));
    return {split_k(d.m_pad / KB, c1, env, MAXB), split_k(d.r_pad / KB, c2, f2, MAXB)};
}

template <int NB, bool FUSE>
hipError_t launch_nb(const fqm_weights& w, const uint16_t* x, void* y, int y_f32, int batch, uint16_t* D1,
                     uint16_t* D2, const MdbfDims& d, const Plan& pl, hipStream_t s) {
    constexpr int MAXB = NB == 1 ? 8 : 4;
    const Split k1 = pl.k1, k2 = pl.k2;
    hipError_t e;
    switch (k1.bpw) {
        case 1: e = launch_pass1<NB, 1, FUSE>(w, x, batch, D1, D2, d, k1.nw, s); break;
        case 2: e = launch_pass1<NB, 2, FUSE>(w, x, batch, D1, D2, d, k1.nw, s); break;
        case 3: e = launch_pass1<NB, 3, FUSE>(w, x, batch, D1, D2, d, k1.nw, s); break;
        case 4: e = launch_pass1<NB, 4, FUSE>(w, x, batch, D1, D2, d, k1.nw, s); break;
        case 5: e = launch_pass1<NB, NB == 1 ? 5 : 4, FUSE>(w, x, batch, D1, D2, d, k1.nw, s); break;
        case 6: e = launch_pass1<NB, NB == 1 ? 6 : 4, FUSE>(w, x, batch, D1, D2, d, k1.nw, s); break;
        case 7: e = launch_pass1<NB, NB == 1 ? 7 : 4, FUSE>(w, x, batch, D1, D2, d, k1.nw, s); break;
        default: e = launch_pass1<NB, MAXB, FUSE>(w, x, batch, D1, D2, d, k1.nw, s); break;
    }
    if (e != hipSuccess) return e;
    switch (k2.bpw) {
        case 1: return launch_pass2<NB, 1>(w, y, y_f32, batch, D2, d, k2.nw, s);
        case 2: return launch_pass2<NB, 2>(w, y, y_f32, batch, D2, d, k2.nw, s);
        case 3: return launch_pass2<NB, 3>(w, y, y_f32, batch, D2, d, k2.nw, s);
        case 4: return launch_pass2<NB, 4>(w, y, y_f32, batch, D2, d, k2.nw, s);
        case 5: return launch_pass2<NB, NB == 1 ? 5 : 4>(w, y, y_f32, batch, D2, d, k2.nw, s);
        case 6: return launch_pass2<NB, NB == 1 ? 6 : 4>(w, y, y_f32, batch, D2, d, k2.nw, s);
        case 7: return launch_pass2<NB, NB == 1 ? 7 : 4>(w, y, y_f32, batch, D2, d, k2.nw, s);
        default: return launch_pass2<NB, MAXB>(w, y, y_f32, batch, D2, d, k2.nw, s);
    }
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
    const Plan pl = d.ncb == 1 ? plan_passes<1>(w, batch, d) : plan_passes<4>(w, batch, d);
    if (fuse_prep(d, md.l, batch, pl.k1.nw)) return launch_nb<1, true>(w, x, y, y_f32, batch, D1, D2, d, pl, s);
    hipLaunchKernelGGL(mdbf_prep, dim3((unsigned)(4 * d.m_pad / KB), (unsigned)(d.nsg * d.ncb), (unsigned)md.P),
                       dim3(256), 0, s, md, x, D1, w.cols, batch, d.nsg, d.ncb, d.m_pad / KB, d.d1_path);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // two to four column blocks share the four-block kernels (a block past
    // ncb re-reads a live column and its results are not read)
    return d.ncb == 1 ? launch_nb<1, false>(w, x, y, y_f32, batch, D1, D2, d, pl, s)
                      : launch_nb<4, false>(w, x, y, y_f32, batch, D1, D2, d, pl, s);
}

}  // namespace fqm
