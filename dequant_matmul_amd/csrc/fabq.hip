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
//
// With vector centroids (corr = V[tier][cb_base + idx_b][k mod 128]) the
// correction of a block does not factor into c * sum x, but it depends on
// the row only through (tier, idx_b): the block's term is
//   G[b][blk][16 tier + idx] = sum_{k in blk} V[tier][cb_base + idx][k mod 128] x[b][k],
// one value per batch row, block and active centroid (4 tiers x 16).  A first
// launch folds x into G (the workspace); the GEMV then adds one G value per
// binary row and block, so no centroid vector is read per weight.
#include "fqm_internal.h"

namespace fqm {
namespace {

constexpr int kWaves = 4;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Eight bf16 +-1.0 from one sign byte: bit e set -> +1.0, clear -> -1.0.
__device__ __forceinline__ bf16x8_t signs_to_bf16(uint32_t byte) {
    const uint32_t nb = ~byte;
    u32x4_t v;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t t = (nb >> (2 * d)) & 3u;  // sign bits of elements 2d, 2d + 1
        v[d] = 0x3F803F80u | (((t | (t << 15)) & 0x10001u) << 15);
    }
    return __builtin_bit_cast(bf16x8_t, v);
}

typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));

// The 32 signs of one sign dword as 16 bf16 pairs of +-1.0 (element 2j in
// the low half of pair j, 2j+1 in the high half; bit set -> +1.0): the two
// 16-bit halves of a dword holding two copies of the relevant half of ~d are
// shifted by different amounts at once, which puts the sign of element 2j at
// bit 15 and that of 2j+1 at bit 31.
__device__ __forceinline__ void signs32_to_bf16(uint32_t d, uint32_t ones, uint32_t (&v)[16]) {
    const uint32_t nd = ~d;
    const uint32_t lo = __builtin_amdgcn_perm(nd, nd, 0x01000100u);  // (nd[15:0], nd[15:0])
    const uint32_t hi = __builtin_amdgcn_perm(nd, nd, 0x03020302u);  // (nd[31:16], nd[31:16])
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const u16x2_t sh = {(uint16_t)(15 - 2 * (j & 7)), (uint16_t)(14 - 2 * (j & 7))};
        const u16x2_t t = __builtin_bit_cast(u16x2_t, j < 8 ? lo : hi) << sh;
        v[j] = (__builtin_bit_cast(uint32_t, t) & 0x80008000u) | ones;  // ones = bf16 (1, 1) in a register
    }
}

// a.lo * b.lo + a.hi * b.hi + c for bf16 pairs, fp32 accumulate
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                          false);
}

// G (vector centroids): one workgroup per (batch row, block).  The 64 active
// centroid vectors' residues the block touches (all 128 for blocks of 128
// columns or more, else the block's own bs) are staged transposed in LDS
// (s_v[j][e], rows of 65 floats: conflict-free stores and reads) and the
// block's x in fp32; thread (q, e) sums the quarter q of the block's columns
// for centroid e, and the four quarters are added in order.
__global__ __launch_bounds__(256) void fabq_vec_fold(fqm_fabq f, const uint16_t* __restrict__ x,
                                                     float* __restrict__ G, int64_t cols, int nblk) {
    __shared__ float s_v[128 * 65];
    __shared__ float s_x[512];
    __shared__ float s_p[4][64];
    const int tid = threadIdx.x, bs = f.blocksize;
    const int blk = blockIdx.x % nblk, b = blockIdx.x / nblk;
    const int64_t k0 = (int64_t)blk * bs;
    const int nj = min(bs, 128);        // residues touched: j0 .. j0 + nj - 1
    const int j0 = (int)(k0 & 127);     // 0 when bs >= 128; bs divides 128 otherwise, so no wrap
    // every load goes out before the first store: float4 piece i = tid + 256 u
    // of the 64 x nj slice (indices past it repeat the last piece), and x
    // elements tid, tid + 256 of the block (clamped likewise)
    const int n4 = 16 * nj;  // float4 pieces
    float4 vv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int i = min(tid + 256 * u, n4 - 1), e = (4 * i) / nj, jj = 4 * i - e * nj;
        vv[u] = *reinterpret_cast<const float4*>(
            f.vcodebook + (int64_t)(64 * (e >> 4) + f.cb_base + (e & 15)) * 128 + j0 + jj);
    }
    uint16_t xb[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) xb[u] = x[(int64_t)b * cols + k0 + min(tid + 256 * u, bs - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int i = min(tid + 256 * u, n4 - 1), e = (4 * i) / nj, jj = 4 * i - e * nj;
        s_v[(jj + 0) * 65 + e] = vv[u].x;
        s_v[(jj + 1) * 65 + e] = vv[u].y;
        s_v[(jj + 2) * 65 + e] = vv[u].z;
        s_v[(jj + 3) * 65 + e] = vv[u].w;
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) s_x[min(tid + 256 * u, bs - 1)] = bf16_to_f32(xb[u]);
    __syncthreads();
    const int e = tid & 63, q = tid >> 6;
    float acc = 0.f;
#pragma unroll 8
    for (int k = q; k < bs; k += 4) acc = fmaf(s_v[(k & (nj - 1)) * 65 + e], s_x[k], acc);
    s_p[q][e] = acc;
    __syncthreads();
    if (tid < 64)
        G[((int64_t)b * nblk + blk) * 64 + tid] = ((s_p[0][tid] + s_p[1][tid]) + s_p[2][tid]) + s_p[3][tid];
}

// Vector-ALU kernel, one stored row per wave (batch 1..3, and every batch
// for blocks of 16 columns or vector centroids).  Every lane runs the same
// number of steps (indices past the row are clamped and their results dropped
// by a select), so each group of U steps issues all its loads before the
// first use; the row's output slot, high-row scale and its 16 active
// centroids (one pair per lane, looked up across lanes; the tier's window in
// the tiered mode) are requested up front.  A sign dword covers 32 columns:
// one block, part of one, or (16-column blocks) two, so its products are
// summed per 16-column half.  VEC: the correction of each block is its G
// value, added by the lane whose dword starts the block.
// XL: x (B rows, cols % 32 == 0) is staged in LDS once per workgroup, every
// wave then reads it there instead of through the vector L1.  16-byte piece
// n of an x row sits at piece slot (n & ~3) | ((n & 3) ^ ((n >> 4) & 3)), so
// that both access patterns hit 16 distinct 16-byte bank slots per 16 lanes:
// a binary row's lane p reads pieces 4p + h (h = 0..3, one instruction each),
// an int row's lane p reads piece p.
template <int B, bool VEC, bool XL>
__global__ __launch_bounds__(64 * kWaves) void fabq_gemv_kernel(fqm_fabq f, const uint16_t* __restrict__ x,
                                                        void* __restrict__ y, int y_f32,
                                                        int64_t rows, int64_t cols, const float* __restrict__ G) {
    constexpr int UI = B == 1 ? 5 : 1;             // high-row steps per group (64 dwords of fields each)
    constexpr int UB = B == 1 ? 3 : 1;             // binary steps per group (64 dwords of 32 signs each)
    extern __shared__ __attribute__((aligned(16))) uint4 s_xl[];
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t np = cols / 8;  // 16-byte x pieces per batch row
    if constexpr (XL) {
        const uint4* xg = reinterpret_cast<const uint4*>(x);
        for (int64_t g = threadIdx.x; g < B * np; g += 64 * kWaves) {
            const int64_t b = g / np, n = g - b * np;
            s_xl[b * np + ((n & ~3) | ((n & 3) ^ ((n >> 4) & 3)))] = xg[g];
        }
        __syncthreads();
    }
    // x piece n (8 columns) of batch row b
    auto xpiece = [&](int b, int64_t n) -> uint4 {
        if constexpr (XL) return s_xl[b * np + ((n & ~3) | ((n & 3) ^ ((n >> 4) & 3)))];
        else return reinterpret_cast<const uint4*>(x + (int64_t)b * cols)[min(n, np - 1)];  // past the row: unused
    };
    const int64_t i_u = (int64_t)blockIdx.x * kWaves + wave;  // stored row
    if (i_u >= rows) return;
    const int64_t i = i_u;
    const int64_t n_lo = rows - f.n_hi;
    const bool has_bin = n_lo > 0;
    const int64_t j = max(i - (int64_t)f.n_hi, (int64_t)0);        // binary row (when i >= n_hi)
    const int tier = (has_bin && f.cb_mode != FQM_CB_SCALAR16) ? f.tier[min(j, n_lo - 1)] : 0;
    const int cbase = 64 * tier + (f.cb_mode != FQM_CB_SCALAR16 ? f.cb_base : 0);
    // unconditional loads (x stands in for an array the matrix does not have)
    const uint32_t cbits = *(reinterpret_cast<const uint32_t*>((has_bin && !VEC) ? f.codebook + cbase : x) +
                             (lane & 7));
    const int32_t out_row = f.row_of[i];
    const uint16_t hbits = *(f.n_hi > 0 ? f.s_hi + min(i, (int64_t)f.n_hi - 1) : x);

    float acc[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = 0.f;

    if (i < f.n_hi && f.hi_bits == 8) {
        // int8 row: two dwords = 8 fields = 8 columns per lane step.
        const uint2* q = reinterpret_cast<const uint2*>(f.q4 + i * f.ld_q4);
        const int64_t nw = cols / 8;
        for (int64_t p0 = 0; p0 < nw; p0 += 64 * UI) {
            uint2 d[UI];
            uint4 xv[UI][B];
#pragma unroll
            for (int u = 0; u < UI; ++u) {
                const int64_t p = min(p0 + 64 * u + lane, nw - 1);
                d[u] = q[p];
#pragma unroll
                for (int b = 0; b < B; ++b) xv[u][b] = xpiece(b, p);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < UI; ++u) {
                const bool ok = p0 + 64 * u + lane < nw;
                float wq[8];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    wq[jj] = (float)((int32_t)(d[u].x << (24 - 8 * jj)) >> 24);
                    wq[4 + jj] = (float)((int32_t)(d[u].y << (24 - 8 * jj)) >> 24);
                }
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    const uint32_t xs[4] = {xv[u][b].x, xv[u][b].y, xv[u][b].z, xv[u][b].w};
                    float a = acc[b];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        a = fmaf(wq[2 * jj], bf16lo(xs[jj]), a);
                        a = fmaf(wq[2 * jj + 1], bf16hi(xs[jj]), a);
                    }
                    acc[b] = ok ? a : acc[b];
                }
            }
        }
        const float s = fp16_to_f32(hbits);
#pragma unroll
        for (int b = 0; b < B; ++b) acc[b] *= s;
    } else if (i < f.n_hi) {
        // int4 row: one dword = 8 nibbles = 8 columns per lane step.
        const uint32_t* q = reinterpret_cast<const uint32_t*>(f.q4 + i * f.ld_q4);
        const int64_t nw = cols / 8;
        for (int64_t p0 = 0; p0 < nw; p0 += 64 * UI) {
            uint32_t d[UI];
            uint4 xv[UI][B];
#pragma unroll
            for (int u = 0; u < UI; ++u) {
                const int64_t p = min(p0 + 64 * u + lane, nw - 1);
                d[u] = q[p];
#pragma unroll
                for (int b = 0; b < B; ++b) xv[u][b] = xpiece(b, p);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < UI; ++u) {
                const bool ok = p0 + 64 * u + lane < nw;
                float wq[8];
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) wq[jj] = (float)((int32_t)(d[u] << (28 - 4 * jj)) >> 28);
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    const uint32_t xs[4] = {xv[u][b].x, xv[u][b].y, xv[u][b].z, xv[u][b].w};
                    float a = acc[b];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        a = fmaf(wq[2 * jj], bf16lo(xs[jj]), a);
                        a = fmaf(wq[2 * jj + 1], bf16hi(xs[jj]), a);
                    }
                    acc[b] = ok ? a : acc[b];
                }
            }
        }
        const float s = fp16_to_f32(hbits);
#pragma unroll
        for (int b = 0; b < B; ++b) acc[b] *= s;
    } else {
        // binary row: one dword = 32 sign bits, columns 32 p .. 32 p + 31.
        uint32_t ones = 0x3F803F80u;  // bf16 (1, 1), held in a register
        asm volatile("" : "+v"(ones));
        const uint32_t* sg = reinterpret_cast<const uint32_t*>(f.signs + j * f.ld_signs);
        const int64_t nb = cols / f.blocksize;
        const uint16_t* sb = f.s_blk + j * nb;
        const uint8_t* ib = f.idx + j * f.ld_idx;
        const bool bs16 = f.blocksize == 16;
        const int wshift = bs16 ? 0 : __builtin_ctz((unsigned)f.blocksize) - 5;  // log2(sign dwords per block)
        const int nw = (int)((cols + 31) / 32);  // 16-column blocks: the last dword may hold one block
        for (int p0 = 0; p0 < nw; p0 += 64 * UB) {
            uint32_t d[UB];
            uint16_t sbits[UB][2];
            uint8_t ibits[UB];
            int bodd[UB];
            uint4 xv[UB][B][4];
#pragma unroll
            for (int u = 0; u < UB; ++u) {
                const int p = min(p0 + 64 * u + lane, nw - 1);
                const int blk = bs16 ? 2 * p : p >> wshift;  // block of the dword's first half
                d[u] = sg[p];
                sbits[u][0] = sb[blk];
                sbits[u][1] = sb[bs16 ? min(blk + 1, (int)nb - 1) : blk];
                ibits[u] = ib[blk >> 1];
                bodd[u] = blk & 1;
#pragma unroll
                for (int b = 0; b < B; ++b)
#pragma unroll
                    for (int h = 0; h < 4; ++h)
                        xv[u][b][h] = xpiece(b, 4 * (int64_t)p + h);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < UB; ++u) {
                const bool ok = p0 + 64 * u + lane < nw;
                const float s0 = fp16_to_f32(sbits[u][0]), s1 = fp16_to_f32(sbits[u][1]);
                // centroid of each half: bs16 -> the byte's two nibbles, else one nibble twice
                const int id0 = bs16 ? (ibits[u] & 15) : (ibits[u] >> (4 * bodd[u])) & 15;
                const int id1 = bs16 ? (ibits[u] >> 4) : id0;
                float c0 = 0.f, c1 = 0.f;
                // VEC: this dword starts block blk0 (always with 16-column
                // blocks, whose second half is block blk0 + 1 when it exists)
                int blk0 = 0;
                bool first = false, second = false;
                if (VEC) {
                    const int p = min(p0 + 64 * u + lane, nw - 1);
                    blk0 = bs16 ? 2 * p : p >> wshift;
                    first = bs16 || (p & ((1 << wshift) - 1)) == 0;
                    second = bs16 && 32 * (int64_t)p + 16 < cols;
                } else {
                    const uint32_t cp0 = (uint32_t)__shfl((int)cbits, id0 >> 1);
                    const uint32_t cp1 = (uint32_t)__shfl((int)cbits, id1 >> 1);
                    c0 = fp16_to_f32((uint16_t)(cp0 >> (16 * (id0 & 1))));
                    c1 = fp16_to_f32((uint16_t)(cp1 >> (16 * (id1 & 1))));
                }
                // the 32 signs as bf16 +-1.0 pairs: products with x are exact
                uint32_t sv[16];
                signs32_to_bf16(d[u], ones, sv);
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    float ps[2] = {0.f, 0.f}, xsum[2] = {0.f, 0.f};
                    float g0 = 0.f, g1 = 0.f;
                    if (VEC) {
                        const float* gb = G + (int64_t)b * nb * 64 + 16 * (tier & 3);
                        if (first) g0 = gb[(int64_t)blk0 * 64 + id0];
                        if (second) g1 = gb[(int64_t)(blk0 + 1) * 64 + id1];
                    }
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        const int half = h >> 1;
                        const uint32_t xs[4] = {xv[u][b][h].x, xv[u][b][h].y, xv[u][b][h].z, xv[u][b][h].w};
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            ps[half] = dot2_bf16(sv[4 * h + t], xs[t], ps[half]);
                            if (!VEC) xsum[half] = dot2_bf16(ones, xs[t], xsum[half]);
                        }
                    }
                    if (32 * (p0 + 64 * u + lane) + 16 >= cols) {  // the dword's second half is past the row
                        ps[1] = 0.f;
                        xsum[1] = 0.f;
                    }
                    float a = acc[b];
                    if (VEC) {
                        a = fmaf(s0, ps[0], fmaf(s1, ps[1], a + (g0 + g1)));
                    } else {
                        a = fmaf(s0, ps[0], fmaf(c0, xsum[0], a));
                        a = fmaf(s1, ps[1], fmaf(c1, xsum[1], a));
                    }
                    acc[b] = ok ? a : acc[b];
                }
            }
        }
    }
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

// ---------------------------------------------------------------------------
// Matrix-core kernel (batch >= 4, blocks of 32 columns or more, scalar
// centroids).  A workgroup owns 16 stored rows
// (one v_mfma_f32_16x16x32_bf16 row block); its 8 waves split the row's
// 32-wide k slices.  Every weight enters the product exactly as a bf16: a
// sign bit as +-1.0, an int4 or int8 value as itself (HI8: int8 high rows),
// and x is bf16 already, so each product is exact and sums in fp32.  Per block a wave scales its partial
// sum: binary rows add s_b * (sum of +-x) over the wave's slices of the
// block (linear, so the waves' parts add up to the block's); int4 rows add
// the plain sum and take the row scale at the end.  The codebook term
// c[idx_b] * (sum of x over the wave's slices of block b) takes its sum of x
// from a second MFMA per slice with an all-ones row operand (the matrix
// cores are otherwise idle; no vector instructions per slice).  The per-block
// scales and centroid values of the 16 rows (the row's tier window in the
// tiered mode) are staged in LDS first, so a flush reads LDS only.  The waves' results are added in
// wave order.  A row block that is all binary (or all int4) decodes only its
// own kind; a mixed one decodes both and selects per lane.
// Latency shapes the loop: the first slices' loads go out before the tables
// are filled, and each group's loads go out before the previous group's
// products; no global load depends on another.
// ---------------------------------------------------------------------------

constexpr int kMW = 8;        // waves per workgroup
constexpr int kGS = 2;        // slices whose loads a wave issues together (2: -15 % against 8; 1 within 2 %)
constexpr int kMaxNB = 256;   // blocks per row the LDS tables hold (larger: VALU kernel)

// Eight bf16 from eight 8-bit two's complement fields (field e at bits 8e of
// the 64-bit lo | hi << 32), exact.
__device__ __forceinline__ bf16x8_t bytes_to_bf16(uint32_t lo, uint32_t hi) {
    u32x4_t v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t d = e < 2 ? lo : hi;
        const int sh = 16 * (e & 1);
        const float a = (float)((int32_t)(d << (24 - sh)) >> 24);
        const float b = (float)((int32_t)(d << (16 - sh)) >> 24);
        v[e] = (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xFFFF0000u);
    }
    return __builtin_bit_cast(bf16x8_t, v);
}

// Eight bf16 from eight 4-bit two's complement fields (field e at bits 4e), exact.
__device__ __forceinline__ bf16x8_t nibbles_to_bf16(uint32_t d) {
    u32x4_t v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float lo = (float)((int32_t)(d << (28 - 8 * e)) >> 28);
        const float hi = (float)((int32_t)(d << (24 - 8 * e)) >> 28);
        v[e] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
    }
    return __builtin_bit_cast(bf16x8_t, v);
}

template <bool HI8>
__global__ __launch_bounds__(64 * kMW) __attribute__((amdgpu_waves_per_eu(HI8 ? 2 : 4))) void fabq_gemv_mfma_kernel(fqm_fabq f, const uint16_t* __restrict__ x,
                                                                  void* __restrict__ y, int y_f32, int rows,
                                                                  int cols, int batch, const float* __restrict__ G) {
    __shared__ float s_sc[16 * kMaxNB];     // [row][blk]: s_b (binary) or 1 (high rows)
    __shared__ float s_cv[16 * kMaxNB];     // [row][blk]: the block's centroid (binary) or 0 (high rows, vector centroids)
    __shared__ uint8_t s_e[16 * kMaxNB];    // vector centroids: [row][blk] the G entry 16 tier + idx of binary rows
    __shared__ f32x4_t s_red[kMW * 64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r0 = blockIdx.x * 16;
    const int bs = f.blocksize, nblk = cols / bs, spb = bs / 32;

    // A operand: stored row r0 + lane % 16, k = 32 t + 8 g + e (g = lane / 16)
    const int g = lane >> 4;
    const int ra = min(r0 + (lane & 15), rows - 1);
    const bool a_int4 = ra < f.n_hi;  // a high-precision row (int4, or int8 with HI8)
    // the same loads either way (no branch around them): int4 rows the dword
    // of 8 fields at byte 16 t + 4 g, int8 rows the two dwords of 8 fields at
    // byte 32 t + 8 g, binary rows the dword at byte 4 t holding sign byte g
    // (read twice where int8 rows read two)
    const uint8_t* arow = a_int4 ? f.q4 + (int64_t)ra * f.ld_q4 + (HI8 ? 8 : 4) * g
                                 : f.signs + (int64_t)(ra - f.n_hi) * f.ld_signs;
    const int astep = a_int4 ? (HI8 ? 32 : 16) : 4;
    const int ahi = (HI8 && a_int4) ? 4 : 0;
    const int ashift = a_int4 ? 0 : 8 * g;
    // B operand: batch row lane % 16 (rows past the batch repeat the last one; never stored)
    const uint16_t* xrow = x + (int64_t)min(lane & 15, batch - 1) * cols + 8 * g;
    // D rows of this lane: 4 g + i (i = 0..3), column (batch row) lane % 16

    const int ns = cols / 32;
    const int t0 = (wave * ns) / kMW, t1 = ((wave + 1) * ns) / kMW;  // this wave's slices
    // loads of the group of slices starting at base into register set q
    // (indices past the wave's last slice repeat it, or slice 0 for a wave
    // without slices; never used)
    uint32_t wq[2][kGS];
    uint32_t wq2[2][HI8 ? kGS : 1];
    u32x4_t xv[2][kGS];
    auto load_group = [&](int q, int base) {
#pragma unroll
        for (int u = 0; u < kGS; ++u) {
            const int t = max(min(base + u, t1 - 1), 0);
            wq[q][u] = *reinterpret_cast<const uint32_t*>(arow + astep * t);
            if constexpr (HI8) wq2[q][u] = *reinterpret_cast<const uint32_t*>(arow + astep * t + ahi);
            xv[q][u] = *reinterpret_cast<const u32x4_t*>(xrow + 32 * t);
        }
    };
    // Per-block scales and indices of the 16 rows (rows past the end repeat
    // the last): table item e = tid + 64 kMW p goes to [row][blk].  The raw
    // fields of the first pass are requested before the first group of
    // weights and stored after it, so the two latencies overlap; their loads
    // are unconditional (clamped index; x stands in for the binary-row arrays
    // when there are no binary rows, and the values are then not used).
    const int ne = 16 * nblk;
    const bool has_bin = f.n_hi < rows;
    const int e0 = min(tid, ne - 1);
    const int er = e0 / nblk, eb = e0 - er * nblk;
    const int esr = min(r0 + er, rows - 1);
    const int64_t ejb = max(esr - f.n_hi, 0);
    const uint16_t* ps = has_bin ? f.s_blk + ejb * nblk + eb : x;
    const uint8_t* pi = has_bin ? f.idx + ejb * f.ld_idx + (eb >> 1) : reinterpret_cast<const uint8_t*>(x);
    const bool tiered = f.cb_mode == FQM_CB_TIERED, vec = f.cb_mode == FQM_CB_VECTOR;
    const uint8_t* pt = (has_bin && f.cb_mode != FQM_CB_SCALAR16) ? f.tier + ejb : reinterpret_cast<const uint8_t*>(x);
    const uint16_t sraw = *ps;
    const uint8_t iraw = *pi, traw = *pt;
    __builtin_amdgcn_sched_barrier(0);
    load_group(0, t0);  // unconditional, so the waits below count exactly
    // the output row and int4 row scale this thread stores at the end
    const int srow = min(r0 + ((tid >> 4) & 15), rows - 1);
    const int32_t out_row = f.row_of[srow];
    const uint16_t hraw = *(f.n_hi > 0 ? f.s_hi + min(srow, f.n_hi - 1) : x);  // used for int4 rows only

    // centroid of binary row jb's block: the codebook entry, or the row's
    // tier window entry
    auto centroid = [&](int64_t jb, uint32_t id, uint32_t t) {
        return vec ? 0.f : fp16_to_f32(f.codebook[(tiered ? 64 * t + f.cb_base : 0) + id]);
    };
    if (tid < ne) {
        const bool bin = esr >= f.n_hi;
        const uint32_t id = (iraw >> ((eb & 1) * 4)) & 15u;
        s_sc[er * kMaxNB + eb] = bin ? fp16_to_f32(sraw) : 1.f;
        s_cv[er * kMaxNB + eb] = bin ? centroid(ejb, id, traw) : 0.f;
        s_e[er * kMaxNB + eb] = (uint8_t)(16 * (traw & 3u) + id);
    }
    for (int e = tid + 64 * kMW; e < ne; e += 64 * kMW) {  // blocks shorter than 5120 / 32 columns
        const int r = e / nblk, blk = e - r * nblk;
        const int sr = min(r0 + r, rows - 1);
        float sc = 1.f, cv = 0.f;
        uint32_t ge = 0;
        if (sr >= f.n_hi) {
            const int64_t jb = sr - f.n_hi;
            const uint32_t id = (f.idx[jb * f.ld_idx + (blk >> 1)] >> ((blk & 1) * 4)) & 15u;
            const uint32_t t = f.cb_mode != FQM_CB_SCALAR16 ? f.tier[jb] : 0u;
            sc = fp16_to_f32(f.s_blk[jb * nblk + blk]);
            cv = centroid(jb, id, t);
            ge = 16 * (t & 3u) + id;
        }
        s_sc[r * kMaxNB + blk] = sc;
        s_cv[r * kMaxNB + blk] = cv;
        s_e[r * kMaxNB + blk] = (uint8_t)ge;
    }
    __syncthreads();  // tables

    f32x4_t total = {0.f, 0.f, 0.f, 0.f}, acc = {0.f, 0.f, 0.f, 0.f};
    f32x4_t accx = {0.f, 0.f, 0.f, 0.f};  // every row: the sum of x over the block's slices so far
    const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
    auto flush = [&](int blk) {
        const float xb = accx[0];  // the wave's part of the block's sum of x, batch row lane % 16
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i;
            const float cv = s_cv[r * kMaxNB + blk];
            total[i] = fmaf(s_sc[r * kMaxNB + blk], acc[i], fmaf(cv, xb, total[i]));
            acc[i] = 0.f;
            accx[i] = 0.f;
        }
    };
    // kind of the row block: 0 all binary, 1 all int4, 2 mixed (uniform)
    const int kind = r0 >= f.n_hi ? 0 : (min(r0 + 16, rows) <= f.n_hi ? 1 : 2);
    int cur = t0 / spb;  // block of the running sums
    auto group = [&](auto qc, int base) {
        constexpr int q = decltype(qc)::value;
        if (base + kGS < t1) load_group(q ^ 1, base + kGS);
#pragma unroll
        for (int u = 0; u < kGS; ++u) {
            const int t = base + u;
            if (t >= t1) break;
            const int blk = t / spb;
            if (blk != cur) {
                flush(cur);
                cur = blk;
            }
            bf16x8_t av;
            auto high = [&]() {
                if constexpr (HI8) return bytes_to_bf16(wq[q][u], wq2[q][u]);
                else return nibbles_to_bf16(wq[q][u]);
            };
            if (kind == 0) {
                av = signs_to_bf16((wq[q][u] >> ashift) & 255u);
            } else if (kind == 1) {
                av = high();
            } else {
                const u32x4_t ai = __builtin_bit_cast(u32x4_t, high());
                const u32x4_t as = __builtin_bit_cast(u32x4_t, signs_to_bf16((wq[q][u] >> ashift) & 255u));
                av = __builtin_bit_cast(bf16x8_t, a_int4 ? ai : as);
            }
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, xv[q][u]), acc, 0, 0, 0);
            accx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, __builtin_bit_cast(bf16x8_t, xv[q][u]), accx, 0, 0, 0);
        }
    };
    for (int base = t0; base < t1; base += 2 * kGS) {
        group(std::integral_constant<int, 0>{}, base);
        if (base + kGS < t1) group(std::integral_constant<int, 1>{}, base + kGS);
    }
    if (t0 < t1) flush(cur);

    // waves' results in wave order; int4 rows take their row scale
    s_red[wave * 64 + lane] = total;
    __syncthreads();
    if (tid < 256) {
        const int row = tid >> 4, col = tid & 15;  // stored row r0 + row, batch row col
        const int l = 16 * (row >> 2) + col, i = row & 3;
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < kMW; ++w) v += s_red[w * 64 + l][i];
        const int sr = r0 + row;
        if (sr < rows && col < batch) {
            v *= srow < f.n_hi ? fp16_to_f32(hraw) : 1.f;
            if (vec && srow >= f.n_hi) {  // vector centroids: the binary row's G values, block by block
                const float* gb = G + (int64_t)col * nblk * 64;
                float gs = 0.f;
                for (int blk = 0; blk < nblk; ++blk) gs += gb[(int64_t)blk * 64 + s_e[row * kMaxNB + blk]];
                v += gs;
            }
            const int64_t o = (int64_t)col * rows + out_row;
            if (y_f32)
                reinterpret_cast<float*>(y)[o] = v;
            else
                reinterpret_cast<uint16_t*>(y)[o] = f32_to_bf16(v);
        }
    }
}

// x goes through LDS when it takes at most this many bytes (B rows).
constexpr int64_t kMaxXL = 64 * 1024;

template <int B>
hipError_t launch_b(const fqm_weights& w, const uint16_t* x, void* y, int y_f32, const float* G, hipStream_t s) {
    const unsigned grid = (unsigned)((w.rows + kWaves - 1) / kWaves);
    const int64_t xl = (int64_t)B * w.cols * 2;
    const bool use_xl = w.cols % 32 == 0 && xl <= kMaxXL;
    if (w.fabq.cb_mode == FQM_CB_VECTOR) {
        if (use_xl)
            hipLaunchKernelGGL((fabq_gemv_kernel<B, true, true>), dim3(grid), dim3(64 * kWaves), (size_t)xl, s,
                               w.fabq, x, y, y_f32, w.rows, w.cols, G);
        else
            hipLaunchKernelGGL((fabq_gemv_kernel<B, true, false>), dim3(grid), dim3(64 * kWaves), 0, s, w.fabq, x,
                               y, y_f32, w.rows, w.cols, G);
    } else {
        if (use_xl)
            hipLaunchKernelGGL((fabq_gemv_kernel<B, false, true>), dim3(grid), dim3(64 * kWaves), (size_t)xl, s,
                               w.fabq, x, y, y_f32, w.rows, w.cols, G);
        else
            hipLaunchKernelGGL((fabq_gemv_kernel<B, false, false>), dim3(grid), dim3(64 * kWaves), 0, s, w.fabq, x, y,
                               y_f32, w.rows, w.cols, G);
    }
    return hipGetLastError();
}

}  // namespace

// Vector centroids need G: batch x blocks x 64 fp32 in the workspace, when
// the layer has binary rows.
size_t fabq_workspace_bytes(const fqm_weights& w, int batch) {
    const fqm_fabq& f = w.fabq;
    if (f.cb_mode != FQM_CB_VECTOR || w.rows <= f.n_hi || w.cols <= 0 || f.blocksize <= 0) return 0;
    const size_t n = (size_t)batch * (size_t)(w.cols / f.blocksize) * 64 * sizeof(float);
    return (n + 15) / 16 * 16;
}

// The matrix-core kernel takes batch >= 4 when blocks are at least 32 columns
// (a 32-wide k slice never holds two blocks), the per-block tables of 16 rows
// fit its LDS (cols / blocksize <= 256) and the sizes fit 32 bits; the VALU
// kernel takes the rest (at batch 1 it is the faster one: 8.8 against 19 us on
// the 5120 x 5120 layer, where 8 batch rows take 31 against 23 us).
hipError_t launch_fabq_gemv(const fqm_weights& w, const uint16_t* x, void* y, int y_f32,
                            int batch, float* ws, hipStream_t s) {
    fqm_weights v = w;
    if (!v.fabq.hi_bits) v.fabq.hi_bits = 4;
    const fqm_fabq& f = v.fabq;
    const float* G = nullptr;
    if (fabq_workspace_bytes(v, batch)) {
        if (!ws || v.cols / f.blocksize > 0x7fffffff / 16 || (int64_t)batch * (v.cols / f.blocksize) > 0x7fffffff)
            return hipErrorInvalidValue;
        const int nblk = (int)(v.cols / f.blocksize);
        hipLaunchKernelGGL(fabq_vec_fold, dim3((unsigned)(batch * nblk)), dim3(256), 0, s, f, x, ws, v.cols, nblk);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        G = ws;
    }
    if (batch >= 4 && f.blocksize >= 32 && v.cols / f.blocksize <= kMaxNB && v.rows <= 0x7fffffff &&
        v.cols <= 0x7fffffff) {
        if (f.hi_bits == 8)
            hipLaunchKernelGGL(fabq_gemv_mfma_kernel<true>, dim3((unsigned)((v.rows + 15) / 16)), dim3(64 * kMW), 0, s,
                               f, x, y, y_f32, (int)v.rows, (int)v.cols, batch, G);
        else
            hipLaunchKernelGGL(fabq_gemv_mfma_kernel<false>, dim3((unsigned)((v.rows + 15) / 16)), dim3(64 * kMW), 0,
                               s, f, x, y, y_f32, (int)v.rows, (int)v.cols, batch, G);
        return hipGetLastError();
    }
    switch (batch) {
        case 1: return launch_b<1>(v, x, y, y_f32, G, s);
        case 2: return launch_b<2>(v, x, y, y_f32, G, s);
        case 3: return launch_b<3>(v, x, y, y_f32, G, s);
        case 4: return launch_b<4>(v, x, y, y_f32, G, s);
        case 5: return launch_b<5>(v, x, y, y_f32, G, s);
        case 6: return launch_b<6>(v, x, y, y_f32, G, s);
        case 7: return launch_b<7>(v, x, y, y_f32, G, s);
        case 8: return launch_b<8>(v, x, y, y_f32, G, s);
        case 9: return launch_b<9>(v, x, y, y_f32, G, s);
        case 10: return launch_b<10>(v, x, y, y_f32, G, s);
        case 11: return launch_b<11>(v, x, y, y_f32, G, s);
        case 12: return launch_b<12>(v, x, y, y_f32, G, s);
        case 13: return launch_b<13>(v, x, y, y_f32, G, s);
        case 14: return launch_b<14>(v, x, y, y_f32, G, s);
        case 15: return launch_b<15>(v, x, y, y_f32, G, s);
        case 16: return launch_b<16>(v, x, y, y_f32, G, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fqm
