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

// Vector-ALU kernel (batch 1..3), one stored row per wave.  Every lane runs
// the same number of steps (indices past the row are clamped and their
// results dropped by a select), so each group of U steps issues all its loads
// before the first use; the row's output slot, int4 scale and the codebook
// (one centroid per lane, looked up across lanes) are requested up front.
template <int B>
__global__ __launch_bounds__(256) void fabq_gemv_kernel(fqm_fabq f, const uint16_t* __restrict__ x,
                                                        void* __restrict__ y, int y_f32,
                                                        int64_t rows, int64_t cols) {
    constexpr int UI = B == 1 ? 5 : 1;  // int4 steps per group (64 dwords of 8 fields each)
    constexpr int UB = B == 1 ? 3 : 1;  // binary steps per group (64 dwords of 32 signs each)
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t i_u = (int64_t)blockIdx.x * kWaves + wave;  // stored row
    if (i_u >= rows) return;
    const int64_t i = i_u;
    const bool has_bin = f.n_hi < rows;
    // unconditional loads (x stands in for an array the matrix does not have)
    const uint32_t cbits = *(reinterpret_cast<const uint32_t*>(has_bin ? f.codebook : x) + (lane & 7));
    const int32_t out_row = f.row_of[i];
    const uint16_t hbits = *(f.n_hi > 0 ? f.s_hi + min(i, (int64_t)f.n_hi - 1) : x);

    float acc[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = 0.f;

    if (i < f.n_hi) {
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
                for (int b = 0; b < B; ++b) xv[u][b] = *reinterpret_cast<const uint4*>(x + (int64_t)b * cols + 8 * p);
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
        // binary row: one dword = 32 sign bits; a block (>= 64 columns) holds whole dwords.
        // centroids 2 (lane % 8) and 2 (lane % 8) + 1 (fp16 pairs), read across lanes where used
        uint32_t ones = 0x3F803F80u;  // bf16 (1, 1), held in a register
        asm volatile("" : "+v"(ones));
        const int64_t j = i - f.n_hi;
        const uint32_t* sg = reinterpret_cast<const uint32_t*>(f.signs + j * f.ld_signs);
        const int64_t nb = cols / f.blocksize;
        const uint16_t* sb = f.s_blk + j * nb;
        const uint8_t* ib = f.idx + j * f.ld_idx;
        const int wshift = __builtin_ctz((unsigned)f.blocksize) - 5;  // log2(sign dwords per block)
        const int nw = (int)(cols / 32);
        for (int p0 = 0; p0 < nw; p0 += 64 * UB) {
            uint32_t d[UB];
            uint16_t sbits[UB];
            uint8_t ibits[UB];
            int bodd[UB];
            uint4 xv[UB][B][4];
#pragma unroll
            for (int u = 0; u < UB; ++u) {
                const int p = min(p0 + 64 * u + lane, nw - 1);
                const int blk = p >> wshift;
                d[u] = sg[p];
                sbits[u] = sb[blk];
                ibits[u] = ib[blk >> 1];
                bodd[u] = blk & 1;
#pragma unroll
                for (int b = 0; b < B; ++b)
#pragma unroll
                    for (int h = 0; h < 4; ++h)
                        xv[u][b][h] = reinterpret_cast<const uint4*>(x + (int64_t)b * cols + 32 * p)[h];
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < UB; ++u) {
                const bool ok = p0 + 64 * u + lane < nw;
                const float s = fp16_to_f32(sbits[u]);
                const int id = (ibits[u] >> (4 * bodd[u])) & 15;
                const uint32_t cpair = (uint32_t)__shfl((int)cbits, id >> 1);
                const float c = fp16_to_f32((uint16_t)(cpair >> (16 * (id & 1))));
                // the 32 signs as bf16 +-1.0 pairs: products with x are exact
                uint32_t sv[16];
                signs32_to_bf16(d[u], ones, sv);
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    float ps = 0.f, xsum = 0.f;
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        const uint32_t xs[4] = {xv[u][b][h].x, xv[u][b][h].y, xv[u][b][h].z, xv[u][b][h].w};
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            ps = dot2_bf16(sv[4 * h + t], xs[t], ps);
                            xsum = dot2_bf16(ones, xs[t], xsum);
                        }
                    }
                    const float a = fmaf(s, ps, fmaf(c, xsum, acc[b]));
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
// Matrix-core kernel (every batch 1..16).  A workgroup owns 16 stored rows
// (one v_mfma_f32_16x16x32_bf16 row block); its 8 waves split the row's
// 32-wide k slices.  Every weight enters the product exactly as a bf16: a
// sign bit as +-1.0, an int4 value as itself, and x is bf16 already, so each
// product is exact and sums in fp32.  Per block a wave scales its partial
// sum: binary rows add s_b * (sum of +-x) over the wave's slices of the
// block (linear, so the waves' parts add up to the block's); int4 rows add
// the plain sum and take the row scale at the end.  The codebook term
// c[idx_b] * (sum of x over the wave's slices of block b) takes its sum of x
// from a second MFMA per slice with an all-ones row operand (the matrix
// cores are otherwise idle; no vector instructions per slice).  The per-block scales and centroids of the 16 rows are staged in LDS
// first, so a flush reads LDS only.  The waves' results are added in
// wave order.  A row block that is all binary (or all int4) decodes only its
// own kind; a mixed one decodes both and selects per lane.
// Latency shapes the loop: the first slices' loads go out before the tables
// are filled, and each group's loads go out before the previous group's
// products; no global load depends on another.
// ---------------------------------------------------------------------------

constexpr int kMW = 8;        // waves per workgroup
constexpr int kGS = 8;        // slices whose loads a wave issues together
constexpr int kMaxNB = 256;   // blocks per row the LDS tables hold (larger: VALU kernel)

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

__global__ __launch_bounds__(64 * kMW) __attribute__((amdgpu_waves_per_eu(4))) void fabq_gemv_mfma_kernel(fqm_fabq f, const uint16_t* __restrict__ x,
                                                                  void* __restrict__ y, int y_f32, int rows,
                                                                  int cols, int batch) {
    __shared__ float s_sc[16 * kMaxNB];     // [row][blk]: s_b (binary) or 1 (int4)
    __shared__ uint8_t s_ix[16 * kMaxNB];   // [row][blk]: idx_b (binary) or 16 (int4: centroid 0)
    __shared__ float s_cb[17];              // centroids, and 0 at 16
    __shared__ f32x4_t s_red[kMW * 64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r0 = blockIdx.x * 16;
    const int bs = f.blocksize, nblk = cols / bs, spb = bs / 32;

    // A operand: stored row r0 + lane % 16, k = 32 t + 8 g + e (g = lane / 16)
    const int g = lane >> 4;
    const int ra = min(r0 + (lane & 15), rows - 1);
    const bool a_int4 = ra < f.n_hi;
    // one dword per slice either way (no branch around the loads): int4 rows
    // the dword of 8 fields at byte 16 t + 4 g, binary rows the dword at byte
    // 4 t holding sign byte g
    const uint8_t* arow = a_int4 ? f.q4 + (int64_t)ra * f.ld_q4 + 4 * g
                                 : f.signs + (int64_t)(ra - f.n_hi) * f.ld_signs;
    const int astep = a_int4 ? 16 : 4;
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
    u32x4_t xv[2][kGS];
    auto load_group = [&](int q, int base) {
#pragma unroll
        for (int u = 0; u < kGS; ++u) {
            const int t = max(min(base + u, t1 - 1), 0);
            wq[q][u] = *reinterpret_cast<const uint32_t*>(arow + astep * t);
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
    const uint16_t* pcb = has_bin ? f.codebook + (tid & 15) : x;
    const uint16_t sraw = *ps, craw = *pcb;
    const uint8_t iraw = *pi;
    __builtin_amdgcn_sched_barrier(0);
    load_group(0, t0);  // unconditional, so the waits below count exactly
    // the output row and int4 row scale this thread stores at the end
    const int srow = min(r0 + ((tid >> 4) & 15), rows - 1);
    const int32_t out_row = f.row_of[srow];
    const uint16_t hraw = *(f.n_hi > 0 ? f.s_hi + min(srow, f.n_hi - 1) : x);  // used for int4 rows only

    if (tid < ne) {
        const bool bin = esr >= f.n_hi;
        s_sc[er * kMaxNB + eb] = bin ? fp16_to_f32(sraw) : 1.f;
        s_ix[er * kMaxNB + eb] = bin ? (uint8_t)((iraw >> ((eb & 1) * 4)) & 15u) : (uint8_t)16;
    }
    for (int e = tid + 64 * kMW; e < ne; e += 64 * kMW) {  // blocks shorter than 5120 / 32 columns
        const int r = e / nblk, blk = e - r * nblk;
        const int sr = min(r0 + r, rows - 1);
        float sc = 1.f;
        uint32_t ix = 16u;
        if (sr >= f.n_hi) {
            const int64_t jb = sr - f.n_hi;
            sc = fp16_to_f32(f.s_blk[jb * nblk + blk]);
            ix = (f.idx[jb * f.ld_idx + (blk >> 1)] >> ((blk & 1) * 4)) & 15u;
        }
        s_sc[r * kMaxNB + blk] = sc;
        s_ix[r * kMaxNB + blk] = (uint8_t)ix;
    }
    if (tid < 17) s_cb[tid] = (tid < 16 && has_bin) ? fp16_to_f32(craw) : 0.f;
    __syncthreads();  // tables

    f32x4_t total = {0.f, 0.f, 0.f, 0.f}, acc = {0.f, 0.f, 0.f, 0.f};
    f32x4_t accx = {0.f, 0.f, 0.f, 0.f};  // every row: the sum of x over the block's slices so far
    const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
    auto flush = [&](int blk) {
        const float xb = accx[0];  // the wave's part of the block's sum of x, batch row lane % 16
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i;
            const float cv = s_cb[s_ix[r * kMaxNB + blk]];
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
            if (kind == 0) {
                av = signs_to_bf16((wq[q][u] >> ashift) & 255u);
            } else if (kind == 1) {
                av = nibbles_to_bf16(wq[q][u]);
            } else {
                const u32x4_t ai = __builtin_bit_cast(u32x4_t, nibbles_to_bf16(wq[q][u]));
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
            const int64_t o = (int64_t)col * rows + out_row;
            if (y_f32)
                reinterpret_cast<float*>(y)[o] = v;
            else
                reinterpret_cast<uint16_t*>(y)[o] = f32_to_bf16(v);
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

// The matrix-core kernel takes batch >= 4 when the per-block tables of 16
// rows fit its LDS (cols / blocksize <= 256) and the sizes fit 32 bits; the
// VALU kernel takes the rest (at batch 1 it is the faster one: 8.8 against
// 19 us on the 5120 x 5120 layer, where 8 batch rows take 31 against 23 us).
hipError_t launch_fabq_gemv(const fqm_weights& w, const uint16_t* x, void* y, int y_f32,
                            int batch, hipStream_t s) {
    if (batch >= 4 && w.cols / w.fabq.blocksize <= kMaxNB && w.rows <= 0x7fffffff && w.cols <= 0x7fffffff) {
        hipLaunchKernelGGL(fabq_gemv_mfma_kernel, dim3((unsigned)((w.rows + 15) / 16)), dim3(64 * kMW), 0, s,
                           w.fabq, x, y, y_f32, (int)w.rows, (int)w.cols, batch);
        return hipGetLastError();
    }
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
