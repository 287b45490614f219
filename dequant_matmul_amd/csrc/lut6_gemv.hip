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

// ---------------------------------------------------------------------------
// Batch 1, cols a multiple of 1024.
//
// A "cell" is 1024 consecutive weights of one row: 64 lanes x one 12-byte
// piece (16 codes) each, 768 contiguous bytes, so a cell is one fully
// coalesced load instruction.  Workgroup g owns rows [g*rows/G, (g+1)*rows/G)
// (at least one row per wave); it stages x (cols bf16) and its rows' tables
// (128 B each) in LDS once, and its waves split the group's cells, taken row
// by row, into equal contiguous ranges of at most NC cells, so no row spans
// more than two waves.  A wave issues the loads of all its cells at once
// (its only HBM traffic) and then works through them in order with no
// branches, so the compiler can overlap one cell's gathers with the next
// cell's address arithmetic.  Per cell a lane does 16 gathers from the row's
// table (one row per instruction: lanes hit distinct banks or share a
// dword), pairs them, and meets the matching x pair in v_dot2_f32_bf16 (fp32
// accumulate).  Each lane stores its running sum into an LDS partial slot
// when a row ends (into a discard slot otherwise); after a barrier every row
// adds its two slots per lane and reduces across the wave with DPP, in a
// fixed order, so the result does not depend on timing.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) const uint16_t lds_u16;
typedef __attribute__((address_space(3))) const u32x4_t lds_u4;
typedef __attribute__((address_space(3))) float lds_f32;

__device__ __forceinline__ float dot2(uint32_t w, uint32_t x, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w),
                                          __builtin_bit_cast(bf16x2_t, x), acc, false);
}

// Code j of a 12-byte piece, shifted so that its 6 bits sit at bits 1..6
// (the byte offset of its table entry) with other bits still to be masked.
template <int J>
__device__ __forceinline__ uint32_t code_x2(uint32_t d0, uint32_t d1, uint32_t d2) {
    constexpr int bit = 6 * J;
    if constexpr (bit == 0) return d0 << 1;
    else if constexpr (bit + 6 <= 32) return d0 >> (bit - 1);
    else if constexpr (bit < 32) return __builtin_amdgcn_alignbit(d1, d0, bit - 1);
    else if constexpr (bit == 32) return d1 << 1;
    else if constexpr (bit + 6 <= 64) return d1 >> (bit - 33);
    else if constexpr (bit < 64) return __builtin_amdgcn_alignbit(d2, d1, bit - 33);
    else if constexpr (bit == 64) return d2 << 1;
    else return d2 >> (bit - 65);
}

constexpr int kB1Waves = 8;    // waves per workgroup (2 per SIMD; two groups per CU)
constexpr int kB1Cells = 22;   // most cells per wave
constexpr int kB1Ring = 8;     // cells in flight per wave
constexpr int kB1Stage = 5;    // 16-byte staging pieces per thread (x and tables)

template <int NC, int D, int CPR>
__global__ __launch_bounds__(64 * kB1Waves) __attribute__((amdgpu_waves_per_eu(4))) void lut6_gemv_b1(
    const uint8_t* __restrict__ packed, int64_t ld, const uint16_t* __restrict__ lut,
    const uint16_t* __restrict__ x, void* __restrict__ y, int y_f32, int rq, int rr) {
    // Workgroup g owns R = rq (+1 for g < rr) rows starting at r0; its cells,
    // row by row, go to the kB1Waves waves in equal contiguous ranges.
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int nw = kB1Waves;
    constexpr int cpr = CPR;  // cells per row = cols / 1024
    constexpr int cols = 1024 * CPR;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = blockIdx.x;
    const int r0 = g * rq + min(g, rr);
    const int R = rq + (g < rr ? 1 : 0);
    const int C = R * cpr;
    const int cb = (w * C) / nw, ce = ((w + 1) * C) / nw;
    const int n = ce - cb;  // cells of this wave, cpr..NC
    const int rl0 = cb / cpr, cj0 = cb - rl0 * cpr;

    // LDS: x [cols] bf16 (swizzled, see staging) | tables [R][64] bf16 |
    //      partials [R][2][64] fp32 | discard slots [nw][64] fp32
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_u8*)smem;
    const uint32_t x_off = lds0;
    const uint32_t tab_off = lds0 + (uint32_t)(cols * 2);
    const uint32_t part_off = tab_off + (uint32_t)R * 128u;
    const uint32_t drop_off = part_off + (uint32_t)R * 512u + (uint32_t)w * 256u;

    // Staging loads for x and the tables go out first (kB1Stage 16-byte
    // pieces per thread), then the cell loads; the staging stores below then
    // wait only for the staging loads.
    const int nx = (int)(cols >> 3), nst = nx + R * 8;
    const u32x4_t* xs = reinterpret_cast<const u32x4_t*>(x);
    const u32x4_t* ts = reinterpret_cast<const u32x4_t*>(lut + r0 * 64);
    u32x4_t stage[kB1Stage];
#pragma unroll
    for (int u = 0; u < kB1Stage; ++u) {
        const int k = min(tid + u * (64 * nw), nst - 1);  // clamped: no branches
        stage[u] = *(k < nx ? xs + k : ts + (k - nx));
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the staging loads ahead of the cell loads

    // Per-cell bookkeeping, computed once: lane e (< NC) holds the values of
    // the wave's cell e, and each cell reads them with v_readlane.  (Done per
    // cell in scalar code this is ~30 SALU instructions a cell, and the CU's
    // scalar pipe, shared by its waves, becomes the bottleneck.)
    // Cell e is column block (cj0 + e) % cpr of row rl0 + (cj0 + e) / cpr;
    // cells past n stand for the last cell (its bytes are read again, an L2
    // hit; its sum is discarded), so every load is issued unconditionally and
    // every wait is exact.
    const uint8_t* wbase = packed + (int64_t)(r0 + rl0) * ld + 768 * cj0;  // wave-uniform
    const uint32_t lofs = 12u * lane;
    uint32_t t_load, t_base, t_xoff, t_dst;
    float t_keep;
    {
        const int e = min(lane, n - 1);
        const int t = cj0 + e, rl = rl0 + t / cpr, cj = t % cpr;
        t_load = (uint32_t)(t / cpr) * (uint32_t)ld + 768u * (uint32_t)(cj - cj0);
        t_base = tab_off + (uint32_t)rl * 128u;
        t_xoff = x_off + (uint32_t)cj * 2048u;
        const bool end = lane < n && (cj == cpr - 1 || lane == n - 1);
        const uint32_t sl = (rl == rl0 && cj0 != 0) ? 1u : 0u;
        t_dst = end ? part_off + ((uint32_t)rl * 2u + sl) * 256u : drop_off;
        t_keep = end ? 0.f : 1.f;
    }
    auto cell_ptr = [&](int e) {
        return reinterpret_cast<const uint32_t*>(wbase + __builtin_amdgcn_readlane(t_load, e) + lofs);
    };
    // A window of D cells is in flight per wave: cell e + D is requested as
    // soon as cell e's codes have been turned into addresses, so requests
    // go out (and return) roughly in cell order.
    uint32_t ring[D][3];
#pragma unroll
    for (int e = 0; e < D; ++e) {
        const uint32_t* q = cell_ptr(e);
        ring[e][0] = __builtin_nontemporal_load(q);
        ring[e][1] = __builtin_nontemporal_load(q + 1);
        ring[e][2] = __builtin_nontemporal_load(q + 2);
    }
    __builtin_amdgcn_sched_barrier(0);

    {
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(smem);
#pragma unroll
        for (int u = 0; u < kB1Stage; ++u) {
            // x piece p = 64*cj + lane (32 bytes, halves h = 0, 1) goes to
            // 16-byte slot cj*128 + h*64 + lane, so that each of a cell's two
            // x reads covers 1 KB of consecutive LDS (no bank conflicts).
            const int k = min(tid + u * (64 * nw), nst - 1);
            const int slot = k < nx ? (((k >> 7) << 7) | ((k & 1) << 6) | ((k >> 1) & 63)) : k;
            dst[slot] = stage[u];  // clamped duplicates store equal values
        }
    }
    __syncthreads();

    uint32_t mask = 0x7Eu;
    asm volatile("" : "+v"(mask));  // keep the mask in a VGPR: v_and_or_b32 takes no literal
    float acc0 = 0.f, acc1 = 0.f;
    // Cell d of this wave is column block cj = (cj0 + d) % cpr of row
    // rl0 + (cj0 + d) / cpr.  Slots past n hold the last cell again: they are
    // computed like the others (no branch) and their sums are discarded.
#pragma unroll
    for (int d = 0; d < NC; ++d) {
        const uint32_t base = __builtin_amdgcn_readlane(t_base, d);
        const uint32_t d0 = ring[d % D][0], d1 = ring[d % D][1], d2 = ring[d % D][2];
        uint32_t a[16];
        a[0] = (code_x2<0>(d0, d1, d2) & mask) | base;
        a[1] = (code_x2<1>(d0, d1, d2) & mask) | base;
        a[2] = (code_x2<2>(d0, d1, d2) & mask) | base;
        a[3] = (code_x2<3>(d0, d1, d2) & mask) | base;
        a[4] = (code_x2<4>(d0, d1, d2) & mask) | base;
        a[5] = (code_x2<5>(d0, d1, d2) & mask) | base;
        a[6] = (code_x2<6>(d0, d1, d2) & mask) | base;
        a[7] = (code_x2<7>(d0, d1, d2) & mask) | base;
        a[8] = (code_x2<8>(d0, d1, d2) & mask) | base;
        a[9] = (code_x2<9>(d0, d1, d2) & mask) | base;
        a[10] = (code_x2<10>(d0, d1, d2) & mask) | base;
        a[11] = (code_x2<11>(d0, d1, d2) & mask) | base;
        a[12] = (code_x2<12>(d0, d1, d2) & mask) | base;
        a[13] = (code_x2<13>(d0, d1, d2) & mask) | base;
        a[14] = (code_x2<14>(d0, d1, d2) & mask) | base;
        a[15] = (code_x2<15>(d0, d1, d2) & mask) | base;
        if (d + D < NC) {  // compile-time condition: refill this slot with cell d + D
            const uint32_t* q = cell_ptr(d + D);
            ring[d % D][0] = __builtin_nontemporal_load(q);
            ring[d % D][1] = __builtin_nontemporal_load(q + 1);
            ring[d % D][2] = __builtin_nontemporal_load(q + 2);
        }
        // x pairs of this lane's piece (halves 1 KB apart, see the staging)
        const uint32_t xa = __builtin_amdgcn_readlane(t_xoff, d) + 16u * lane;
        const u32x4_t xl = *(lds_u4*)(uintptr_t)xa, xh = *(lds_u4*)(uintptr_t)(xa + 1024);
        const uint32_t xv[8] = {xl[0], xl[1], xl[2], xl[3], xh[0], xh[1], xh[2], xh[3]};
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
            // two gathered bf16 -> one dword: bytes [lo.0, lo.1, hi.0, hi.1] (v_perm_b32)
            const uint32_t w0 = __builtin_amdgcn_perm(*(lds_u16*)(uintptr_t)a[2 * j + 1],
                                                      *(lds_u16*)(uintptr_t)a[2 * j], 0x05040100u);
            const uint32_t w1 = __builtin_amdgcn_perm(*(lds_u16*)(uintptr_t)a[2 * j + 3],
                                                      *(lds_u16*)(uintptr_t)a[2 * j + 2], 0x05040100u);
            acc0 = dot2(w0, xv[j], acc0);
            acc1 = dot2(w1, xv[j + 1], acc1);
        }
        // Row end: this lane's sum goes to partial slot [row][s] (s = 1 only
        // for a row an earlier wave started) and the sums restart; otherwise
        // the store goes to the discard slot and keep = 1.
        const uint32_t dst = __builtin_amdgcn_readlane(t_dst, d);
        *(lds_f32*)(uintptr_t)(dst + 4u * lane) = acc0 + acc1;
        const float keep = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t_keep), d));
        acc0 *= keep;
        acc1 *= keep;
    }
    __syncthreads();
    const float* part = reinterpret_cast<const float*>(smem + cols * 2 + R * 128);
    for (int i = w; i < R; i += nw) {
        // Slot 1 holds data only if a wave range starts strictly inside row i.
        bool split = false;
#pragma unroll
        for (int k = 1; k < nw; ++k) {
            const int b = (k * C) / nw;
            split |= b > i * cpr && b < (i + 1) * cpr;
        }
        float v = part[i * 128 + lane];
        if (split) v += part[i * 128 + 64 + lane];
        const float sum = wave_sum_lane63(v);
        if (lane == 63) {
            if (y_f32)
                reinterpret_cast<float*>(y)[r0 + i] = sum;
            else
                reinterpret_cast<uint16_t*>(y)[r0 + i] = f32_to_bf16(sum);
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

// Cells per row (cols / 1024) with a compiled variant; other widths take the
// generic kernel.  5 and 17 are the 27B-class MLP widths (5120, 17408).
bool b1_cpr_supported(int64_t cpr) {
    switch (cpr) {
        case 1: case 2: case 3: case 4: case 5: case 6: case 8: case 12: case 16: case 17: case 20:
            return true;
        default:
            return false;
    }
}

// Grid: 512 workgroups (two per CU on 256 CUs) when the row count allows,
// with every workgroup holding at least one row per wave (so a row spans at
// most two waves) and at most kB1Cells cells per wave.
constexpr int64_t kB1MaxLds = 64 * 1024;  // dynamic LDS per workgroup

bool b1_fits(const fqm_weights& w, int64_t* groups, size_t* lds) {
    if (w.cols <= 0 || (w.cols & 1023) || w.rows < kB1Waves || w.rows > 0x7fffffff) return false;
    if (w.lut6.ld > 0xffffffffLL / (kB1Cells + 1)) return false;  // 32-bit cell offsets
    const int64_t cpr = w.cols >> 10;
    if (cpr > kB1Cells || !b1_cpr_supported(cpr)) return false;
    const int64_t rmax = (int64_t)kB1Cells * kB1Waves / cpr;   // rows per group, at most
    const int64_t lo = (w.rows + rmax - 1) / rmax;              // fewest groups
    const int64_t hi = w.rows / kB1Waves;                        // most groups
    int64_t g = 512;
    if (g < lo) g = lo;
    if (g > hi) g = hi;
    if (g < lo || g > 0x7fffffff) return false;
    const int64_t r = (w.rows + g - 1) / g;
    const int64_t bytes = w.cols * 2 + r * (128 + 512) + kB1Waves * 256;
    if (bytes > kB1MaxLds) return false;
    if (w.cols / 8 + r * 8 > (int64_t)kB1Stage * 64 * kB1Waves) return false;
    *groups = g;
    *lds = (size_t)bytes;
    return true;
}

template <int CPR>
hipError_t launch_b1_cpr(const fqm_weights& w, const uint16_t* x, void* y, int y_f32,
                         int64_t groups, size_t lds, hipStream_t s) {
    hipLaunchKernelGGL((lut6_gemv_b1<kB1Cells, kB1Ring, CPR>), dim3((unsigned)groups),
                       dim3(64 * kB1Waves), lds, s, w.lut6.packed, w.lut6.ld, w.lut6.lut, x, y, y_f32,
                       (int)(w.rows / groups), (int)(w.rows % groups));
    return hipGetLastError();
}

hipError_t launch_b1(const fqm_weights& w, const uint16_t* x, void* y, int y_f32, int64_t groups,
                     size_t lds, hipStream_t s) {
    switch (w.cols >> 10) {
        case 1: return launch_b1_cpr<1>(w, x, y, y_f32, groups, lds, s);
        case 2: return launch_b1_cpr<2>(w, x, y, y_f32, groups, lds, s);
        case 3: return launch_b1_cpr<3>(w, x, y, y_f32, groups, lds, s);
        case 4: return launch_b1_cpr<4>(w, x, y, y_f32, groups, lds, s);
        case 5: return launch_b1_cpr<5>(w, x, y, y_f32, groups, lds, s);
        case 6: return launch_b1_cpr<6>(w, x, y, y_f32, groups, lds, s);
        case 8: return launch_b1_cpr<8>(w, x, y, y_f32, groups, lds, s);
        case 12: return launch_b1_cpr<12>(w, x, y, y_f32, groups, lds, s);
        case 16: return launch_b1_cpr<16>(w, x, y, y_f32, groups, lds, s);
        case 17: return launch_b1_cpr<17>(w, x, y, y_f32, groups, lds, s);
        case 20: return launch_b1_cpr<20>(w, x, y, y_f32, groups, lds, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_lut6_gemv(const fqm_weights& w, const uint16_t* x, void* y, int y_f32,
                            int batch, hipStream_t s) {
    int64_t groups = 0;
    size_t lds = 0;
    if (batch == 1 && b1_fits(w, &groups, &lds)) return launch_b1(w, x, y, y_f32, groups, lds, s);
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
