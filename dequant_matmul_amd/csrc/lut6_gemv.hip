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

// ---------------------------------------------------------------------------
// Batch 1, cols a multiple of 1024.  A row is CPR chunks of 1024 weights; in
// chunk c lane i owns the 12-byte piece i (16 codes, bytes [768c + 12i, +12)
// of the row: one fully coalesced 768-byte load per chunk) and the matching
// 16 x values (32 bytes), read from the x block the workgroup stages in LDS
// once.  Each row is split over S waves (wave s takes chunks
// [s*CPR/S, (s+1)*CPR/S)); a workgroup holds WPG waves, i.e. WPG/S rows.
// Codes are requested PC chunks ahead, every load unconditional within the
// unrolled chunk loop, so the compiler's waits are exact.  A wave's row table
// sits in its own 128-byte LDS slot (a multiple of 128, held in a scalar
// register), so a code becomes a gather address in two VALU ops (shift, then
// mask and OR of the slot in one v_and_or_b32) and all 64 lanes of a gather
// read one 128-byte table (distinct banks or a shared dword).  Two gathered
// bf16 are paired (v_perm_b32) and meet the x pair in v_dot2_f32_bf16 (fp32
// accumulate).  Each wave reduces its partial row sum once with DPP; with
// S > 1 the S partials are added in wave order through LDS, so the result
// does not depend on timing.
// ---------------------------------------------------------------------------
template <int CPR, int S, int WPG, int PC>
__global__ __launch_bounds__(64 * WPG) void lut6_gemv_rows(const uint8_t* __restrict__ packed,
                                                           int64_t ld,
                                                           const uint16_t* __restrict__ lut,
                                                           const uint16_t* __restrict__ x,
                                                           void* __restrict__ y, int y_f32,
                                                           int rows) {
    constexpr int RPG = WPG / S;                           // rows per workgroup
    constexpr int NCH = (CPR + S - 1) / S;                 // most chunks per wave
    constexpr int NX = CPR * 128;                          // x in 16-byte pieces
    constexpr int XS = (NX + 64 * WPG - 1) / (64 * WPG);   // staging pieces per thread
    __shared__ __attribute__((aligned(16))) u32x4_t s_x[NX];
    __shared__ __attribute__((aligned(16))) uint32_t s_tab[WPG][32];
    __shared__ float s_part[WPG];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rr = wv / S, sp = wv - rr * S;   // row within the group, split index
    const int row_u = blockIdx.x * RPG + rr;
    const int row = min(row_u, rows - 1);  // rows past the end repeat the last row (not stored)
    const int cs = (sp * CPR) / S, n = ((sp + 1) * CPR) / S - cs;  // this wave's chunks [cs, cs + n)
    const uint8_t* rowp = packed + (int64_t)row * ld + 768 * cs + 12 * lane;

    // x staging loads and the table load go out first, then the first PC
    // chunks of codes; the LDS stores below wait only for the former.
    u32x4_t xs[XS];
#pragma unroll
    for (int u = 0; u < XS; ++u)
        xs[u] = reinterpret_cast<const u32x4_t*>(x)[min(tid + u * 64 * WPG, NX - 1)];
    const uint32_t tv = reinterpret_cast<const uint32_t*>(lut + (int64_t)row * 64)[lane & 31];
    __builtin_amdgcn_sched_barrier(0);

    uint32_t cr[PC + 1][3];
    // chunk c of this wave (c < NCH); c >= n repeats the wave's last chunk
    auto load_codes = [&](int c) {
        const uint32_t* q = reinterpret_cast<const uint32_t*>(rowp + 768 * min(c, n - 1));
        cr[c % (PC + 1)][0] = __builtin_nontemporal_load(q);
        cr[c % (PC + 1)][1] = __builtin_nontemporal_load(q + 1);
        cr[c % (PC + 1)][2] = __builtin_nontemporal_load(q + 2);
    };
#pragma unroll
    for (int c = 0; c < PC && c < NCH; ++c) load_codes(c);
    __builtin_amdgcn_sched_barrier(0);

    // x piece p = 64*cj + l (32 bytes = 16-byte halves h = 0, 1) goes to
    // slot cj*128 + h*64 + l, so that each half-read of a chunk covers 1 KB of
    // consecutive LDS (no bank conflicts).
#pragma unroll
    for (int u = 0; u < XS; ++u) {
        const int k = min(tid + u * 64 * WPG, NX - 1);
        s_x[((k >> 7) << 7) | ((k & 1) << 6) | ((k >> 1) & 63)] = xs[u];  // clamped duplicates store equal values
    }
    s_tab[wv][lane & 31] = tv;  // unconditional (lanes 32-63 repeat 0-31), so the load stays ahead of the codes
    __syncthreads();

    const uint32_t base = (uint32_t)(uintptr_t)(lds_u8*)s_tab + 128u * wv;  // multiple of 128
    uint32_t mask = 0x7Eu;
    asm volatile("" : "+v"(mask));  // in a VGPR: (code & mask) | base is one v_and_or_b32
    const uint32_t xb = (uint32_t)(uintptr_t)(lds_u8*)s_x + 2048u * cs + 16u * lane;
    float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        if (c + PC < NCH) load_codes(c + PC);
        const uint32_t cc = (uint32_t)min(c, n - 1);
        const u32x4_t xl = *(lds_u4*)(uintptr_t)(xb + 2048u * cc);
        const u32x4_t xh = *(lds_u4*)(uintptr_t)(xb + 2048u * cc + 1024u);
        const uint32_t xv[8] = {xl[0], xl[1], xl[2], xl[3], xh[0], xh[1], xh[2], xh[3]};
        const uint32_t d0 = cr[c % (PC + 1)][0], d1 = cr[c % (PC + 1)][1], d2 = cr[c % (PC + 1)][2];
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
        float p0 = 0.f, p1 = 0.f;
        float& s0 = (NCH * S == CPR) ? acc0 : p0;  // uneven split: the repeated chunk is dropped
        float& s1 = (NCH * S == CPR) ? acc1 : p1;
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
            const uint32_t w0 = __builtin_amdgcn_perm(*(lds_u16*)(uintptr_t)a[2 * j + 1],
                                                      *(lds_u16*)(uintptr_t)a[2 * j], 0x05040100u);
            const uint32_t w1 = __builtin_amdgcn_perm(*(lds_u16*)(uintptr_t)a[2 * j + 3],
                                                      *(lds_u16*)(uintptr_t)a[2 * j + 2], 0x05040100u);
            s0 = dot2(w0, xv[j], s0);
            s1 = dot2(w1, xv[j + 1], s1);
        }
        if (NCH * S != CPR) {
            const float keep = c < n ? 1.f : 0.f;
            acc0 = fmaf(p0, keep, acc0);
            acc1 = fmaf(p1, keep, acc1);
        }
    }
    const float sum = wave_sum_lane63(acc0 + acc1);
    if (S == 1) {
        if (lane == 63 && row_u < rows) {
            if (y_f32)
                reinterpret_cast<float*>(y)[row_u] = sum;
            else
                reinterpret_cast<uint16_t*>(y)[row_u] = f32_to_bf16(sum);
        }
    } else {
        // the S partial sums of a row are added in wave order
        if (lane == 63) s_part[wv] = sum;
        __syncthreads();
        if (sp == 0 && lane == 0 && row_u < rows) {
            float t = s_part[wv];
#pragma unroll
            for (int q = 1; q < S; ++q) t += s_part[wv + q];
            if (y_f32)
                reinterpret_cast<float*>(y)[row_u] = t;
            else
                reinterpret_cast<uint16_t*>(y)[row_u] = f32_to_bf16(t);
        }
    }
}

// Batch rows B > 1 on the same layout: the workgroup stages B x blocks in LDS
// (batch row b at piece offset b * CPR * 128, swizzled as above), every
// pair of gathered weights meets the B x pairs in B v_dot2 (one decode for
// all batch rows), and each wave reduces B row sums.  A scheduling barrier
// closes every chunk and the sums are pinned there, so the unrolled loop
// keeps one chunk's operands live at a time.
template <int CPR, int WPG, int PC, int B>
__global__ __launch_bounds__(64 * WPG) void lut6_gemv_rows_batch(const uint8_t* __restrict__ packed,
                                                                 int64_t ld,
                                                                 const uint16_t* __restrict__ lut,
                                                                 const uint16_t* __restrict__ x,
                                                                 void* __restrict__ y, int y_f32,
                                                                 int rows) {
    constexpr int NX = CPR * 128;                              // x of one batch row in 16-byte pieces
    constexpr int XS = (B * NX + 64 * WPG - 1) / (64 * WPG);   // staging pieces per thread
    __shared__ __attribute__((aligned(16))) u32x4_t s_x[B * NX];
    __shared__ __attribute__((aligned(16))) uint32_t s_tab[WPG][32];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int row_u = blockIdx.x * WPG + wv;
    const int row = min(row_u, rows - 1);  // rows past the end repeat the last row (not stored)
    const uint8_t* rowp = packed + (int64_t)row * ld + 12 * lane;

    u32x4_t xs[XS];
#pragma unroll
    for (int u = 0; u < XS; ++u)
        xs[u] = reinterpret_cast<const u32x4_t*>(x)[min(tid + u * 64 * WPG, B * NX - 1)];
    const uint32_t tv = reinterpret_cast<const uint32_t*>(lut + (int64_t)row * 64)[lane & 31];
    __builtin_amdgcn_sched_barrier(0);

    uint32_t cr[PC + 1][3];
    auto load_codes = [&](int c) {
        const uint32_t* q = reinterpret_cast<const uint32_t*>(rowp + 768 * c);
        cr[c % (PC + 1)][0] = __builtin_nontemporal_load(q);
        cr[c % (PC + 1)][1] = __builtin_nontemporal_load(q + 1);
        cr[c % (PC + 1)][2] = __builtin_nontemporal_load(q + 2);
    };
#pragma unroll
    for (int c = 0; c < PC && c < CPR; ++c) load_codes(c);
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int u = 0; u < XS; ++u) {
        const int t = min(tid + u * 64 * WPG, B * NX - 1), k = t % NX;  // batch row t / NX, piece k
        s_x[(t - k) + (((k >> 7) << 7) | ((k & 1) << 6) | ((k >> 1) & 63))] = xs[u];
    }
    s_tab[wv][lane & 31] = tv;
    __syncthreads();

    const uint32_t base = (uint32_t)(uintptr_t)(lds_u8*)s_tab + 128u * wv;
    uint32_t mask = 0x7Eu;
    asm volatile("" : "+v"(mask));
    const uint32_t xb = (uint32_t)(uintptr_t)(lds_u8*)s_x + 16u * lane;
    float acc0[B], acc1[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc0[b] = acc1[b] = 0.f;
#pragma unroll
    for (int c = 0; c < CPR; ++c) {
        if (c + PC < CPR) load_codes(c + PC);
        const uint32_t d0 = cr[c % (PC + 1)][0], d1 = cr[c % (PC + 1)][1], d2 = cr[c % (PC + 1)][2];
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
        uint32_t w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            w[j] = __builtin_amdgcn_perm(*(lds_u16*)(uintptr_t)a[2 * j + 1], *(lds_u16*)(uintptr_t)a[2 * j],
                                         0x05040100u);
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const u32x4_t xl = *(lds_u4*)(uintptr_t)(xb + 16u * NX * b + 2048u * c);
            const u32x4_t xh = *(lds_u4*)(uintptr_t)(xb + 16u * NX * b + 2048u * c + 1024u);
            const uint32_t xv[8] = {xl[0], xl[1], xl[2], xl[3], xh[0], xh[1], xh[2], xh[3]};
#pragma unroll
            for (int j = 0; j < 8; j += 2) {
                acc0[b] = dot2(w[j], xv[j], acc0[b]);
                acc1[b] = dot2(w[j + 1], xv[j + 1], acc1[b]);
            }
            // the sums pass through an empty asm at every chunk: without it the
            // compiler sank whole dot2 chains to their last use, keeping every
            // chunk's gathered weights and x live (registers grew with the chunks)
            asm volatile("" : "+v"(acc0[b]), "+v"(acc1[b]));
        }
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const float sum = wave_sum_lane63(acc0[b] + acc1[b]);
        if (lane == 63 && row_u < rows) {
            if (y_f32)
                reinterpret_cast<float*>(y)[(int64_t)b * rows + row_u] = sum;
            else
                reinterpret_cast<uint16_t*>(y)[(int64_t)b * rows + row_u] = f32_to_bf16(sum);
        }
    }
}

template <int CPR, int S, int WPG, int PC>
hipError_t launch_rows(const fqm_weights& w, const uint16_t* x, void* y, int y_f32, hipStream_t s) {
    constexpr int RPG = WPG / S;
    const unsigned grid = (unsigned)((w.rows + RPG - 1) / RPG);
    hipLaunchKernelGGL((lut6_gemv_rows<CPR, S, WPG, PC>), dim3(grid), dim3(64 * WPG), 0, s,
                       w.lut6.packed, w.lut6.ld, w.lut6.lut, x, y, y_f32, (int)w.rows);
    return hipGetLastError();
}

template <int B>
hipError_t launch_b(const fqm_weights& w, const uint16_t* x, void* y, int y_f32, hipStream_t s) {
    const unsigned grid = (unsigned)((w.rows + kWaves - 1) / kWaves);
    hipLaunchKernelGGL(lut6_gemv_generic<B>, dim3(grid), dim3(64 * kWaves), 0, s, w.lut6.packed,
                       w.lut6.ld, w.lut6.lut, x, y, y_f32, w.rows, w.cols);
    return hipGetLastError();
}

// Batch-1 variants by cells per row (cols / 1024), 1 to kMaxCells: rows of at
// most 8 cells use 4-wave workgroups, longer rows 10-wave workgroups (x for a
// 17408-column row is 34 KB of LDS, so a CU holds four such groups); codes are
// requested four cells ahead.  Other widths take the generic kernel.
constexpr int kMaxCells = 31;  // x (2 KB per cell) and the tables stay under 64 KB of LDS

bool rows_supported(const fqm_weights& w) {
    return w.cols > 0 && (w.cols & 1023) == 0 && (w.cols >> 10) <= kMaxCells && w.rows > 0 &&
           w.rows <= 0x7fffffff;
}

template <int CPR>
hipError_t launch_cells(const fqm_weights& w, const uint16_t* x, void* y, int y_f32, hipStream_t s) {
    if constexpr (CPR > kMaxCells) {
        return hipErrorInvalidValue;
    } else {
        if ((w.cols >> 10) != CPR) return launch_cells<CPR + 1>(w, x, y, y_f32, s);
        if constexpr (CPR <= 8) return launch_rows<CPR, 1, 4, 4>(w, x, y, y_f32, s);
        else return launch_rows<CPR, 1, 10, 4>(w, x, y, y_f32, s);
    }
}

hipError_t launch_b1(const fqm_weights& w, const uint16_t* x, void* y, int y_f32, hipStream_t s) {
    return launch_cells<1>(w, x, y, y_f32, s);
}

// Batches 2 and 3 take the batch-row kernel while two 10-wave groups still
// fit a CU (B * cells <= 38, at most 76 KB of x per group).  Measured against
// the matrix-core kernel (same box, graph replays): 17408 x 5120 batch 2
// 17.7-19.8 us against 26.5 us, batch 3 22.1-22.8 against 26.5-27.2 us, batch
// 4 28.6-28.9 against 25.1 us; 5120 x 17408 batch 2 19.7-21.8 against
// 26.0-27.4 us.  Batches 4-16 stay on the matrix cores.
constexpr int kRowsMaxBatch = 3;
constexpr int batch_max_cells(int b) { return 38 / b; }

bool rows_batch_supported(const fqm_weights& w, int batch) {
    return batch >= 2 && batch <= kRowsMaxBatch && rows_supported(w) && (w.cols >> 10) <= batch_max_cells(batch);
}

template <int CPR, int B>
hipError_t launch_cells_batch(const fqm_weights& w, const uint16_t* x, void* y, int y_f32, hipStream_t s) {
    if constexpr (CPR > batch_max_cells(B)) {
        return hipErrorInvalidValue;
    } else {
        if ((w.cols >> 10) != CPR) return launch_cells_batch<CPR + 1, B>(w, x, y, y_f32, s);
        constexpr int WPG = CPR <= 8 ? 4 : 10;
        const unsigned grid = (unsigned)((w.rows + WPG - 1) / WPG);
        hipLaunchKernelGGL((lut6_gemv_rows_batch<CPR, WPG, 4, B>), dim3(grid), dim3(64 * WPG), 0, s,
                           w.lut6.packed, w.lut6.ld, w.lut6.lut, x, y, y_f32, (int)w.rows);
        return hipGetLastError();
    }
}

hipError_t launch_rows_batch(const fqm_weights& w, const uint16_t* x, void* y, int y_f32, int batch,
                             hipStream_t s) {
    if (batch == 2) return launch_cells_batch<1, 2>(w, x, y, y_f32, s);
    if (batch == 3) return launch_cells_batch<1, 3>(w, x, y, y_f32, s);
    return hipErrorInvalidValue;
}

}  // namespace

bool lut6_gemv_rows_path(const fqm_weights& w, int batch) {
    return batch == 1 ? rows_supported(w) : rows_batch_supported(w, batch);
}

bool lut6_gemv_fast_path(const fqm_weights& w, int batch) {
    return lut6_gemv_rows_path(w, batch) || (batch > 1 && lut_gemv_mfma_supported(w, batch));
}

hipError_t launch_lut6_gemv(const fqm_weights& w, const uint16_t* x, void* y, int y_f32,
                            int batch, float* ws, hipStream_t s) {
    if (batch == 1 && rows_supported(w)) return launch_b1(w, x, y, y_f32, s);
    if (rows_batch_supported(w, batch)) return launch_rows_batch(w, x, y, y_f32, batch, s);
    if (lut_gemv_mfma_supported(w, batch)) return launch_lut_gemv_mfma(w, x, y, y_f32, batch, ws, s);
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
