// Per-row LUT 4-bit GEMV: y[b][r] = sum_k lut[r][code[r][k]] * x[b][k] with
// 16-entry tables.
//
// Source: "Qwen3.8-27B - BenQ 6-bit": the card's "Why equal-width shells"
// table places 8 tiers in 4 bits beside 32 tiers in 6 bits; read as the 6-bit
// format is read ("What BenQ stores"), a 4-bit code (1 sign + 3 tier bits)
// selects one of the row's 16 signed bf16 levels, and the product gathers
// from the table inside the matmul.
//
// Codes are two per byte (code 2j in the low nibble of byte j), so a row of
// 1024 weights is 512 bytes: half the bytes of the 6-bit format for the same
// decode work per weight.
#include "fqm_internal.h"

namespace fqm {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) const uint16_t lds_u16;
typedef __attribute__((address_space(3))) const uint32_t lds_u32c;
typedef __attribute__((address_space(3))) const u32x4_t lds_u4;

constexpr int kWaves = 4;

__device__ __forceinline__ float dot2(uint32_t w, uint32_t x, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), __builtin_bit_cast(bf16x2_t, x), acc,
                                          false);
}

// Code j (0..15) of an 8-byte piece d0, d1 shifted so that its 4 bits sit at
// bits 1..4 (the byte offset of its table entry), other bits still to be masked.
template <int J>
__device__ __forceinline__ uint32_t code4_x2(uint32_t d0, uint32_t d1) {
    constexpr int o = (4 * J) & 31;
    const uint32_t d = J < 8 ? d0 : d1;
    if constexpr (o == 0) return d << 1;
    else return d >> (o - 1);
}

// ---------------------------------------------------------------------------
// Batch 1, cols = 1024 CPR.  The batch-1 LUT6 kernel's structure with 4-bit
// codes: in chunk c lane i owns the 8-byte piece i (16 codes, bytes
// [512c + 8i, +8): one coalesced 512-byte load per chunk) and the matching 16
// x values from the x block staged once per workgroup in LDS (the same
// swizzle: each half-read of a chunk covers 1 KB of consecutive LDS).  A
// wave's 32-byte table sits in its own LDS slot (a multiple of 32), so a code
// becomes a gather address in a shift and one v_and_or_b32; the 64 lanes read
// 8 dwords in 8 distinct banks.  Codes are requested PC chunks ahead, every
// load unconditional; the row sum is one DPP reduction per wave.
// With PT the wave's slot holds a 1 KB table of weight pairs instead: entry p
// is lut[p & 15] | lut[p >> 4] << 16, so byte j of a lane's codes (codes 2j
// and 2j + 1) addresses the pair that meets x pair j in v_dot2 directly: one
// shift, one v_and_or_b32 and one 32-bit gather per two weights, and no
// v_perm_b32.  The dot2 operands and their order are those of the 16-entry
// path, so the result is the same bit for bit.  Building the pairs costs
// five table loads and four LDS stores per lane and row, which only rows of
// many cells repay.
// ---------------------------------------------------------------------------
template <int CPR, int WPG, int PC, bool PT>
__global__ __launch_bounds__(64 * WPG) void lut4_gemv_cells(const uint8_t* __restrict__ packed, int64_t ld,
                                                            const uint16_t* __restrict__ lut,
                                                            const uint16_t* __restrict__ x,
                                                            void* __restrict__ y, int y_f32, int rows) {
    constexpr int NX = CPR * 128;                          // x in 16-byte pieces
    constexpr int XS = (NX + 64 * WPG - 1) / (64 * WPG);   // staging pieces per thread
    __shared__ __attribute__((aligned(16))) u32x4_t s_x[NX];
    __shared__ __attribute__((aligned(PT ? 1024 : 32))) uint32_t s_tab[WPG][PT ? 256 : 8];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int row_u = blockIdx.x * WPG + wv;
    const int row = min(row_u, rows - 1);  // rows past the end repeat the last row (not stored)
    const uint8_t* rowp = packed + (int64_t)row * ld + 8 * lane;

    u32x4_t xs[XS];
#pragma unroll
    for (int u = 0; u < XS; ++u)
        xs[u] = reinterpret_cast<const u32x4_t*>(x)[min(tid + u * 64 * WPG, NX - 1)];
    const uint16_t* lr = lut + (int64_t)row * 16;
    const uint32_t tv = PT ? (uint32_t)lr[lane & 15] : reinterpret_cast<const uint32_t*>(lr)[lane & 7];
    uint32_t t_hi[4];  // PT: entries (lane >> 4) + 4 t, the high halves of pairs lane + 64 t
#pragma unroll
    for (int t = 0; t < 4; ++t) t_hi[t] = PT ? lr[(lane >> 4) + 4 * t] : 0u;
    __builtin_amdgcn_sched_barrier(0);

    uint32_t cr[PC + 1][2];
    auto load_codes = [&](int c) {
        const uint32_t* q = reinterpret_cast<const uint32_t*>(rowp + 512 * c);
        cr[c % (PC + 1)][0] = __builtin_nontemporal_load(q);
        cr[c % (PC + 1)][1] = __builtin_nontemporal_load(q + 1);
    };
#pragma unroll
    for (int c = 0; c < PC && c < CPR; ++c) load_codes(c);
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int u = 0; u < XS; ++u) {
        const int k = min(tid + u * 64 * WPG, NX - 1);
        s_x[((k >> 7) << 7) | ((k & 1) << 6) | ((k >> 1) & 63)] = xs[u];  // clamped duplicates store equal values
    }
    if constexpr (PT) {
#pragma unroll
        for (int t = 0; t < 4; ++t) s_tab[wv][lane + 64 * t] = tv | (t_hi[t] << 16);
    } else {
        s_tab[wv][lane & 7] = tv;  // unconditional (lanes repeat), so the load stays ahead of the codes
    }
    __syncthreads();

    const uint32_t base = (uint32_t)(uintptr_t)(lds_u8*)s_tab + (PT ? 1024u : 32u) * wv;  // multiple of the slot
    uint32_t mask = PT ? 0x3FCu : 0x1Eu;
    asm volatile("" : "+v"(mask));  // in a VGPR: (code & mask) | base is one v_and_or_b32
    const uint32_t xb = (uint32_t)(uintptr_t)(lds_u8*)s_x + 16u * lane;
    float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
    for (int c = 0; c < CPR; ++c) {
        if (c + PC < CPR) load_codes(c + PC);
        const u32x4_t xl = *(lds_u4*)(uintptr_t)(xb + 2048u * c);
        const u32x4_t xh = *(lds_u4*)(uintptr_t)(xb + 2048u * c + 1024u);
        const uint32_t xv[8] = {xl[0], xl[1], xl[2], xl[3], xh[0], xh[1], xh[2], xh[3]};
        const uint32_t d0 = cr[c % (PC + 1)][0], d1 = cr[c % (PC + 1)][1];
        if constexpr (PT) {
            uint32_t p[8];  // byte j of the lane's codes, as the LDS address of its pair
            p[0] = ((d0 << 2) & mask) | base;
            p[1] = ((d0 >> 6) & mask) | base;
            p[2] = ((d0 >> 14) & mask) | base;
            p[3] = ((d0 >> 22) & mask) | base;
            p[4] = ((d1 << 2) & mask) | base;
            p[5] = ((d1 >> 6) & mask) | base;
            p[6] = ((d1 >> 14) & mask) | base;
            p[7] = ((d1 >> 22) & mask) | base;
#pragma unroll
            for (int j = 0; j < 8; j += 2) {
                acc0 = dot2(*(lds_u32c*)(uintptr_t)p[j], xv[j], acc0);
                acc1 = dot2(*(lds_u32c*)(uintptr_t)p[j + 1], xv[j + 1], acc1);
            }
            continue;
        }
        uint32_t a[16];
        a[0] = (code4_x2<0>(d0, d1) & mask) | base;
        a[1] = (code4_x2<1>(d0, d1) & mask) | base;
        a[2] = (code4_x2<2>(d0, d1) & mask) | base;
        a[3] = (code4_x2<3>(d0, d1) & mask) | base;
        a[4] = (code4_x2<4>(d0, d1) & mask) | base;
        a[5] = (code4_x2<5>(d0, d1) & mask) | base;
        a[6] = (code4_x2<6>(d0, d1) & mask) | base;
        a[7] = (code4_x2<7>(d0, d1) & mask) | base;
        a[8] = (code4_x2<8>(d0, d1) & mask) | base;
        a[9] = (code4_x2<9>(d0, d1) & mask) | base;
        a[10] = (code4_x2<10>(d0, d1) & mask) | base;
        a[11] = (code4_x2<11>(d0, d1) & mask) | base;
        a[12] = (code4_x2<12>(d0, d1) & mask) | base;
        a[13] = (code4_x2<13>(d0, d1) & mask) | base;
        a[14] = (code4_x2<14>(d0, d1) & mask) | base;
        a[15] = (code4_x2<15>(d0, d1) & mask) | base;
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
            const uint32_t w0 = __builtin_amdgcn_perm(*(lds_u16*)(uintptr_t)a[2 * j + 1],
                                                      *(lds_u16*)(uintptr_t)a[2 * j], 0x05040100u);
            const uint32_t w1 = __builtin_amdgcn_perm(*(lds_u16*)(uintptr_t)a[2 * j + 3],
                                                      *(lds_u16*)(uintptr_t)a[2 * j + 2], 0x05040100u);
            acc0 = dot2(w0, xv[j], acc0);
            acc1 = dot2(w1, xv[j + 1], acc1);
        }
    }
    const float sum = wave_sum_lane63(acc0 + acc1);
    if (lane == 63 && row_u < rows) {
        if (y_f32)
            reinterpret_cast<float*>(y)[row_u] = sum;
        else
            reinterpret_cast<uint16_t*>(y)[row_u] = f32_to_bf16(sum);
    }
}

// Batches 2 and 3: the batch-1 structure with every batch row's x block in
// LDS (row b at piece offset b * CPR * 128); each pair of gathered weights
// meets the B x pairs in B v_dot2, so a weight is decoded once for all batch
// rows.  Every chunk ends in a scheduling barrier and passes the sums through
// an empty asm, so the compiler cannot sink the dot2 chains to the final
// reduction (that kept every chunk's operands live).
template <int CPR, int WPG, int PC, int B>
__global__ __launch_bounds__(64 * WPG) void lut4_gemv_cells_batch(const uint8_t* __restrict__ packed, int64_t ld,
                                                                  const uint16_t* __restrict__ lut,
                                                                  const uint16_t* __restrict__ x,
                                                                  void* __restrict__ y, int y_f32, int rows) {
    constexpr int NX = CPR * 128;                              // x of one batch row in 16-byte pieces
    constexpr int XS = (B * NX + 64 * WPG - 1) / (64 * WPG);   // staging pieces per thread
    __shared__ __attribute__((aligned(16))) u32x4_t s_x[B * NX];
    __shared__ __attribute__((aligned(32))) uint32_t s_tab[WPG][8];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int row_u = blockIdx.x * WPG + wv;
    const int row = min(row_u, rows - 1);  // rows past the end repeat the last row (not stored)
    const uint8_t* rowp = packed + (int64_t)row * ld + 8 * lane;

    u32x4_t xs[XS];
#pragma unroll
    for (int u = 0; u < XS; ++u)
        xs[u] = reinterpret_cast<const u32x4_t*>(x)[min(tid + u * 64 * WPG, B * NX - 1)];
    const uint32_t tv = reinterpret_cast<const uint32_t*>(lut + (int64_t)row * 16)[lane & 7];
    __builtin_amdgcn_sched_barrier(0);

    uint32_t cr[PC + 1][2];
    auto load_codes = [&](int c) {
        const uint32_t* q = reinterpret_cast<const uint32_t*>(rowp + 512 * c);
        cr[c % (PC + 1)][0] = __builtin_nontemporal_load(q);
        cr[c % (PC + 1)][1] = __builtin_nontemporal_load(q + 1);
    };
#pragma unroll
    for (int c = 0; c < PC && c < CPR; ++c) load_codes(c);
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int u = 0; u < XS; ++u) {
        const int t = min(tid + u * 64 * WPG, B * NX - 1), k = t % NX;  // batch row t / NX, piece k
        s_x[(t - k) + (((k >> 7) << 7) | ((k & 1) << 6) | ((k >> 1) & 63))] = xs[u];
    }
    s_tab[wv][lane & 7] = tv;
    __syncthreads();

    const uint32_t base = (uint32_t)(uintptr_t)(lds_u8*)s_tab + 32u * wv;
    uint32_t mask = 0x1Eu;
    asm volatile("" : "+v"(mask));
    const uint32_t xb = (uint32_t)(uintptr_t)(lds_u8*)s_x + 16u * lane;
    float acc0[B], acc1[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc0[b] = acc1[b] = 0.f;
#pragma unroll
    for (int c = 0; c < CPR; ++c) {
        if (c + PC < CPR) load_codes(c + PC);
        const uint32_t d0 = cr[c % (PC + 1)][0], d1 = cr[c % (PC + 1)][1];
        uint32_t a[16];
        a[0] = (code4_x2<0>(d0, d1) & mask) | base;
        a[1] = (code4_x2<1>(d0, d1) & mask) | base;
        a[2] = (code4_x2<2>(d0, d1) & mask) | base;
        a[3] = (code4_x2<3>(d0, d1) & mask) | base;
        a[4] = (code4_x2<4>(d0, d1) & mask) | base;
        a[5] = (code4_x2<5>(d0, d1) & mask) | base;
        a[6] = (code4_x2<6>(d0, d1) & mask) | base;
        a[7] = (code4_x2<7>(d0, d1) & mask) | base;
        a[8] = (code4_x2<8>(d0, d1) & mask) | base;
        a[9] = (code4_x2<9>(d0, d1) & mask) | base;
        a[10] = (code4_x2<10>(d0, d1) & mask) | base;
        a[11] = (code4_x2<11>(d0, d1) & mask) | base;
        a[12] = (code4_x2<12>(d0, d1) & mask) | base;
        a[13] = (code4_x2<13>(d0, d1) & mask) | base;
        a[14] = (code4_x2<14>(d0, d1) & mask) | base;
        a[15] = (code4_x2<15>(d0, d1) & mask) | base;
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

// Any width (cols % 16 == 0) and batch 1..16: one row per wave, lane i takes
// the 8-byte pieces i, i + 64, ..., decodes its 16 codes through the row's
// table in LDS and adds the B products in fp32.
template <int B>
__global__ __launch_bounds__(256) void lut4_gemv_generic(const uint8_t* __restrict__ packed, int64_t ld,
                                                         const uint16_t* __restrict__ lut,
                                                         const uint16_t* __restrict__ x, void* __restrict__ y,
                                                         int y_f32, int64_t rows, int64_t cols) {
    __shared__ uint32_t s_lut[kWaves][8];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kWaves + wave;
    if (row < rows && lane < 8) s_lut[wave][lane] = reinterpret_cast<const uint32_t*>(lut + row * 16)[lane];
    __syncthreads();
    if (row >= rows) return;
    const uint16_t* tab = reinterpret_cast<const uint16_t*>(s_lut[wave]);
    float acc[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = 0.f;
    const uint8_t* prow = packed + row * ld;
    for (int64_t p = lane; p < cols / 16; p += 64) {
        const uint2 q = *reinterpret_cast<const uint2*>(prow + 8 * p);
        float w[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) w[j] = bf16_to_f32(tab[((j < 8 ? q.x : q.y) >> (4 * (j & 7))) & 15u]);
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

__global__ __launch_bounds__(256) void lut4_dequant_kernel(const uint8_t* __restrict__ packed, int64_t ld,
                                                           const uint16_t* __restrict__ lut,
                                                           uint16_t* __restrict__ W, int64_t rows, int64_t cols) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= rows * cols) return;
    const int64_t r = t / cols, k = t - r * cols;
    W[t] = lut[r * 16 + ((packed[r * ld + (k >> 1)] >> (4 * (k & 1))) & 15u)];
}

constexpr int kMaxCells = 31;  // x (2 KB per cell) and the tables stay under 64 KB of LDS

template <int CPR>
hipError_t launch_cells(const fqm_weights& w, const uint16_t* x, void* y, int y_f32, hipStream_t s) {
    if constexpr (CPR > kMaxCells) {
        return hipErrorInvalidValue;
    } else {
        if ((w.cols >> 10) != CPR) return launch_cells<CPR + 1>(w, x, y, y_f32, s);
        constexpr int WPG = CPR <= 8 ? 4 : 10;
        const unsigned grid = (unsigned)((w.rows + WPG - 1) / WPG);
        // pair tables on rows of more than 8 cells: 5120 x 17408 took 14.4-14.6 us
        // against 15.2-15.4 us; on 17408 x 5120 they cost 8 % (14.9-15.0 against 13.8 us)
        hipLaunchKernelGGL((lut4_gemv_cells<CPR, WPG, 4, (CPR > 8)>), dim3(grid), dim3(64 * WPG), 0, s, w.lut4.packed,
                           w.lut4.ld, w.lut4.lut, x, y, y_f32, (int)w.rows);
        return hipGetLastError();
    }
}

// Batches 2 and 3 while two groups of the batch kernel fit a CU (B * cells
// <= 38, as for the 6-bit codes).
constexpr int kRowsMaxBatch = 3;
constexpr int batch_max_cells(int b) { return 38 / b; }

template <int CPR, int B>
hipError_t launch_cells_batch(const fqm_weights& w, const uint16_t* x, void* y, int y_f32, hipStream_t s) {
    if constexpr (CPR > batch_max_cells(B)) {
        return hipErrorInvalidValue;
    } else {
        if ((w.cols >> 10) != CPR) return launch_cells_batch<CPR + 1, B>(w, x, y, y_f32, s);
        constexpr int WPG = CPR <= 8 ? 4 : 10;
        const unsigned grid = (unsigned)((w.rows + WPG - 1) / WPG);
        hipLaunchKernelGGL((lut4_gemv_cells_batch<CPR, WPG, 4, B>), dim3(grid), dim3(64 * WPG), 0, s,
                           w.lut4.packed, w.lut4.ld, w.lut4.lut, x, y, y_f32, (int)w.rows);
        return hipGetLastError();
    }
}

template <int B>
hipError_t launch_generic(const fqm_weights& w, const uint16_t* x, void* y, int y_f32, hipStream_t s) {
    const unsigned grid = (unsigned)((w.rows + kWaves - 1) / kWaves);
    hipLaunchKernelGGL(lut4_gemv_generic<B>, dim3(grid), dim3(64 * kWaves), 0, s, w.lut4.packed, w.lut4.ld,
                       w.lut4.lut, x, y, y_f32, w.rows, w.cols);
    return hipGetLastError();
}

template <int B>
hipError_t launch_batch(const fqm_weights& w, const uint16_t* x, void* y, int y_f32, int batch, hipStream_t s) {
    if constexpr (B > 16) {
        return hipErrorInvalidValue;
    } else {
        if (batch != B) return launch_batch<B + 1>(w, x, y, y_f32, batch, s);
        return launch_generic<B>(w, x, y, y_f32, s);
    }
}

}  // namespace

static bool cells_supported(const fqm_weights& w) {
    return w.cols > 0 && (w.cols & 1023) == 0 && (w.cols >> 10) <= kMaxCells;
}

bool lut4_gemv_rows_path(const fqm_weights& w, int batch) {
    if (batch == 1) return cells_supported(w);
    return batch >= 2 && batch <= kRowsMaxBatch && cells_supported(w) && (w.cols >> 10) <= batch_max_cells(batch);
}

bool lut4_gemv_fast_path(const fqm_weights& w, int batch) {
    return lut4_gemv_rows_path(w, batch) || (batch > 1 && lut_gemv_mfma_supported(w, batch));
}

hipError_t launch_lut4_gemv(const fqm_weights& w, const uint16_t* x, void* y, int y_f32, int batch,
                            float* ws, hipStream_t s) {
    if (w.rows > 0x7fffffff) return hipErrorInvalidValue;
    if (batch == 1 && cells_supported(w))
        return launch_cells<1>(w, x, y, y_f32, s);
    if (lut4_gemv_rows_path(w, batch)) {
        if (batch == 2) return launch_cells_batch<1, 2>(w, x, y, y_f32, s);
        return launch_cells_batch<1, 3>(w, x, y, y_f32, s);
    }
    if (lut_gemv_mfma_supported(w, batch)) return launch_lut_gemv_mfma(w, x, y, y_f32, batch, ws, s);
    return launch_batch<1>(w, x, y, y_f32, batch, s);
}

hipError_t launch_dequant_lut4(const fqm_weights& w, uint16_t* W, hipStream_t s) {
    const int64_t n = w.rows * w.cols;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(lut4_dequant_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, w.lut4.packed,
                       w.lut4.ld, w.lut4.lut, W, w.rows, w.cols);
    return hipGetLastError();
}

}  // namespace fqm
