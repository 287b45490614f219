// Per-row LUT 6-bit GEMV for batch 2..16: y[b][r] = sum_k lut[r][code[r][k]] * x[b][k].
//
// Source: "Qwen3.8-27B - BenQ 6-bit", "What BenQ stores": a weight is its
// row's table entry selected by the 6-bit code, gathered inside the matmul.
//
// With more than one activation row the multiply-adds per weight grow with
// the batch, so the contraction runs on the matrix cores
// (v_mfma_f32_16x16x32_bf16, fp32 accumulate) and the decode stays the
// batch-independent part:
//   - A workgroup owns 16 rows (one MFMA row block) and a range of 1024-wide
//     K chunks.  Wave w decodes rows w, w+4, w+8, w+12 of the block: per
//     chunk lane i loads the row's 12-byte piece i (a coalesced 768-byte
//     load per wave instruction) and gathers its 16 weights from the row's
//     128-byte table in LDS (all 64 lanes of a gather read one table: no bank
//     conflicts).
//   - The decoded 16 x 1024 bf16 block goes to LDS (double-buffered) as
//     2048-byte rows whose 16-byte chunks are XOR-swizzled, then every wave
//     reads MFMA row fragments from it for a quarter of the chunk's 32-wide
//     k slices; the x fragments (batch row b = lane % 16, rows past the batch
//     repeat the last one and are never stored) come straight from L2.
//   - The four waves' 16 x 16 partial results are added in wave order; with
//     K split over several workgroups the partials go to the workspace and a
//     second kernel adds them in split order.
#include <algorithm>
#include <type_traits>

#include "fqm_internal.h"

namespace fqm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds8;
typedef __attribute__((address_space(3))) const uint16_t lds16c;
typedef __attribute__((address_space(3))) u32x4 lds128;
typedef __attribute__((address_space(3))) const u32x4 lds128c;
typedef __attribute__((address_space(3))) f32x4 ldsf4;

constexpr int RB = 16;                         // rows per workgroup
constexpr int NW = 4;                          // waves per workgroup
constexpr int CH = 1024;                       // k per chunk
constexpr int PC = 2;                          // code chunks requested ahead
constexpr int WT_BYTES = RB * CH * 2;          // one decoded block (32 KB)
constexpr int OFF_TAB = 2 * WT_BYTES;
constexpr int OFF_RED = OFF_TAB + RB * 128;
constexpr int LDS_BYTES = OFF_RED + NW * 64 * 16;
constexpr int SLICES = CH / 32 / NW;           // k slices per wave per chunk (8)

__device__ __forceinline__ uint32_t perm_lo16(uint32_t hi, uint32_t lo) {
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
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

// Byte offset of 16-byte chunk q (k = 8q .. 8q+7) of row r in a decoded block.
// Row r's chunks are XORed with r (and chunk bit 4 into bit 0), so a quarter
// wave reading one chunk of 16 rows, or writing chunks 2i (or 2i+1) of one
// row for 16 consecutive i, touches 16 distinct bank groups.
__device__ __forceinline__ uint32_t wpos(uint32_t r, uint32_t q) {
    return r * 2048u + 16u * (q ^ r ^ ((q >> 4) & 1u));
}

__global__ __launch_bounds__(64 * NW) void lut6_gemv_mfma_kernel(
    const uint8_t* __restrict__ packed, int64_t ld, const uint16_t* __restrict__ lut,
    const uint16_t* __restrict__ x, void* __restrict__ y, int y_f32, float* __restrict__ part,
    int rows, int cols, int batch, int nblocks, int cps) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds8*)smem;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int blk = blockIdx.x % nblocks, ks = blockIdx.x / nblocks;
    const int n0 = blk * RB;
    const int nch = cols / CH;
    const int c0 = ks * cps, c1 = min(c0 + cps, nch);  // this workgroup's chunks [c0, c1)
    const int n = c1 - c0;

    // row tables
    if (tid < RB * 8) {
        const int r = tid >> 3, part8 = tid & 7;
        const u32x4 v = *reinterpret_cast<const u32x4*>(lut + (int64_t)min(n0 + r, rows - 1) * 64 + part8 * 8);
        *(lds128*)(uintptr_t)(lds0 + OFF_TAB + 16u * (uint32_t)tid) = v;
    }

    // this wave decodes rows wave + 4u (u = 0..3)
    const uint8_t* prow[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
        prow[u] = packed + (int64_t)min(n0 + wave + 4 * u, rows - 1) * ld + (int64_t)768 * c0 + 12 * lane;
    uint32_t cr[PC + 1][4][3];
    // codes of chunk c0 + c of the four rows (clamped to the last chunk) into
    // register slot cs % (PC + 1) (cs: a compile-time number congruent to c)
    auto load_codes = [&](int cs, int c) {
        const int cc = min(c, n - 1);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t* q = reinterpret_cast<const uint32_t*>(prow[u] + 768 * cc);
            cr[cs % (PC + 1)][u][0] = __builtin_nontemporal_load(q);
            cr[cs % (PC + 1)][u][1] = __builtin_nontemporal_load(q + 1);
            cr[cs % (PC + 1)][u][2] = __builtin_nontemporal_load(q + 2);
        }
    };
    // x fragments: batch row min(lane % 16, batch - 1), k = 1024 c + 32 s + 8 (lane / 16)
    const uint16_t* xrow = x + (int64_t)min(lane & 15, batch - 1) * cols + (int64_t)CH * c0 + 8 * (lane >> 4) +
                           32 * wave;
    bf16x8 xf[2][SLICES];
    auto load_x = [&](int c, int buf) {
        const int cc = min(c, n - 1);
#pragma unroll
        for (int s = 0; s < SLICES; ++s)
            xf[buf][s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xrow + CH * cc + 128 * s));
    };

    uint32_t mask = 0x7Eu;
    asm volatile("" : "+v"(mask));  // in a VGPR: (code & mask) | base is one v_and_or_b32
    const uint32_t tab = lds0 + OFF_TAB + 128u * (uint32_t)wave;  // + 512 u; multiple of 128
    // decode the chunk whose codes sit in register slot cs % (PC + 1) into buffer buf
    auto decode = [&](int cs, int buf) {
        const uint32_t wb = lds0 + (uint32_t)buf * WT_BYTES;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t d0 = cr[cs % (PC + 1)][u][0], d1 = cr[cs % (PC + 1)][u][1], d2 = cr[cs % (PC + 1)][u][2];
            const uint32_t tb = tab + 512u * u;
            uint32_t a[16];
            a[0] = (code_x2<0>(d0, d1, d2) & mask) | tb;
            a[1] = (code_x2<1>(d0, d1, d2) & mask) | tb;
            a[2] = (code_x2<2>(d0, d1, d2) & mask) | tb;
            a[3] = (code_x2<3>(d0, d1, d2) & mask) | tb;
            a[4] = (code_x2<4>(d0, d1, d2) & mask) | tb;
            a[5] = (code_x2<5>(d0, d1, d2) & mask) | tb;
            a[6] = (code_x2<6>(d0, d1, d2) & mask) | tb;
            a[7] = (code_x2<7>(d0, d1, d2) & mask) | tb;
            a[8] = (code_x2<8>(d0, d1, d2) & mask) | tb;
            a[9] = (code_x2<9>(d0, d1, d2) & mask) | tb;
            a[10] = (code_x2<10>(d0, d1, d2) & mask) | tb;
            a[11] = (code_x2<11>(d0, d1, d2) & mask) | tb;
            a[12] = (code_x2<12>(d0, d1, d2) & mask) | tb;
            a[13] = (code_x2<13>(d0, d1, d2) & mask) | tb;
            a[14] = (code_x2<14>(d0, d1, d2) & mask) | tb;
            a[15] = (code_x2<15>(d0, d1, d2) & mask) | tb;
            uint32_t wv[8];
#pragma unroll
            for (int p = 0; p < 8; ++p)
                wv[p] = perm_lo16(*(lds16c*)(uintptr_t)a[2 * p + 1], *(lds16c*)(uintptr_t)a[2 * p]);
            const uint32_t r = (uint32_t)(wave + 4 * u);
            *(lds128*)(uintptr_t)(wb + wpos(r, 2u * lane)) = u32x4{wv[0], wv[1], wv[2], wv[3]};
            *(lds128*)(uintptr_t)(wb + wpos(r, 2u * lane + 1u)) = u32x4{wv[4], wv[5], wv[6], wv[7]};
        }
    };
    // A fragments: row lane % 16, slice 4 s' + wave (s' = 0..7), chunk q = 4 slice + lane / 16
    const uint32_t arow = (uint32_t)(lane & 15);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    auto mma = [&](int buf, int xb) {
        const uint32_t wb = lds0 + (uint32_t)buf * WT_BYTES;
#pragma unroll
        for (int s = 0; s < SLICES; ++s) {
            const uint32_t q = (uint32_t)(4 * (4 * s + wave) + (lane >> 4));
            const bf16x8 af = __builtin_bit_cast(bf16x8, *(lds128c*)(uintptr_t)(wb + wpos(arow, q)));
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, xf[xb][s], acc, 0, 0, 0);
        }
    };

#pragma unroll
    for (int c = 0; c < PC; ++c) load_codes(c, c);
    load_x(0, 0);
    __syncthreads();  // tables
    decode(0, 0);
    load_codes(PC, PC);
    __syncthreads();

    // Chunk c: request x of c + 1 and the codes of c + PC + 1, decode c + 1
    // into the other buffer, multiply c.  Past the end the chunk index is
    // clamped; the extra decode lands in a buffer that is never read.  The
    // loop is unrolled by 6 so that every register slot (codes: c % 3, x and
    // LDS buffers: c % 2) is a compile-time index.
    auto step = [&](auto cm, int c) {
        constexpr int C6 = decltype(cm)::value;
        load_x(c + 1, (C6 + 1) & 1);
        decode(C6 + 1, (C6 + 1) & 1);
        load_codes(C6 + 1 + PC, c + 1 + PC);
        mma(C6 & 1, C6 & 1);
        __syncthreads();
    };
    for (int c = 0; c < n; c += 6) {
        step(std::integral_constant<int, 0>{}, c);
        if (c + 1 < n) step(std::integral_constant<int, 1>{}, c + 1);
        if (c + 2 < n) step(std::integral_constant<int, 2>{}, c + 2);
        if (c + 3 < n) step(std::integral_constant<int, 3>{}, c + 3);
        if (c + 4 < n) step(std::integral_constant<int, 4>{}, c + 4);
        if (c + 5 < n) step(std::integral_constant<int, 5>{}, c + 5);
    }

    // D layout of a 16x16 block: lane l, item i -> row 4 (l / 16) + i, column l % 16.
    *(ldsf4*)(uintptr_t)(lds0 + OFF_RED + 16u * (uint32_t)(64 * wave + lane)) = acc;
    __syncthreads();
    {
        const int row = tid >> 4, col = tid & 15;  // output row n0 + row, batch row col
        const int l = 16 * (row >> 2) + col, i = row & 3;
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w)
            v += *(__attribute__((address_space(3))) const float*)(uintptr_t)(lds0 + OFF_RED + 16u * (uint32_t)(64 * w + l) + 4u * i);
        const int nr = n0 + row;
        if (nr < rows && col < batch) {
            if (part)
                part[((int64_t)ks * batch + col) * rows + nr] = v;
            else if (y_f32)
                reinterpret_cast<float*>(y)[(int64_t)col * rows + nr] = v;
            else
                reinterpret_cast<uint16_t*>(y)[(int64_t)col * rows + nr] = f32_to_bf16(v);
        }
    }
}

// y[b][r] = sum over splits s (in order) of part[s][b][r]
__global__ __launch_bounds__(256) void lut6_gemv_split_sum(const float* __restrict__ part, void* __restrict__ y,
                                                           int y_f32, int64_t n, int nsplit) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    float v = part[i];
    for (int s = 1; s < nsplit; ++s) v += part[(int64_t)s * n + i];
    if (y_f32)
        reinterpret_cast<float*>(y)[i] = v;
    else
        reinterpret_cast<uint16_t*>(y)[i] = f32_to_bf16(v);
}

}  // namespace

// K split: enough workgroups to cover the chip about four times over.
void lut6_mfma_split(const fqm_weights& w, int64_t* nblocks, int* nsplit, int* cps) {
    const int64_t nb = (w.rows + RB - 1) / RB;
    const int nch = (int)(w.cols / CH);
    int want = (int)std::min<int64_t>(nch, std::max<int64_t>(1, (1024 + nb - 1) / nb));
    const int per = (nch + want - 1) / want;
    *nblocks = nb;
    *cps = per;
    *nsplit = (nch + per - 1) / per;
}

bool lut6_gemv_mfma_supported(const fqm_weights& w, int batch) {
    return batch >= 2 && batch <= 16 && w.cols > 0 && w.cols % CH == 0 && w.cols <= 0x7fffffff &&
           w.rows > 0 && w.rows <= 0x7fffffff;
}

size_t lut6_gemv_mfma_workspace(const fqm_weights& w, int batch) {
    if (!lut6_gemv_mfma_supported(w, batch)) return 0;
    int64_t nb;
    int ns, cps;
    lut6_mfma_split(w, &nb, &ns, &cps);
    return ns > 1 ? (size_t)ns * (size_t)batch * (size_t)w.rows * sizeof(float) : 0;
}

hipError_t launch_lut6_gemv_mfma(const fqm_weights& w, const uint16_t* x, void* y, int y_f32, int batch,
                                 float* ws, hipStream_t s) {
    int64_t nb;
    int ns, cps;
    lut6_mfma_split(w, &nb, &ns, &cps);
    if (nb * ns > 0x7fffffff) return hipErrorInvalidValue;
    float* part = ns > 1 ? ws : nullptr;
    if (ns > 1 && !ws) return hipErrorInvalidValue;
    // more than 64 KB of dynamic LDS per workgroup
    const hipError_t ea = hipFuncSetAttribute(reinterpret_cast<const void*>(&lut6_gemv_mfma_kernel),
                                              hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    if (ea != hipSuccess) return ea;
    hipLaunchKernelGGL(lut6_gemv_mfma_kernel, dim3((unsigned)(nb * ns)), dim3(64 * NW), LDS_BYTES, s,
                       w.lut6.packed, w.lut6.ld, w.lut6.lut, x, y, y_f32, part, (int)w.rows, (int)w.cols, batch,
                       (int)nb, cps);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || ns == 1) return e;
    const int64_t total = (int64_t)batch * w.rows;
    hipLaunchKernelGGL(lut6_gemv_split_sum, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, part, y, y_f32,
                       total, ns);
    return hipGetLastError();
}

}  // namespace fqm
