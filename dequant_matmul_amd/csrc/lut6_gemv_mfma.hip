// Per-row LUT 6-bit GEMV for batch 2..16: y[b][r] = sum_k lut[r][code[r][k]] * x[b][k].
//
// Source: "Qwen3.8-27B - BenQ 6-bit", "What BenQ stores": a weight is its
// row's table entry selected by the 6-bit code, gathered inside the matmul.
//
// With more than one activation row the multiply-adds per weight grow with
// the batch, so the contraction runs on the matrix cores
// (v_mfma_f32_16x16x32_bf16, fp32 accumulate) and the decode stays the
// batch-independent part:
//   - A workgroup owns 16 rows (one MFMA row block) and a range of 512-wide
//     K chunks.  A wave instruction decodes two rows (32 lanes each; the two
//     tables sit in opposite halves of the 64 banks): lane j loads the row's
//     12-byte piece j (16 codes) and gathers its 16 weights from the row's
//     128-byte table in LDS.
//   - The decoded 16 x 512 bf16 block and the 16 x 512 x block (batch rows
//     past the batch are not loaded; their output columns are not stored)
//     sit in LDS, double-buffered, as 1024-byte rows whose 16-byte chunks
//     are permuted and XOR-swizzled, so the decode writes, the x stores (x
//     staged through registers with coalesced loads one chunk ahead) and
//     both MFMA operand reads are free of bank conflicts.  Every wave multiplies a quarter of
//     the chunk's 32-wide k slices.
//   - The waves' 16 x 16 partial results are added in wave order; K is
//     split over workgroups so that the grid covers the chip several times,
//     the partials go to the workspace and a second kernel adds them in
//     split order.
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
typedef __attribute__((address_space(3))) const float ldsf;

constexpr int RB = 16;                         // rows per workgroup
constexpr int NW = 8;                          // waves per workgroup
constexpr int PPW = RB / 2 / NW;               // row pairs each wave decodes per chunk
constexpr int CH = 512;                        // k per chunk
constexpr int PC = 2;                          // code chunks requested ahead
constexpr int TILE = RB * CH * 2;              // one decoded W block (16 KB); an x block is XROWS KB
constexpr int SLICES = CH / 32 / NW;           // k slices per wave per chunk
constexpr int SPLIT_TARGET = 1024;             // aim for at least this many workgroups

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

// Byte offset of 16-byte chunk q (k = 8q .. 8q+7) of row r in a [16][512]
// bf16 tile.  Row r's chunks are XORed with r (and chunk bit 4 into bit 0), so
// a quarter wave reading one chunk of 16 rows, or writing chunks 2i (or
// 2i+1) of one row for 16 consecutive i, touches 16 distinct bank groups.
__device__ __forceinline__ uint32_t tpos(uint32_t r, uint32_t q) {
    return r * 1024u + 16u * (q ^ r ^ ((q >> 4) & 1u));
}

// W block layout: chunk q of row r at slot ((q / 2) | (q % 2) * 32) ^ r.  A
// decode write instruction covers chunks 2j (or 2j + 1) of a row for 32
// consecutive j, i.e. 32 consecutive slots; with the layout above (stride-2
// chunks) those writes measured about 8 bank-conflict cycles per
// instruction, with this one none, and the MFMA row-fragment reads (16 rows,
// one chunk) stay conflict-free.
__device__ __forceinline__ uint32_t wpos(uint32_t r, uint32_t q) {
    return r * 1024u + 16u * (((q >> 1) | ((q & 1u) << 5)) ^ (r & 15u));
}

// XROWS: batch rows an x block holds (8 or 16, >= batch); XPT = XROWS / 8
// 16-byte x pieces per thread per chunk.  With XROWS = 8 a workgroup uses
// about 50 KB of LDS and three fit on a CU.
template <int XROWS>
__global__ __launch_bounds__(64 * NW) void lut6_gemv_mfma_kernel(
    const uint8_t* __restrict__ packed, int64_t ld, const uint16_t* __restrict__ lut,
    const uint16_t* __restrict__ x, void* __restrict__ y, int y_f32, float* __restrict__ part,
    int rows, int cols, int batch, int nblocks, int cps) {
    __shared__ __attribute__((aligned(1024))) uint8_t s_tab[RB * 128];  // low addresses: immediate offsets
    __shared__ __attribute__((aligned(16))) uint8_t s_w0[TILE];
    __shared__ __attribute__((aligned(16))) uint8_t s_w1[TILE];
    constexpr int XPT = XROWS / 8;
    __shared__ __attribute__((aligned(16))) uint8_t s_x0[XROWS * 1024];
    __shared__ __attribute__((aligned(16))) uint8_t s_x1[XROWS * 1024];
    static_assert(NW * 64 * 16 <= TILE, "the reduction reuses a W buffer");
    lds8* const TAB = (lds8*)s_tab;
    lds8* const WS[2] = {(lds8*)s_w0, (lds8*)s_w1};
    lds8* const XS[2] = {(lds8*)s_x0, (lds8*)s_x1};
    lds8* const RED = (lds8*)s_w0;  // after the K loop

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, j = lane & 31;
    const int blk = blockIdx.x % nblocks, ks = blockIdx.x / nblocks;
    const int n0 = blk * RB;
    const int nch = cols / CH;
    const int c0 = ks * cps, c1 = min(c0 + cps, nch);  // this workgroup's chunks [c0, c1)
    const int n = c1 - c0;

    // row tables
    if (tid < RB * 8) {
        const int r = tid >> 3, part8 = tid & 7;
        const u32x4 v = *reinterpret_cast<const u32x4*>(lut + (int64_t)min(n0 + r, rows - 1) * 64 + part8 * 8);
        *(lds128*)(TAB + 16 * tid) = v;
    }

    // this wave decodes rows 2 (wave + NW u) + h, u < PPW; lane j takes piece j
    const uint8_t* prow[PPW];
    uint32_t tabrow[PPW];  // table offsets, multiples of 128: (code & mask) | tabrow is one v_and_or_b32
#pragma unroll
    for (int u = 0; u < PPW; ++u) {
        const int r = 2 * (wave + NW * u) + h;
        prow[u] = packed + (int64_t)min(n0 + r, rows - 1) * ld + (int64_t)384 * c0 + 12 * j;
        tabrow[u] = (uint32_t)(128 * r);
    }
    uint32_t cr[PC + 1][PPW][3];
    // codes of chunk c0 + c of the two rows (clamped to the last chunk) into
    // register slot cs % (PC + 1) (cs: a compile-time number congruent to c)
    auto load_codes = [&](int cs, int c) {
        const int cc = min(c, n - 1);
#pragma unroll
        for (int u = 0; u < PPW; ++u) {
            const uint32_t* q = reinterpret_cast<const uint32_t*>(prow[u] + 384 * cc);
            cr[cs % (PC + 1)][u][0] = __builtin_nontemporal_load(q);
            cr[cs % (PC + 1)][u][1] = __builtin_nontemporal_load(q + 1);
            cr[cs % (PC + 1)][u][2] = __builtin_nontemporal_load(q + 2);
        }
    };
    // x block of chunk c0 + c: piece p = tid + 256 u is batch row p / 64,
    // 16-byte chunk p % 64 (pieces past the batch repeat the last one: same
    // bytes to the same address).  Loaded one chunk ahead into registers.
    const uint16_t* xsrc[XPT];
    uint32_t xdst[XPT];
#pragma unroll
    for (int u = 0; u < XPT; ++u) {
        const int pc = min(tid + 64 * NW * u, 64 * batch - 1);
        xsrc[u] = x + (int64_t)(pc >> 6) * cols + (int64_t)CH * c0 + 8 * (pc & 63);
        xdst[u] = tpos((uint32_t)(pc >> 6), (uint32_t)(pc & 63));
    }
    u32x4 xw[2][XPT];
    auto load_x = [&](int set, int c) {
        const int cc = min(c, n - 1);
#pragma unroll
        for (int u = 0; u < XPT; ++u) xw[set][u] = *reinterpret_cast<const u32x4*>(xsrc[u] + CH * cc);
    };
    auto store_x = [&](int set, int buf) {
#pragma unroll
        for (int u = 0; u < XPT; ++u) *(lds128*)(XS[buf] + xdst[u]) = xw[set][u];
    };

    uint32_t mask = 0x7Eu;
    asm volatile("" : "+v"(mask));  // in a VGPR: (code & mask) | row is one v_and_or_b32
    // Gather the weights of the chunk whose codes sit in register slot
    // cs % (PC + 1); they are written to LDS one chunk later.
    uint32_t g[PPW][16];
    auto gather = [&](int cs) {
#pragma unroll
        for (int u = 0; u < PPW; ++u) {
            const uint32_t d0 = cr[cs % (PC + 1)][u][0], d1 = cr[cs % (PC + 1)][u][1], d2 = cr[cs % (PC + 1)][u][2];
            const uint32_t tb = tabrow[u];
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
#pragma unroll
            for (int e = 0; e < 16; ++e) g[u][e] = *(lds16c*)(TAB + a[e]);
        }
    };
    // Write the gathered weights as bf16 pairs into W buffer buf.
    auto write_w = [&](int buf) {
#pragma unroll
        for (int u = 0; u < PPW; ++u) {
            uint32_t wv[8];
#pragma unroll
            for (int p = 0; p < 8; ++p) wv[p] = perm_lo16(g[u][2 * p + 1], g[u][2 * p]);
            const uint32_t r = (uint32_t)(2 * (wave + NW * u) + h);
            *(lds128*)(WS[buf] + wpos(r, 2u * j)) = u32x4{wv[0], wv[1], wv[2], wv[3]};
            *(lds128*)(WS[buf] + wpos(r, 2u * j + 1u)) = u32x4{wv[4], wv[5], wv[6], wv[7]};
        }
    };
    // operand offsets: row (W) or batch row (x) lane % 16, slice NW s + wave, chunk 4 slice + lane / 16
    uint32_t wopos[SLICES], xopos[SLICES];
#pragma unroll
    for (int s2 = 0; s2 < SLICES; ++s2) {
        const uint32_t q = (uint32_t)(4 * (NW * s2 + wave) + (lane >> 4));
        wopos[s2] = wpos((uint32_t)(lane & 15), q);
        xopos[s2] = tpos((uint32_t)(lane & 15 & (XROWS - 1)), q);  // columns >= XROWS are never stored
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};

    // ---- prologue: W(0) and x(0) in LDS, W(1) gathered, x(1) loaded --------------
#pragma unroll
    for (int c = 0; c < PC + 1; ++c) load_codes(c, c);
    load_x(0, 0);
    store_x(0, 0);
    load_x(1, 1);
    __syncthreads();  // tables, x block 0
    gather(0);
    write_w(0);
    gather(1);
    load_codes(PC + 1, PC + 1);
    __syncthreads();

    // Chunk c: read its MFMA operands first; then write W(c+1) (gathered one
    // chunk earlier), store x(c+1) (loaded one chunk earlier), gather W(c+2),
    // request x(c+2) and the codes of c + PC + 2; then the MFMAs of c.  Past
    // the end the chunk index is clamped; the extra work lands in buffers that
    // are never read.  The loop is unrolled by 6 so that every register slot
    // (codes: c % 3, x: c % 2) and buffer (c % 2) is a compile-time index.
    auto step = [&](auto cm, int c) {
        constexpr int C6 = decltype(cm)::value;
        constexpr int B = C6 & 1;
        bf16x8 af[SLICES], bf[SLICES];
#pragma unroll
        for (int s2 = 0; s2 < SLICES; ++s2) {
            af[s2] = __builtin_bit_cast(bf16x8, *(lds128c*)(WS[B] + wopos[s2]));
            bf[s2] = __builtin_bit_cast(bf16x8, *(lds128c*)(XS[B] + xopos[s2]));
        }
        write_w(B ^ 1);
        store_x(B ^ 1, B ^ 1);
        gather(C6 + 2);
        load_x(B, c + 2);
        load_codes(C6 + 2 + PC, c + 2 + PC);
#pragma unroll
        for (int s2 = 0; s2 < SLICES; ++s2) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s2], bf[s2], acc, 0, 0, 0);
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
    *(ldsf4*)(RED + 16 * (64 * wave + lane)) = acc;
    __syncthreads();
    if (tid < RB * 16) {
        const int row = tid >> 4, col = tid & 15;  // output row n0 + row, batch row col
        const int l = 16 * (row >> 2) + col, i = row & 3;
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) v += *(ldsf*)(RED + 16 * (64 * w + l) + 4 * i);
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

// K split: enough workgroups to cover the chip several times over (two
// resident per CU), with the chunks spread evenly over the splits.
void lut6_mfma_split(const fqm_weights& w, int64_t* nblocks, int* nsplit, int* cps) {
    const int64_t nb = (w.rows + RB - 1) / RB;
    const int nch = (int)(w.cols / CH);
    const int want = (int)std::min<int64_t>(nch, std::max<int64_t>(1, (SPLIT_TARGET + nb - 1) / nb));
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
    const dim3 grid((unsigned)(nb * ns)), block(64 * NW);
    if (batch <= 8)
        hipLaunchKernelGGL(lut6_gemv_mfma_kernel<8>, grid, block, 0, s, w.lut6.packed, w.lut6.ld, w.lut6.lut, x, y,
                           y_f32, part, (int)w.rows, (int)w.cols, batch, (int)nb, cps);
    else
        hipLaunchKernelGGL(lut6_gemv_mfma_kernel<16>, grid, block, 0, s, w.lut6.packed, w.lut6.ld, w.lut6.lut, x, y,
                           y_f32, part, (int)w.rows, (int)w.cols, batch, (int)nb, cps);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || ns == 1) return e;
    const int64_t total = (int64_t)batch * w.rows;
    hipLaunchKernelGGL(lut6_gemv_split_sum, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, part, y, y_f32,
                       total, ns);
    return hipGetLastError();
}

}  // namespace fqm
