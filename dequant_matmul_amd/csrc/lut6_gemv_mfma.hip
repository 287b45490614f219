// Per-row LUT GEMV for batch 2..16: y[b][r] = sum_k lut[r][code[r][k]] * x[b][k],
// 6-bit codes (64-entry tables, 4 codes per 3 bytes) or 4-bit codes (16-entry
// tables, 2 codes per byte).
//
// Source: "Qwen3.8-27B - BenQ 6-bit", "What BenQ stores": a weight is its
// row's table entry selected by the 6-bit code, gathered inside the matmul;
// "Why equal-width shells" places 8 tiers in 4 bits, read the same way.
//
// With more than one activation row the multiply-adds per weight grow with
// the batch, so the contraction runs on the matrix cores
// (v_mfma_f32_16x16x32_bf16, fp32 accumulate) and the decode stays the
// batch-independent part:
//   - A workgroup owns 16 rows (one MFMA row block) and a range of 512-wide
//     K chunks; wave w takes k [64 w, 64 w + 64) of every chunk.
//   - Codes arrive with coalesced loads (a wave instruction reads 384
//     (6-bit) or 256 (4-bit) contiguous bytes of each of two rows) four
//     chunks ahead and pass through a small LDS buffer (16 rows x one chunk),
//     because the operand layout wants 16 rows per wave instruction.
//   - Weights are gathered straight into the MFMA row operand: lane
//     (r = lane % 16, g = lane / 16) reads the 12- (8-) byte piece of row r holding
//     codes [16 g, 16 g + 16) of the wave's 64 k, gathers the 16 bf16 values
//     from row r's table and packs them into the operands of the wave's two
//     32-wide k slices (slice s uses codes 16 g + 8 s + e; the x operand is
//     read in the same k order).  W never passes through LDS as a tile.
//   - Tables: each row's table is held four times, one copy per lane group
//     g, entry e of (row r, copy g) at 256 e + 4 (16 g + r): the 64 lanes of a
//     gather hit 64 distinct banks, whatever the codes.
//   - x chunks (batch rows past the batch are not loaded; their output
//     columns are not stored) sit in LDS, double-buffered, as 1024-byte rows
//     with XOR-swizzled 16-byte chunks; x is staged through registers with
//     coalesced loads one chunk ahead.  The gathers run one chunk ahead of
//     their MFMAs.
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
typedef __attribute__((address_space(3))) uint16_t lds16;
typedef __attribute__((address_space(3))) uint32_t lds32;
typedef __attribute__((address_space(3))) const uint16_t lds16c;
typedef __attribute__((address_space(3))) u32x4 lds128;
typedef __attribute__((address_space(3))) const u32x4 lds128c;
typedef __attribute__((address_space(3))) f32x4 ldsf4;
typedef __attribute__((address_space(3))) const float ldsf;

constexpr int RB = 16;                         // rows per workgroup
constexpr int NW = 8;                          // waves per workgroup
constexpr int CH = 512;                        // k per chunk
constexpr int CSLOTS = 4;                      // code register slots: chunks are loaded 4 steps ahead
constexpr int SLICES = CH / 32 / NW;           // k slices per wave per chunk
constexpr int SPLIT_TARGET = 1024;             // aim for at least this many workgroups
static_assert(SLICES == 2 && CH == 64 * NW, "a wave takes 64 k of a chunk: 16 codes per lane");

// Workgroup barrier that waits for nothing: the caller has made its LDS
// stores complete already (the LDS reads still in flight are gathers from
// the tables, which no wave rewrites inside the loop).
__device__ __forceinline__ void barrier_no_wait() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t perm_lo16(uint32_t hi, uint32_t lo) {
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// Per code width: piece bytes (16 codes), table entries, code buffer row
// stride (a chunk's bytes + 16, so that a read of 16 rows starts in 16
// different bank groups), table bytes (4 copies x 16 rows x
// entries, 4-byte slots; at least what the final reduction reuses).
template <int BITS>
struct LutFmt {
    static constexpr int PB = 2 * BITS;
    static constexpr int ND = PB / 4;
    static constexpr int ENTRIES = 1 << BITS;
    static constexpr int CHB = CH * BITS / 8;
    static constexpr int CB_ROW = CHB + 16;
    static constexpr int TAB_BYTES = std::max(ENTRIES * 256, NW * 64 * 16);
};

// Table offset of code J of a piece d[0..ND): the code's bits moved to bits
// 8.. (entry stride 256 bytes), other bits still to be masked.
template <int BITS, int J>
__device__ __forceinline__ uint32_t code_x256(const uint32_t* d) {
    constexpr int bit = BITS * J, w = bit >> 5, o = bit & 31;
    if constexpr (o + BITS <= 32) {
        if constexpr (o >= 8) return d[w] >> (o - 8);
        else return d[w] << (8 - o);
    } else {
        return __builtin_amdgcn_alignbit(d[w + 1], d[w], o - 8);
    }
}

// Byte offset of 16-byte chunk q (k = 8q .. 8q+7) of row r in a [16][512]
// bf16 tile.  Rows are 1024 bytes, so every row starts in bank 0; row r's
// chunks are XORed with a permutation of r's bits (bit 0 -> 0, 1 -> 3, 2 -> 1,
// 3 -> 2).  The operand read of a wave (lane (r, g) reads chunk 2 g + s of
// row r % rows, s fixed) then spreads its 16-byte pieces evenly over the 16
// bank groups of 64 banks: two per group for 8 batch rows (32 distinct
// pieces), four for 16 (64 pieces), the minimum for 512 and 1024 bytes.
// A wave storing the 64 chunks of one row is conflict-free for any XOR.
__device__ __forceinline__ uint32_t tpos(uint32_t r, uint32_t q) {
    const uint32_t sw = (r & 1u) | ((r & 2u) << 2) | ((r & 4u) >> 1) | ((r & 8u) >> 1);
    return r * 1024u + 16u * (q ^ sw);
}

// XROWS: batch rows an x block holds (8 or 16, >= batch); XPT = XROWS / 8
// 16-byte x pieces per thread per chunk.
template <int BITS, int XROWS>
__device__ __forceinline__ void gemv_mfma_body(
    const uint8_t* __restrict__ packed, int64_t ld, const uint16_t* __restrict__ lut,
    const uint16_t* __restrict__ x, void* __restrict__ y, int y_f32, float* __restrict__ part,
    int rows, int cols, int batch, int nblocks, int cps) {
    using F = LutFmt<BITS>;
    constexpr int PB = F::PB, ND = F::ND, CHB = F::CHB, CB_ROW = F::CB_ROW, TAB_BYTES = F::TAB_BYTES;
    __shared__ __attribute__((aligned(16))) uint8_t s_tab[TAB_BYTES];
    constexpr int XPT = XROWS / 8;
    __shared__ __attribute__((aligned(16))) uint8_t s_x0[XROWS * 1024];
    __shared__ __attribute__((aligned(16))) uint8_t s_x1[XROWS * 1024];
    __shared__ __attribute__((aligned(16))) uint8_t s_c0[RB * CB_ROW];
    __shared__ __attribute__((aligned(16))) uint8_t s_c1[RB * CB_ROW];
    lds8* const CB[2] = {(lds8*)s_c0, (lds8*)s_c1};
    lds8* const TAB = (lds8*)s_tab;
    lds8* const XS[2] = {(lds8*)s_x0, (lds8*)s_x1};
    lds8* const RED = (lds8*)s_tab;  // after the K loop
    static_assert(NW * 64 * 16 <= TAB_BYTES, "the reduction reuses the tables");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, g = lane >> 4;
    const int blk = blockIdx.x % nblocks, ks = blockIdx.x / nblocks;
    const int n0 = blk * RB;
    const int nch = cols / CH;
    const int c0 = ks * cps, c1 = min(c0 + cps, nch);  // this workgroup's chunks [c0, c1)
    const int n = c1 - c0;

    // row tables, four copies: thread t writes copy t / 128 of entries
    // EPT (t % 8) .. + EPT - 1 of row (t / 8) % 16 (loaded here, stored to LDS
    // once the first code and x loads are out, so that their latencies overlap)
    constexpr int EPT = F::ENTRIES / 8;  // entries per thread: 8 (6-bit) or 2 (4-bit)
    const int tr = (tid >> 3) & 15, tpart = tid & 7, tcp = tid >> 7;
    uint32_t tv[EPT / 2];
    {
        const uint32_t* tsrc =
            reinterpret_cast<const uint32_t*>(lut + (int64_t)min(n0 + tr, rows - 1) * F::ENTRIES + tpart * EPT);
#pragma unroll
        for (int i = 0; i < EPT / 2; ++i) tv[i] = tsrc[i];
    }
    static_assert(64 * NW == RB * 8 * 4, "one table item per thread");

    // Global code loads: wave w, lane half h, lane j = lane % 32 loads the
    // piece j of row 2 w + h.  Chunk c goes to register slot c % CSLOTS, then
    // to the code buffer.
    const int crow = 2 * wave + (lane >> 5), cpiece = lane & 31;
    const uint8_t* prow = packed + (int64_t)min(n0 + crow, rows - 1) * ld + (int64_t)CHB * c0 + PB * cpiece;
    uint32_t cr[CSLOTS][ND];
    auto load_codes = [&](int cs, int c) {
        const int cc = min(c, n - 1);
        const uint32_t* q = reinterpret_cast<const uint32_t*>(prow + CHB * cc);
#pragma unroll
        for (int i = 0; i < ND; ++i) cr[cs % CSLOTS][i] = __builtin_nontemporal_load(q + i);
    };
    auto store_codes = [&](int cs, int buf) {
        lds8* d = CB[buf] + CB_ROW * crow + PB * cpiece;
#pragma unroll
        for (int i = 0; i < ND; ++i) *(lds32*)(d + 4 * i) = cr[cs % CSLOTS][i];
    };
    // lane (r16, g): row n0 + r16, codes [64 wave + 16 g, + 16) of each chunk
    const uint32_t cread = (uint32_t)(CB_ROW * r16 + 4 * PB * wave + PB * g);
    const uint32_t tabrow = (uint32_t)(4 * (16 * g + r16));  // (code << 8) | tabrow

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

    uint32_t mask = (uint32_t)(F::ENTRIES - 1) << 8;
    asm volatile("" : "+v"(mask));  // in a VGPR: (code & mask) | row is one v_and_or_b32
    // Gather the 16 weights of the chunk whose codes sit in code buffer buf;
    // they feed the MFMAs one chunk later.
    uint32_t gv[16];
    auto gather = [&](int buf) {
        const lds8* q = CB[buf] + cread;
        uint32_t d[ND];
#pragma unroll
        for (int i = 0; i < ND; ++i) d[i] = *(const lds32*)(q + 4 * i);
        uint32_t a[16];
        a[0] = (code_x256<BITS, 0>(d) & mask) | tabrow;
        a[1] = (code_x256<BITS, 1>(d) & mask) | tabrow;
        a[2] = (code_x256<BITS, 2>(d) & mask) | tabrow;
        a[3] = (code_x256<BITS, 3>(d) & mask) | tabrow;
        a[4] = (code_x256<BITS, 4>(d) & mask) | tabrow;
        a[5] = (code_x256<BITS, 5>(d) & mask) | tabrow;
        a[6] = (code_x256<BITS, 6>(d) & mask) | tabrow;
        a[7] = (code_x256<BITS, 7>(d) & mask) | tabrow;
        a[8] = (code_x256<BITS, 8>(d) & mask) | tabrow;
        a[9] = (code_x256<BITS, 9>(d) & mask) | tabrow;
        a[10] = (code_x256<BITS, 10>(d) & mask) | tabrow;
        a[11] = (code_x256<BITS, 11>(d) & mask) | tabrow;
        a[12] = (code_x256<BITS, 12>(d) & mask) | tabrow;
        a[13] = (code_x256<BITS, 13>(d) & mask) | tabrow;
        a[14] = (code_x256<BITS, 14>(d) & mask) | tabrow;
        a[15] = (code_x256<BITS, 15>(d) & mask) | tabrow;
#pragma unroll
        for (int e = 0; e < 16; ++e) gv[e] = *(lds16c*)(TAB + a[e]);
    };
    // x operand of slice s: batch row lane % 16, 16-byte chunk 8 wave + 2 g + s
    uint32_t xopos[SLICES];
#pragma unroll
    for (int s2 = 0; s2 < SLICES; ++s2)
        xopos[s2] = tpos((uint32_t)(r16 & (XROWS - 1)), (uint32_t)(8 * wave + 2 * g + s2));  // columns >= XROWS are never stored
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};

    // ---- prologue: x(0) and the codes of chunks 0, 1 in LDS, W(0) gathered ------
#pragma unroll
    for (int c = 0; c < CSLOTS; ++c) load_codes(c, c);
    load_x(0, 0);
    {
        lds8* dst = TAB + 256 * EPT * tpart + 4 * (16 * tcp + tr);
#pragma unroll
        for (int e = 0; e < EPT; ++e) *(lds16*)(dst + 256 * e) = (uint16_t)(tv[e >> 1] >> (16 * (e & 1)));
    }
    store_codes(0, 0);
    store_codes(1, 1);
    store_x(0, 0);
    load_x(1, 1);
    __syncthreads();  // tables, x block 0, code buffers
    gather(0);        // its code reads finish before the gathers go out
    barrier_no_wait();  // code buffer 0 is rewritten in chunk 0

    // Chunk c: read its x operands, store x(c+1) (loaded one chunk earlier)
    // and the codes of c+2 (loaded two chunks earlier), pack the weights
    // gathered one chunk earlier into the row operands, request x(c+2) and
    // the codes of c+4; wait for this chunk's LDS reads and stores; gather
    // W(c+1) (codes in the buffer since the previous chunk); then the MFMAs
    // of c and a barrier that does not wait for the gathers (their results
    // are used one chunk later).  Past the end the chunk index is clamped;
    // the extra work lands in buffers that are never read.  The loop is
    // unrolled by 4 so that every register slot (codes: c % 4, x: c % 2) and
    // buffer (c % 2) is a compile-time index.
    auto step = [&](auto cm, int c) {
        constexpr int C4 = decltype(cm)::value;
        constexpr int B = C4 & 1;
        bf16x8 af[SLICES], bf[SLICES];
#pragma unroll
        for (int s2 = 0; s2 < SLICES; ++s2) bf[s2] = __builtin_bit_cast(bf16x8, *(lds128c*)(XS[B] + xopos[s2]));
        store_x(B ^ 1, B ^ 1);
        store_codes(C4 + 2, B);
#pragma unroll
        for (int s2 = 0; s2 < SLICES; ++s2)
            af[s2] = __builtin_bit_cast(
                bf16x8, u32x4{perm_lo16(gv[8 * s2 + 1], gv[8 * s2]), perm_lo16(gv[8 * s2 + 3], gv[8 * s2 + 2]),
                              perm_lo16(gv[8 * s2 + 5], gv[8 * s2 + 4]), perm_lo16(gv[8 * s2 + 7], gv[8 * s2 + 6])});
        load_x(B, c + 2);
        load_codes(C4 + CSLOTS, c + CSLOTS);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) only: this chunk's LDS reads and stores are done
        asm volatile("" ::: "memory");
        gather(B ^ 1);
#pragma unroll
        for (int s2 = 0; s2 < SLICES; ++s2) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s2], bf[s2], acc, 0, 0, 0);
        barrier_no_wait();
    };
    for (int c = 0; c < n; c += 4) {
        step(std::integral_constant<int, 0>{}, c);
        if (c + 1 < n) step(std::integral_constant<int, 1>{}, c + 1);
        if (c + 2 < n) step(std::integral_constant<int, 2>{}, c + 2);
        if (c + 3 < n) step(std::integral_constant<int, 3>{}, c + 3);
    }

    __syncthreads();  // every wave's last gathers have read the tables, which RED overwrites
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

#define GEMV_MFMA_ARGS                                                                                     \
    const uint8_t *__restrict__ packed, int64_t ld, const uint16_t *__restrict__ lut,                       \
        const uint16_t *__restrict__ x, void *__restrict__ y, int y_f32, float *__restrict__ part, int rows, \
        int cols, int batch, int nblocks, int cps

template <int XROWS>
__global__ __launch_bounds__(64 * NW) void lut6_gemv_mfma_kernel(GEMV_MFMA_ARGS) {
    gemv_mfma_body<6, XROWS>(packed, ld, lut, x, y, y_f32, part, rows, cols, batch, nblocks, cps);
}

template <int XROWS>
__global__ __launch_bounds__(64 * NW) void lut4_gemv_mfma_kernel(GEMV_MFMA_ARGS) {
    gemv_mfma_body<4, XROWS>(packed, ld, lut, x, y, y_f32, part, rows, cols, batch, nblocks, cps);
}
#undef GEMV_MFMA_ARGS

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
void lut_mfma_split(const fqm_weights& w, int64_t* nblocks, int* nsplit, int* cps) {
    const int64_t nb = (w.rows + RB - 1) / RB;
    const int nch = (int)(w.cols / CH);
    const int want = (int)std::min<int64_t>(nch, std::max<int64_t>(1, (SPLIT_TARGET + nb - 1) / nb));
    const int per = (nch + want - 1) / want;
    *nblocks = nb;
    *cps = per;
    *nsplit = (nch + per - 1) / per;
}

bool lut_gemv_mfma_supported(const fqm_weights& w, int batch) {
    return batch >= 2 && batch <= 16 && w.cols > 0 && w.cols % CH == 0 && w.cols <= 0x7fffffff &&
           w.rows > 0 && w.rows <= 0x7fffffff;
}

size_t lut_gemv_mfma_workspace(const fqm_weights& w, int batch) {
    if (!lut_gemv_mfma_supported(w, batch)) return 0;
    // the one-row-per-wave kernels take these batches
    if (w.format == FQM_LUT6 ? lut6_gemv_rows_path(w, batch) : lut4_gemv_rows_path(w, batch)) return 0;
    int64_t nb;
    int ns, cps;
    lut_mfma_split(w, &nb, &ns, &cps);
    return ns > 1 ? (size_t)ns * (size_t)batch * (size_t)w.rows * sizeof(float) : 0;
}

hipError_t launch_lut_gemv_mfma(const fqm_weights& w, const uint16_t* x, void* y, int y_f32, int batch,
                                float* ws, hipStream_t s) {
    if (w.format != FQM_LUT6 && w.format != FQM_LUT4) return hipErrorInvalidValue;
    int64_t nb;
    int ns, cps;
    lut_mfma_split(w, &nb, &ns, &cps);
    if (nb * ns > 0x7fffffff) return hipErrorInvalidValue;
    float* part = ns > 1 ? ws : nullptr;
    if (ns > 1 && !ws) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(nb * ns)), block(64 * NW);
    const bool six = w.format == FQM_LUT6;
    const uint8_t* packed = six ? w.lut6.packed : w.lut4.packed;
    const int64_t ld = six ? w.lut6.ld : w.lut4.ld;
    const uint16_t* lut = six ? w.lut6.lut : w.lut4.lut;
    const int r = (int)w.rows, c = (int)w.cols, n = (int)nb;
    if (six && batch <= 8)
        hipLaunchKernelGGL(lut6_gemv_mfma_kernel<8>, grid, block, 0, s, packed, ld, lut, x, y, y_f32, part, r, c,
                           batch, n, cps);
    else if (six)
        hipLaunchKernelGGL(lut6_gemv_mfma_kernel<16>, grid, block, 0, s, packed, ld, lut, x, y, y_f32, part, r, c,
                           batch, n, cps);
    else if (batch <= 8)
        hipLaunchKernelGGL(lut4_gemv_mfma_kernel<8>, grid, block, 0, s, packed, ld, lut, x, y, y_f32, part, r, c,
                           batch, n, cps);
    else
        hipLaunchKernelGGL(lut4_gemv_mfma_kernel<16>, grid, block, 0, s, packed, ld, lut, x, y, y_f32, part, r, c,
                           batch, n, cps);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || ns == 1) return e;
    const int64_t total = (int64_t)batch * w.rows;
    hipLaunchKernelGGL(lut6_gemv_split_sum, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, part, y, y_f32,
                       total, ns);
    return hipGetLastError();
}

}  // namespace fqm
