// Per-row LUT 6-bit GEMM (prefill): Y[m][n] = sum_k X[m][k] * lut[n][code[n][k]].
//
// Source: "Qwen3.8-27B - BenQ 6-bit", "What BenQ stores": decode is the
// row-wise gather of codes into the row's table, fused into the matrix
// product so the decoded matrix is never written out.  Each workgroup owns a
// BM x BN tile of Y; per K step of BK it decodes the BN x BK block of W into
// LDS as bf16 (exact: the table entries are bf16), stages the BM x BK block of
// X, and contracts them on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16,
// fp32 accumulate).
//
// Data movement per K step (one workgroup, 8 waves):
//   - X block: 32 KB, four 16-byte loads per thread into registers one step
//     ahead, then ds_write_b128 into the X tile.
//   - codes: the 128 rows x 48 bytes of the step, one 16-byte load per thread
//     into a small LDS code buffer, so the global loads carry each code byte
//     once.
//   - decode: a wave instruction covers two rows, 32 lanes each; lane j takes
//     the code pair (2j, 2j+1) of its row from one 8-byte LDS read, gathers
//     both bf16 values from the row table (the two tables sit in opposite
//     halves of the 64 banks: no conflicts) and stores them as one dword.
// X and W tiles are 128-byte rows whose 16-byte chunks are XOR-swizzled by
// (row / 2) % 8, so the MFMA operand reads (16 rows per quarter wave, same
// chunk) hit 16 distinct bank groups.
//
// Pipeline: the decode is spread over steps (codes read one step before
// their gathers; gathers, X stores and W writes issued between the MFMAs of
// the current step) so no wave waits on an LDS round trip with its matrix
// instructions idle.  The order inside a step is fixed in the source with
// scheduling barriers.  One workgroup barrier per step.
//
// Tile order: workgroups are dispatched round-robin over the 8 XCDs, and
// workgroup b computes M tile b % 8 (for M = 8 * BM), so each XCD keeps one
// X panel (BM x K bf16, 2.6 MB at K = 5120) in its own L2 while the W panels
// stream through; other M take the same mapping modulo the M tile count.
#include <type_traits>

#include "fqm_internal.h"

namespace fqm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef u32x2 u32x2_a4 __attribute__((aligned(4)));
typedef __attribute__((address_space(3))) uint8_t lds8;
typedef __attribute__((address_space(3))) const uint16_t lds16c;
typedef __attribute__((address_space(3))) uint32_t lds32;
typedef __attribute__((address_space(3))) const u32x2_a4 lds64c;
typedef __attribute__((address_space(3))) u32x4 lds128;
typedef __attribute__((address_space(3))) const u32x4 lds128c;

constexpr int BM = 256, BN = 128, BK = 64;
constexpr int NWAVE = 8;                     // 4 (M) x 2 (N) waves, 64 x 64 outputs each
constexpr int XT_BYTES = BM * BK * 2;        // one X tile, 128-byte rows
constexpr int WT_BYTES = BN * BK * 2;        // one W tile, 128-byte rows
constexpr int TAB_BYTES = BN * 128;          // BN row tables
constexpr int CODE_BYTES = BN * BK * 3 / 4;  // one step of codes, 48 bytes per row
constexpr int CODE_SLACK = 16;               // bytes before and after each code buffer
constexpr int CPT = CODE_BYTES / 16;         // 16-byte code pieces per step
constexpr int PAIRS = BN / NWAVE / 2;        // row pairs each wave decodes per step
constexpr int XDMA = XT_BYTES / 1024 / NWAVE;  // 1 KB direct-to-LDS X loads per wave per step
static_assert(CPT <= 64 * NWAVE && PAIRS == 8 && XDMA == 4, "tile constants");

template <int BUF>
using Buf = std::integral_constant<int, BUF>;

typedef __attribute__((address_space(1))) const void gvoid;
typedef __attribute__((address_space(3))) void lvoid;

__global__ __launch_bounds__(64 * NWAVE) void lut6_gemm_kernel(const uint16_t* __restrict__ X,
                                                               const uint8_t* __restrict__ packed,
                                                               int64_t ld,
                                                               const uint16_t* __restrict__ lut,
                                                               uint16_t* __restrict__ Y, int M,
                                                               int N, int K, int mtiles) {
    // Separate LDS objects per buffer: the X tiles are written by direct
    // global -> LDS loads, and distinct objects let the compiler see that the
    // other buffers' reads and writes do not wait for those loads.
    __shared__ __attribute__((aligned(16))) uint8_t s_x0[XT_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t s_x1[XT_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t s_w0[WT_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t s_w1[WT_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t s_tab[TAB_BYTES];  // low addresses: immediate offsets
    // The code buffers keep 16 bytes of slack on both sides: the first lane
    // pair of a row reads the dword before the row, the last one the dword
    // after it (both only feed bits that are masked off).
    __shared__ __attribute__((aligned(16))) uint8_t s_c0[CODE_BYTES + 2 * CODE_SLACK];
    __shared__ __attribute__((aligned(16))) uint8_t s_c1[CODE_BYTES + 2 * CODE_SLACK];
    lds8* const XS[2] = {(lds8*)s_x0, (lds8*)s_x1};
    lds8* const WS[2] = {(lds8*)s_w0, (lds8*)s_w1};
    lds8* const CS[2] = {(lds8*)s_c0, (lds8*)s_c1};
    lds8* const TAB = (lds8*)s_tab;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int b = blockIdx.x;
    const int mt = b % mtiles, nt = b / mtiles;
    const int m0 = mt * BM, n0 = nt * BN;
    const int wm = wave >> 1, wn = wave & 1;  // this wave's 64 x 64 output block
    const int h = lane >> 5, j = lane & 31;

    // ---- row tables (resident for the whole K loop) ---------------------------
    for (int i = tid; i < BN * 8; i += 64 * NWAVE) {
        const int r = i >> 3, part = i & 7;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (n0 + r < N) v = *reinterpret_cast<const u32x4*>(lut + (int64_t)(n0 + r) * 64 + part * 8);
        *(lds128*)(TAB + 16 * i) = v;
    }

    // ---- X: direct global -> LDS, 1 KB (8 rows) per wave instruction -----------
    // Load u of wave w fills rows 8 (8u + w) .. + 7; lane l lands at byte 16 l
    // of that kilobyte (row + l / 8, stored chunk l % 8) and fetches the
    // logical chunk that the swizzle puts there, (l % 8) ^ ((row / 2) % 8).
    const uint16_t* xsrc[XDMA];
#pragma unroll
    for (int u = 0; u < XDMA; ++u) {
        const int row = 8 * (8 * u + wave) + (lane >> 3);
        const int chunk = (lane & 7) ^ ((row >> 1) & 7);
        xsrc[u] = X + (int64_t)min(m0 + row, M - 1) * K + 8 * chunk;
    }
    auto dma_x = [&](int buf, int t, int u) {
        __builtin_amdgcn_global_load_lds((gvoid*)(xsrc[u] + t * BK), (lvoid*)(XS[buf] + 1024 * (8 * u + wave)), 16, 0, 0);
    };
    // Code piece of this thread: 16 bytes of row p / 3 (threads past the last
    // piece repeat an earlier one: same bytes to the same address).
    const int cp = tid < CPT ? tid : tid - CPT;
    const uint8_t* csrc = packed + (int64_t)min(n0 + cp / 3, N - 1) * ld + 16 * (cp % 3);
    const int cdst = CODE_SLACK + 16 * cp;

    // ---- decode constants ------------------------------------------------------
    // Wave w decodes rows 2w + 16 p + h (p = 0..7); lane j of each half takes
    // the codes 2j and 2j + 1, bits [12j, 12j + 12) of the row's 48 bytes.  A
    // funnel shift by 12j - 1 of the dword pair holding bit 12j - 1 puts code
    // 2j at bits 1..6 (its table byte offset) and code 2j + 1 at bits 7..12.
    const int q12 = 12 * j - 1;
    const int crd = CODE_SLACK + 48 * (2 * wave + h) + 4 * (q12 >> 5);
    const uint32_t csh = (uint32_t)(q12 & 31);
    // table offset of row 2w + 16p + h: a multiple of 128, so (v & mask) | off is one v_and_or_b32
    uint32_t tabp[PAIRS];
#pragma unroll
    for (int p = 0; p < PAIRS; ++p) tabp[p] = (uint32_t)(128 * (2 * wave + h) + 2048 * p);
    const int wst = 128 * (2 * wave + h) + 16 * ((j >> 2) ^ wave) + 4 * (j & 3);
    uint32_t vmask = 0x7Eu;
    asm volatile("" : "+v"(vmask));  // in a VGPR: (v & mask) | row is one v_and_or_b32

    // ---- MFMA operand offsets --------------------------------------------------
    // A: row wm*64 + 32 i + (lane % 32) of the X tile, B: row wn*64 + 32 jj +
    // (lane % 32) of the W tile; k slice q, 8 elements at 8 h: chunk 2q + h.
    int aq[BK / 16], bq[BK / 16];
#pragma unroll
    for (int q = 0; q < BK / 16; ++q) {
        const int c = 16 * ((2 * q + h) ^ ((lane >> 1) & 7));
        aq[q] = 128 * (wm * 64 + j) + c;
        bq[q] = 128 * (wn * 64 + j) + c;
    }

    const int steps = K / BK;
    u32x4 cw;               // a 16-byte code piece, three steps ahead
    u32x2 cc[PAIRS];        // this lane's code dwords for the next W tile
    uint32_t g0[PAIRS], g1[PAIRS];  // gathered bf16 values of the next W tile
    auto load_c = [&](int t) { cw = *reinterpret_cast<const u32x4*>(csrc + t * (BK * 3 / 4)); };
    auto store_c = [&](int buf) { *(lds128*)(CS[buf] + cdst) = cw; };
    auto read_codes = [&](int buf, int p) { cc[p] = *(lds64c*)(CS[buf] + crd + 768 * p); };
    auto gather = [&](int p) {
        const uint32_t v = __builtin_amdgcn_alignbit(cc[p].y, cc[p].x, csh);
        g0[p] = *(lds16c*)(TAB + ((v & vmask) | tabp[p]));
        g1[p] = *(lds16c*)(TAB + (((v >> 6) & vmask) | tabp[p]));
    };
    auto write_w = [&](int buf, int p) {
        *(lds32*)(WS[buf] + wst + 2048 * p) = g0[p] | (g1[p] << 16);
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][jj][r] = 0.f;

    // ---- prologue ----------------------------------------------------------------
    // State at the top of step t (buffer B = t % 2): X and W buffers B hold
    // X(t) and W(t); cc holds the codes of step t+1; code buffer B holds the
    // codes of step t+2; cw holds (or is loading) the codes of step t+3.
#pragma unroll
    for (int u = 0; u < XDMA; ++u) dma_x(0, 0, u);
    load_c(0);
    store_c(0);
    load_c(min(1, steps - 1));
    store_c(1);
    __syncthreads();  // tables, X(0), codes of steps 0 and 1
#pragma unroll
    for (int p = 0; p < PAIRS; ++p) read_codes(0, p);
#pragma unroll
    for (int p = 0; p < PAIRS; ++p) gather(p);
#pragma unroll
    for (int p = 0; p < PAIRS; ++p) write_w(0, p);
#pragma unroll
    for (int p = 0; p < PAIRS; ++p) read_codes(1, p);
    load_c(min(2, steps - 1));
    __syncthreads();  // W(0) written, code buffer 0 free
    store_c(0);
    load_c(min(3, steps - 1));
    __builtin_amdgcn_s_waitcnt(0x0F71);  // X(0) landed (the code load may stay in flight)
    __syncthreads();

    // ---- main loop -----------------------------------------------------------------
    // Step t first stores the codes of step t+3 (loaded one step earlier),
    // requests the codes of step t+4 and issues the direct loads of X(t+1)
    // (all complete by the step's closing barrier), then, with the MFMAs of
    // step t spread between them: the gathers of W(t+1) (codes read one step
    // earlier), the code reads of step t+2 and the writes of W(t+1).  Past the end the
    // indices are clamped; the extra work lands in buffers that are never read.
    auto step = [&](auto bufc, int t) {
        constexpr int B = decltype(bufc)::value;
        const int tn = min(t + 1, steps - 1);
        bf16x8 a[2][2], bb[2][2];
        auto frag = [&](int q) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
                a[q & 1][i] = __builtin_bit_cast(bf16x8, *(lds128c*)(XS[B] + aq[q] + 4096 * i));
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
                bb[q & 1][jj] = __builtin_bit_cast(bf16x8, *(lds128c*)(WS[B] + bq[q] + 4096 * jj));
        };
        auto mma = [&](int q, int i, int jj) {
            acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[q & 1][i], bb[q & 1][jj], acc[i][jj], 0, 0, 0);
        };
#define FQM_SLOT __builtin_amdgcn_sched_barrier(0)
        store_c(B ^ 1);  // its buffer held the codes of step t+1, read in step t-1
        load_c(min(t + 4, steps - 1));
        FQM_SLOT;
        dma_x(B ^ 1, tn, 0);
        dma_x(B ^ 1, tn, 1);
        frag(0);
        frag(1);
        dma_x(B ^ 1, tn, 2);
        dma_x(B ^ 1, tn, 3);
        FQM_SLOT;
        mma(0, 0, 0); gather(0); gather(1); FQM_SLOT;
        mma(0, 0, 1); gather(2); gather(3); FQM_SLOT;
        mma(0, 1, 0); gather(4); gather(5); FQM_SLOT;
        mma(0, 1, 1); gather(6); gather(7); FQM_SLOT;
        frag(2); FQM_SLOT;
        mma(1, 0, 0); read_codes(B, 0); read_codes(B, 1); FQM_SLOT;
        mma(1, 0, 1); read_codes(B, 2); read_codes(B, 3); FQM_SLOT;
        mma(1, 1, 0); read_codes(B, 4); read_codes(B, 5); FQM_SLOT;
        mma(1, 1, 1); read_codes(B, 6); read_codes(B, 7); FQM_SLOT;
        frag(3); FQM_SLOT;
        mma(2, 0, 0); write_w(B ^ 1, 0); FQM_SLOT;
        mma(2, 0, 1); write_w(B ^ 1, 1); write_w(B ^ 1, 2); FQM_SLOT;
        mma(2, 1, 0); write_w(B ^ 1, 3); write_w(B ^ 1, 4); FQM_SLOT;
        mma(2, 1, 1); write_w(B ^ 1, 5); write_w(B ^ 1, 6); FQM_SLOT;
        mma(3, 0, 0); write_w(B ^ 1, 7); FQM_SLOT;
        mma(3, 0, 1); FQM_SLOT;
        mma(3, 1, 0); FQM_SLOT;
        mma(3, 1, 1); FQM_SLOT;
#undef FQM_SLOT
        // The direct loads of X(t+1) (and the code load before them) must
        // have landed before the barrier publishes them: vmcnt(0).
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
    };
    for (int t = 0; t < steps; t += 2) {
        step(Buf<0>{}, t);
        if (t + 1 < steps) step(Buf<1>{}, t + 1);
    }

    // D layout of a 32x32 block: lane l, item r -> row (r % 4) + 8 * (r / 4) + 4 * (l / 32), column l % 32.
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * 64 + 32 * i + (r & 3) + 8 * (r >> 2) + 4 * h;
                const int n = n0 + wn * 64 + 32 * jj + j;
                if (m < M && n < N) Y[(int64_t)m * N + n] = f32_to_bf16(acc[i][jj][r]);
            }
}

}  // namespace

hipError_t launch_lut6_gemm(const fqm_weights& w, const uint16_t* X, uint16_t* Y, int64_t M,
                            hipStream_t s) {
    if (w.cols % BK || w.rows > 0x7fffffff || M > 0x7fffffff || w.cols > 0x7fffffff)
        return hipErrorInvalidValue;
    const int mtiles = (int)((M + BM - 1) / BM);
    const int64_t ntiles = (w.rows + BN - 1) / BN;
    if (ntiles * mtiles > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(lut6_gemm_kernel, dim3((unsigned)(ntiles * mtiles)), dim3(64 * NWAVE), 0, s,
                       X, w.lut6.packed, w.lut6.ld, w.lut6.lut, Y, (int)M, (int)w.rows, (int)w.cols,
                       mtiles);
    return hipGetLastError();
}

}  // namespace fqm
