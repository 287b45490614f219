// Per-row LUT GEMM (prefill): Y[m][n] = sum_k X[m][k] * lut[n][code[n][k]],
// 6-bit codes (64-entry tables) or 4-bit codes (16-entry tables).
//
// Source: "Qwen3.8-27B - BenQ 6-bit", "What BenQ stores": decode is the
// row-wise gather of codes into the row's table, fused into the matrix
// product so the decoded matrix is never written out ("Why equal-width
// shells" places 8 tiers in 4 bits, read the same way).  The text below
// gives the 6-bit sizes; 4-bit codes take 16 bytes per lane per step and
// 2 KB table planes.  Each workgroup owns a
// BM x BN tile of Y and contracts it on the bf16 matrix cores
// (v_mfma_f32_32x32x16_bf16, fp32 accumulate); the decoded weights are exact
// (the table entries are bf16).
//
// Decode straight into matrix operands.  The workgroup's 8 waves share the
// 256 X rows of the tile; each wave owns 32 rows of W (columns of Y).  For
// each 16-wide k slice, lane (j, g) of the wave
// (j = lane % 32, g = lane / 32) needs 8 consecutive weights of W row j as its
// B operand: it takes the 8 codes from registers (loaded from global memory
// three steps ahead, 24 bytes per lane per step), gathers the 8 bf16 values from
// row j's table in LDS and packs them into the operand.  The same B operand
// feeds eight MFMAs (the tile's eight 32-row blocks of X), so each gathered
// weight serves 256 rows of X.  W never passes through LDS as a tile, and no
// code bytes are staged in LDS.
//
// k order.  Inside a K step of 64, lane half g takes the step's codes
// [32 g, 32 g + 32) (bytes [24 g, 24 g + 24) of the row's 48-byte chunk) and
// slice q of the step uses k = 32 g + 8 q + e (e = 0..7).  The X operand reads
// use the same k order (16-byte chunk 4 g + q of the X row), so each product
// pairs the right X and W values; only the order of the fp32 sums differs
// from the plain k order.
//
// Table layout (bank-sliced).  Entry e of tile row r (0..255) sits at
//   8192 (r / 64) + 128 e + 4 (r % 32) + 2 ((r / 32) % 2),
// so the 32 lanes of a half-wave (the 32 rows of one 32-row group, any
// codes) hit 32 distinct banks: gathers never conflict.  A code c becomes the
// gather address (c << 7) | base_lane, i.e. one shift and one v_and_or_b32.
//
// X: three 256 x 64 bf16 tile buffers (128-byte rows, 16-byte chunks
// XOR-swizzled by (row / 2) % 8 so the operand reads of 16 rows hit 16
// distinct bank groups), filled by direct global -> LDS loads one step ahead.
// One workgroup barrier per step publishes the next X tile; with three
// buffers it needs no wait for the wave's LDS reads, so the operand reads
// and gathers stay one and two slices ahead of the MFMAs across it.  LDS:
// 96 KB of X and 32 KB of tables, one workgroup per compute unit.
//
// Tile order: workgroups are dispatched round-robin over the 8 XCDs, and
// workgroup b computes M tile b % mtiles, so with M = 8 * BM each XCD keeps
// one X panel (BM x K bf16, 2.6 MB at K = 5120) in its own L2 while the W
// panels stream through.
#include <algorithm>
#include <type_traits>

#include "fqm_internal.h"

namespace fqm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef u32x4 u32x4_a8 __attribute__((aligned(8)));
typedef u32x2 u32x2_a8 __attribute__((aligned(8)));
typedef __attribute__((address_space(3))) uint8_t lds8;
typedef __attribute__((address_space(3))) uint16_t lds16;
typedef __attribute__((address_space(3))) const uint16_t lds16c;
typedef __attribute__((address_space(3))) const u32x4 lds128c;
typedef __attribute__((address_space(3))) void lvoid;

// Tile heights: BM rows of X per workgroup (256 for prefill; 64 for small M,
// where a 256-row tile would mostly multiply padding).
constexpr int BM_BIG = 256, BM_SMALL = 64;
constexpr int BN = 256, BK = 64;
constexpr int NWAVE = 8;                       // 8 waves along N, BM x 32 outputs each
constexpr int NXB = 3;                         // X tile buffers (and code slots): the loop is unrolled by 3
static_assert(BN == 32 * NWAVE, "tile constants");
template <int BM>
struct TileShape {
    static constexpr int MB = BM / 32;                    // 32-row blocks of X per wave
    static constexpr int XT_BYTES = BM * BK * 2;          // one X tile, 128-byte rows
    static constexpr int XDMA = XT_BYTES / 1024 / NWAVE;  // 1 KB direct-to-LDS X loads per wave per step
    static_assert(XDMA >= 1 && BM % 64 == 0, "every wave loads whole kilobytes of the X tile");
};

// Per code width: table entries, a table plane (64 rows' tables, bank-sliced),
// the code bytes a lane reads per K step (32 codes) and a row's bytes per step.
template <int BITS>
struct GemmFmt {
    static constexpr int ENTRIES = 1 << BITS;
    static constexpr int PLANE = 128 * ENTRIES;  // 8 KB (6-bit), 2 KB (4-bit)
    static constexpr int TAB_BYTES = (BN / 64) * PLANE;
    static constexpr int ND = BITS;              // dwords of code per lane per step
    static constexpr int STEP_BYTES = 8 * BITS;  // a row's 64 codes
    static constexpr int CODE_LOADS = ND == 6 ? 2 : 1;  // global loads per lane per step (16 + 8 or 16 bytes)
};

template <int BUF>
using Buf = std::integral_constant<int, BUF>;

// Table offset of code C (0..31) of a lane's code run d[0..ND): the code's
// bits moved to bits 7.. and OR-ed into the lane's row offset.
template <int BITS, int C, int ND>
__device__ __forceinline__ uint32_t code_addr(const uint32_t (&d)[ND], uint32_t mask, uint32_t base) {
    constexpr int bit = BITS * C, w = bit >> 5, o = bit & 31;
    uint32_t v;
    if constexpr (o + BITS <= 32) {
        if constexpr (o >= 7) v = d[w] >> (o - 7);
        else v = d[w] << (7 - o);
    } else {
        v = __builtin_amdgcn_alignbit(d[w + 1], d[w], o - 7);
    }
    return (v & mask) | base;
}

// The 8 gather addresses of slice Q (codes 8 Q .. 8 Q + 7).
template <int BITS, int Q, int ND>
__device__ __forceinline__ void slice_addrs(const uint32_t (&d)[ND], uint32_t mask, uint32_t base, uint32_t (&ad)[8]) {
    ad[0] = code_addr<BITS, 8 * Q + 0>(d, mask, base);
    ad[1] = code_addr<BITS, 8 * Q + 1>(d, mask, base);
    ad[2] = code_addr<BITS, 8 * Q + 2>(d, mask, base);
    ad[3] = code_addr<BITS, 8 * Q + 3>(d, mask, base);
    ad[4] = code_addr<BITS, 8 * Q + 4>(d, mask, base);
    ad[5] = code_addr<BITS, 8 * Q + 5>(d, mask, base);
    ad[6] = code_addr<BITS, 8 * Q + 6>(d, mask, base);
    ad[7] = code_addr<BITS, 8 * Q + 7>(d, mask, base);
}

template <int Q>
using Slice = std::integral_constant<int, Q>;

// Workgroup barrier after all but this wave's last N vector-memory loads have
// completed (loads complete in issue order).  LDS reads may stay in flight:
// the buffers they read are not rewritten before the next barrier.  The wait
// is the waitcnt builtin, so the compiler's own wait bookkeeping sees it; the
// barrier is the bare instruction between two compiler memory barriers (a
// workgroup fence would also wait for the loads left in flight).
template <int N>
__device__ __forceinline__ void barrier_after_loads() {
    static_assert(N >= 0 && N < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0F70 | N);  // vmcnt(N) expcnt(7) lgkmcnt(15)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Workgroup b computes tile (M tile tt % mtiles, N tile nt0 + tt / mtiles),
// tt = b / ksplit, over K steps [t0, t1) of its split b % ksplit.  PARTIAL:
// the fp32 tile (all BM x BN values) goes to part[b]; otherwise the bf16
// outputs inside M x N go to Y.
template <int BITS, bool PARTIAL, int BM>
__device__ __forceinline__ void gemm_tile(const uint16_t* __restrict__ X,
                                                               const uint8_t* __restrict__ packed,
                                                               int64_t ld,
                                                               const uint16_t* __restrict__ lut,
                                                               uint16_t* __restrict__ Y, float* __restrict__ part,
                                                               int M, int N, int K, int mtiles, int nt0,
                                                               int ksplit) {
    constexpr int MB = TileShape<BM>::MB, XT_BYTES = TileShape<BM>::XT_BYTES, XDMA = TileShape<BM>::XDMA;
    using F = GemmFmt<BITS>;
    constexpr int TAB_BYTES = F::TAB_BYTES, PLANE = F::PLANE, ND = F::ND, EPT = F::ENTRIES / 8;
    // Separate LDS objects: the X tiles are written by direct global -> LDS
    // loads, and distinct objects let the compiler see that the table
    // gathers do not wait for those loads.
    __shared__ __attribute__((aligned(8192))) uint8_t s_tab[TAB_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t s_x0[XT_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t s_x1[XT_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t s_x2[XT_BYTES];
    lds8* const XS[NXB] = {(lds8*)s_x0, (lds8*)s_x1, (lds8*)s_x2};
    lds8* const TAB = (lds8*)s_tab;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int b = blockIdx.x;
    const int tt = b / ksplit, ks = b - tt * ksplit;
    const int mt = tt % mtiles, nt = nt0 + tt / mtiles;
    const int m0 = mt * BM, n0 = nt * BN;
    const int wn = wave;  // W rows 32 wn .. 32 wn + 31 of the tile
    const int g = lane >> 5, j = lane & 31;

    // ---- row tables, bank-sliced (resident for the whole K loop) ------------------
    for (int i = tid; i < BN * 8; i += 64 * NWAVE) {
        const int r = i >> 3, part = i & 7;  // entries EPT part .. + EPT - 1 of tile row r
        uint32_t v[4] = {0u, 0u, 0u, 0u};
        if (n0 + r < N) {
            const uint16_t* src = lut + (int64_t)(n0 + r) * F::ENTRIES + part * EPT;
            if constexpr (EPT == 8) {
                const u32x4 q = *reinterpret_cast<const u32x4*>(src);
                v[0] = q[0]; v[1] = q[1]; v[2] = q[2]; v[3] = q[3];
            } else {
                v[0] = *reinterpret_cast<const uint32_t*>(src);
            }
        }
        lds8* dst = TAB + PLANE * (r >> 6) + 4 * (r & 31) + 2 * ((r >> 5) & 1) + 128 * EPT * part;
#pragma unroll
        for (int e = 0; e < EPT; ++e) *(lds16*)(dst + 128 * e) = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
    }
    // this lane's row 32 wn + j: plane wn / 2, half wn % 2 (bits below the code's and above them only)
    const uint32_t tbase = (uint32_t)PLANE * (wn >> 1) + 4u * j + 2u * (wn & 1);
    uint32_t cmask = (uint32_t)(F::ENTRIES - 1) << 7;
    asm volatile("" : "+v"(cmask));  // in a VGPR: (v & mask) | base is one v_and_or_b32

    // ---- X: direct global -> LDS, 1 KB (8 rows) per wave instruction -----------
    // Buffer loads with an LDS destination from the tile's X panel (the
    // compiler tracks these exactly; the flat-address form makes it wait for
    // every LDS read while one is in flight).  Load u of wave w fills rows
    // 8 (8u + w) .. + 7; lane l lands at byte 16 l of that kilobyte (row +
    // l / 8, stored chunk l % 8) and fetches the logical chunk that the
    // swizzle puts there, (l % 8) ^ ((row / 2) % 8).  Rows past M repeat row
    // M - 1 (never stored).
    // X as one buffer (the host keeps M * K * 2 below 2^31); the tile's first
    // row goes into the scalar offset.
    const __amdgpu_buffer_rsrc_t xrsrc = __builtin_amdgcn_make_buffer_rsrc((void*)X, (short)0, 0x7fffffff, 0x00020000);
    const uint32_t xtile = (uint32_t)m0 * (uint32_t)K * 2u;
    uint32_t xoff[XDMA];
#pragma unroll
    for (int u = 0; u < XDMA; ++u) {
        const int row = 8 * (8 * u + wave) + (lane >> 3);
        const int chunk = (lane & 7) ^ ((row >> 1) & 7);
        xoff[u] = (uint32_t)(min(row, M - 1 - m0) * K + 8 * chunk) * 2u;
    }
    auto dma_x = [&](int buf, int t) {
#pragma unroll
        for (int u = 0; u < XDMA; ++u)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xrsrc, (lvoid*)(XS[buf] + 1024 * (8 * u + wave)), 16, xoff[u],
                                                     xtile + (uint32_t)t * (BK * 2), 0, 0);
    };

    // ---- codes: 24 bytes of row 32 wn + j per lane per step ------------------------
    const uint8_t* csrc = packed + (int64_t)min(n0 + 32 * wn + j, N - 1) * ld + 4 * ND * g;
    uint32_t cw[NXB][ND];
    auto load_codes = [&](int slot, int t) {
        const uint8_t* p = csrc + F::STEP_BYTES * t;
        const u32x4 lo = *reinterpret_cast<const u32x4_a8*>(p);
        cw[slot][0] = lo[0]; cw[slot][1] = lo[1]; cw[slot][2] = lo[2]; cw[slot][3] = lo[3];
        if constexpr (ND == 6) {
            const u32x2 hi = *reinterpret_cast<const u32x2_a8*>(p + 16);
            cw[slot][4] = hi[0]; cw[slot][5] = hi[1];
        }
    };

    // ---- X operand offsets ------------------------------------------------------
    // A of block i, slice q: X tile row 32 i + j, logical chunk 4 g + q.
    int aoff[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) aoff[q] = 128 * j + 16 * ((4 * g + q) ^ ((j >> 1) & 7));

    f32x16 acc[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

    const int ksteps = K / BK;
    const int t0 = (int)((int64_t)ks * ksteps / ksplit), t1 = (int)((int64_t)(ks + 1) * ksteps / ksplit);
    const int steps = t1 - t0;  // >= 1
    __builtin_assume(steps > 0);

    // ---- operands: A one slice ahead, table gathers two slices ahead ----------------
    // a[i] and bop hold the operands of the slice whose MFMAs issue next, wv
    // the gathered table entries of the slice after it.  A slice first packs
    // wv into the next B operand; while its MFMAs run, the wave reads the next
    // slice's A operands (a[i] right after the MFMA that consumes it) and
    // gathers the entries of the slice after that.  The order is pinned with
    // scheduling groups, one MFMA at a time.
    bf16x8 a[MB];
    bf16x8 bop;
    uint32_t wv[8];
    auto pack_b = [&]() {
        u32x4 bw;
#pragma unroll
        for (int e = 0; e < 4; ++e) bw[e] = __builtin_amdgcn_perm(wv[2 * e + 1], wv[2 * e], 0x05040100u);
        return __builtin_bit_cast(bf16x8, bw);
    };
    auto read_a = [&](int buf, auto qc) {
        constexpr int q = decltype(qc)::value;
#pragma unroll
        for (int i = 0; i < MB; ++i) a[i] = __builtin_bit_cast(bf16x8, *(lds128c*)(XS[buf] + aoff[q] + 4096 * i));
    };
    auto gather = [&](auto qc, int slot) {
        constexpr int q = decltype(qc)::value;
        uint32_t ad[8];
        slice_addrs<BITS, q>(cw[slot], cmask, tbase, ad);
#pragma unroll
        for (int e = 0; e < 8; ++e) wv[e] = *(lds16c*)(TAB + ad[e]);
    };
    // Gathers ride with the first half of the slice's MFMAs (GPM per MFMA), so
    // that the perms at the start of the next slice wait only for LDS reads
    // issued half a slice earlier.
    constexpr int HALF = MB / 2, GPM = 8 / HALF;
    static_assert(GPM * HALF == 8, "8 gathers per slice");
    // The MFMAs of the current slice; A of slice AQ from X buffer AB, gathers of
    // slice GQ from code slot GS.
    auto slice = [&](auto aqc, int ab, auto gqc, int gs) {
        constexpr int aq = decltype(aqc)::value, gq = decltype(gqc)::value;
        __builtin_amdgcn_sched_barrier(0);
        const bf16x8 bnext = pack_b();
        uint32_t ad[8];
        slice_addrs<BITS, gq>(cw[gs], cmask, tbase, ad);
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bop, acc[i], 0, 0, 0);
            a[i] = __builtin_bit_cast(bf16x8, *(lds128c*)(XS[ab] + aoff[aq] + 4096 * i));
            if (i < HALF) {
#pragma unroll
                for (int e = GPM * i; e < GPM * (i + 1); ++e) wv[e] = *(lds16c*)(TAB + ad[e]);
            }
        }
        bop = bnext;
        // perms and the first addresses; per MFMA: the MFMA, its A read (and in
        // the first half its gathers), then the next gathers' addresses
        __builtin_amdgcn_sched_group_barrier(0x0002, 4 + 2 * GPM, 0);
#pragma unroll
        for (int i = 0; i < HALF; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x0100, 1 + GPM, 0);
            __builtin_amdgcn_sched_group_barrier(0x0002, 2 * GPM, 0);
        }
#pragma unroll
        for (int i = HALF; i < MB; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- prologue: X(t0) and the codes of steps t0, t0 + 1 in place; then, as
    // after every barrier, the next X tile and codes requested; operands of
    // slice 0 read and entries of slices 0 and 1 gathered
    dma_x(0, t0);
    load_codes(0, t0);
    load_codes(1, t0 + min(1, steps - 1));
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();                     // tables and X(t0) visible
    dma_x(1, t0 + min(1, steps - 1));
    __builtin_amdgcn_sched_barrier(0);  // the X loads go out before the code loads
    load_codes(2, t0 + min(2, steps - 1));
    gather(Slice<0>{}, 0);
    read_a(0, Slice<0>{});
    bop = pack_b();
    gather(Slice<1>{}, 0);

    // ---- main loop -----------------------------------------------------------------
    // Step t0 + t uses X buffer and code slot P = t % 3.  Its slices 0..2 issue
    // their MFMAs while reading A of slices 1..3 and gathering for slices 2, 3
    // and slice 0 of step t+1; then the wave waits until X(t+1) (requested one
    // step earlier) has landed, the workgroup barrier publishes it, and slice 3
    // reads A of slice 0 of step t+1 from it and gathers for that step's slice
    // 1.  After the barrier every wave has consumed X(t-1) (its MFMAs read those
    // operands), so that buffer takes X(t+2); the codes of step t+3 go into
    // slot P (its last gathers were issued in slice 1).  Memory loads complete
    // in issue order: after the barrier a step issues X(t+2) and then
    // codes(t+3), so at the next barrier only this step's code loads may still
    // be in flight.  Past the end the indices are clamped; the extra reads land
    // in buffers and registers that are never used.
    auto step = [&](auto pc, int t) {
        constexpr int P = decltype(pc)::value, P1 = (P + 1) % NXB, P2 = (P + 2) % NXB;
        slice(Slice<1>{}, P, Slice<2>{}, P);
        slice(Slice<2>{}, P, Slice<3>{}, P);
        slice(Slice<3>{}, P, Slice<0>{}, P1);
        barrier_after_loads<F::CODE_LOADS>();
        dma_x(P2, t0 + min(t + 2, steps - 1));
        __builtin_amdgcn_sched_barrier(0);  // the X loads go out before the code loads
        load_codes(P, t0 + min(t + 3, steps - 1));
        slice(Slice<0>{}, P1, Slice<1>{}, P1);
    };
    int t = 0;
    for (; t + 2 < steps; t += 3) {
        step(Buf<0>{}, t);
        step(Buf<1>{}, t + 1);
        step(Buf<2>{}, t + 2);
    }
    if (t < steps) step(Buf<0>{}, t);
    if (t + 1 < steps) step(Buf<1>{}, t + 1);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no X load may still be writing this workgroup's LDS

    // D layout of a 32x32 block: lane l, item r -> row (r % 4) + 8 * (r / 4) + 4 * (l / 32), column l % 32.
    if constexpr (PARTIAL) {
        float* pt = part + (size_t)b * (BM * BN) + 32 * wn + j;
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) pt[(32 * i + (r & 3) + 8 * (r >> 2) + 4 * g) * BN] = acc[i][r];
    } else {
        const int n = n0 + 32 * wn + j;
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + 32 * i + (r & 3) + 8 * (r >> 2) + 4 * g;
                if (m < M && n < N) Y[(int64_t)m * N + n] = f32_to_bf16(acc[i][r]);
            }
    }
}

#define FQM_GEMM_ARGS                                                                                    \
    const uint16_t *__restrict__ X, const uint8_t *__restrict__ packed, int64_t ld,                      \
        const uint16_t *__restrict__ lut, uint16_t *__restrict__ Y, float *__restrict__ part, int M, int N, \
        int K, int mtiles, int nt0, int ksplit
template <bool PARTIAL>
__global__ __launch_bounds__(64 * NWAVE) void lut6_gemm_kernel(FQM_GEMM_ARGS) {
    gemm_tile<6, PARTIAL, BM_BIG>(X, packed, ld, lut, Y, part, M, N, K, mtiles, nt0, ksplit);
}
// 64-row tiles: 56 KB of LDS and at most 128 VGPRs (four waves per SIMD), so
// two workgroups share a CU
template <bool PARTIAL>
__global__ __launch_bounds__(64 * NWAVE) __attribute__((amdgpu_waves_per_eu(4))) void lut6_gemm_small_kernel(
    FQM_GEMM_ARGS) {
    gemm_tile<6, PARTIAL, BM_SMALL>(X, packed, ld, lut, Y, part, M, N, K, mtiles, nt0, ksplit);
}
template <bool PARTIAL>
__global__ __launch_bounds__(64 * NWAVE) void lut4_gemm_kernel(FQM_GEMM_ARGS) {
    gemm_tile<4, PARTIAL, BM_BIG>(X, packed, ld, lut, Y, part, M, N, K, mtiles, nt0, ksplit);
}
template <bool PARTIAL>
__global__ __launch_bounds__(64 * NWAVE) __attribute__((amdgpu_waves_per_eu(4))) void lut4_gemm_small_kernel(
    FQM_GEMM_ARGS) {
    gemm_tile<4, PARTIAL, BM_SMALL>(X, packed, ld, lut, Y, part, M, N, K, mtiles, nt0, ksplit);
}
#undef FQM_GEMM_ARGS

// Y for the split tiles: the ksplit fp32 partial tiles of tile tt summed in
// split order (a fixed order), rounded once to bf16.  Thread: 4 consecutive
// columns of one tile row.
template <int BM>
__global__ __launch_bounds__(256) void lut6_gemm_reduce(const float* __restrict__ part, uint16_t* __restrict__ Y,
                                                        int M, int N, int mtiles, int nt0, int ksplit,
                                                        int64_t groups) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (tile, row, column group)
    if (e >= groups) return;
    constexpr int G = BN / 4;
    const int64_t tt = e / (BM * G);
    const int rem = (int)(e - tt * (BM * G));
    const int ml = rem / G, nl = 4 * (rem - ml * G);
    const int mt = (int)(tt % mtiles), nt = nt0 + (int)(tt / mtiles);
    const int m = mt * BM + ml, n = nt * BN + nl;
    if (m >= M) return;
    const float* p = part + (size_t)tt * ksplit * (BM * BN) + ml * BN + nl;
    float4 sum = *reinterpret_cast<const float4*>(p);
    for (int k = 1; k < ksplit; ++k) {
        const float4 v = *reinterpret_cast<const float4*>(p + (size_t)k * (BM * BN));
        sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
    }
    uint16_t* y = Y + (int64_t)m * N + n;
    if (n + 0 < N) y[0] = f32_to_bf16(sum.x);
    if (n + 1 < N) y[1] = f32_to_bf16(sum.y);
    if (n + 2 < N) y[2] = f32_to_bf16(sum.z);
    if (n + 3 < N) y[3] = f32_to_bf16(sum.w);
}

// Tile plan.  Whole rounds of tiles (one per resident workgroup: one per
// compute unit for 256-row tiles, two for 64-row tiles)
// run as one launch.  The N tiles left for a last, partial round are split
// along K into ksplit parts (of at least MIN_SPLIT_STEPS steps; at most
// MAX_SPLIT_SMALL parts for 64-row tiles, whose fp32 partials would
// otherwise outweigh the weights) and their fp32 partial tiles are reduced
// afterwards.  ksplit minimises the last round's length in K steps,
// ceil(tail * k / slots) * ceil(steps / k): for 32 tail tiles of 80 steps on
// 256 slots that is 8 parts (one round of 10 steps); for 160 tiles of 272
// steps (the 5120 x 17408 layer at 2048 rows) 3 parts, two rounds of 91
// steps instead of one round of 272 on 160 of the 256 compute units.  Ties
// take the fewer parts, and the partials are capped at MAX_SPLIT_BYTES.
constexpr int MIN_SPLIT_STEPS = 8;
constexpr int MAX_SPLIT_SMALL = 4;
constexpr int64_t MAX_SPLIT_BYTES = (int64_t)256 << 20;
constexpr int64_t SMALL_M_MAX = 64;  // M up to this takes 64-row tiles (measured: faster up to 64 rows, slower at 128 and 256)

struct GemmPlan {
    int bm = BM_BIG;      // tile height
    int mtiles = 0, ntiles = 0;
    int nt_main = 0;      // N tiles [0, nt_main) in the direct launch
    int ksplit = 1;       // K parts of each remaining tile
    int64_t tail = 0;     // remaining tiles ((ntiles - nt_main) * mtiles)
    size_t ws_bytes = 0;  // tail * ksplit fp32 partial tiles
};

GemmPlan gemm_plan(int64_t rows, int64_t cols, int64_t M, int cus) {
    GemmPlan p;
    const bool small = M <= SMALL_M_MAX;
    p.bm = small ? BM_SMALL : BM_BIG;
    p.mtiles = (int)((M + p.bm - 1) / p.bm);
    p.ntiles = (int)((rows + BN - 1) / BN);
    p.nt_main = p.ntiles;
    const int64_t tiles = (int64_t)p.mtiles * p.ntiles, slots = (int64_t)std::max(cus, 1) * (small ? 2 : 1);
    if (tiles % slots == 0) return p;
    const int nt_main = (int)((tiles / slots) * slots / p.mtiles);
    const int64_t tail = (int64_t)(p.ntiles - nt_main) * p.mtiles;
    const int64_t steps = cols / BK;
    int64_t kmax = steps / MIN_SPLIT_STEPS;
    if (small) kmax = std::min<int64_t>(kmax, MAX_SPLIT_SMALL);
    int64_t ksplit = 1, best = ((tail + slots - 1) / slots) * steps;
    for (int64_t k = 2; k <= kmax; ++k) {
        if (tail * k * p.bm * BN * (int64_t)sizeof(float) > MAX_SPLIT_BYTES) break;
        const int64_t len = ((tail * k + slots - 1) / slots) * ((steps + k - 1) / k);
        if (len < best) best = len, ksplit = k;
    }
    if (ksplit < 2) return p;
    p.nt_main = nt_main;
    p.ksplit = (int)ksplit;
    p.tail = tail;
    p.ws_bytes = (size_t)tail * ksplit * p.bm * BN * sizeof(float);
    return p;
}

template <int BITS, int BM>
hipError_t launch_plan(const fqm_weights& w, const uint16_t* X, uint16_t* Y, int64_t M, void* ws,
                       const GemmPlan& p, hipStream_t s) {
    hipError_t e;
    const int64_t main_tiles = (int64_t)p.nt_main * p.mtiles;
    auto kernel = [](bool partial) {
        if constexpr (BITS == 4 && BM == BM_SMALL)
            return partial ? lut4_gemm_small_kernel<true> : lut4_gemm_small_kernel<false>;
        else if constexpr (BITS == 4)
            return partial ? lut4_gemm_kernel<true> : lut4_gemm_kernel<false>;
        else if constexpr (BM == BM_SMALL)
            return partial ? lut6_gemm_small_kernel<true> : lut6_gemm_small_kernel<false>;
        else
            return partial ? lut6_gemm_kernel<true> : lut6_gemm_kernel<false>;
    };
    const uint8_t* packed = BITS == 4 ? w.lut4.packed : w.lut6.packed;
    const int64_t ld = BITS == 4 ? w.lut4.ld : w.lut6.ld;
    const uint16_t* lut = BITS == 4 ? w.lut4.lut : w.lut6.lut;
    if (main_tiles > 0) {
        hipLaunchKernelGGL(kernel(false), dim3((unsigned)main_tiles), dim3(64 * NWAVE), 0, s, X,
                           packed, ld, lut, Y, nullptr, (int)M, (int)w.rows, (int)w.cols,
                           p.mtiles, 0, 1);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (p.tail > 0) {
        float* part = static_cast<float*>(ws);
        hipLaunchKernelGGL(kernel(true), dim3((unsigned)(p.tail * p.ksplit)), dim3(64 * NWAVE), 0, s,
                           X, packed, ld, lut, Y, part, (int)M, (int)w.rows, (int)w.cols,
                           p.mtiles, p.nt_main, p.ksplit);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const int64_t groups = p.tail * BM * (BN / 4);
        hipLaunchKernelGGL(lut6_gemm_reduce<BM>, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, s, part, Y,
                           (int)M, (int)w.rows, p.mtiles, p.nt_main, p.ksplit, groups);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t device_cus(int* cus) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
    return e;
}

}  // namespace

size_t lut_gemm_workspace(const fqm_weights& w, int64_t M) {
    int cus = 0;
    if (M <= 0 || device_cus(&cus) != hipSuccess) return 0;
    return gemm_plan(w.rows, w.cols, M, cus).ws_bytes;
}

hipError_t launch_lut_gemm(const fqm_weights& w, const uint16_t* X, uint16_t* Y, int64_t M, void* ws,
                           size_t ws_bytes, hipStream_t s) {
    if ((w.format != FQM_LUT6 && w.format != FQM_LUT4) || w.cols % BK || w.rows > 0x7fffffff || M > 0x7fffffff || w.cols > 0x7fffffff ||
        M * w.cols * 2 > 0x7fffffff)
        return hipErrorInvalidValue;
    int cus = 0;
    hipError_t e = device_cus(&cus);
    if (e != hipSuccess) return e;
    const GemmPlan p = gemm_plan(w.rows, w.cols, M, cus);
    if ((int64_t)p.ntiles * p.mtiles > 0x7fffffff) return hipErrorInvalidValue;
    if (p.ws_bytes > ws_bytes || (p.ws_bytes && !ws)) return hipErrorInvalidValue;
    if (w.format == FQM_LUT4)
        return p.bm == BM_SMALL ? launch_plan<4, BM_SMALL>(w, X, Y, M, ws, p, s)
                                : launch_plan<4, BM_BIG>(w, X, Y, M, ws, p, s);
    return p.bm == BM_SMALL ? launch_plan<6, BM_SMALL>(w, X, Y, M, ws, p, s)
                            : launch_plan<6, BM_BIG>(w, X, Y, M, ws, p, s);
}

}  // namespace fqm
