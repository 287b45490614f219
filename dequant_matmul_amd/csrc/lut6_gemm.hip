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
// Decode: one row's 64 codes of a K step sit on the 64 lanes of a wave (lane
// l takes code l, bits [6l, 6l+6) of the row's 48-byte segment), so every
// gather of an instruction reads the same 128-byte table (distinct banks or a
// shared dword: no bank conflicts), and each lane stores its bf16 value at
// its column.  The BN row tables stay in LDS for the whole K loop.
//
// Pipeline: LDS tiles are double-buffered; while the waves run the MFMAs of
// step t they decode step t+1 (codes already in registers) into the other
// buffer, store the prefetched X block of step t+1, and issue the global
// loads of step t+2.  One barrier per step.
//
// Tile order: workgroups are dispatched round-robin over the 8 XCDs, and
// workgroup b computes M tile b % 8 (for M = 8 * BM), so each XCD keeps one
// X panel (BM x K bf16, 2.6 MB at K = 5120) in its own L2 while the W panels
// stream through; other M take the same mapping modulo the M tile count.
#include "fqm_internal.h"

namespace fqm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) uint8_t lds8;
typedef __attribute__((address_space(3))) const uint16_t lds16c;
typedef __attribute__((address_space(3))) uint16_t lds16;
typedef __attribute__((address_space(3))) u32x4 lds128;
typedef __attribute__((address_space(3))) const u32x4 lds128c;

constexpr int BM = 256, BN = 128, BK = 64;
constexpr int NWAVE = 8;                  // 4 (M) x 2 (N) waves, 64 x 64 outputs each
constexpr int LDT = BK + 8;               // LDS row stride of the X and W tiles, bf16 elements
constexpr int XT_BYTES = BM * LDT * 2;    // one X tile
constexpr int WT_BYTES = BN * LDT * 2;    // one W tile
constexpr int TAB_BYTES = BN * 128;       // BN row tables
constexpr int LDS_BYTES = 2 * XT_BYTES + 2 * WT_BYTES + TAB_BYTES;
constexpr int ROWS_PER_WAVE = BN / NWAVE; // W rows each wave decodes per step
constexpr int XPT = BM * BK * 2 / 16 / (64 * NWAVE);  // 16-byte X pieces per thread per step

__global__ __launch_bounds__(64 * NWAVE) void lut6_gemm_kernel(const uint16_t* __restrict__ X,
                                                               const uint8_t* __restrict__ packed,
                                                               int64_t ld,
                                                               const uint16_t* __restrict__ lut,
                                                               uint16_t* __restrict__ Y, int M,
                                                               int N, int K, int mtiles) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds8*)smem;
    const uint32_t xt0 = lds0, wt0 = lds0 + 2 * XT_BYTES;
    const uint32_t tab0 = wt0 + 2 * WT_BYTES;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int b = blockIdx.x;
    const int mt = b % mtiles, nt = b / mtiles;
    const int m0 = mt * BM, n0 = nt * BN;
    const int wm = wave >> 1, wn = wave & 1;  // this wave's 64 x 64 output block

    // ---- row tables (resident) -------------------------------------------------
    for (int i = tid; i < BN * 8; i += 64 * NWAVE) {
        const int r = i >> 3, part = i & 7;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (n0 + r < N) v = *reinterpret_cast<const u32x4*>(lut + (int64_t)(n0 + r) * 64 + part * 8);
        *(lds128*)(uintptr_t)(tab0 + (uint32_t)i * 16u) = v;
    }

    // ---- per-lane decode constants --------------------------------------------
    // Lane l owns code l of a 64-code segment, bits [6l, 6l+6).  A funnel shift
    // by p = 6l - 1 of the dword pair holding bit p puts the code at bits 1..6
    // (its table byte offset); lane 0 shifts its first dword left by one
    // (pair (d0, d0), shift 31).  Lanes 59..63 end inside dword 11 and read no
    // dword past it.
    const int p6 = 6 * lane - 1;
    const uint32_t clo = lane == 0 ? 0u : (uint32_t)(p6 >> 5);
    const uint32_t chi = lane == 0 ? 0u : (clo < 11u ? clo + 1u : 11u);
    const uint32_t csh = (uint32_t)(p6 & 31);
    uint32_t vmask = 0x7Eu;
    asm volatile("" : "+v"(vmask));  // in a VGPR: (v & mask) | base is one v_and_or_b32

    // this wave decodes rows wave + NWAVE*i of the tile
    const uint8_t* crow[ROWS_PER_WAVE];
#pragma unroll
    for (int i = 0; i < ROWS_PER_WAVE; ++i) {
        const int r = min(n0 + wave + NWAVE * i, N - 1);
        crow[i] = packed + (int64_t)r * ld;
    }
    // X pieces of this thread: row xr, 16-byte piece xc (8 per 64-element row)
    const uint16_t* xsrc[XPT];
    uint32_t xdst[XPT];
#pragma unroll
    for (int u = 0; u < XPT; ++u) {
        const int p = tid + u * 64 * NWAVE;
        const int xr = p >> 3, xc = p & 7;
        xsrc[u] = X + (int64_t)min(m0 + xr, M - 1) * K + 8 * xc;
        xdst[u] = (uint32_t)(xr * LDT + 8 * xc) * 2u;
    }

    const int steps = K / BK;
    uint32_t cw[ROWS_PER_WAVE][2];  // codes of the next step to decode
    u32x4 xw[XPT];            // X pieces of the next step to store
    auto load_step = [&](int t) {
        const int kb = t * BK;
#pragma unroll
        for (int i = 0; i < ROWS_PER_WAVE; ++i) {
            const uint32_t* seg = reinterpret_cast<const uint32_t*>(crow[i] + (kb * 3) / 4);
            cw[i][0] = seg[clo];
            cw[i][1] = seg[chi];
        }
#pragma unroll
        for (int u = 0; u < XPT; ++u) xw[u] = *reinterpret_cast<const u32x4*>(xsrc[u] + kb);
    };
    auto store_step = [&](int buf) {
        const uint32_t xt = xt0 + (uint32_t)buf * XT_BYTES, wt = wt0 + (uint32_t)buf * WT_BYTES;
#pragma unroll
        for (int u = 0; u < XPT; ++u) *(lds128*)(uintptr_t)(xt + xdst[u]) = xw[u];
        // all gathers first, then the stores: the table reads of the rows overlap
        uint32_t w16[ROWS_PER_WAVE];
#pragma unroll
        for (int i = 0; i < ROWS_PER_WAVE; ++i) {
            const uint32_t tb = tab0 + 128u * (uint32_t)(wave + NWAVE * i);  // multiple of 128
            const uint32_t v = __builtin_amdgcn_alignbit(cw[i][1], cw[i][0], csh);
            w16[i] = *(lds16c*)(uintptr_t)((v & vmask) | tb);
        }
        const uint32_t wl = wt + (uint32_t)(wave * LDT + lane) * 2u;
#pragma unroll
        for (int i = 0; i < ROWS_PER_WAVE; ++i)
            *(lds16*)(uintptr_t)(wl + (uint32_t)(NWAVE * i * LDT) * 2u) = (uint16_t)w16[i];
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    load_step(0);
    __syncthreads();  // tables in LDS
    store_step(0);
    load_step(min(1, steps - 1));
    __syncthreads();

    // MFMA operand addresses: A rows wm*64 + 32*i + (lane % 32), B rows wn*64 + 32*j + (lane % 32),
    // 8 consecutive k at 8*(lane / 32) within each 16-wide k slice.
    const uint32_t aoff = (uint32_t)((wm * 64 + (lane & 31)) * LDT + 8 * (lane >> 5)) * 2u;
    const uint32_t boff = (uint32_t)((wn * 64 + (lane & 31)) * LDT + 8 * (lane >> 5)) * 2u;
    for (int t = 0; t < steps; ++t) {
        const int buf = t & 1;
        const uint32_t xt = xt0 + (uint32_t)buf * XT_BYTES + aoff;
        const uint32_t wt = wt0 + (uint32_t)buf * WT_BYTES + boff;
        // Operand fragments are double-buffered across the four 16-wide k slices.
        bf16x8 a[2][2], bb[2][2];
        auto frag = [&](int kk, int f) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
                a[f][i] = __builtin_bit_cast(bf16x8, *(lds128c*)(uintptr_t)(xt + (uint32_t)(32 * i * LDT + kk) * 2u));
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bb[f][j] = __builtin_bit_cast(bf16x8, *(lds128c*)(uintptr_t)(wt + (uint32_t)(32 * j * LDT + kk) * 2u));
        };
        frag(0, 0);
#pragma unroll
        for (int q = 0; q < BK / 16; ++q) {
            if (q + 1 < BK / 16) frag(16 * (q + 1), (q + 1) & 1);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[q & 1][i], bb[q & 1][j], acc[i][j], 0, 0, 0);
        }
        // Decode step t+1 into the other buffer and request step t+2, in the
        // same basic block as the MFMAs so the two interleave.  Past the end
        // the step index is clamped: the extra decode lands in a buffer that is
        // never read and the extra loads re-read the last step.
        store_step(buf ^ 1);
        load_step(min(t + 2, steps - 1));
        // Interleave: each MFMA followed by a share of the decode's VALU, LDS
        // and global-load instructions (scheduling hint only).
#pragma unroll
        for (int g = 0; g < 16; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS read
            __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS write
            __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);  // global load
        }
        __syncthreads();
    }

    // D layout of a 32x32 block: lane l, item r -> row (r % 4) + 8 * (r / 4) + 4 * (l / 32), column l % 32.
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * 64 + 32 * i + (r & 3) + 8 * (r >> 2) + 4 * (lane >> 5);
                const int n = n0 + wn * 64 + 32 * j + (lane & 31);
                if (m < M && n < N) Y[(int64_t)m * N + n] = f32_to_bf16(acc[i][j][r]);
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
    // more than 64 KB of dynamic LDS per workgroup
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&lut6_gemm_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lut6_gemm_kernel, dim3((unsigned)(ntiles * mtiles)), dim3(64 * NWAVE), LDS_BYTES, s,
                       X, w.lut6.packed, w.lut6.ld, w.lut6.lut, Y, (int)M, (int)w.rows, (int)w.cols,
                       mtiles);
    return hipGetLastError();
}

}  // namespace fqm
