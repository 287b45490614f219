// Internal declarations shared by the library's HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fqm.h"

namespace fqm {

// ---- small device helpers -------------------------------------------------

// bf16 bits -> fp32 (exact: a bf16 is the top half of an fp32).
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}
// The two bf16 halves of a packed dword.
__device__ __forceinline__ float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// fp16 bits -> fp32 (exact).
__device__ __forceinline__ float fp16_to_f32(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// Sum over the 64 lanes of a wavefront; every lane receives the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Sum over the 64 lanes with DPP moves only (no LDS traffic); the total is
// exact in lane 63 only.  Steps: pairs and quads (quad_perm), 8 lanes
// (row_half_mirror), 16 lanes (row_mirror), then row 0 -> 1 and 2 -> 3
// (row_bcast:15 into rows 1 and 3) and rows 0-1 -> 2-3 (row_bcast:31 into
// rows 2 and 3).  Rows left out of a broadcast add zero.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_or_zero(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xF, false));
}
__device__ __forceinline__ float wave_sum_lane63(float v) {
    v += dpp_or_zero<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
    v += dpp_or_zero<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
    v += dpp_or_zero<0x141, 0xF>(v);  // row_half_mirror
    v += dpp_or_zero<0x140, 0xF>(v);  // row_mirror
    v += dpp_or_zero<0x142, 0xA>(v);  // row_bcast:15
    v += dpp_or_zero<0x143, 0xC>(v);  // row_bcast:31
    return v;
}

// The 16 six-bit codes of a 12-byte piece (three little-endian dwords):
// code j sits at bits [6j, 6j+6) of the 96-bit value.
__device__ __forceinline__ void codes16(uint32_t d0, uint32_t d1, uint32_t d2, uint32_t c[16]) {
#pragma unroll
    for (int j = 0; j < 5; ++j) c[j] = (d0 >> (6 * j)) & 63u;
    c[5] = __builtin_amdgcn_alignbit(d1, d0, 30) & 63u;
#pragma unroll
    for (int j = 6; j < 10; ++j) c[j] = (d1 >> (6 * j - 32)) & 63u;
    c[10] = __builtin_amdgcn_alignbit(d2, d1, 28) & 63u;
#pragma unroll
    for (int j = 11; j < 16; ++j) c[j] = (d2 >> (6 * j - 64)) & 63u;
}

// ---- launchers (host side, one per kernel family) ---------------------------

hipError_t launch_pack_bits(const uint8_t* vals, uint8_t* out, int64_t rows, int64_t cols,
                            int bits, int64_t ld, int32_t* d_err, hipStream_t s);
// Zeroes n elements of elem_bytes (2 or 4) at p, with a kernel (graph-safe).
hipError_t launch_zero_fill(void* p, int64_t n, int elem_bytes, hipStream_t s);
hipError_t launch_unpack6(const uint8_t* packed, uint8_t* codes, int64_t rows, int64_t cols,
                          int64_t ld, hipStream_t s);
hipError_t launch_dequant_lut6(const fqm_weights& w, uint16_t* W, hipStream_t s);
hipError_t launch_dequant_lut4(const fqm_weights& w, uint16_t* W, hipStream_t s);
hipError_t launch_lut4_gemv(const fqm_weights& w, const uint16_t* x, void* y, int y_f32, int batch,
                            float* ws, hipStream_t s);
// true when launch_lut4_gemv takes a tuned kernel for this shape and batch
// (the cell kernel at batch 1, the matrix-core kernel at 2..16)
bool lut4_gemv_fast_path(const fqm_weights& w, int batch);
// true when launch_lut4_gemv takes the one-row-per-wave kernels (batch 1 on
// 1-31 whole cells, batch 2 on 1-19, batch 3 on 1-12); no workspace
bool lut4_gemv_rows_path(const fqm_weights& w, int batch);
hipError_t launch_dequant_fabq(const fqm_weights& w, uint16_t* W, hipStream_t s);

hipError_t launch_lut6_gemv(const fqm_weights& w, const uint16_t* x, void* y, int y_f32,
                            int batch, float* ws, hipStream_t s);
// Batch 2..16 of either LUT format (6- or 4-bit codes) on the matrix cores
// (cols a multiple of 512); K may be split over workgroups, with fp32 partial
// sums in the caller's workspace.  Support and workspace depend on the shape
// and batch only.
bool lut_gemv_mfma_supported(const fqm_weights& w, int batch);
// true when launch_lut6_gemv takes a tuned kernel for this shape and batch
// (the cell kernel at batch 1, the matrix-core kernel at 2..16)
bool lut6_gemv_fast_path(const fqm_weights& w, int batch);
// true when launch_lut6_gemv takes the one-row-per-wave kernels (batch 1 on
// 1-31 whole 1024-column cells, batch 2 on 1-19, batch 3 on 1-12); they need
// no workspace
bool lut6_gemv_rows_path(const fqm_weights& w, int batch);
size_t lut_gemv_mfma_workspace(const fqm_weights& w, int batch);
hipError_t launch_lut_gemv_mfma(const fqm_weights& w, const uint16_t* x, void* y, int y_f32, int batch,
                                float* ws, hipStream_t s);
// Prefill GEMM of either LUT format (6- or 4-bit codes); the tile plan and
// its workspace depend on the shape, M and the device only.
size_t lut_gemm_workspace(const fqm_weights& w, int64_t M);
hipError_t launch_lut_gemm(const fqm_weights& w, const uint16_t* X, uint16_t* Y, int64_t M, void* ws,
                           size_t ws_bytes, hipStream_t s);
// FABQ: ws holds the vector-centroid terms G (fabq_workspace_bytes; other
// codebook modes need none and ws may be null).
size_t fabq_workspace_bytes(const fqm_weights& w, int batch);
hipError_t launch_fabq_gemv(const fqm_weights& w, const uint16_t* x, void* y, int y_f32,
                            int batch, float* ws, hipStream_t s);
// MDBF: workspace holds the bf16 hi/lo dense operands of both passes.
size_t mdbf_workspace_bytes(const fqm_weights& w, int batch);
hipError_t launch_mdbf_gemv(const fqm_weights& w, const uint16_t* x, void* y, int y_f32, int batch, void* ws,
                            hipStream_t s);

}  // namespace fqm
