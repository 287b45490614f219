// C ABI: argument checks on the host, then stream-ordered launches.
// Nothing here allocates, synchronises or keeps state between calls.
#include <string.h>

#include <cstdint>

#include "fqm_internal.h"

using namespace fqm;

namespace {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool ld_ok(int64_t ld, int64_t need) { return ld >= need && (ld & 15) == 0; }
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline fqm_status hip_status(hipError_t e) { return e == hipSuccess ? FQM_OK : FQM_E_HIP; }

// Checks a descriptor; on success returns FQM_OK.  Only host memory is read.
fqm_status check_weights(const fqm_weights* w) {
    if (!w) return FQM_E_NULL;
    if (w->rows < 0 || w->cols < 0) return FQM_E_SHAPE;
    switch (w->format) {
        case FQM_LUT6: {
            const fqm_lut6& f = w->lut6;
            if (w->cols % 64) return FQM_E_SHAPE;
            if (w->rows == 0) return FQM_OK;
            if (!f.packed || !f.lut) return FQM_E_NULL;
            if (!aligned16(f.packed) || !aligned16(f.lut)) return FQM_E_ALIGN;
            if (f.ld < w->cols * 3 / 4) return FQM_E_SHAPE;
            if (f.ld & 15) return FQM_E_ALIGN;
            return FQM_OK;
        }
        case FQM_LUT4: {
            const fqm_lut4& f = w->lut4;
            if (w->cols % 64) return FQM_E_SHAPE;
            if (w->rows == 0) return FQM_OK;
            if (!f.packed || !f.lut) return FQM_E_NULL;
            if (!aligned16(f.packed) || !aligned16(f.lut)) return FQM_E_ALIGN;
            if (f.ld < w->cols / 2) return FQM_E_SHAPE;
            if (f.ld & 15) return FQM_E_ALIGN;
            return FQM_OK;
        }
        case FQM_FABQ: {
            const fqm_fabq& f = w->fabq;
            const int bs = f.blocksize;
            if (bs != 64 && bs != 128 && bs != 256 && bs != 512) return FQM_E_FORMAT;
            if (w->cols % bs) return FQM_E_SHAPE;
            if (f.n_hi < 0 || f.n_hi > w->rows) return FQM_E_SHAPE;
            if (w->rows == 0) return FQM_OK;
            const int64_t n_lo = w->rows - f.n_hi;
            const int64_t nb = w->cols / bs;
            if (!f.row_of) return FQM_E_NULL;
            if (!aligned16(f.row_of)) return FQM_E_ALIGN;
            if (f.n_hi > 0) {
                if (!f.q4 || !f.s_hi) return FQM_E_NULL;
                if (!aligned16(f.q4) || !aligned16(f.s_hi)) return FQM_E_ALIGN;
                if (f.ld_q4 < w->cols / 2) return FQM_E_SHAPE;
                if (f.ld_q4 & 15) return FQM_E_ALIGN;
            }
            if (n_lo > 0) {
                if (!f.signs || !f.s_blk || !f.idx || !f.codebook) return FQM_E_NULL;
                if (!aligned16(f.signs) || !aligned16(f.s_blk) || !aligned16(f.idx) ||
                    !aligned16(f.codebook))
                    return FQM_E_ALIGN;
                if (f.ld_signs < w->cols / 8 || f.ld_idx < (nb + 1) / 2) return FQM_E_SHAPE;
                if ((f.ld_signs & 15) || (f.ld_idx & 15)) return FQM_E_ALIGN;
            }
            return FQM_OK;
        }
        case FQM_MDBF: {
            const fqm_mdbf& f = w->mdbf;
            if (f.l < 1 || f.l > 16 || (f.P != 1 && f.P != 2)) return FQM_E_FORMAT;
            if (f.r < 1 || f.r > 65536) return FQM_E_FORMAT;
            if (w->cols % 32) return FQM_E_SHAPE;
            if (w->rows == 0) return FQM_OK;
            for (int p = 0; p < f.P; ++p) {
                const fqm_mdbf_path& q = f.path[p];
                if (!q.S_A || !q.S_B || !q.A_amp || !q.B_amp || !q.Q_U || !q.Q_V) return FQM_E_NULL;
                if (!aligned16(q.S_A) || !aligned16(q.S_B) || !aligned16(q.A_amp) ||
                    !aligned16(q.B_amp) || !aligned16(q.Q_U) || !aligned16(q.Q_V))
                    return FQM_E_ALIGN;
                if (q.ld_A < (f.r + 7) / 8 || q.ld_B < w->cols / 8) return FQM_E_SHAPE;
                if ((q.ld_A & 15) || (q.ld_B & 15)) return FQM_E_ALIGN;
            }
            return FQM_OK;
        }
        default:
            return FQM_E_FORMAT;
    }
}

}  // namespace

extern "C" {

int32_t fqm_version(void) { return FQM_VERSION; }

const char* fqm_status_str(int32_t status) {
    switch (status) {
        case FQM_OK: return "ok";
        case FQM_E_NULL: return "a required pointer is NULL";
        case FQM_E_ALIGN: return "a base pointer or row stride is not 16-byte aligned";
        case FQM_E_SHAPE: return "sizes negative, out of range or inconsistent";
        case FQM_E_FORMAT: return "unknown format or format parameter out of range";
        case FQM_E_WORKSPACE: return "workspace missing or too small";
        case FQM_E_UNSUPPORTED: return "combination not supported";
        case FQM_E_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

fqm_status fqm_pack_bits(const uint8_t* vals, uint8_t* out, int64_t rows, int64_t cols,
                         int32_t bits, int64_t ld, int32_t* d_err, void* stream) {
    if (bits != 1 && bits != 4 && bits != 6) return FQM_E_FORMAT;
    if (rows < 0 || cols < 0) return FQM_E_SHAPE;
    if (rows == 0) return FQM_OK;
    if (!out || (cols > 0 && !vals)) return FQM_E_NULL;
    if (!aligned16(out)) return FQM_E_ALIGN;
    if (ld < (cols * bits + 7) / 8) return FQM_E_SHAPE;
    if (ld & 15) return FQM_E_ALIGN;
    return hip_status(launch_pack_bits(vals, out, rows, cols, bits, ld, d_err, as_stream(stream)));
}

fqm_status fqm_pack(const uint8_t* codes, uint8_t* packed, int64_t rows, int64_t cols, int64_t ld,
                    int32_t* d_err, void* stream) {
    return fqm_pack_bits(codes, packed, rows, cols, 6, ld, d_err, stream);
}

fqm_status fqm_unpack(const uint8_t* packed, uint8_t* codes, int64_t rows, int64_t cols, int64_t ld,
                      void* stream) {
    if (rows < 0 || cols < 0 || (cols & 3)) return FQM_E_SHAPE;
    if (rows == 0 || cols == 0) return FQM_OK;
    if (!packed || !codes) return FQM_E_NULL;
    if (!aligned16(packed)) return FQM_E_ALIGN;
    if (ld < cols * 3 / 4) return FQM_E_SHAPE;
    if (ld & 15) return FQM_E_ALIGN;
    return hip_status(launch_unpack6(packed, codes, rows, cols, ld, as_stream(stream)));
}

fqm_status fqm_dequant(const fqm_weights* w, uint16_t* W, void* stream) {
    const fqm_status st = check_weights(w);
    if (st != FQM_OK) return st;
    if (w->format == FQM_MDBF) return FQM_E_UNSUPPORTED;
    if (w->rows == 0 || w->cols == 0) return FQM_OK;
    if (!W) return FQM_E_NULL;
    if (!aligned16(W)) return FQM_E_ALIGN;
    if (w->format == FQM_LUT6) return hip_status(launch_dequant_lut6(*w, W, as_stream(stream)));
    if (w->format == FQM_LUT4) return hip_status(launch_dequant_lut4(*w, W, as_stream(stream)));
    return hip_status(launch_dequant_fabq(*w, W, as_stream(stream)));
}

size_t fqm_workspace_size(const fqm_weights* w, int32_t batch) {
    if (check_weights(w) != FQM_OK || batch < 1 || batch > 16) return 0;
    if (w->format == FQM_LUT6 || w->format == FQM_LUT4) return fqm::lut_gemv_mfma_workspace(*w, batch);
    if (w->format != FQM_MDBF) return 0;
    return fqm::mdbf_workspace_bytes(*w, batch);
}

fqm_status fqm_gemv(const fqm_weights* w, const uint16_t* x, void* y, int32_t y_dtype,
                    int32_t batch, void* workspace, size_t ws_bytes, void* stream) {
    const fqm_status st = check_weights(w);
    if (st != FQM_OK) return st;
    if (batch < 1 || batch > 16) return FQM_E_SHAPE;
    if (y_dtype != FQM_BF16 && y_dtype != FQM_F32) return FQM_E_FORMAT;
    if (w->rows == 0) return FQM_OK;
    if (!y || (w->cols > 0 && !x)) return FQM_E_NULL;
    if (!aligned16(y) || (x && !aligned16(x))) return FQM_E_ALIGN;
    const int y_f32 = y_dtype == FQM_F32;
    hipStream_t s = as_stream(stream);
    switch (w->format) {
        case FQM_LUT6: {
            const size_t need = fqm_workspace_size(w, batch);
            if (need && (!workspace || ws_bytes < need)) return FQM_E_WORKSPACE;
            if (need && !aligned16(workspace)) return FQM_E_ALIGN;
            return hip_status(
                launch_lut6_gemv(*w, x, y, y_f32, batch, static_cast<float*>(workspace), s));
        }
        case FQM_LUT4: {
            const size_t need = fqm_workspace_size(w, batch);
            if (need && (!workspace || ws_bytes < need)) return FQM_E_WORKSPACE;
            if (need && !aligned16(workspace)) return FQM_E_ALIGN;
            return hip_status(
                launch_lut4_gemv(*w, x, y, y_f32, batch, static_cast<float*>(workspace), s));
        }
        case FQM_FABQ: return hip_status(launch_fabq_gemv(*w, x, y, y_f32, batch, s));
        case FQM_MDBF: {
            const size_t need = fqm_workspace_size(w, batch);
            if (!workspace || ws_bytes < need) return FQM_E_WORKSPACE;
            if (!aligned16(workspace)) return FQM_E_ALIGN;
            return hip_status(
                launch_mdbf_gemv(*w, x, y, y_f32, batch, workspace, s));
        }
    }
    return FQM_E_FORMAT;
}

// Up to 16 rows of X go to the GEMV kernels when they have a tuned kernel
// for the shape: the prefill tiles are 256 rows tall, so below that the
// matrix cores would mostly multiply padding (measured on the 17408 x 5120
// layer: 14-31 us through the GEMV path against 68-71 us as a GEMM).
static bool gemm_as_gemv(const fqm_weights& w, int64_t M) {
    if (M < 1 || M > 16) return false;
    return w.format == FQM_LUT4 ? fqm::lut4_gemv_fast_path(w, (int)M) : fqm::lut6_gemv_fast_path(w, (int)M);
}

static bool lut_format(const fqm_weights& w) { return w.format == FQM_LUT6 || w.format == FQM_LUT4; }

size_t fqm_gemm_workspace_size(const fqm_weights* w, int64_t M) {
    if (check_weights(w) != FQM_OK || !lut_format(*w) || M <= 0 || w->rows == 0) return 0;
    if (w->cols % 64 || M * w->cols * 2 > INT32_MAX) return 0;
    if (gemm_as_gemv(*w, M)) return fqm::lut_gemv_mfma_workspace(*w, (int)M);
    return fqm::lut_gemm_workspace(*w, M);
}

fqm_status fqm_gemm(const fqm_weights* w, const uint16_t* X, uint16_t* Y, int64_t M, void* workspace,
                    size_t ws_bytes, void* stream) {
    const fqm_status st = check_weights(w);
    if (st != FQM_OK) return st;
    if (!lut_format(*w)) return FQM_E_UNSUPPORTED;
    if (M < 0) return FQM_E_SHAPE;
    if (M > (int64_t)65535 * 128) return FQM_E_SHAPE;
    if (M == 0 || w->rows == 0) return FQM_OK;
    if (w->cols % 64 || M * w->cols * 2 > INT32_MAX) return FQM_E_SHAPE;
    if (!Y || !X) return FQM_E_NULL;
    if (!aligned16(Y) || !aligned16(X)) return FQM_E_ALIGN;
    const size_t need = fqm_gemm_workspace_size(w, M);
    if (need && (!workspace || ws_bytes < need)) return FQM_E_WORKSPACE;
    if (need && !aligned16(workspace)) return FQM_E_ALIGN;
    float* gws = static_cast<float*>(workspace);
    if (gemm_as_gemv(*w, M))  // Y[M][rows] bf16 is the GEMV's y[batch][rows]
        return hip_status(w->format == FQM_LUT4 ? launch_lut4_gemv(*w, X, Y, 0, (int)M, gws, as_stream(stream))
                                                : launch_lut6_gemv(*w, X, Y, 0, (int)M, gws, as_stream(stream)));
    return hip_status(launch_lut_gemm(*w, X, Y, M, workspace, ws_bytes, as_stream(stream)));
}

}  // extern "C"
