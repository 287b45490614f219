// C ABI: argument checks on the host, then stream-ordered launches.
// Nothing here allocates, synchronises or keeps state between calls.
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <cstdint>
#include <mutex>

#include "fqm_internal.h"

using namespace fqm;

namespace {

// ---- the static scratch of fqm_gemv_static ----------------------------------
// One array per GPU the library runs on, held until the process ends.  Host
// code never uses the array's name as an address (on the host it is only a
// stand-in): each device's address is looked up once, with that device
// current, and kept in scratch_addr.
__device__ __align__(256) uint8_t scratch[FQM_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_addr[kMaxDevices];
std::mutex scratch_mu;

// The current device's copy of `scratch`.
hipError_t scratch_for_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(scratch_mu);
        p = scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

// ---- debug checks --------------------------------------------------------------
// -1 until the first call reads FQM_DEBUG; then 0 (off) or 1 (on).
std::atomic<int> debug_state{-1};

bool debug_on() {
    int v = debug_state.load(std::memory_order_relaxed);
    if (v < 0) {
        const char* e = getenv("FQM_DEBUG");
        const int from_env = (e && *e && strcmp(e, "0") != 0) ? 1 : 0;
        int expected = -1;
        debug_state.compare_exchange_strong(expected, from_env);
        v = debug_state.load(std::memory_order_relaxed);
    }
    return v > 0;
}

// [p, p + bytes) lies inside one device allocation (nothing to check when
// bytes <= 0).
bool in_allocation(const void* p, int64_t bytes) {
    if (bytes <= 0) return true;
    if (!p) return false;
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, const_cast<void*>(p)) != hipSuccess) {
        (void)hipGetLastError();  // not device memory: clear the sticky error
        return false;
    }
    const uintptr_t b = reinterpret_cast<uintptr_t>(base), q = reinterpret_cast<uintptr_t>(p);
    return q >= b && (uint64_t)(q - b) + (uint64_t)bytes <= (uint64_t)size;
}

// Bytes that `rows` rows `ld` apart span when the last one needs `last` bytes.
inline int64_t span(int64_t rows, int64_t ld, int64_t last) { return rows > 0 ? (rows - 1) * ld + last : 0; }

// Every buffer of a descriptor (already checked by check_weights) at the
// extent the kernels may touch.
fqm_status check_weight_buffers(const fqm_weights& w) {
    const int64_t R = w.rows, C = w.cols;
    if (R == 0) return FQM_OK;
    bool ok = true;
    switch (w.format) {
        case FQM_LUT6:
            ok = in_allocation(w.lut6.packed, span(R, w.lut6.ld, C * 3 / 4)) && in_allocation(w.lut6.lut, R * 128);
            break;
        case FQM_LUT4:
            ok = in_allocation(w.lut4.packed, span(R, w.lut4.ld, C / 2)) && in_allocation(w.lut4.lut, R * 32);
            break;
        case FQM_FABQ: {
            const fqm_fabq& f = w.fabq;
            const int64_t n_lo = R - f.n_hi, nb = C / f.blocksize;
            const int hb = f.hi_bits ? f.hi_bits : 4;
            ok = in_allocation(f.row_of, R * 4);
            if (f.n_hi > 0)
                ok = ok && in_allocation(f.q4, span(f.n_hi, f.ld_q4, C * hb / 8)) && in_allocation(f.s_hi, f.n_hi * 2);
            if (n_lo > 0) {
                ok = ok && in_allocation(f.signs, span(n_lo, f.ld_signs, C / 8)) &&
                     in_allocation(f.s_blk, n_lo * nb * 2) && in_allocation(f.idx, span(n_lo, f.ld_idx, (nb + 1) / 2));
                if (f.cb_mode == FQM_CB_SCALAR16) ok = ok && in_allocation(f.codebook, 16 * 2);
                if (f.cb_mode == FQM_CB_TIERED) ok = ok && in_allocation(f.codebook, 4 * 64 * 2);
                if (f.cb_mode == FQM_CB_VECTOR) ok = ok && in_allocation(f.vcodebook, 4 * 64 * 128 * 4);
                if (f.cb_mode != FQM_CB_SCALAR16) ok = ok && in_allocation(f.tier, n_lo);
            }
            break;
        }
        case FQM_MDBF: {
            const fqm_mdbf& f = w.mdbf;
            for (int p = 0; p < f.P && ok; ++p) {
                const fqm_mdbf_path& q = f.path[p];
                ok = in_allocation(q.S_A, span(R, q.ld_A, ((f.r + 7) / 8 + 15) & ~15)) &&
                     in_allocation(q.S_B, span(f.r, q.ld_B, (C / 8 + 15) & ~15)) &&
                     in_allocation(q.A_amp, R * f.l * 2) && in_allocation(q.B_amp, C * f.l * 2) &&
                     in_allocation(q.Q_U, (int64_t)f.r * f.l * 2) && in_allocation(q.Q_V, (int64_t)f.r * f.l * 2);
            }
            break;
        }
        default:
            break;
    }
    return ok ? FQM_OK : FQM_E_BOUNDS;
}

// After a call's launches: with the checks on (and the stream not being
// captured), wait for the stream and turn a kernel failure into FQM_E_HIP.
fqm_status debug_finish(fqm_status st, hipStream_t s) {
    if (st != FQM_OK || !debug_on()) return st;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) return FQM_E_HIP;
    if (cs != hipStreamCaptureStatusNone) return st;
    if (hipStreamSynchronize(s) != hipSuccess || hipGetLastError() != hipSuccess) return FQM_E_HIP;
    return st;
}

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
            if (bs != 16 && bs != 32 && bs != 64 && bs != 128 && bs != 256 && bs != 512) return FQM_E_FORMAT;
            if (f.hi_bits != 0 && f.hi_bits != 4 && f.hi_bits != 8) return FQM_E_FORMAT;
            if (f.cb_mode < FQM_CB_SCALAR16 || f.cb_mode > FQM_CB_VECTOR) return FQM_E_FORMAT;
            if (f.cb_mode != FQM_CB_SCALAR16 && (f.cb_base < 0 || f.cb_base > 48 || (f.cb_base & 15)))
                return FQM_E_FORMAT;
            if (w->cols % bs) return FQM_E_SHAPE;
            if (f.n_hi < 0 || f.n_hi > w->rows) return FQM_E_SHAPE;
            if (w->rows == 0) return FQM_OK;
            const int64_t n_lo = w->rows - f.n_hi;
            const int64_t nb = w->cols / bs;
            const int hb = f.hi_bits ? f.hi_bits : 4;
            if (!f.row_of) return FQM_E_NULL;
            if (!aligned16(f.row_of)) return FQM_E_ALIGN;
            if (f.n_hi > 0) {
                if (!f.q4 || !f.s_hi) return FQM_E_NULL;
                if (!aligned16(f.q4) || !aligned16(f.s_hi)) return FQM_E_ALIGN;
                if (f.ld_q4 < w->cols * hb / 8) return FQM_E_SHAPE;
                if (f.ld_q4 & 15) return FQM_E_ALIGN;
            }
            if (n_lo > 0) {
                if (!f.signs || !f.s_blk || !f.idx) return FQM_E_NULL;
                if (f.cb_mode == FQM_CB_VECTOR ? !f.vcodebook : !f.codebook) return FQM_E_NULL;
                if (f.cb_mode != FQM_CB_SCALAR16 && !f.tier) return FQM_E_NULL;
                if (!aligned16(f.signs) || !aligned16(f.s_blk) || !aligned16(f.idx) ||
                    (f.codebook && !aligned16(f.codebook)) || (f.tier && !aligned16(f.tier)) ||
                    (f.vcodebook && !aligned16(f.vcodebook)))
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

int32_t fqm_set_debug(int32_t on) {
    const int prev = debug_on() ? 1 : 0;
    debug_state.store(on ? 1 : 0, std::memory_order_relaxed);
    return prev;
}

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
        case FQM_E_SCRATCH: return "needs more scratch than fqm_gemv_static's static maximum";
        case FQM_E_BOUNDS: return "debug checks: a buffer is not inside one device allocation of its size";
        default: return "unknown status";
    }
}

fqm_status fqm_pack_bits(const uint8_t* vals, uint8_t* out, int64_t rows, int64_t cols,
                         int32_t bits, int64_t ld, int32_t* d_err, void* stream) {
    if (bits != 1 && bits != 4 && bits != 6 && bits != 8) return FQM_E_FORMAT;
    if (rows < 0 || cols < 0) return FQM_E_SHAPE;
    if (rows == 0) return FQM_OK;
    if (!out || (cols > 0 && !vals)) return FQM_E_NULL;
    if (!aligned16(out)) return FQM_E_ALIGN;
    if (ld < (cols * bits + 7) / 8) return FQM_E_SHAPE;
    if (ld & 15) return FQM_E_ALIGN;
    if (debug_on() && !(in_allocation(vals, rows * cols) && in_allocation(out, span(rows, ld, (cols * bits + 7) / 8)) &&
                        (!d_err || in_allocation(d_err, 4))))
        return FQM_E_BOUNDS;
    return debug_finish(hip_status(launch_pack_bits(vals, out, rows, cols, bits, ld, d_err, as_stream(stream))),
                        as_stream(stream));
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
    if (debug_on() && !(in_allocation(packed, span(rows, ld, cols * 3 / 4)) && in_allocation(codes, rows * cols)))
        return FQM_E_BOUNDS;
    return debug_finish(hip_status(launch_unpack6(packed, codes, rows, cols, ld, as_stream(stream))), as_stream(stream));
}

fqm_status fqm_dequant(const fqm_weights* w, uint16_t* W, void* stream) {
    const fqm_status st = check_weights(w);
    if (st != FQM_OK) return st;
    if (w->format == FQM_MDBF) return FQM_E_UNSUPPORTED;
    if (w->rows == 0 || w->cols == 0) return FQM_OK;
    if (!W) return FQM_E_NULL;
    if (!aligned16(W)) return FQM_E_ALIGN;
    if (debug_on() && (check_weight_buffers(*w) != FQM_OK || !in_allocation(W, w->rows * w->cols * 2)))
        return FQM_E_BOUNDS;
    hipStream_t s = as_stream(stream);
    if (w->format == FQM_LUT6) return debug_finish(hip_status(launch_dequant_lut6(*w, W, s)), s);
    if (w->format == FQM_LUT4) return debug_finish(hip_status(launch_dequant_lut4(*w, W, s)), s);
    return debug_finish(hip_status(launch_dequant_fabq(*w, W, s)), s);
}

size_t fqm_workspace_size(const fqm_weights* w, int32_t batch) {
    if (check_weights(w) != FQM_OK || batch < 1 || batch > 16) return 0;
    if (w->format == FQM_LUT6 || w->format == FQM_LUT4) return fqm::lut_gemv_mfma_workspace(*w, batch);
    if (w->format == FQM_FABQ) return fqm::fabq_workspace_bytes(*w, batch);
    if (w->format != FQM_MDBF) return 0;
    return fqm::mdbf_workspace_bytes(*w, batch);
}

}  // extern "C"

namespace {

// The launches of fqm_gemv once its arguments have passed the checks.
fqm_status gemv_launch(const fqm_weights* w, const uint16_t* x, void* y, int y_f32, int32_t batch,
                       void* workspace, size_t ws_bytes, hipStream_t s) {
    if (w->cols == 0)  // an empty sum: y = 0 whatever the format (x is not read)
        return hip_status(launch_zero_fill(y, (int64_t)batch * w->rows, y_f32 ? 4 : 2, s));
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
        case FQM_FABQ: {
            const size_t need = fqm_workspace_size(w, batch);
            if (need && (!workspace || ws_bytes < need)) return FQM_E_WORKSPACE;
            if (need && !aligned16(workspace)) return FQM_E_ALIGN;
            return hip_status(launch_fabq_gemv(*w, x, y, y_f32, batch, static_cast<float*>(workspace), s));
        }
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

// fqm_gemv; static_ws: the workspace is fqm_gemv_static's scratch array (a
// device symbol, not an allocation the debug checks can look up).
fqm_status gemv_impl(const fqm_weights* w, const uint16_t* x, void* y, int32_t y_dtype, int32_t batch,
                     void* workspace, size_t ws_bytes, void* stream, bool static_ws) {
    const fqm_status st = check_weights(w);
    if (st != FQM_OK) return st;
    if (batch < 1 || batch > 16) return FQM_E_SHAPE;
    if (y_dtype != FQM_BF16 && y_dtype != FQM_F32) return FQM_E_FORMAT;
    if (w->rows == 0) return FQM_OK;
    if (!y || (w->cols > 0 && !x)) return FQM_E_NULL;
    if (!aligned16(y) || (x && !aligned16(x))) return FQM_E_ALIGN;
    const int y_f32 = y_dtype == FQM_F32;
    hipStream_t s = as_stream(stream);
    if (!debug_on()) return gemv_launch(w, x, y, y_f32, batch, workspace, ws_bytes, s);
    const size_t need = w->cols > 0 ? fqm_workspace_size(w, batch) : 0;
    if (check_weight_buffers(*w) != FQM_OK || !in_allocation(x, (int64_t)batch * w->cols * 2) ||
        !in_allocation(y, (int64_t)batch * w->rows * (y_f32 ? 4 : 2)) ||
        (!static_ws && workspace && !in_allocation(workspace, (int64_t)need)))
        return FQM_E_BOUNDS;
    return debug_finish(gemv_launch(w, x, y, y_f32, batch, workspace, ws_bytes, s), s);
}

}  // namespace

extern "C" {

fqm_status fqm_gemv(const fqm_weights* w, const uint16_t* x, void* y, int32_t y_dtype,
                    int32_t batch, void* workspace, size_t ws_bytes, void* stream) {
    return gemv_impl(w, x, y, y_dtype, batch, workspace, ws_bytes, stream, false);
}

fqm_status fqm_gemv_static(const fqm_weights* w, const uint16_t* x, void* y, int32_t y_dtype,
                           int32_t batch, void* stream) {
    const fqm_status st = check_weights(w);
    if (st != FQM_OK) return st;
    if (batch < 1 || batch > 16) return FQM_E_SHAPE;
    const size_t need = fqm_workspace_size(w, batch);
    if (need > FQM_STATIC_SCRATCH_BYTES) return FQM_E_SCRATCH;
    void* ws = nullptr;
    if (need && scratch_for_current_device(&ws) != hipSuccess) return FQM_E_HIP;
    return gemv_impl(w, x, y, y_dtype, batch, ws, need, stream, true);
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
    if (w->cols == 0) return 0;  // Y is zero-filled, no K parts
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
    if (!Y || (w->cols > 0 && !X)) return FQM_E_NULL;
    if (!aligned16(Y) || (X && !aligned16(X))) return FQM_E_ALIGN;
    const size_t need = fqm_gemm_workspace_size(w, M);
    if (need && (!workspace || ws_bytes < need)) return FQM_E_WORKSPACE;
    if (need && !aligned16(workspace)) return FQM_E_ALIGN;
    hipStream_t s = as_stream(stream);
    if (debug_on() && (check_weight_buffers(*w) != FQM_OK || !in_allocation(X, M * w->cols * 2) ||
                       !in_allocation(Y, M * w->rows * 2) || (need && !in_allocation(workspace, (int64_t)need))))
        return FQM_E_BOUNDS;
    fqm_status r;
    if (w->cols == 0)  // an empty sum: Y = 0 (the tile kernels assume at least one K step)
        r = hip_status(launch_zero_fill(Y, M * w->rows, 2, s));
    else if (gemm_as_gemv(*w, M))  // Y[M][rows] bf16 is the GEMV's y[batch][rows]
        r = hip_status(w->format == FQM_LUT4
                           ? launch_lut4_gemv(*w, X, Y, 0, (int)M, static_cast<float*>(workspace), s)
                           : launch_lut6_gemv(*w, X, Y, 0, (int)M, static_cast<float*>(workspace), s));
    else
        r = hip_status(launch_lut_gemm(*w, X, Y, M, workspace, ws_bytes, s));
    return debug_finish(r, s);
}

}  // extern "C"
