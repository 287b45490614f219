// Packing of bit fields, and the test-only unpack / dequant kernels.
//
// Bit-field rule (all formats): field k of a row occupies bits [b*k, b*k+b)
// of the row's little-endian bit stream.  6-bit fields hold the per-row LUT
// codes of "Qwen3.8-27B - BenQ 6-bit" ("What BenQ stores"); 1-bit fields the
// signs of the FABQ-RC binary rows and the MDBF sign matrices; 4-bit fields
// int4 weights and codebook indices.
#include "fqm_internal.h"

namespace fqm {
namespace {

// One thread per output dword: gathers the (at most 32/b + 2) fields whose
// bits overlap the dword.  Bytes past the row's last field come out zero.
__global__ __launch_bounds__(256) void pack_bits_kernel(const uint8_t* __restrict__ vals,
                                                        uint32_t* __restrict__ out,
                                                        int64_t rows, int64_t cols, int bits,
                                                        int64_t ld_words,
                                                        int32_t* __restrict__ d_err) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= rows * ld_words) return;
    const int64_t r = t / ld_words;
    const int64_t d = t - r * ld_words;
    const int64_t bit0 = 32 * d;
    const uint32_t mask = (1u << bits) - 1u;
    int64_t k0 = bit0 / bits;
    int64_t k1 = (bit0 + 31) / bits;
    if (k1 > cols - 1) k1 = cols - 1;
    uint64_t acc = 0;
    bool bad = false;
    const uint8_t* rv = vals + r * cols;
    for (int64_t k = k0; k <= k1; ++k) {
        uint32_t v = rv[k];
        bad |= v > mask;
        v &= mask;
        const int64_t p = k * bits - bit0;  // may be negative for the first field
        acc |= p >= 0 ? ((uint64_t)v << p) : ((uint64_t)v >> (-p));
    }
    out[r * ld_words + d] = (uint32_t)acc;
    if (bad && d_err) atomicOr(d_err, 1);
}

__global__ __launch_bounds__(256) void unpack6_kernel(const uint8_t* __restrict__ packed,
                                                      uint8_t* __restrict__ codes, int64_t rows,
                                                      int64_t cols, int64_t ld) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= rows * cols) return;
    const int64_t r = t / cols;
    const int64_t k = t - r * cols;
    const uint8_t* p = packed + r * ld;
    const int64_t bit = 6 * k;
    const int sh = (int)(bit & 7);
    uint32_t v = p[bit >> 3];
    if (sh > 2) v |= (uint32_t)p[(bit >> 3) + 1] << 8;
    codes[t] = (uint8_t)((v >> sh) & 63u);
}

__global__ __launch_bounds__(256) void dequant_lut6_kernel(const uint8_t* __restrict__ packed,
                                                           int64_t ld,
                                                           const uint16_t* __restrict__ lut,
                                                           uint16_t* __restrict__ W, int64_t rows,
                                                           int64_t cols) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= rows * cols) return;
    const int64_t r = t / cols;
    const int64_t k = t - r * cols;
    const uint8_t* p = packed + r * ld;
    const int64_t bit = 6 * k;
    const int sh = (int)(bit & 7);
    uint32_t v = p[bit >> 3];
    if (sh > 2) v |= (uint32_t)p[(bit >> 3) + 1] << 8;
    W[t] = lut[r * 64 + ((v >> sh) & 63u)];
}

// Round an fp64 value to the nearest bf16 (ties to even) from its bits, with
// no intermediate fp32 rounding.  Finite inputs.
__device__ uint16_t f64_to_bf16_rne(double v) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t sign = (uint32_t)(u >> 63) << 15;
    const uint64_t a = u & 0x7FFFFFFFFFFFFFFFull;
    if (a == 0) return (uint16_t)sign;
    int e = (int)(a >> 52);                      // biased fp64 exponent (0 = subnormal)
    uint64_t sig = a & 0xFFFFFFFFFFFFFull;
    if (e) sig |= 1ull << 52; else e = 1;
    int be = e - 1023 + 127;                     // bf16 biased exponent of a normal result
    int shift = 45;                              // keep 8 significant bits
    if (be <= 0) { shift += 1 - be; be = 0; }    // bf16 subnormal: fixed quantum 2^-133
    if (shift > 63) return (uint16_t)sign;
    uint64_t kept = sig >> shift;
    const uint64_t rem = sig & ((1ull << shift) - 1);
    const uint64_t half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (kept & 1))) ++kept;
    // kept carries the implicit bit for normals; a carry into bit 8 bumps the exponent.
    uint32_t bits;
    if (be == 0) {
        bits = (uint32_t)kept;                   // subnormal (or rounded up to the smallest normal)
    } else {
        if (kept >> 8) { kept >>= 1; ++be; }
        bits = ((uint32_t)be << 7) | ((uint32_t)kept & 0x7Fu);
    }
    return (uint16_t)(sign | bits);
}

__device__ __forceinline__ uint32_t field(const uint8_t* row, int64_t k, int b) {
    const int64_t bit = (int64_t)b * k;
    const int sh = (int)(bit & 7);
    uint32_t v = row[bit >> 3];
    if (sh + b > 8) v |= (uint32_t)row[(bit >> 3) + 1] << 8;
    return (v >> sh) & ((1u << b) - 1u);
}

__global__ __launch_bounds__(256) void dequant_fabq_kernel(fqm_fabq f, int64_t rows, int64_t cols,
                                                           uint16_t* __restrict__ W) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= rows * cols) return;
    const int64_t i = t / cols;          // stored row
    const int64_t k = t - i * cols;
    const int64_t out_row = f.row_of[i];
    double w;
    if (i < f.n_hi) {
        const int hb = f.hi_bits ? f.hi_bits : 4;
        int q = (int)field(f.q4 + i * f.ld_q4, k, hb);
        q = q >= (1 << (hb - 1)) ? q - (1 << hb) : q;
        w = (double)q * (double)fp16_to_f32(f.s_hi[i]);
    } else {
        const int64_t j = i - f.n_hi;
        const int64_t nb = cols / f.blocksize;
        const int64_t blk = k / f.blocksize;
        const double s = (double)fp16_to_f32(f.s_blk[j * nb + blk]);
        const uint32_t id = field(f.idx + j * f.ld_idx, blk, 4);
        double c;
        if (f.cb_mode == FQM_CB_SCALAR16) {
            c = (double)fp16_to_f32(f.codebook[id]);
        } else {
            const int64_t cid = 64 * (int64_t)f.tier[j] + f.cb_base + id;
            c = f.cb_mode == FQM_CB_TIERED ? (double)fp16_to_f32(f.codebook[cid])
                                           : (double)f.vcodebook[cid * 128 + (k & 127)];
        }
        w = (field(f.signs + j * f.ld_signs, k, 1) ? s : -s) + c;   // exact in fp64
    }
    W[out_row * cols + k] = f64_to_bf16_rne(w);
}

// Zeroes n 16-bit or 32-bit elements (an empty product: cols == 0).  A fill
// kernel rather than hipMemsetAsync, so the call can sit in a captured graph.
__global__ __launch_bounds__(256) void zero_fill_kernel(uint32_t* __restrict__ p, int64_t words,
                                                        uint16_t* __restrict__ tail) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t < words) p[t] = 0u;
    if (t == 0 && tail) *tail = 0;
}

inline unsigned grid_for(int64_t n, int block) { return (unsigned)((n + block - 1) / block); }

}  // namespace

hipError_t launch_zero_fill(void* p, int64_t n, int elem_bytes, hipStream_t s) {
    const int64_t bytes = n * elem_bytes;
    if (bytes == 0) return hipSuccess;
    const int64_t words = bytes / 4;  // p is 16-byte aligned (checked by the callers)
    uint16_t* tail = (bytes & 2) ? reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(p) + 4 * words) : nullptr;
    hipLaunchKernelGGL(zero_fill_kernel, dim3(grid_for(words > 0 ? words : 1, 256)), dim3(256), 0, s,
                       static_cast<uint32_t*>(p), words, tail);
    return hipGetLastError();
}

hipError_t launch_pack_bits(const uint8_t* vals, uint8_t* out, int64_t rows, int64_t cols,
                            int bits, int64_t ld, int32_t* d_err, hipStream_t s) {
    const int64_t words = ld / 4;
    const int64_t n = rows * words;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(pack_bits_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, vals,
                       reinterpret_cast<uint32_t*>(out), rows, cols, bits, words, d_err);
    return hipGetLastError();
}

hipError_t launch_unpack6(const uint8_t* packed, uint8_t* codes, int64_t rows, int64_t cols,
                          int64_t ld, hipStream_t s) {
    const int64_t n = rows * cols;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(unpack6_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, packed, codes,
                       rows, cols, ld);
    return hipGetLastError();
}

hipError_t launch_dequant_lut6(const fqm_weights& w, uint16_t* W, hipStream_t s) {
    const int64_t n = w.rows * w.cols;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(dequant_lut6_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s,
                       w.lut6.packed, w.lut6.ld, w.lut6.lut, W, w.rows, w.cols);
    return hipGetLastError();
}

hipError_t launch_dequant_fabq(const fqm_weights& w, uint16_t* W, hipStream_t s) {
    const int64_t n = w.rows * w.cols;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(dequant_fabq_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, w.fabq,
                       w.rows, w.cols, W);
    return hipGetLastError();
}

}  // namespace fqm
