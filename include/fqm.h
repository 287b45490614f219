/*
 * fqm.h - fused low-bit dequant-matmul for AMD MI355X (gfx950), C ABI.
 *
 * The library computes the weight-only quantized products y = W x (GEMV,
 * batch 1..16) and Y = X W^T (GEMM) where W is stored in one of three packed
 * formats and is decoded inside the kernels; W is never written out in full
 * (fqm_dequant exists for testing only).
 *
 * Formats (pages named by title and section):
 *   FQM_LUT6  "Qwen3.8-27B - BenQ 6-bit", "What BenQ stores": one 6-bit code
 *             per weight (1 sign bit + 5 magnitude-tier bits) indexing its
 *             output row's own table of 64 signed bf16 levels (32 negative in
 *             ascending order, then 32 positive); decoding W is the row-wise
 *             gather of codes into the tables, and the card's kernel fuses
 *             that gather into the matrix product.  Codes are packed four per
 *             three bytes, the packing its usage note says the format needs.
 *   FQM_LUT4  the same card, "Why equal-width shells": its 8-tier, 4-bit
 *             placement read as the 6-bit format is - one 4-bit code (1 sign
 *             + 3 tier bits) per weight indexing the row's table of 16 signed
 *             bf16 levels (8 negative ascending, then 8 positive); codes two
 *             per byte.
 *   FQM_FABQ  "FABQ-RC" README "Key Ideas" and the FABQ-RC model card
 *             "How It Works" / "Quantization Details": the top 5 % of output
 *             rows as int4 (model card) or int8 (README) with an fp16 row
 *             scale, the rest binary +-1 with an fp16 scale per block of
 *             `blocksize` columns plus a per-block 4-bit index into a residual
 *             codebook whose centroid is added back at inference:
 *                 w = s_b * (+-1) + corr,
 *             corr = c[idx_b] (one 16-entry fp16 codebook), or, with the
 *             card's 4 tiered codebooks of 64 centroids (a binary row's tier
 *             its importance quartile; 16 active centroids per layer from
 *             cb_base), C[tier][cb_base + idx_b] (fp16 centroids) or
 *             V[tier][cb_base + idx_b][k mod 128] (the card's
 *             4 x 64 x 128 x 4-byte storage read as 128-float vectors).
 *   FQM_MDBF  OneCompression "MDBF", "Algorithm": W = sum_p F_p G_p with
 *             F = S_A (.) (A_amp Q_U^T), G = S_B (.) (Q_V B_amp^T), sign
 *             matrices packed 8 per byte and fp16 envelopes; evaluated as
 *                 z = sum_k q_V,k (.) (S_B (b_k (.) x)),
 *                 y = sum_k a_k (.) (S_A (q_U,k (.) z)).
 *
 * Packed bit fields.  Every packed tensor uses one rule: a row of `cols`
 * fields of b bits is a little-endian bit stream; field k occupies stream
 * bits [b*k, b*k + b), least significant bit first, and stream bit i is bit
 * (i mod 8) of byte (i div 8).  Rows start every `ld` bytes; bytes after the
 * last field are zero (fqm_pack writes them) and are ignored by the kernels.
 *   b = 6: LUT6 codes.  b = 1: signs, bit 1 = +1, bit 0 = -1.
 *   b = 4: int4 weights (two's complement) and codebook indices.
 *   b = 8: int8 weights (two's complement).
 *
 * Numbers.  bf16 and fp16 values are passed as their uint16_t bit patterns.
 * Products accumulate in fp32; bf16 outputs are rounded to nearest even.
 *
 * Conventions shared by every call.
 *   - Ownership: the caller allocates and frees every buffer.  All tensor
 *     pointers are DEVICE pointers unless stated otherwise; descriptor
 *     structs (fqm_weights) are HOST memory and are read during the call
 *     only.  The library allocates nothing, frees nothing and keeps no
 *     pointer after returning; calls on different streams may run
 *     concurrently.  The one piece of global state is the per-GPU static
 *     scratch array of fqm_gemv_static (see there).
 *   - Ordering: every call only enqueues work on `stream` (a hipStream_t
 *     passed as void*, NULL = the null stream) and returns; inputs must stay
 *     valid and unmodified, and outputs unread, until the stream passes the
 *     call.
 *   - Errors: arguments are checked on the host before anything is enqueued.
 *     A non-zero fqm_status means nothing was enqueued, except FQM_E_HIP
 *     (a launch failed; earlier kernels of the same call may have run).
 *     Data-dependent errors (a value too wide for its field in fqm_pack*)
 *     are reported through a device flag instead.
 *   - Alignment: every tensor base pointer must be 16-byte aligned and every
 *     row stride `ld` a multiple of 16 bytes (FQM_E_ALIGN otherwise).
 *   - Empty work: rows == 0 or M == 0 enqueue nothing and return FQM_OK;
 *     cols == 0 writes zeros to y (fqm_gemv) or Y (fqm_gemm), and x / X may
 *     then be NULL.
 */
#ifndef FQM_H
#define FQM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FQM_VERSION 5

/* Bytes of the device scratch array fqm_gemv_static uses on each GPU. */
#define FQM_STATIC_SCRATCH_BYTES ((size_t)16 << 20)

typedef enum fqm_status {
    FQM_OK = 0,
    FQM_E_NULL = 1,        /* a required pointer is NULL */
    FQM_E_ALIGN = 2,       /* a base pointer or row stride breaks the 16-byte rule */
    FQM_E_SHAPE = 3,       /* sizes negative, out of range or inconsistent */
    FQM_E_FORMAT = 4,      /* unknown format tag or format parameter out of range */
    FQM_E_WORKSPACE = 5,   /* workspace missing or smaller than fqm_workspace_size */
    FQM_E_UNSUPPORTED = 6, /* valid request this build does not implement */
    FQM_E_HIP = 7,         /* a HIP launch failed */
    FQM_E_SCRATCH = 8,     /* fqm_gemv_static: needs more than FQM_STATIC_SCRATCH_BYTES */
    FQM_E_BOUNDS = 9       /* debug checks: a buffer is not inside one device allocation of its size */
} fqm_status;

enum fqm_format { FQM_LUT6 = 1, FQM_FABQ = 2, FQM_MDBF = 3, FQM_LUT4 = 4 };
enum fqm_dtype { FQM_BF16 = 0, FQM_F32 = 1 };

/* Per-row LUT, 6-bit codes (rows = N outputs, cols = K inputs).
 * cols must be a multiple of 64 (one 48-byte group holds 64 codes). */
typedef struct fqm_lut6 {
    const uint8_t* packed;  /* [rows][ld] bytes, 6-bit fields */
    const uint16_t* lut;    /* [rows][64] bf16, entry j is the level of code j */
    int64_t ld;             /* bytes per packed row, >= cols*3/4 */
} fqm_lut6;

/* Per-row LUT, 4-bit codes (rows = N outputs, cols = K inputs).
 * cols must be a multiple of 64. */
typedef struct fqm_lut4 {
    const uint8_t* packed;  /* [rows][ld] bytes, 4-bit fields (code 2j in the low nibble of byte j) */
    const uint16_t* lut;    /* [rows][16] bf16, entry j is the level of code j */
    int64_t ld;             /* bytes per packed row, >= cols/2 */
} fqm_lut4;

/* FABQ-RC-style core (rows = N, cols = K).  Stored row i (0 <= i < rows)
 * produces output row row_of[i]; stored rows 0..n_hi-1 are high-precision
 * rows, stored rows n_hi..rows-1 are binary rows (binary row j = stored row
 * n_hi + j).  row_of must be a permutation of 0..rows-1 (not checked: a
 * repeated entry makes two rows write the same output).  A zeroed hi_bits /
 * cb_mode means 4 / FQM_CB_SCALAR16. */
enum fqm_cb_mode {
    FQM_CB_SCALAR16 = 0,  /* codebook: [16] fp16; corr = codebook[idx] */
    FQM_CB_TIERED = 1,    /* codebook: [4][64] fp16; corr = codebook[tier][cb_base + idx] */
    FQM_CB_VECTOR = 2     /* vcodebook: [4][64][128] fp32; corr = vcodebook[tier][cb_base + idx][k % 128] */
};
typedef struct fqm_fabq {
    int32_t blocksize;          /* 16, 32, 64, 128, 256 or 512; divides cols */
    int32_t n_hi;               /* high-precision rows, 0..rows */
    const int32_t* row_of;      /* [rows] */
    const uint8_t* q4;          /* [n_hi][ld_q4], hi_bits-wide two's complement fields */
    int64_t ld_q4;              /* >= cols*hi_bits/8 */
    const uint16_t* s_hi;       /* [n_hi] fp16 row scales */
    const uint8_t* signs;       /* [rows-n_hi][ld_signs], 1-bit fields */
    int64_t ld_signs;           /* >= cols/8 */
    const uint16_t* s_blk;      /* [rows-n_hi][cols/blocksize] fp16, dense */
    const uint8_t* idx;         /* [rows-n_hi][ld_idx], 4-bit fields, one per block */
    int64_t ld_idx;             /* >= ceil(cols/blocksize/2) */
    const uint16_t* codebook;   /* FQM_CB_SCALAR16: [16] fp16; FQM_CB_TIERED: [4][64] fp16 */
    int32_t hi_bits;            /* 4 or 8 (0 = 4) */
    int32_t cb_mode;            /* enum fqm_cb_mode */
    int32_t cb_base;            /* tiered modes: 0, 16, 32 or 48 */
    const uint8_t* tier;        /* tiered modes: [rows-n_hi], 0..3 per binary row */
    const float* vcodebook;     /* FQM_CB_VECTOR: [4][64][128] fp32 */
} fqm_fabq;

/* One MDBF path (rows = n outputs, cols = m inputs, rank r, envelope rank l). */
typedef struct fqm_mdbf_path {
    const uint8_t* S_A;         /* [n][ld_A], 1-bit fields along r; each row is read up to
                                   ceil(r/8) rounded up to a multiple of 16 bytes */
    int64_t ld_A;               /* >= ceil(r/8) */
    const uint8_t* S_B;         /* [r][ld_B], 1-bit fields along m; each row is read up to
                                   m/8 rounded up to a multiple of 16 bytes */
    int64_t ld_B;               /* >= m/8 */
    const uint16_t* A_amp;      /* [n][l] fp16 */
    const uint16_t* B_amp;      /* [m][l] fp16 */
    const uint16_t* Q_U;        /* [r][l] fp16 */
    const uint16_t* Q_V;        /* [r][l] fp16 */
} fqm_mdbf_path;

typedef struct fqm_mdbf {
    int32_t r;                  /* 1..65536 */
    int32_t l;                  /* 1..16 */
    int32_t P;                  /* 1 or 2; path[0..P-1] are used */
    fqm_mdbf_path path[2];
} fqm_mdbf;

/* Weight descriptor: `format` selects which member is read. */
typedef struct fqm_weights {
    int32_t format;             /* enum fqm_format */
    int64_t rows;               /* outputs (N, or n for MDBF) */
    int64_t cols;               /* inputs  (K, or m for MDBF; MDBF needs m % 32 == 0) */
    fqm_lut6 lut6;
    fqm_fabq fabq;
    fqm_mdbf mdbf;
    fqm_lut4 lut4;              /* last, so the earlier members keep their offsets */
} fqm_weights;

/* Library version (FQM_VERSION). */
int32_t fqm_version(void);

/* Debug checks on (on != 0) or off for every later call in this process;
 * returns the previous setting.  The setting starts from the environment
 * variable FQM_DEBUG (on unless unset, empty or "0"), read on first use.
 * With the checks on, each call also (1) checks, before enqueuing anything,
 * that every device buffer it would read or write, at the extent its shape
 * and strides give, lies inside one device allocation
 * (hipMemGetAddressRange), returning FQM_E_BOUNDS otherwise; a view into a
 * larger allocation (a caching allocator's block) passes when it stays
 * inside that allocation, and the static scratch of fqm_gemv_static is not
 * checked; and (2) after enqueuing, unless the stream is being captured,
 * waits for the stream and returns FQM_E_HIP if the call's kernels failed.
 * The checks cost a host round trip per buffer and a stream synchronisation
 * per call: they are for finding caller bugs, not for production runs. */
int32_t fqm_set_debug(int32_t on);

/* Static, human-readable name of a status code (never NULL). */
const char* fqm_status_str(int32_t status);

/* Pack `bits`-wide unsigned fields (bits = 1, 4, 6 or 8): vals [rows][cols]
 * uint8, one field per byte, row-major and dense; out [rows][ld] bytes under
 * the packed-field rule above, padding bytes zeroed.  A value >= 2^bits is
 * packed as (value & (2^bits - 1)) and sets bit 0 of *d_err (a device int32
 * the caller zeroes beforehand; may be NULL).  Signed int4 values are passed
 * as (q & 15).  Requires ld >= ceil(cols*bits/8); vals needs no alignment.
 * The bit-field rule is this project's convention; the pages fix only the
 * field widths (see the format list above). */
fqm_status fqm_pack_bits(const uint8_t* vals, uint8_t* out, int64_t rows, int64_t cols,
                         int32_t bits, int64_t ld, int32_t* d_err, void* stream);

/* Pack LUT6 codes (0..63), four per three bytes: fqm_pack_bits with bits = 6.
 * Source: "Qwen3.8-27B - BenQ 6-bit", usage note on packing the stored
 * uint8 codes to 6 bits (~28 GB -> ~21 GB). */
fqm_status fqm_pack(const uint8_t* codes, uint8_t* packed, int64_t rows, int64_t cols,
                    int64_t ld, int32_t* d_err, void* stream);

/* Test helper: unpack 6-bit codes back to one byte per code, codes [rows][cols]
 * dense.  Requires cols % 4 == 0.  The inverse of fqm_pack: each group of three
 * bytes (little-endian 24 bits) yields four codes of 6 bits, lowest first.
 * Source: "Qwen3.8-27B - BenQ 6-bit", "What BenQ stores" (one 6-bit code per
 * weight) and its usage note on packing the stored uint8 codes to 6 bits. */
fqm_status fqm_unpack(const uint8_t* packed, uint8_t* codes, int64_t rows, int64_t cols,
                      int64_t ld, void* stream);

/* Test helper: write the decoded weights W [rows][cols] as bf16, row-major,
 * row index = output row.  Sources: LUT6 / LUT4 "Qwen3.8-27B - BenQ 6-bit",
 * "What BenQ stores" (decode is a gather of the code's entry in the row's
 * table); FABQ the FABQ-RC model card "Quantization Details" and the FABQ-RC
 * README "Key Ideas" (scale times sign or int4 / int8 level, plus the residual
 * codebook correction).  LUT6 and LUT4: W[r][k] = lut[r][code] (an exact copy).
 * FABQ: the exact value of q*s or s_b*(+-1) + corr rounded once to bf16
 * (nearest even).  MDBF: FQM_E_UNSUPPORTED (W is a product of factors). */
fqm_status fqm_dequant(const fqm_weights* w, uint16_t* W, void* stream);

/* Bytes of device workspace fqm_gemv needs for this descriptor and batch:
 * MDBF 32*P*S*C*(roundup(m,512) + roundup(r,512)) with S = ceil(batch / bs),
 * bs = 1 if 3*l >= 64 else floor(64 / (3*l)) and C = ceil(3*l*min(bs, batch) / 16)
 * (the dense operands of both passes: each fp32 value as three bf16 parts,
 * in C blocks of 16 columns per batch slice of bs rows); LUT6 and LUT4 with batch >= 2 and
 * cols a multiple of 512 split K over workgroups unless rows > 16368, and
 * then need S*batch*rows*4 (S fp32 partial sums per output, S <= cols / 512,
 * a function of rows and cols only, the same for both formats), else 0;
 * LUT6 at batch 2 with cols = 1024*c, 1 <= c <= 19, and at batch 3 with
 * 1 <= c <= 12 needs none (one row per wave, every batch row from one decode);
 * FABQ with FQM_CB_VECTOR and at least one binary row
 * batch*(cols/blocksize)*64*4 rounded up to 16 (per batch row, block and
 * active centroid 16*tier + idx, the block's sum over its columns k of
 * vcodebook[tier][cb_base + idx][k % 128] * x[k] in fp32, formed by a first
 * launch; the GEMV then adds one such term per binary row and block), other
 * FABQ modes 0.
 * Returns 0 for an invalid descriptor. */
size_t fqm_workspace_size(const fqm_weights* w, int32_t batch);

/* y = W x for `batch` activation rows (1..16).
 * x: [batch][cols] bf16, row-major.  y: [batch][rows], bf16 (y_dtype =
 * FQM_BF16) or fp32 (FQM_F32).  workspace: device memory of at least
 * fqm_workspace_size(w, batch) bytes (may be NULL when that is 0); its
 * contents on entry do not matter and are clobbered.
 * LUT6 and LUT4 follow the BenQ card's decode (a gather into the row's table)
 * fused into the product; FABQ and MDBF follow the decode stated with each format
 * above; every decoded weight stays in fp32 (never rounded to bf16). */
fqm_status fqm_gemv(const fqm_weights* w, const uint16_t* x, void* y, int32_t y_dtype,
                    int32_t batch, void* workspace, size_t ws_bytes, void* stream);

/* fqm_gemv without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The same kernels and results as fqm_gemv (bit for
 * bit); where fqm_gemv would use the caller's workspace, this call uses a
 * static device array of FQM_STATIC_SCRATCH_BYTES (16 MiB) that the library
 * holds on each GPU it runs on until the process ends.  The array of the
 * current device (hipGetDevice) is used, so `stream` must belong to that
 * device; its address is looked up on the first call on each device that
 * needs scratch.  Nothing is allocated, freed or cleared (the kernels need no
 * zeroed scratch: every word they read they first write in the same call).
 * Calls that overlap on one GPU (concurrent streams, host threads, or graph
 * replays in flight together) share the array and RACE: serialise them.
 * Returns FQM_E_SCRATCH, enqueuing nothing, when fqm_workspace_size(w,
 * batch) exceeds FQM_STATIC_SCRATCH_BYTES (for example MDBF with many
 * envelopes at large batch on the 27B-class MLP shapes); FQM_E_HIP if the
 * address lookup fails; otherwise as fqm_gemv. */
fqm_status fqm_gemv_static(const fqm_weights* w, const uint16_t* x, void* y, int32_t y_dtype,
                           int32_t batch, void* stream);

/* Bytes of device workspace fqm_gemm needs for this LUT6 or LUT4 descriptor and M on
 * the current device: for M <= 16 on a shape the GEMV kernels cover (batch 1:
 * cols = 1024 c, 1 <= c <= 31; batch 2..16: cols a multiple of 512) it is
 * fqm_workspace_size(w, M), since fqm_gemm then runs those kernels; otherwise
 * 256 * 256 * 4 bytes per K part of each 256 x 256 output tile of a last,
 * partial round of tiles (one round = one tile per compute unit), when such
 * tiles are split along K, and 0 when nothing is split.  A function of rows,
 * cols, M and the device's compute-unit count (the same for both formats).
 * Returns 0 for an invalid, FABQ or MDBF descriptor. */
size_t fqm_gemm_workspace_size(const fqm_weights* w, int64_t M);

/* Y = X W^T for a LUT6 or LUT4 descriptor (prefill): X [M][cols] bf16, Y [M][rows]
 * bf16, both row-major.  Source: "Qwen3.8-27B - BenQ 6-bit", "What BenQ stores":
 * the gather of the decode fused into the GEMM so that the decoded matrix is
 * never written out.  Shapes: cols a multiple of 64 and M * cols * 2 < 2^31
 * (FQM_E_SHAPE otherwise).  Each weight is gathered from its row's table
 * (exact: the levels are bf16) straight into the operands of the bf16 matrix
 * cores, fp32 accumulation.  workspace: device memory of at least
 * fqm_gemm_workspace_size(w, M) bytes, 16-byte aligned (may be NULL when that
 * is 0); its contents on entry do not matter and are clobbered.  Split tiles
 * add their fp32 K parts in a fixed order, so results do not depend on timing.
 * Up to 16 rows of X on a shape the GEMV kernels cover run those kernels (the
 * same product as fqm_gemv with batch = M and bf16 output; the 256-row tiles
 * would mostly multiply padding there).
 * FABQ / MDBF descriptors return FQM_E_UNSUPPORTED. */
fqm_status fqm_gemm(const fqm_weights* w, const uint16_t* X, uint16_t* Y, int64_t M,
                    void* workspace, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FQM_H */
