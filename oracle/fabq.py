"""FABQ-RC-style binary core: decode and product (oracle side).

Test infrastructure only.

Sources: "FABQ-RC" README, "Key Ideas" (top 5 % channels kept at higher
precision - int8 there -, the rest binary +-1, a blocksize per layer swept
over {16, 32, 64, 128, 256}, a k-means residual codebook whose centroid is
added back at inference) and the FABQ-RC model card, "How It Works" and
"Quantization Details" (int4 for the top channels, binary +-1 with per-block
scaling, blocksizes {64, 128, 256, 512}, "4 tiered k-means codebooks (64
centroids each, Fisher quartile-based)", 4-bit indices per block with 16
active centroids per layer cluster, and a codebook storage of
4 x 64 x 128 x 4 bytes).

Reading taken where the pages are open or disagree:
  * high-precision rows: ``hi_bits`` = 4 (model card) or 8 (README), signed
    two's-complement fields with one fp16 scale per row and no zero point;
  * binary rows in blocks of ``bs`` consecutive columns, bs in
    {16, 32, 64, 128, 256, 512}, each with an fp16 scale s_b and a 4-bit index;
  * the residual correction, binary rows only, by ``cb_mode``:
      0  one per-layer 16-entry fp16 codebook c:      corr = c[idx_b]
      1  4 tiers x 64 fp16 centroids C; a binary row's tier is the quartile
         of its importance among the binary rows; the layer uses the 16
         consecutive centroids starting at ``cb_base`` of its row's tier:
                                                      corr = C[tier, cb_base + idx_b]
      2  4 tiers x 64 centroids that are vectors of 128 fp32 values V (the
         4 x 64 x 128 x 4-byte storage); weight k takes element k mod 128:
                                                      corr = V[tier, cb_base + idx_b, k mod 128]
Stored row i is output row ``row_of[i]``; the ``n_hi`` high-precision rows
come first.

  high row:    W[row_of[i], k] = q[i, k] * s_hi[i]
  binary row:  W[row_of[n_hi + j], k] = s_blk[j, k // bs] * (+1 if bit else -1) + corr
  y = x W^T    (fp64)

Parity status: unpinned by the pages (no worked example; the pages'
descriptions of the codebook conflict).  Pinned against the reading above by
weights constructed to be exactly representable, closed forms for zero
codebooks and for high-precision-only layers, reductions between the
codebook modes, brute force over bits, a hand-worked example
(tests/golden/fabq_variants.txt), and one-hot x.
"""
import numpy as np

from . import bits
from .numerics import fp16_to_f64, bf16_to_f64


def idx_row_bytes(cols: int, bs: int) -> int:
    nb = cols // bs
    return ((nb + 1) // 2 + 3) // 4 * 4   # nibbles, padded to 4 bytes


def pack(inp):
    """Packed stored tensors (dict of numpy arrays) from an unpacked input.
    The codebook mode and its parameters travel with them."""
    nb = inp.cols // inp.blocksize
    hb = getattr(inp, "hi_bits", 4)
    mode = getattr(inp, "cb_mode", 0)
    p = dict(
        q4=bits.pack(inp.q4, hb),
        signs=bits.pack(inp.signs, 1),
        idx=bits.pack(inp.idx, 4, idx_row_bytes(inp.cols, inp.blocksize)),
        s_hi=np.asarray(inp.s_hi, dtype=np.uint16),
        s_blk=np.asarray(inp.s_blk, dtype=np.uint16).reshape(-1, nb),
        codebook=np.asarray(inp.codebook, dtype=np.uint16),
        row_of=np.asarray(inp.row_of, dtype=np.int32),
        hi_bits=hb, cb_mode=mode, cb_base=int(getattr(inp, "cb_base", 0)),
    )
    if mode in (1, 2):
        p["tier"] = np.asarray(inp.tier, dtype=np.uint8)
    if mode == 2:
        p["vcodebook"] = np.asarray(inp.vcodebook, dtype=np.float32).reshape(4, 64, 128)
    return p


def correction(p, idx, cols: int, bs: int) -> np.ndarray:
    """fp64 residual correction [n_lo][cols] of the binary rows."""
    mode = p.get("cb_mode", 0)
    blk = np.arange(cols) // bs
    if mode == 0:
        return fp16_to_f64(p["codebook"])[idx][:, blk]
    tier = np.asarray(p["tier"], dtype=np.int64)[:, None]           # [n_lo][1]
    cid = p["cb_base"] + idx                                          # [n_lo][nb]
    if mode == 1:
        C = fp16_to_f64(p["codebook"]).reshape(4, 64)
        return C[tier, cid][:, blk]
    V = np.asarray(p["vcodebook"], dtype=np.float32).astype(np.float64).reshape(4, 64, 128)
    return V[tier, cid[:, blk], (np.arange(cols) % 128)[None, :]]


def decode(p, rows: int, cols: int, bs: int, n_hi: int) -> np.ndarray:
    """fp64 W[rows][cols] from packed tensors."""
    nb = cols // bs
    hb = p.get("hi_bits", 4)
    W = np.zeros((rows, cols), dtype=np.float64)
    row_of = np.asarray(p["row_of"], dtype=np.int64)
    if n_hi:
        q = bits.to_signed(bits.unpack(p["q4"], cols, hb), hb).astype(np.float64)
        W[row_of[:n_hi]] = q * fp16_to_f64(p["s_hi"])[:, None]
    n_lo = rows - n_hi
    if n_lo:
        pm1 = np.where(bits.unpack(p["signs"], cols, 1) == 1, 1.0, -1.0)
        idx = bits.unpack(p["idx"], nb, 4)
        s = fp16_to_f64(p["s_blk"])                       # [n_lo][nb]
        blk = np.arange(cols) // bs
        W[row_of[n_hi:]] = s[:, blk] * pm1 + correction(p, idx, cols, bs)
    return W


def gemv(p, x_bits, rows: int, cols: int, bs: int, n_hi: int) -> np.ndarray:
    return bf16_to_f64(x_bits) @ decode(p, rows, cols, bs, n_hi).T


def bpw(rows: int, cols: int, bs: int, n_hi: int, n_codes: int = 16, hi_bits: int = 4,
        cb_mode: int = 0) -> float:
    """Stored bits per weight: high-precision rows + fp16 row scales, sign
    bits + fp16 block scales + 4-bit indices, the codebook (16 fp16; 4 x 64
    fp16; or 4 x 64 x 128 fp32 = 128 KB), one tier byte per binary row in the
    tiered modes, and a 32-bit row map."""
    n_lo = rows - n_hi
    nb = cols // bs
    cb_bits = {0: n_codes * 16, 1: 4 * 64 * 16, 2: 4 * 64 * 128 * 32}[cb_mode]
    tier_bits = 8 * n_lo if cb_mode in (1, 2) else 0
    total = (n_hi * cols * hi_bits + n_hi * 16 + n_lo * cols + n_lo * nb * (16 + 4)
             + cb_bits + tier_bits + rows * 32)
    return total / (rows * cols)
