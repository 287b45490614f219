"""FABQ-RC-style binary core: decode and product (oracle side).

Test infrastructure only.

Sources: "FABQ-RC" README, "Key Ideas" (top 5 % channels kept at higher
precision, the rest binary +-1, per-layer blocksize, a k-means residual
codebook whose centroid is added back at inference) and the FABQ-RC model
card, "How It Works" and "Quantization Details" (int4 for the top channels,
binary +-1 with per-block scaling, 4-bit indices into 16 active centroids).

Reading taken where the pages are open or disagree: int4 rows (the model card)
with one fp16 scale per row and no zero point; binary rows in blocks of
``bs`` consecutive columns, each with an fp16 scale s_b and a 4-bit index into
one per-layer 16-entry fp16 codebook c; the codebook correction applies to
binary rows only.  Stored row i is output row ``row_of[i]``; the ``n_hi`` int4
rows come first.

  int4 row:    W[row_of[i], k] = q[i, k] * s_hi[i]
  binary row:  W[row_of[n_hi + j], k] = s_blk[j, k // bs] * (+1 if bit else -1)
                                         + c[idx[j, k // bs]]
  y = x W^T    (fp64)

Parity status: unpinned by the pages (no worked example; the pages'
descriptions of the codebook conflict).  Pinned against the reading above by
weights constructed to be exactly representable, closed forms for an all-zero
codebook and for int4-only layers, brute force over bits, and one-hot x.
"""
import numpy as np

from . import bits
from .numerics import fp16_to_f64, bf16_to_f64


def idx_row_bytes(cols: int, bs: int) -> int:
    nb = cols // bs
    return ((nb + 1) // 2 + 3) // 4 * 4   # nibbles, padded to 4 bytes


def pack(inp):
    """Packed stored tensors (dict of numpy arrays) from an unpacked input."""
    nb = inp.cols // inp.blocksize
    return dict(
        q4=bits.pack(inp.q4, 4),
        signs=bits.pack(inp.signs, 1),
        idx=bits.pack(inp.idx, 4, idx_row_bytes(inp.cols, inp.blocksize)),
        s_hi=np.asarray(inp.s_hi, dtype=np.uint16),
        s_blk=np.asarray(inp.s_blk, dtype=np.uint16).reshape(-1, nb),
        codebook=np.asarray(inp.codebook, dtype=np.uint16),
        row_of=np.asarray(inp.row_of, dtype=np.int32),
    )


def decode(p, rows: int, cols: int, bs: int, n_hi: int) -> np.ndarray:
    """fp64 W[rows][cols] from packed tensors."""
    nb = cols // bs
    W = np.zeros((rows, cols), dtype=np.float64)
    row_of = np.asarray(p["row_of"], dtype=np.int64)
    if n_hi:
        q = bits.to_signed(bits.unpack(p["q4"], cols, 4), 4).astype(np.float64)
        W[row_of[:n_hi]] = q * fp16_to_f64(p["s_hi"])[:, None]
    n_lo = rows - n_hi
    if n_lo:
        pm1 = np.where(bits.unpack(p["signs"], cols, 1) == 1, 1.0, -1.0)
        idx = bits.unpack(p["idx"], nb, 4)
        s = fp16_to_f64(p["s_blk"])                       # [n_lo][nb]
        c = fp16_to_f64(p["codebook"])[idx]               # [n_lo][nb]
        blk = np.arange(cols) // bs
        W[row_of[n_hi:]] = s[:, blk] * pm1 + c[:, blk]
    return W


def gemv(p, x_bits, rows: int, cols: int, bs: int, n_hi: int) -> np.ndarray:
    return bf16_to_f64(x_bits) @ decode(p, rows, cols, bs, n_hi).T


def bpw(rows: int, cols: int, bs: int, n_hi: int, n_codes: int = 16) -> float:
    """Stored bits per weight: int4 rows + fp16 row scales, sign bits + fp16
    block scales + 4-bit indices, the fp16 codebook, and a 32-bit row map."""
    n_lo = rows - n_hi
    nb = cols // bs
    total = (n_hi * cols * 4 + n_hi * 16 + n_lo * cols + n_lo * nb * (16 + 4)
             + n_codes * 16 + rows * 32)
    return total / (rows * cols)
