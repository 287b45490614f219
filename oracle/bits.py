"""Bit-field packing used by every stored format (oracle side).

Test infrastructure only.  One rule covers all three field widths: a row of
``cols`` fields of ``b`` bits is a little-endian bit stream in which field k
occupies stream bits [b*k, b*k + b), least significant bit first, and stream
bit i is bit (i mod 8) of byte (i div 8).  Rows start every ``ld`` bytes; bytes
past the last field are zero.

  b = 6 : four LUT codes per three bytes, the packing the BenQ model card
          says would shrink its stored uint8 codes to ~21 GB ("Requires ~28 GB
          ... packing to 6-bit").  The bit order is this project's convention.
  b = 1 : sign bits, 1 -> +1 (MDBF "packed into uint8 (8:1)"; FABQ binary rows).
  b = 4 : int4 weights (two's complement) and 4-bit codebook indices.

Implemented with ``np.unpackbits`` / ``np.packbits`` over explicit bit
matrices, i.e. the definition above written out bit by bit.
"""
import numpy as np


def packed_row_bytes(cols: int, b: int) -> int:
    return (cols * b + 7) // 8


def pack(vals, b: int, ld: int | None = None, chunk_rows: int = 256) -> np.ndarray:
    vals = np.asarray(vals)
    rows, cols = vals.shape
    nbytes = packed_row_bytes(cols, b)
    ld = nbytes if ld is None else ld
    if ld < nbytes:
        raise ValueError("row stride too small")
    out = np.zeros((rows, ld), dtype=np.uint8)
    for r0 in range(0, rows, chunk_rows):
        v = vals[r0:r0 + chunk_rows].astype(np.int64) & ((1 << b) - 1)
        bitmat = ((v[:, :, None] >> np.arange(b)) & 1).astype(np.uint8)  # [rows][cols][b]
        stream = bitmat.reshape(v.shape[0], cols * b)
        out[r0:r0 + chunk_rows, :nbytes] = np.packbits(stream, axis=1, bitorder="little")
    return out


def unpack(packed, cols: int, b: int, chunk_rows: int = 256) -> np.ndarray:
    """Unsigned field values [rows][cols] (int64)."""
    packed = np.asarray(packed, dtype=np.uint8)
    rows = packed.shape[0]
    nbytes = packed_row_bytes(cols, b)
    out = np.empty((rows, cols), dtype=np.int64)
    weights = (1 << np.arange(b)).astype(np.int64)
    for r0 in range(0, rows, chunk_rows):
        stream = np.unpackbits(packed[r0:r0 + chunk_rows, :nbytes], axis=1,
                               bitorder="little")[:, :cols * b]
        bitmat = stream.reshape(stream.shape[0], cols, b).astype(np.int64)
        out[r0:r0 + chunk_rows] = bitmat @ weights
    return out


def to_signed(u, b: int) -> np.ndarray:
    """Two's-complement reinterpretation of unsigned b-bit fields."""
    u = np.asarray(u, dtype=np.int64)
    return np.where(u >= (1 << (b - 1)), u - (1 << b), u)
