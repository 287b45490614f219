"""Per-row LUT 6-bit weights: decode and product (oracle side).

Test infrastructure only.

Source: "Qwen3.8-27B - BenQ 6-bit" model card, section "What BenQ stores":
each weight is a 6-bit code (1 sign bit, 5 magnitude-tier bits) that indexes
its output row's own table of 64 signed bf16 magnitudes, 32 negative in
ascending order then 32 positive; decoding a weight matrix is the row-wise
gather of the codes into the tables; the bits-per-weight table counts 6.000
for the code and 64 bf16 entries per row amortised over the row's columns.

  W[r, k] = lut[r, code[r, k]]            (exact copy of a bf16 value)
  y[b, r] = sum_k W[r, k] * x[b, k]       (fp64 matmul)

Parity status: the decode and the product are pinned (library gather,
brute force, one-hot, mirror, scaling, constructed exact weights).  The byte
layout of the packed codes is this project's own convention (the pages state
only that packing to 6 bits is possible); it is pinned by hand-computed bytes
and a round trip, not by the pages.
"""
import numpy as np

from . import bits
from .numerics import bf16_to_f64


def pack_codes(codes, ld: int | None = None) -> np.ndarray:
    return bits.pack(codes, 6, ld)


def unpack_codes(packed, cols: int) -> np.ndarray:
    return bits.unpack(packed, cols, 6).astype(np.uint8)


def decode(codes, lut_bits) -> np.ndarray:
    """fp64 W[rows][cols] = lut[r][codes[r][k]]."""
    lut = bf16_to_f64(lut_bits)
    return np.take_along_axis(lut, np.asarray(codes, dtype=np.int64), axis=1)


def gemv(packed, lut_bits, x_bits, cols: int) -> np.ndarray:
    """y[batch][rows] in fp64 from packed codes, bf16 tables and bf16 x."""
    W = decode(unpack_codes(packed, cols), lut_bits)
    x = bf16_to_f64(x_bits)
    return x @ W.T


def gemm(packed, lut_bits, X_bits, cols: int) -> np.ndarray:
    """Y[M][rows] = X W^T in fp64 (same definition as gemv with batch = M)."""
    return gemv(packed, lut_bits, X_bits, cols)


def bpw(cols: int) -> float:
    """Bits per weight of one matrix: 6 code bits + 64 x 16 table bits per row."""
    return 6.0 + 64.0 * 16.0 / cols
