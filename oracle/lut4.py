"""Per-row LUT 4-bit weights: decode and product (oracle side).

Test infrastructure only.

Source: "Qwen3.8-27B - BenQ 6-bit" model card, section "Why equal-width
shells": the placement table compares level placements at 8 tiers / 4 bits
beside 32 tiers / 6 bits.  This module is the 4-bit row of that table read
the same way as the 6-bit format ("What BenQ stores"): a code is 1 sign bit
and 3 tier bits and indexes its output row's own table of 16 signed bf16
levels, 8 negative in ascending order then 8 positive.

  W[r, k] = lut[r, code[r, k]]            (exact copy of a bf16 value)
  y[b, r] = sum_k W[r, k] * x[b, k]       (fp64 matmul)

Codes are stored two per byte with the same bit-stream rule as every other
field here (field k at stream bits [4k, 4k + 4), least significant first), a
layout of this project's own (the pages give the bit count only).

Parity status: the decode and the product are pinned (library gather, brute
force, one-hot, constant codes, mirror, hand-computed bytes and a round trip).
"""
import numpy as np

from . import bits
from .numerics import bf16_to_f64


def pack_codes(codes, ld: int | None = None) -> np.ndarray:
    return bits.pack(codes, 4, ld)


def unpack_codes(packed, cols: int) -> np.ndarray:
    return bits.unpack(packed, cols, 4).astype(np.uint8)


def decode(codes, lut_bits) -> np.ndarray:
    """fp64 W[rows][cols] = lut[r][codes[r][k]] (16-entry tables)."""
    lut = bf16_to_f64(lut_bits)
    return np.take_along_axis(lut, np.asarray(codes, dtype=np.int64), axis=1)


def gemv(packed, lut_bits, x_bits, cols: int) -> np.ndarray:
    """y[batch][rows] in fp64 from packed codes, bf16 tables and bf16 x."""
    W = decode(unpack_codes(packed, cols), lut_bits)
    x = bf16_to_f64(x_bits)
    return x @ W.T


def bpw(cols: int) -> float:
    """Bits per weight of one matrix: 4 code bits + 16 x 16 table bits per row."""
    return 4.0 + 16.0 * 16.0 / cols
