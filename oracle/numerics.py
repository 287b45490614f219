"""Exact conversions between stored 16-bit floats and fp64 (oracle side).

Test infrastructure only.  bf16 is the top half of an IEEE binary32; fp16 is
IEEE binary16.  Both widen to fp64 exactly.  ``f64_to_bf16_rne`` rounds an fp64
value straight to the nearest bf16 (ties to even), without an fp32 step, and is
used only by the comparison rule for bf16 outputs.
"""
import numpy as np


def bf16_to_f64(bits) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def fp16_to_f64(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def f64_to_bf16_rne(v) -> np.ndarray:
    """Round fp64 to the nearest bf16 value (8 significant bits), ties to even.

    Returned as fp64 values.  Below 2^-126 the quantum is fixed at 2^-133
    (bf16 subnormals).  Values beyond the bf16 range are not expected here.
    """
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)                     # v = m * 2^e with 0.5 <= |m| < 1
    q = np.maximum(e - 8, -133)            # weight of the last kept bit
    scale = np.ldexp(1.0, q)
    return np.rint(v / scale) * scale      # rint rounds half to even; /scale is exact


def bf16_bits_from_f64_rne(v) -> np.ndarray:
    """bf16 bit patterns of ``f64_to_bf16_rne(v)`` (the value is exact in fp32)."""
    f = f64_to_bf16_rne(v).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
