"""MDBF double binary factorisation: product and bit accounting (oracle side).

Test infrastructure only.

Source: OneCompression documentation page "MDBF (Multi-Envelope Double Binary
Factorization)":
  * "Algorithm": W ~ sum_p F_p G_p with F = S_A (.) (A_amp Q_U^T) and
    G = S_B (.) (Q_V B_amp^T); S_A in {+-1}^{n x r}, S_B in {+-1}^{r x m}, one
    bit per sign packed into uint8; A_amp n x l, B_amp m x l, Q_U r x l,
    Q_V r x l in fp16.
  * "Choosing l and P": (l, P) = (1, 1) is DBF, (1, 2) is LittleBit.
  * "The matrix shape caps the reachable BPW": r <= min(n, m) and the b_max
    ceiling; targets above it are clamped with a warning.
  * "Bit-width and rank": b_eff and its inversion for r; scale_bits is an
    accounting parameter (default 16).
  * "Save and Load": signs unpacked on the fly at inference, envelopes fp16.
  * DBF comparison paragraph: W ~ A diag(d) B.

Two independent routes compute y = W x:
  dense    - form F, G, W in fp64, multiply.
  factored - z = sum_k q_V,k (.) (S_B (b_k (.) x)),
             y = sum_k a_k (.) (S_A (q_U,k (.) z)).

Parity status: pinned (route agreement, the DBF and LittleBit reductions, the
all-ones-sign rank-l closed form, and the page's accounting formulas checked
against the stored byte counts).  Sign bit layout (bits along the last
dimension, LSB first, 1 -> +1, rows padded to 16 bytes) is this project's
convention.
"""
import math
import warnings

import numpy as np

from . import bits
from .numerics import fp16_to_f64, bf16_to_f64


def sign_row_bytes(cols: int) -> int:
    return (bits.packed_row_bytes(cols, 1) + 15) // 16 * 16


def pack(inp):
    paths = []
    for p in range(inp.P):
        paths.append(dict(
            S_A=bits.pack(inp.S_A[p], 1, sign_row_bytes(inp.r)),
            S_B=bits.pack(inp.S_B[p], 1, sign_row_bytes(inp.m)),
            A_amp=np.asarray(inp.A_amp[p], dtype=np.uint16),
            B_amp=np.asarray(inp.B_amp[p], dtype=np.uint16),
            Q_U=np.asarray(inp.Q_U[p], dtype=np.uint16),
            Q_V=np.asarray(inp.Q_V[p], dtype=np.uint16),
        ))
    return paths


def _signs(packed, cols):
    return np.where(bits.unpack(packed, cols, 1) == 1, 1.0, -1.0)


def factors(path, n, m, r):
    """fp64 (F, G) of one path."""
    S_A = _signs(path["S_A"], r)
    S_B = _signs(path["S_B"], m)
    A, B = fp16_to_f64(path["A_amp"]), fp16_to_f64(path["B_amp"])
    QU, QV = fp16_to_f64(path["Q_U"]), fp16_to_f64(path["Q_V"])
    F = S_A * (A @ QU.T)
    G = S_B * (QV @ B.T)
    return F, G


def dense_weight(paths, n, m, r) -> np.ndarray:
    W = np.zeros((n, m))
    for path in paths:
        F, G = factors(path, n, m, r)
        W += F @ G
    return W


def gemv_dense(paths, x_bits, n, m, r) -> np.ndarray:
    return bf16_to_f64(x_bits) @ dense_weight(paths, n, m, r).T


def gemv_factored(paths, x_bits, n, m, r, return_z: bool = False):
    """Two sign-matrix passes per path; x is [batch][m]; returns y [batch][n]."""
    x = bf16_to_f64(x_bits)
    y = np.zeros((x.shape[0], n))
    zs = []
    for path in paths:
        S_A = _signs(path["S_A"], r)
        S_B = _signs(path["S_B"], m)
        A, B = fp16_to_f64(path["A_amp"]), fp16_to_f64(path["B_amp"])
        QU, QV = fp16_to_f64(path["Q_U"]), fp16_to_f64(path["Q_V"])
        l = A.shape[1]
        z = np.zeros((x.shape[0], r))
        for k in range(l):
            z += QV[:, k][None, :] * ((B[:, k][None, :] * x) @ S_B.T)
        for k in range(l):
            y += A[:, k][None, :] * ((QU[:, k][None, :] * z) @ S_A.T)
        zs.append(z)
    return (y, zs) if return_z else y


def b_eff(n, m, r, l, P, scale_bits=16) -> float:
    return P * (r * (n + m) + scale_bits * l * (n + m + 2 * r)) / (n * m)


def b_max(n, m, l, P, scale_bits=16) -> float:
    s, t = min(n, m), max(n, m)
    return P * (s * (s + t) + scale_bits * l * (t + 3 * s)) / (s * t)


def rank(b, n, m, l, P, scale_bits=16) -> int:
    """Rank for a target bit-width: the page's inversion, floored so the layer
    stays within budget, clamped to [1, min(n, m)] with a warning."""
    raw = (b * n * m / P - scale_bits * l * (n + m)) / ((n + m) + 2 * scale_bits * l)
    r = math.floor(raw)
    lo, hi = 1, min(n, m)
    if r > hi or r < lo:
        warnings.warn(f"target bit-width {b} needs rank {raw:.1f}; clamped to [{lo}, {hi}]")
        r = min(max(r, lo), hi)
    return r
