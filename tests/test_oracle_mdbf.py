"""Pins for the MDBF oracle (OneCompression "MDBF")."""
import warnings

import numpy as np
import pytest

import synth
from conftest import read_golden
from oracle import mdbf
from oracle.numerics import fp16_to_f64


@pytest.mark.parametrize("l,P", [(1, 1), (2, 1), (1, 2), (4, 2)])
def test_dense_and_factored_routes_agree(l, P):
    inp = synth.mdbf_input(48, 40, 24, l, P, seed=31)
    paths = mdbf.pack(inp)
    x = synth.activations(3, 40, seed=31)
    y1 = mdbf.gemv_dense(paths, x, 48, 40, 24)
    y2 = mdbf.gemv_factored(paths, x, 48, 40, 24)
    assert np.allclose(y1, y2, rtol=1e-12, atol=1e-18)


def test_dbf_reduction():
    """(l, P) = (1, 1) is DBF: W = A diag(d) B with A = diag(a) S_A,
    d = q_U * q_V and B = S_B diag(b)."""
    inp = synth.mdbf_input(30, 26, 12, 1, 1, seed=32)
    W = mdbf.dense_weight(mdbf.pack(inp), 30, 26, 12)
    SA = np.where(inp.S_A[0] == 1, 1.0, -1.0)
    SB = np.where(inp.S_B[0] == 1, 1.0, -1.0)
    a = fp16_to_f64(inp.A_amp[0])[:, 0]
    b = fp16_to_f64(inp.B_amp[0])[:, 0]
    d = fp16_to_f64(inp.Q_U[0])[:, 0] * fp16_to_f64(inp.Q_V[0])[:, 0]
    A = a[:, None] * SA
    B = SB * b[None, :]
    assert np.allclose(W, A @ np.diag(d) @ B, rtol=1e-13, atol=1e-20)


def test_littlebit_is_two_dbf_paths():
    inp = synth.mdbf_input(30, 26, 12, 1, 2, seed=33)
    paths = mdbf.pack(inp)
    W = mdbf.dense_weight(paths, 30, 26, 12)
    W1 = mdbf.dense_weight(paths[:1], 30, 26, 12)
    W2 = mdbf.dense_weight(paths[1:], 30, 26, 12)
    assert np.allclose(W, W1 + W2, rtol=1e-13, atol=1e-20)
    assert not np.allclose(W, W1)


def test_all_ones_signs_give_the_rank_l_envelope_product():
    inp = synth.mdbf_input(20, 18, 10, 3, 1, seed=34)
    inp.S_A[0][:] = 1
    inp.S_B[0][:] = 1
    W = mdbf.dense_weight(mdbf.pack(inp), 20, 18, 10)
    A, B = fp16_to_f64(inp.A_amp[0]), fp16_to_f64(inp.B_amp[0])
    QU, QV = fp16_to_f64(inp.Q_U[0]), fp16_to_f64(inp.Q_V[0])
    assert np.allclose(W, A @ (QU.T @ QV) @ B.T, rtol=1e-13, atol=1e-20)
    assert np.linalg.matrix_rank(W) <= 3


def test_accounting_golden_values():
    for line in read_golden("mdbf_accounting.txt"):
        lhs, rhs = line.split("=")
        f, *args = lhs.split()
        if f == "rank":
            b, n, m, l, P, sb = float(args[0]), *map(int, args[1:])
            assert mdbf.rank(b, n, m, l, P, sb) == int(rhs)
        elif f == "b_eff":
            n, m, r, l, P, sb = map(int, args)
            assert mdbf.b_eff(n, m, r, l, P, sb) == pytest.approx(float(rhs), rel=1e-15)
        elif f == "b_max":
            n, m, l, P, sb = map(int, args)
            assert mdbf.b_max(n, m, l, P, sb) == pytest.approx(float(rhs), rel=1e-15)


def test_accounting_identities():
    for (n, m, l, P) in [(4096, 4096, 2, 1), (5120, 17408, 2, 1), (300, 70, 4, 2)]:
        s = min(n, m)
        assert mdbf.b_eff(n, m, s, l, P) == pytest.approx(mdbf.b_max(n, m, l, P), rel=1e-14)
        for b in (0.5, 1.0, 1.3):
            if not (mdbf.b_eff(n, m, 1, l, P) <= b < mdbf.b_max(n, m, l, P)):
                continue  # outside the reachable range the rank is clamped
            r = mdbf.rank(b, n, m, l, P)
            if r < s:
                assert mdbf.b_eff(n, m, r, l, P) <= b < mdbf.b_eff(n, m, r + 1, l, P)
    with warnings.catch_warnings(record=True) as rec:
        warnings.simplefilter("always")
        assert mdbf.rank(3.0, 5120, 17408, 2, 1) == 5120   # above b_max: clamped, warned
        assert rec


def test_b_eff_counts_the_stored_bits():
    """b_eff with scale_bits = 16 equals the stored bits: one bit per sign
    (unpadded) plus the fp16 envelopes A (n x l), B (m x l), Q_U and Q_V (r x l)."""
    n, m, r, l, P = 64, 48, 40, 2, 2
    inp = synth.mdbf_input(n, m, r, l, P, seed=35)
    total = 0
    for p in range(P):
        total += inp.S_A[p].size + inp.S_B[p].size
        total += 16 * (inp.A_amp[p].size + inp.B_amp[p].size + inp.Q_U[p].size + inp.Q_V[p].size)
    assert total / (n * m) == pytest.approx(mdbf.b_eff(n, m, r, l, P, 16), rel=1e-15)


def test_config_rank_is_2000():
    c = synth.CONFIGS["mdbf"]
    assert mdbf.rank(1.0, c["n"], c["m"], c["l"], c["P"]) == c["r"] == 2000
