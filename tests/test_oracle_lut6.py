"""Pins for the per-row LUT 6-bit oracle ("Qwen3.8-27B - BenQ 6-bit")."""
import numpy as np
import pytest
import torch

import oracle
import synth
from conftest import read_golden
from oracle import bits, lut6
from oracle.numerics import bf16_to_f64


def _golden_rows(b_want):
    out = []
    for line in read_golden("bitfields.txt"):
        b, vals, by = [s.strip() for s in line.split(";")]
        if int(b) == b_want:
            out.append(([int(t) for t in vals.split()], bytes.fromhex(by.replace(" ", ""))))
    return out


@pytest.mark.parametrize("b", [6, 1, 4])
def test_pack_hand_bytes(b):
    for vals, expect in _golden_rows(b):
        got = bits.pack(np.array([vals]), b)[0].tobytes()
        assert got == expect, (vals, got.hex(), expect.hex())
        back = bits.unpack(np.frombuffer(expect, np.uint8)[None], len(vals), b)[0]
        if b == 4:
            back = bits.to_signed(back, 4)
        assert list(back) == vals


def test_pack_roundtrip_and_size():
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 64, size=(37, 320), dtype=np.uint8)
    p = lut6.pack_codes(codes)
    assert p.shape == (37, 240)  # 4 codes per 3 bytes
    assert np.array_equal(lut6.unpack_codes(p, 320), codes)
    p2 = lut6.pack_codes(codes, ld=256)
    assert np.all(p2[:, 240:] == 0)
    assert np.array_equal(lut6.unpack_codes(p2, 320), codes)


def test_decode_is_the_library_gather():
    """The card defines decode as the row-wise gather of codes into the tables."""
    inp = synth.lut6_input(256, 512, seed=1)
    W = lut6.decode(inp.codes, inp.lut)
    lut_t = torch.from_numpy(inp.lut.view(np.int16).copy()).view(torch.bfloat16)
    Wt = lut_t.gather(1, torch.from_numpy(inp.codes.astype(np.int64)))
    assert np.array_equal(W, Wt.to(torch.float64).numpy())


def test_generator_table_invariants():
    inp = synth.lut6_input(256, 512, seed=1)
    lv = bf16_to_f64(inp.lut)
    assert np.all(np.diff(lv, axis=1) > 0)                       # ascending by value
    assert np.all(lv[:, :32] < 0) and np.all(lv[:, 32:] > 0)      # 32 negative, then 32 positive
    assert np.array_equal(lv[:, ::-1], -lv)                       # code c and 63-c are mirror levels
    # regenerate the weights to check the top level = bf16(63/64 * max|w|)
    rng = np.random.default_rng(1)
    sigma = np.exp(rng.uniform(np.log(0.005), np.log(0.05), size=256))
    w = rng.standard_normal((256, 512)) * sigma[:, None]
    top = np.abs(w).max(1) * 63 / 64
    assert np.allclose(lv[:, 63], top, rtol=2 ** -8)
    # equal-width shells put most weights in the inner tiers
    tier = np.where(inp.codes >= 32, inp.codes - 32, 31 - inp.codes.astype(int))
    hist = np.bincount(tier.ravel(), minlength=32)
    assert hist[:8].sum() > hist[8:].sum()
    assert hist[17:].sum() / hist.sum() < 0.1


def test_generator_shell_shortcut_equals_full_argmin():
    a = synth.lut6_input(256, 512, seed=1)
    b = synth.lut6_input(256, 512, seed=1, exact_argmin=True)
    assert np.array_equal(a.codes, b.codes)


def _brute_gemv(packed, lut_bits, x_bits, rows, cols):
    """Pure-Python loops, reading each code straight from the bytes."""
    lut = bf16_to_f64(lut_bits)
    x = bf16_to_f64(x_bits)
    y = [[0.0] * rows for _ in range(x.shape[0])]
    for r in range(rows):
        row = packed[r]
        for k in range(cols):
            bit0 = 6 * k
            v = 0
            for j in range(6):
                i = bit0 + j
                v |= ((int(row[i >> 3]) >> (i & 7)) & 1) << j
            w = float(lut[r, v])
            for b in range(x.shape[0]):
                y[b][r] += w * float(x[b, k])
    return np.array(y)


def test_gemv_brute_force_tiny():
    inp = synth.lut6_input(24, 64, seed=11)
    x = synth.activations(2, 64, seed=11)
    p = lut6.pack_codes(inp.codes)
    y = lut6.gemv(p, inp.lut, x, 64)
    yb = _brute_gemv(p, inp.lut, x, 24, 64)
    assert np.allclose(y, yb, rtol=1e-12, atol=1e-15)


def test_gemv_c1_against_pure_python():
    inp = synth.lut6_input(256, 512, seed=1)
    x = synth.activations(1, 512, seed=1)
    p = lut6.pack_codes(inp.codes)
    y = lut6.gemv(p, inp.lut, x, 512)
    yb = _brute_gemv(p[:32], inp.lut[:32], x, 32, 512)  # first 32 rows keep it fast
    assert np.max(np.abs(y[:, :32] - yb) / np.abs(yb).max()) < 1e-12


def test_gemv_one_hot_mirror_scaling_linearity():
    inp = synth.lut6_input(40, 128, seed=12)
    p = lut6.pack_codes(inp.codes)
    lv = bf16_to_f64(inp.lut)
    # one-hot x picks one column of the decoded matrix exactly
    for k in (0, 5, 127):
        x = np.zeros((1, 128), np.uint16)
        x[0, k] = 0x3F80  # bf16 1.0
        y = lut6.gemv(p, inp.lut, x, 128)[0]
        assert np.array_equal(y, lv[np.arange(40), inp.codes[:, k]])
    x = synth.activations(3, 128, seed=12)
    y = lut6.gemv(p, inp.lut, x, 128)
    # mirrored codes on a mirror-symmetric table negate y exactly
    pm = lut6.pack_codes(63 - inp.codes)
    assert np.array_equal(lut6.gemv(pm, inp.lut, x, 128), -y)
    # power-of-two scaling of x is exact (bf16 bits: add 2 to the exponent)
    x4 = (x.astype(np.uint32) + (2 << 7)).astype(np.uint16)
    x4[(x & 0x7FFF) == 0] = x[(x & 0x7FFF) == 0]
    assert np.array_equal(lut6.gemv(p, inp.lut, x4, 128), 4 * y)
    # linearity in the batch dimension
    assert np.allclose(lut6.gemv(p, inp.lut, x[1:2], 128)[0], y[1], rtol=0, atol=0)


def test_bpw_formula_and_page_table():
    g = dict(l.replace(" ", "").split("=") for l in read_golden("lut6_bpw.txt"))
    for cols in (512, 5120, 17408):
        inp_rows = 8
        packed_bytes = inp_rows * cols * 3 // 4
        lut_bytes = inp_rows * 64 * 2
        assert (packed_bytes + lut_bytes) * 8 / (inp_rows * cols) == lut6.bpw(cols)
    assert lut6.bpw(512) == 8.0
    lo, hi = lut6.bpw(int(g["cols_max"])), lut6.bpw(int(g["cols_min"]))
    assert lo < float(g["total_bits"]) < hi
    assert float(g["code_bits"]) + float(g["lut_bits"]) == pytest.approx(float(g["total_bits"]), abs=0.005)
    assert lo - 6 < float(g["lut_bits"]) < hi - 6


def test_bpw_counts_the_stored_bytes():
    """bpw times the weight count equals the bits of the arrays actually
    stored: the oracle packer's code bytes (4 codes per 3 bytes, unpadded)
    plus the 64-entry bf16 tables."""
    for rows, cols in ((3, 64), (8, 512), (2, 5120), (2, 17408)):
        inp = synth.lut6_input(rows, cols, seed=cols)
        packed = lut6.pack_codes(inp.codes)
        assert lut6.bpw(cols) * rows * cols == 8 * (packed.nbytes + inp.lut.nbytes)


@pytest.mark.parametrize("jitter", [0.1, 0.3])
def test_jittered_tables_sorted_not_mirror_and_codes_nearest(jitter):
    """Every level moved on its own (a stand-in for a Lloyd-refined table):
    still sorted, 32 negative then 32 positive, but not mirror-symmetric, and
    the shell shortcut still returns the nearest level."""
    a = synth.lut6_input(128, 512, seed=11, level_jitter=jitter)
    b = synth.lut6_input(128, 512, seed=11, level_jitter=jitter, exact_argmin=True)
    lv = bf16_to_f64(a.lut)
    assert np.all(np.diff(lv, axis=1) > 0)
    assert np.all(lv[:, :32] < 0) and np.all(lv[:, 32:] > 0)
    assert np.all(np.any(lv[:, ::-1] != -lv, axis=1))  # no row is a mirror image
    assert np.mean(lv[:, ::-1] != -lv) > 0.5
    assert np.array_equal(a.codes, b.codes)
    # the decode does not assume symmetry: the gather returns each level as stored
    W = lut6.decode(a.codes, a.lut)
    assert np.array_equal(W, lv[np.arange(128)[:, None], a.codes])
