"""Pins for the per-row LUT 4-bit oracle (the 8-tier row of "Qwen3.8-27B -
BenQ 6-bit", "Why equal-width shells", read as the 6-bit format is)."""
import numpy as np
import pytest
import torch

import synth
from oracle import bits, lut4
from oracle.numerics import bf16_to_f64


def test_pack_hand_bytes_and_roundtrip():
    # field k at stream bits [4k, 4k + 4), least significant first: two codes per byte, low nibble first
    p = lut4.pack_codes(np.array([[1, 2, 3, 4, 15, 0]], dtype=np.uint8))
    assert p[0].tobytes() == bytes([0x21, 0x43, 0x0F])
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 16, size=(29, 320), dtype=np.uint8)
    p = lut4.pack_codes(codes)
    assert p.shape == (29, 160)
    assert np.array_equal(lut4.unpack_codes(p, 320), codes)
    p2 = lut4.pack_codes(codes, ld=176)
    assert np.all(p2[:, 160:] == 0) and np.array_equal(lut4.unpack_codes(p2, 320), codes)
    assert np.array_equal(bits.unpack(p, 320, 4), codes)


def test_decode_is_the_library_gather():
    inp = synth.lut4_input(64, 512, seed=2)
    W = lut4.decode(inp.codes, inp.lut)
    lut_t = torch.from_numpy(inp.lut.view(np.int16).copy()).view(torch.bfloat16)
    Wt = lut_t.gather(1, torch.from_numpy(inp.codes.astype(np.int64)))
    assert np.array_equal(W, Wt.to(torch.float64).numpy())


def test_generator_tables_and_nearest_codes():
    inp = synth.lut4_input(64, 512, seed=3)
    lv = bf16_to_f64(inp.lut)
    assert lv.shape == (64, 16) and inp.codes.max() <= 15
    assert np.all(np.diff(lv, axis=1) > 0)                    # ascending
    assert np.all(lv[:, :8] < 0) and np.all(lv[:, 8:] > 0)    # 8 negative, then 8 positive
    assert np.array_equal(lv[:, ::-1], -lv)                   # code c and 15 - c mirror
    # regenerate the weights: every code is the nearest level (ties to the lower index)
    rng = np.random.default_rng([3, 4])
    sigma = np.exp(rng.uniform(np.log(0.005), np.log(0.05), size=64))
    w = rng.standard_normal((64, 512)) * sigma[:, None]
    d = np.abs(w[:, :, None] - lv[:, None, :])
    assert np.array_equal(inp.codes, np.argmin(d, axis=2))
    # top level = bf16(15/16 max|w|)
    top = (7.5 / 8.0) * np.abs(w).max(axis=1)
    assert np.all(np.abs(lv[:, 15] - top) <= top * 2.0 ** -8)


def test_gemv_brute_force():
    rng = np.random.default_rng(6)
    rows, cols = 5, 48
    codes = rng.integers(0, 16, size=(rows, cols), dtype=np.uint8)
    lut = synth.bf16_bits_from_f64(np.sort(rng.standard_normal((rows, 16)), axis=1))
    x = synth.activations(2, cols, 6)
    y = lut4.gemv(lut4.pack_codes(codes), lut, x, cols)
    lv, xv = bf16_to_f64(lut), bf16_to_f64(x)
    for b in range(2):
        for r in range(rows):
            s = 0.0
            for k in range(cols):
                s += float(lv[r, codes[r, k]]) * float(xv[b, k])
            assert abs(y[b, r] - s) <= 1e-12 * max(1.0, abs(s))


def test_gemv_one_hot_constant_and_mirror():
    inp = synth.lut4_input(32, 256, seed=4)
    p = lut4.pack_codes(inp.codes)
    W = lut4.decode(inp.codes, inp.lut)
    # one-hot x picks a column of W exactly
    for k in (0, 77, 255):
        e = np.zeros((1, 256), dtype=np.uint16)
        e[0, k] = 0x3F80  # bf16 1.0
        assert np.array_equal(lut4.gemv(p, inp.lut, e, 256)[0], W[:, k])
    # every code c: y[r] = lut[r][c] * sum(x)
    x = synth.activations(1, 256, 4)
    sx = bf16_to_f64(x).sum()
    for c in (0, 7, 8, 15):
        pc = lut4.pack_codes(np.full((32, 256), c, dtype=np.uint8))
        y = lut4.gemv(pc, inp.lut, x, 256)[0]
        assert np.allclose(y, bf16_to_f64(inp.lut)[:, c] * sx, rtol=1e-12, atol=0)
    # mirrored codes on mirror-symmetric tables negate y exactly
    y = lut4.gemv(p, inp.lut, x, 256)
    ym = lut4.gemv(lut4.pack_codes(15 - inp.codes), inp.lut, x, 256)
    assert np.array_equal(ym, -y)


def test_bits_per_weight_counts_the_stored_bytes():
    """bpw times the weight count is exactly the bits of what is stored: the
    packed code array the oracle's own packer writes (two codes per byte, no
    padding at these widths) plus the bf16 tables."""
    for rows, cols in ((3, 64), (17, 1024), (5, 5120), (2, 17408)):
        inp = synth.lut4_input(rows, cols, seed=cols)
        packed = lut4.pack_codes(inp.codes)
        stored_bits = 8 * (packed.nbytes + inp.lut.nbytes)
        assert lut4.bpw(cols) * rows * cols == stored_bits
    assert lut4.bpw(256) == 5.0  # 4 code bits + 256 table bits over 256 columns


@pytest.mark.parametrize("jitter", [0.1, 0.3])
def test_jittered_tables_sorted_not_mirror_and_codes_nearest(jitter):
    """Tables with every level moved on its own stay sorted with 8 negative
    then 8 positive entries but are not mirror-symmetric; the shell shortcut
    still picks the nearest level."""
    a = synth.lut4_input(128, 512, seed=9, level_jitter=jitter)
    b = synth.lut4_input(128, 512, seed=9, level_jitter=jitter, exact_argmin=True)
    lv = bf16_to_f64(a.lut)
    assert np.all(np.diff(lv, axis=1) > 0)
    assert np.all(lv[:, :8] < 0) and np.all(lv[:, 8:] > 0)
    assert np.all(np.any(lv[:, ::-1] != -lv, axis=1))  # no row is a mirror image
    assert np.mean(lv[:, ::-1] != -lv) > 0.5
    assert np.array_equal(a.codes, b.codes)


def test_generator_shell_shortcut_equals_full_argmin():
    a = synth.lut4_input(256, 1024, seed=5)
    b = synth.lut4_input(256, 1024, seed=5, exact_argmin=True)
    assert np.array_equal(a.codes, b.codes)
