"""Pins for the FABQ-RC-style oracle (README "Key Ideas", model card
"How It Works" / "Quantization Details")."""
import numpy as np
import pytest

import synth
from oracle import bits, fabq
from oracle.numerics import bf16_to_f64, fp16_to_f64


def _constructed(rows, cols, bs, seed):
    """Weights the quantizer reproduces exactly: each binary block is
    mu + a*sigma with balanced signs and 0 < |mu| < a (so mean|w| = a, the
    sign of w is sigma, and the residual mean is mu); each int4 row is q*s with
    max|q| = 7.  a, mu, s are exactly representable in fp16 and sums are exact
    in fp64.  The 16 distinct mu values occur equally often, so the k-means
    start (the (i + 1/2)/16 quantiles) already sits on them."""
    rng = np.random.default_rng(seed)
    nb = cols // bs
    mus = (np.arange(16) - 8) * 2.0 ** -12
    importance = rng.uniform(size=rows)
    n_hi = int(round(0.05 * rows))
    hi = set(np.argsort(-importance, kind="stable")[:n_hi].tolist())
    w = np.empty((rows, cols))
    j = 0
    for r in range(rows):
        if r in hi:
            s = rng.integers(1, 64) * 2.0 ** -14
            q = rng.integers(-7, 8, size=cols).astype(np.float64)
            q[rng.integers(0, cols)] = 7.0
            w[r] = q * s
            continue
        for b in range(nb):
            a = rng.integers(40, 80) * 2.0 ** -10
            mu = mus[j % 16]
            j += 1
            sig = np.array([1.0] * (bs // 2) + [-1.0] * (bs // 2))
            rng.shuffle(sig)
            w[r, b * bs:(b + 1) * bs] = mu + a * sig
    assert j % 16 == 0 and j >= 32
    return w, importance


@pytest.mark.parametrize("bs", [64, 128, 256, 512])
def test_decode_reproduces_constructed_weights(bs):
    w, imp = _constructed(40, 4096, bs, seed=bs)
    inp = synth.fabq_quantize(w, imp, bs)
    p = fabq.pack(inp)
    W = fabq.decode(p, 40, 4096, bs, inp.n_hi)
    assert inp.n_hi == 2
    assert np.array_equal(W, w)


def test_zero_codebook_closed_form():
    """With c = 0 and x = 1, a binary row gives sum_b s_b (#pos - #neg)."""
    inp = synth.fabq_input(64, 1024, seed=21, blocksize=128)
    inp.codebook = np.zeros(16, np.uint16)
    p = fabq.pack(inp)
    ones = np.full((1, 1024), 0x3F80, np.uint16)
    y = fabq.gemv(p, ones, 64, 1024, 128, inp.n_hi)[0]
    s = fp16_to_f64(inp.s_blk)
    npos = inp.signs.reshape(-1, 8, 128).astype(np.int64).sum(axis=2)
    expect = (s * (2 * npos - 128)).sum(axis=1)
    assert np.allclose(y[inp.row_of[inp.n_hi:]], expect, rtol=1e-13, atol=0)


def test_int4_only_layer_closed_form():
    inp = synth.fabq_input(20, 256, seed=22, blocksize=64, hi_frac=1.0)
    assert inp.n_hi == 20
    x = synth.activations(1, 256, seed=22)
    y = fabq.gemv(fabq.pack(inp), x, 20, 256, 64, 20)[0]
    xv = bf16_to_f64(x)[0]
    expect = fp16_to_f64(inp.s_hi) * (inp.q4.astype(np.float64) @ xv)
    assert np.allclose(y[inp.row_of], expect, rtol=1e-13, atol=0)


def test_brute_force_from_bytes():
    """Element-by-element decode reading bits straight from the packed bytes."""
    rows, cols, bs = 40, 256, 64
    inp = synth.fabq_input(rows, cols, seed=23, blocksize=bs)
    p = fabq.pack(inp)
    W = fabq.decode(p, rows, cols, bs, inp.n_hi)
    cb = fp16_to_f64(inp.codebook)

    def field(row_bytes, k, b):
        v = 0
        for j in range(b):
            i = b * k + j
            v |= ((int(row_bytes[i >> 3]) >> (i & 7)) & 1) << j
        return v

    for i in range(rows):
        r = int(p["row_of"][i])
        for k in range(0, cols, 7):
            if i < inp.n_hi:
                q = field(p["q4"][i], k, 4)
                q = q - 16 if q >= 8 else q
                expect = q * float(fp16_to_f64(p["s_hi"][i]))
            else:
                j = i - inp.n_hi
                sgn = 1.0 if field(p["signs"][j], k, 1) else -1.0
                blk = k // bs
                expect = float(fp16_to_f64(p["s_blk"][j, blk])) * sgn + cb[field(p["idx"][j], blk, 4)]
            assert W[r, k] == expect


def test_one_hot_selects_a_column():
    inp = synth.fabq_input(60, 512, seed=24, blocksize=256)
    p = fabq.pack(inp)
    W = fabq.decode(p, 60, 512, 256, inp.n_hi)
    x = np.zeros((1, 512), np.uint16)
    x[0, 300] = 0x3F80
    assert np.array_equal(fabq.gemv(p, x, 60, 512, 256, inp.n_hi)[0], W[:, 300])


def test_bpw_values():
    got = [fabq.bpw(5120, 5120, bs, 256) for bs in (64, 128, 256, 512)]
    # worked by hand: (hi 4-bit + 16-bit scales, lo 1-bit + (16+4) bits per block, 16 fp16 codes, 32-bit row map)
    assert np.allclose(got, [38097152 / 26214400, 34205952 / 26214400, 32260352 / 26214400, 31287552 / 26214400], rtol=1e-15)
    # only the largest block size lands in the cards' ~1.15-1.20 band
    assert 1.15 <= got[3] <= 1.20 and got[2] > 1.20
    # the accounting equals the packed byte counts (unpadded) plus the row map
    inp = synth.fabq_input(100, 1024, seed=25, blocksize=128)
    p = fabq.pack(inp)
    nb = 1024 // 128
    nbytes = (p["q4"].nbytes + p["s_hi"].nbytes + p["signs"].nbytes + p["s_blk"].nbytes
              + (inp.rows - inp.n_hi) * nb // 2 + p["codebook"].nbytes + p["row_of"].nbytes)
    assert nbytes * 8 / (100 * 1024) == pytest.approx(fabq.bpw(100, 1024, 128, inp.n_hi), rel=1e-12)
