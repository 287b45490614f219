"""Pins for the FABQ-RC-style oracle (README "Key Ideas", model card
"How It Works" / "Quantization Details")."""
import dataclasses

import numpy as np
import pytest

import synth
from conftest import read_golden
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


# ---- the variants: int8 rows, blocksizes 16 / 32, tiered and vector codebooks ----

def _golden(name):
    g = {k.strip(): v for k, v in (l.split("=", 1) for l in read_golden("fabq_variants.txt"))}
    return [float(v) for v in g[name].split()]


def _fp16(v):
    return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def _layer(rows, cols, bs, n_hi, row_of, q, s_hi, signs, s_blk, idx, hi_bits=4, cb_mode=0,
           cb_base=0, codebook=None, tier=None, vcodebook=None):
    return synth.FabqInput(rows=rows, cols=cols, blocksize=bs, row_of=np.asarray(row_of, np.int32),
                           n_hi=n_hi, q4=np.asarray(q, np.int8).reshape(n_hi, cols),
                           s_hi=_fp16(s_hi), signs=np.asarray(signs, np.uint8),
                           s_blk=_fp16(s_blk), idx=np.asarray(idx, np.uint8),
                           codebook=np.zeros(16, np.uint16) if codebook is None else codebook,
                           seed=0, hi_bits=hi_bits, cb_mode=cb_mode, cb_base=cb_base,
                           tier=None if tier is None else np.asarray(tier, np.uint8),
                           vcodebook=vcodebook)


def test_golden_vector_codebook_int8_bs16():
    """Case A of tests/golden/fabq_variants.txt (hand-worked)."""
    k = np.arange(32)
    q = np.where(k < 31, k - 16, -128)
    signs = np.zeros((2, 32), np.uint8)
    signs[0, :8] = 1
    signs[0, 16:] = 1
    V = np.full((4, 64, 128), 1000.0, np.float32)
    e = np.arange(128)
    V[0, 17] = e / 1024
    V[0, 18] = 1 / 256
    V[3, 16] = -1 / 64
    V[3, 31, 16:32] = (e[16:32] - 16) / 256
    inp = _layer(3, 32, 16, 1, [2, 0, 1], q, [0.25], signs, [[0.5, 0.25], [1.0, 2.0]], [[1, 2], [0, 15]],
                 hi_bits=8, cb_mode=2, cb_base=16, tier=[0, 3], vcodebook=V)
    y = fabq.gemv(fabq.pack(inp), np.full((1, 32), 0x3F80, np.uint16), 3, 32, 16, 1)[0]
    assert np.array_equal(y, _golden("case_a_y"))


def test_golden_vector_element_is_column_mod_128():
    """Case B: a 16-wide block at columns 144-159 reads vector elements 16-31."""
    V = np.full((4, 64, 128), 1000.0, np.float32)
    V[2, 33] = np.arange(128) / 1024
    inp = _layer(1, 256, 16, 0, [0], np.zeros((0, 256)), [], np.ones((1, 256)), np.zeros((1, 16)),
                 np.ones((1, 16)), cb_mode=2, cb_base=32, tier=[2], vcodebook=V)
    p = fabq.pack(inp)
    y1 = fabq.gemv(p, np.full((1, 256), 0x3F80, np.uint16), 1, 256, 16, 0)[0]
    x = np.zeros((1, 256), np.uint16)
    x[0, 150] = 0x3F80
    y2 = fabq.gemv(p, x, 1, 256, 16, 0)[0]
    assert y1[0] == _golden("case_b_y_ones")[0] and y2[0] == _golden("case_b_y_onehot150")[0]


def test_golden_tiered_scalar_bs32():
    """Case C: the row's tier picks the codebook, cb_base + idx the centroid."""
    C = np.full((4, 64), 1000.0)
    C[1, 50], C[1, 63], C[2, 48] = 0.125, -0.5, 0.0625
    signs = np.stack([np.ones(64), np.zeros(64)]).astype(np.uint8)
    inp = _layer(2, 64, 32, 0, [1, 0], np.zeros((0, 64)), [], signs, [[0.5, 0.5], [0.25, 0.75]],
                 [[2, 15], [0, 0]], cb_mode=1, cb_base=48, codebook=_fp16(C), tier=[1, 2])
    y = fabq.gemv(fabq.pack(inp), np.full((1, 64), 0x3F80, np.uint16), 2, 64, 32, 0)[0]
    assert np.array_equal(y, _golden("case_c_y"))


def test_int8_decode_reproduces_constructed_weights():
    """int8 rows q * s with max|q| = 127 and s exact in fp16: the quantizer
    returns q and s, and the decode reproduces w exactly (also -128)."""
    rng = np.random.default_rng(31)
    rows, cols = 40, 512
    w = rng.standard_normal((rows, cols)) * 0.01
    imp = rng.uniform(size=rows)
    hi = np.argsort(-imp, kind="stable")[:2]
    for r in hi:
        s = rng.integers(1, 64) * 2.0 ** -14
        q = rng.integers(-127, 128, size=cols).astype(np.float64)
        q[rng.integers(0, cols)] = 127.0
        w[r] = q * s
    inp = synth.fabq_quantize(w, imp, 64, hi_bits=8)
    W = fabq.decode(fabq.pack(inp), rows, cols, 64, inp.n_hi)
    assert inp.n_hi == 2 and np.array_equal(W[hi], w[hi])
    q = np.arange(-128, 128, dtype=np.int8).reshape(1, 256)
    one = _layer(1, 256, 64, 1, [0], q, [0.5], np.zeros((0, 256)), np.zeros((0, 4)), np.zeros((0, 4)),
                 hi_bits=8)
    assert np.array_equal(fabq.decode(fabq.pack(one), 1, 256, 64, 1)[0], np.arange(-128, 128) * 0.5)


def test_int8_only_layer_closed_form():
    inp = synth.fabq_input(20, 256, seed=32, blocksize=32, hi_frac=1.0, hi_bits=8)
    assert inp.n_hi == 20 and inp.q4.min() < -8
    x = synth.activations(1, 256, seed=32)
    y = fabq.gemv(fabq.pack(inp), x, 20, 256, 32, 20)[0]
    expect = fp16_to_f64(inp.s_hi) * (inp.q4.astype(np.float64) @ bf16_to_f64(x)[0])
    assert np.allclose(y[inp.row_of], expect, rtol=1e-13, atol=0)


@pytest.mark.parametrize("bs", [16, 32])
def test_tiered_with_equal_tiers_is_the_single_codebook(bs):
    """Mode 1 whose four tiers hold the mode-0 codebook in the active window
    decodes exactly like mode 0 (the 48 other entries are never read)."""
    inp = synth.fabq_input(64, 512, seed=33, blocksize=bs)
    C = np.full((4, 64), 77.0)
    C[:, 16:32] = fp16_to_f64(inp.codebook)
    t = np.random.default_rng(1).integers(0, 4, size=64 - inp.n_hi).astype(np.uint8)
    tiered = dataclasses.replace(inp, cb_mode=1, cb_base=16, codebook=_fp16(C), tier=t)
    a = fabq.decode(fabq.pack(inp), 64, 512, bs, inp.n_hi)
    b = fabq.decode(fabq.pack(tiered), 64, 512, bs, inp.n_hi)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("bs", [16, 128, 512])
def test_constant_vectors_are_the_tiered_scalar_codebook(bs):
    """Mode 2 whose centroid vectors are constant (every element the mode-1
    centroid) decodes exactly like mode 1."""
    inp = synth.fabq_input(64, 1024, seed=34, blocksize=bs, cb_mode=1)
    C = fp16_to_f64(inp.codebook).reshape(4, 64)
    V = np.repeat(C[:, :, None], 128, axis=2).astype(np.float32)
    vec = dataclasses.replace(inp, cb_mode=2, vcodebook=V)
    a = fabq.decode(fabq.pack(inp), 64, 1024, bs, inp.n_hi)
    b = fabq.decode(fabq.pack(vec), 64, 1024, bs, inp.n_hi)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("mode,bs", [(1, 16), (1, 32), (2, 16), (2, 32), (0, 16)])
def test_zero_corrections_closed_form(mode, bs):
    """With every correction zero and x = 1, a binary row gives
    sum_b s_b (#pos - #neg), whatever the codebook mode."""
    inp = synth.fabq_input(64, 1024, seed=35, blocksize=bs, cb_mode=mode)
    if mode == 2:
        inp = dataclasses.replace(inp, vcodebook=np.zeros((4, 64, 128), np.float32))
    else:
        inp = dataclasses.replace(inp, codebook=np.zeros_like(inp.codebook))
    ones = np.full((1, 1024), 0x3F80, np.uint16)
    y = fabq.gemv(fabq.pack(inp), ones, 64, 1024, bs, inp.n_hi)[0]
    nb = 1024 // bs
    npos = inp.signs.reshape(-1, nb, bs).astype(np.int64).sum(axis=2)
    expect = (fp16_to_f64(inp.s_blk) * (2 * npos - bs)).sum(axis=1)
    assert np.allclose(y[inp.row_of[inp.n_hi:]], expect, rtol=1e-13, atol=0)


@pytest.mark.parametrize("hi_bits,mode,bs", [(8, 0, 64), (4, 1, 16), (8, 2, 32), (4, 2, 128), (8, 1, 512)])
def test_variants_brute_force_from_bytes(hi_bits, mode, bs):
    """Element-by-element decode read straight from the packed bytes, with
    the tier, window and vector lookups written out per weight."""
    rows, cols = 40, 1024
    inp = synth.fabq_input(rows, cols, seed=36 + bs, blocksize=bs, hi_bits=hi_bits, cb_mode=mode,
                           hi_frac=0.1)
    p = fabq.pack(inp)
    W = fabq.decode(p, rows, cols, bs, inp.n_hi)

    def field(row_bytes, k, b):
        v = 0
        for j in range(b):
            i = b * k + j
            v |= ((int(row_bytes[i >> 3]) >> (i & 7)) & 1) << j
        return v

    code16 = [float(v) for v in np.asarray(inp.codebook, np.uint16).view(np.float16).ravel()]
    for i in range(rows):
        r = int(p["row_of"][i])
        for k in range(3, cols, 37):
            if i < inp.n_hi:
                q = field(p["q4"][i], k, hi_bits)
                q = q - (1 << hi_bits) if q >= 1 << (hi_bits - 1) else q
                expect = q * float(fp16_to_f64(p["s_hi"][i]))
            else:
                j = i - inp.n_hi
                sgn = 1.0 if field(p["signs"][j], k, 1) else -1.0
                blk = k // bs
                c = field(p["idx"][j], blk, 4)
                if mode == 0:
                    corr = code16[c]
                elif mode == 1:
                    corr = code16[64 * int(inp.tier[j]) + inp.cb_base + c]
                else:
                    corr = float(inp.vcodebook[int(inp.tier[j]), inp.cb_base + c, k % 128])
                expect = float(fp16_to_f64(p["s_blk"][j, blk])) * sgn + corr
            assert W[r, k] == expect, (i, k)


def test_tiers_are_importance_quartiles():
    inp = synth.fabq_input(400, 256, seed=37, blocksize=64, cb_mode=1)
    counts = np.bincount(inp.tier, minlength=4)
    assert counts.min() >= len(inp.tier) // 4 and counts.max() <= len(inp.tier) // 4 + 1


def test_bpw_variant_values():
    """Worked by hand for 5120 x 5120, 256 high rows, block 512 (10 blocks):
    int8 rows 256*5120*8 + 256*16; binary 4864*5120 + 4864*10*20;
    codebooks 16*16 (scalar), 4*64*16 (tiered), 4*64*128*32 = 128 KB (vector);
    tier bytes 4864*8 in the tiered modes; row map 5120*32."""
    base = 256 * 5120 * 8 + 256 * 16 + 4864 * 5120 + 4864 * 10 * 20 + 5120 * 32
    n = 5120 * 5120
    assert fabq.bpw(5120, 5120, 512, 256, hi_bits=8) == (base + 256) / n
    assert fabq.bpw(5120, 5120, 512, 256, hi_bits=8, cb_mode=1) == (base + 4096 + 4864 * 8) / n
    assert fabq.bpw(5120, 5120, 512, 256, hi_bits=8, cb_mode=2) == (base + 131072 * 8 + 4864 * 8) / n
