"""GPU parity for the FABQ-RC-style binary-core GEMV."""
import dataclasses
import functools

import numpy as np
import pytest
import torch

import dequant_matmul_amd as fqm
import oracle
import synth
from gpu_common import DEV, assert_close, bf16_dev, canaries_intact, guarded, to_f64

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=None)
def case(rows, cols, seed, bs):
    inp = synth.fabq_input(rows, cols, seed, blocksize=bs)
    return inp, oracle.fabq.pack(inp)


def weights(inp):
    return fqm.FabqWeights.from_arrays(inp.rows, inp.cols, inp.blocksize, inp.n_hi, inp.row_of,
                                       inp.q4, inp.s_hi, inp.signs, inp.s_blk, inp.idx,
                                       inp.codebook, device=DEV)


@pytest.mark.parametrize("bs", [64, 128, 256, 512])
def test_dequant_is_bit_exact(bs):
    inp, p = case(5120, 5120, 5, bs)
    W = fqm.dequant(weights(inp)).view(torch.int16).cpu().numpy().view(np.uint16)
    ref = oracle.numerics.bf16_bits_from_f64_rne(oracle.fabq.decode(p, 5120, 5120, bs, inp.n_hi))
    assert np.array_equal(W, ref)


@pytest.mark.parametrize("bs", [64, 128, 256, 512])
@pytest.mark.parametrize("batch", [1, 8])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_gemv_layer(bs, batch, out):
    inp, p = case(5120, 5120, 5, bs)
    x = synth.activations(batch, 5120, 5)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    buf, y = guarded((batch, 5120), dt)
    fqm.gemv(weights(inp), bf16_dev(x), y=y)
    torch.cuda.synchronize()
    assert canaries_intact(buf)
    assert_close(to_f64(y), oracle.fabq.gemv(p, x, 5120, 5120, bs, inp.n_hi), out, f"bs{bs} b{batch}")


@pytest.mark.parametrize("batch", [1, 3, 4, 16])
def test_gemv_ragged_rows(batch):
    inp, p = case(101, 1536, 51, 256)
    x = synth.activations(batch, 1536, 51)
    y = fqm.gemv(weights(inp), bf16_dev(x), out_dtype=torch.float32)
    assert_close(to_f64(y), oracle.fabq.gemv(p, x, 101, 1536, 256, inp.n_hi), "f32")


@pytest.mark.parametrize("batch", [1, 2, 5])
def test_all_int4_and_all_binary_layers(batch):
    """Batches 1 and 2 take the VALU kernel (batch 1 with its grouped loads),
    batch 5 the matrix-core one (row blocks of one kind only; a layer without
    binary rows has no block scales, indices or codebook to read)."""
    for frac in (1.0, 0.0):
        inp = synth.fabq_input(64, 1024, 52, blocksize=64, hi_frac=frac)
        p = oracle.fabq.pack(inp)
        x = synth.activations(batch, 1024, 52)
        y = fqm.gemv(weights(inp), bf16_dev(x), out_dtype=torch.float32)
        assert_close(to_f64(y), oracle.fabq.gemv(p, x, 64, 1024, 64, inp.n_hi), "f32", f"hi={frac}")


def _full_nibble_range(rows, cols, seed, bs, hi_frac):
    """A layer whose int4 rows hold every value -8..7.  The quantizer's
    max|w|/7 scale never produces -8 (nibble 0x8), so the int4 values are
    drawn directly; the binary rows come from the generator."""
    base = synth.fabq_input(rows, cols, seed, blocksize=bs, hi_frac=hi_frac)
    rng = np.random.default_rng(seed + 1)
    q4 = rng.integers(-8, 8, size=base.q4.shape).astype(np.int8)
    q4[:, :16] = np.arange(-8, 8, dtype=np.int8)
    q4[:, -8:] = -8
    inp = dataclasses.replace(base, q4=q4)
    p = oracle.fabq.pack(inp)
    assert (p["q4"] & 0x0F == 0x08).any() and (p["q4"] >> 4 == 0x08).any()
    return inp, p


@pytest.mark.parametrize("hi_frac", [0.25, 1.0])
def test_int4_minus_eight_dequant_bit_exact(hi_frac):
    inp, p = _full_nibble_range(96, 1024, 53, 128, hi_frac)
    W = fqm.dequant(weights(inp)).view(torch.int16).cpu().numpy().view(np.uint16)
    ref = oracle.numerics.bf16_bits_from_f64_rne(oracle.fabq.decode(p, 96, 1024, 128, inp.n_hi))
    assert np.array_equal(W, ref)


@pytest.mark.parametrize("hi_frac", [0.25, 1.0])
@pytest.mark.parametrize("batch", [1, 2, 4, 8])
def test_int4_minus_eight_gemv(hi_frac, batch):
    """Batches 1-3 on the VALU kernel, 4 and up on the matrix cores; int4 rows
    with -8 in every position of a nibble pair."""
    inp, p = _full_nibble_range(96, 1024, 53, 128, hi_frac)
    x = synth.activations(batch, 1024, 55)
    buf, y = guarded((batch, 96), torch.float32)
    fqm.gemv(weights(inp), bf16_dev(x), y=y)
    torch.cuda.synchronize()
    assert canaries_intact(buf)
    assert_close(to_f64(y), oracle.fabq.gemv(p, x, 96, 1024, 128, inp.n_hi), "f32",
                 f"hi={hi_frac} b{batch}")
