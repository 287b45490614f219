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
                                       inp.codebook, device=DEV, hi_bits=inp.hi_bits,
                                       cb_mode=inp.cb_mode, cb_base=inp.cb_base, tier=inp.tier,
                                       vcodebook=inp.vcodebook)


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


@pytest.mark.parametrize("batch", [1, 5])
def test_vector_centroids_all_int4_and_all_binary_layers(batch):
    """Vector centroids: a layer without binary rows needs no fold and no
    workspace (nothing reads the centroid terms); an all-binary layer folds
    every block.  Batch 1 on the VALU kernel, 5 on the matrix-core one."""
    for frac in (1.0, 0.0):
        inp = synth.fabq_input(64, 1024, 53, blocksize=128, hi_frac=frac, cb_mode=2)
        p = oracle.fabq.pack(inp)
        w = weights(inp)
        assert (fqm.workspace_size(w, batch) == 0) == (frac == 1.0)
        x = synth.activations(batch, 1024, 53)
        y = fqm.gemv(w, bf16_dev(x), out_dtype=torch.float32)
        assert_close(to_f64(y), oracle.fabq.gemv(p, x, 64, 1024, 128, inp.n_hi), "f32", f"vector hi={frac}")


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


# ---- the variants: int8 high rows (README), blocks of 16 and 32 columns
# (README's sweep), tiered codebooks of 4 x 64 centroids with 16 active per
# layer and 128-float vector centroids (model card "Residual Codebook
# Architecture").  Batches 1-3 run the VALU kernel; batch >= 4 the
# matrix-core kernel except for 16-column blocks.  Vector centroids first
# fold x into per-block terms (a second launch, workspace).
VARIANTS = [  # (hi_bits, cb_mode, blocksize)
    (8, 0, 64), (4, 0, 16), (4, 0, 32), (4, 1, 128), (8, 1, 32), (4, 1, 16),
    (4, 2, 128), (8, 2, 16), (4, 2, 512), (8, 2, 32)]


@functools.lru_cache(maxsize=None)
def variant(rows, cols, seed, hi_bits, cb_mode, bs, hi_frac=0.05):
    inp = synth.fabq_input(rows, cols, seed, blocksize=bs, hi_bits=hi_bits, cb_mode=cb_mode,
                           hi_frac=hi_frac)
    return inp, oracle.fabq.pack(inp)


@pytest.mark.parametrize("hi_bits,cb_mode,bs", VARIANTS)
def test_variant_dequant_bit_exact(hi_bits, cb_mode, bs):
    inp, p = variant(301, 1536, 61, hi_bits, cb_mode, bs, 0.1)
    W = fqm.dequant(weights(inp)).view(torch.int16).cpu().numpy().view(np.uint16)
    ref = oracle.numerics.bf16_bits_from_f64_rne(oracle.fabq.decode(p, 301, 1536, bs, inp.n_hi))
    assert np.array_equal(W, ref)


@pytest.mark.parametrize("hi_bits,cb_mode,bs", VARIANTS)
@pytest.mark.parametrize("batch", [1, 3, 4, 16])
def test_variant_gemv_ragged(hi_bits, cb_mode, bs, batch):
    """301 rows (a partial 16-row block, a mixed block of high and binary
    rows), 1536 columns."""
    inp, p = variant(301, 1536, 61, hi_bits, cb_mode, bs, 0.1)
    x = synth.activations(batch, 1536, 62)
    buf, y = guarded((batch, 301), torch.float32)
    print(f"fabq variant hi{hi_bits} cb{cb_mode} bs{bs} batch {batch}", flush=True)
    fqm.gemv(weights(inp), bf16_dev(x), y=y)
    torch.cuda.synchronize()
    assert canaries_intact(buf)
    assert_close(to_f64(y), oracle.fabq.gemv(p, x, 301, 1536, bs, inp.n_hi), "f32",
                 f"hi{hi_bits} cb{cb_mode} bs{bs} b{batch}")


@pytest.mark.parametrize("hi_bits,cb_mode,bs", [(8, 1, 32), (4, 2, 512), (8, 0, 16), (4, 1, 64)])
@pytest.mark.parametrize("batch", [1, 8])
def test_variant_full_layer(hi_bits, cb_mode, bs, batch):
    """The 5120 x 5120 layer of the benchmark (256 high rows) in each variant."""
    inp, p = variant(5120, 5120, 5, hi_bits, cb_mode, bs)
    x = synth.activations(batch, 5120, 5)
    print(f"fabq layer hi{hi_bits} cb{cb_mode} bs{bs} batch {batch}", flush=True)
    y = fqm.gemv(weights(inp), bf16_dev(x))
    assert_close(to_f64(y), oracle.fabq.gemv(p, x, 5120, 5120, bs, inp.n_hi), "bf16",
                 f"hi{hi_bits} cb{cb_mode} bs{bs} b{batch}")


def test_variant_invariants():
    """One-hot x returns a decoded column (fp32 out, exact up to the order of
    two additions); the same call twice gives the same bits."""
    inp, p = variant(301, 1536, 61, 8, 2, 16, 0.1)
    w = weights(inp)
    W = oracle.fabq.decode(p, 301, 1536, 16, inp.n_hi)
    for k in (0, 150, 1535):
        x = np.zeros((1, 1536), np.uint16)
        x[0, k] = 0x3F80
        y = to_f64(fqm.gemv(w, bf16_dev(x), out_dtype=torch.float32))[0]
        assert np.allclose(y, W[:, k], rtol=2 ** -22, atol=0), k
    x = bf16_dev(synth.activations(5, 1536, 63))
    assert torch.equal(fqm.gemv(w, x, out_dtype=torch.float32), fqm.gemv(w, x, out_dtype=torch.float32))


@pytest.mark.parametrize("hi_bits,cb_mode", [(4, 0), (8, 1), (4, 2)])
@pytest.mark.parametrize("batch", [1, 3, 8])
def test_blocks_of_16_with_a_half_sign_dword(hi_bits, cb_mode, batch):
    """16-column blocks on 1040 columns (65 blocks): each binary row's last
    sign dword holds one block, its other half lies past the row.  x goes
    through the L1 here (1040 is not a multiple of 32); dequantisation too."""
    rows, cols, bs = 77, 1040, 16
    inp, p = variant(rows, cols, 63, hi_bits, cb_mode, bs, 0.1)
    x = synth.activations(batch, cols, 64)
    buf, y = guarded((batch, rows), torch.float32)
    print(f"fabq 1040 cols hi{hi_bits} cb{cb_mode} batch {batch}", flush=True)
    w = weights(inp)
    fqm.gemv(w, bf16_dev(x), y=y)
    torch.cuda.synchronize()
    assert canaries_intact(buf)
    assert_close(to_f64(y), oracle.fabq.gemv(p, x, rows, cols, bs, inp.n_hi), "f32",
                 f"1040 hi{hi_bits} cb{cb_mode} b{batch}")
    if batch == 1:
        W = fqm.dequant(w).view(torch.int16).cpu().numpy().view(np.uint16)
        ref = oracle.numerics.bf16_bits_from_f64_rne(oracle.fabq.decode(p, rows, cols, bs, inp.n_hi))
        assert np.array_equal(W, ref)


@pytest.mark.parametrize("batch", [1, 8])
def test_vector_centroids_graph_replays_match_eager(batch):
    """Vector centroids run two kernels per call (the fold into the workspace,
    then the GEMV).  Captured in a HIP graph and replayed with new x, with
    eager work in between, every replay gives the eager result bit for bit."""
    inp, p = variant(5120, 5120, 5, 4, 2, 512)
    w = weights(inp)
    xs = [bf16_dev(synth.activations(batch, 5120, 70 + i)) for i in range(3)]
    x = xs[0].clone()
    need = fqm.workspace_size(w, batch)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    y = torch.empty((batch, 5120), dtype=torch.float32, device=DEV)
    fqm.gemv(w, x, y=y, workspace=ws)  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fqm.gemv(w, x, y=y, workspace=ws)
    for xi in xs:
        x.copy_(xi)
        g.replay()
        torch.cuda.synchronize()
        got = y.clone()
        eager = fqm.gemv(w, xi, out_dtype=torch.float32)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(got, eager)
