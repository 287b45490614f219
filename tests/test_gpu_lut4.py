"""GPU parity for the per-row LUT 4-bit GEMV (16-entry tables, two codes per byte)."""
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
def case(rows, cols, seed):
    inp = synth.lut4_input(rows, cols, seed)
    return inp, oracle.lut4.pack_codes(inp.codes)


def weights(rows, cols, seed):
    inp, _ = case(rows, cols, seed)
    return fqm.Lut4Weights.from_codes(inp.codes, inp.lut, device=DEV)


@pytest.mark.parametrize("rows,cols,seed", [(130, 1024, 1), (77, 3136, 2), (5120, 5120, 3)])
def test_pack_and_dequant_are_bit_exact(rows, cols, seed):
    inp, packed = case(rows, cols, seed)
    w = weights(rows, cols, seed)
    assert np.array_equal(w.packed[:, :cols // 2].cpu().numpy(), packed)
    W = fqm.dequant(w).view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(W, inp.lut[np.arange(rows)[:, None], inp.codes])


# 1, 11 and 31 whole 1024-column cells (the cell kernel), the full layers
CELL_SHAPES = [(77, 1024, 4), (301, 11264, 5), (97, 31744, 6), (17408, 5120, 7), (5120, 17408, 8)]


@pytest.mark.parametrize("rows,cols,seed", CELL_SHAPES)
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_gemv_b1_cells(rows, cols, seed, out):
    inp, packed = case(rows, cols, seed)
    w = weights(rows, cols, seed)
    x = synth.activations(1, cols, seed)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    buf, y = guarded((1, rows), dt)
    fqm.gemv(w, bf16_dev(x), y=y)
    torch.cuda.synchronize()
    assert canaries_intact(buf)
    assert_close(to_f64(y), oracle.lut4.gemv(packed, inp.lut, x, cols), out, f"{rows}x{cols} {out}")


@pytest.mark.parametrize("batch", [1, 2, 5, 8, 16])
def test_gemv_generic_widths_and_batches(batch):
    """Widths that are not whole cells (and every batch above 1) take the
    generic kernel."""
    for rows, cols, seed in ((70, 1088, 9), (33, 4160, 10)):
        inp, packed = case(rows, cols, seed)
        w = weights(rows, cols, seed)
        x = synth.activations(batch, cols, seed)
        buf, y = guarded((batch, rows), torch.float32)
        fqm.gemv(w, bf16_dev(x), y=y)
        torch.cuda.synchronize()
        assert canaries_intact(buf)
        assert_close(to_f64(y), oracle.lut4.gemv(packed, inp.lut, x, cols), "f32", f"{rows}x{cols} b{batch}")


# Batches 2 and 3 on whole 1024-column cells (2: 1-19, 3: 1-12) take the
# one-row-per-wave kernel with every batch row's x in LDS: 4- and 10-wave
# groups, ragged last groups, the largest cell counts and the MLP layers.
@pytest.mark.parametrize("rows,cols,seed,batch", [(5, 1024, 50, 2), (77, 3072, 51, 3), (23, 9216, 52, 2),
                                                  (41, 12288, 53, 3), (11, 19456, 54, 2), (17408, 5120, 55, 2),
                                                  (5120, 17408, 56, 2)])
def test_gemv_batch_rows_kernel(rows, cols, seed, batch):
    inp = synth.lut4_input(rows, cols, seed)
    packed = oracle.lut4.pack_codes(inp.codes)
    w = fqm.Lut4Weights.from_codes(inp.codes, inp.lut, device=DEV)
    assert fqm.workspace_size(w, batch) == 0
    x = synth.activations(batch, cols, seed + 1)
    out = "f32" if rows * cols < 10_000_000 else "bf16"
    buf, y = guarded((batch, rows), torch.float32 if out == "f32" else torch.bfloat16)
    print(f"lut4 batch-{batch} rows kernel {rows}x{cols}", flush=True)
    fqm.gemv(w, bf16_dev(x), y=y)
    torch.cuda.synchronize()
    assert canaries_intact(buf)
    assert_close(to_f64(y), oracle.lut4.gemv(packed, inp.lut, x, cols), out, f"{rows}x{cols} b{batch}")


@pytest.mark.parametrize("batch", [2, 3, 8, 9, 16])
@pytest.mark.parametrize("rows,cols,seed", [(70, 1536, 13), (301, 4096, 14), (16, 512, 15)])
def test_gemv_matrix_cores(batch, rows, cols, seed):
    """cols a multiple of 512, batch 2..16: the matrix-core kernel (ragged
    16-row blocks, batch rows past the batch in an 8- or 16-row x block)."""
    inp, packed = case(rows, cols, seed)
    w = weights(rows, cols, seed)
    x = synth.activations(batch, cols, seed)
    buf, y = guarded((batch, rows), torch.float32)
    fqm.gemv(w, bf16_dev(x), y=y)
    torch.cuda.synchronize()
    assert canaries_intact(buf)
    assert_close(to_f64(y), oracle.lut4.gemv(packed, inp.lut, x, cols), "f32", f"{rows}x{cols} b{batch}")


@pytest.mark.parametrize("rows,cols,seed,batch", [(17408, 5120, 7, 8), (5120, 17408, 8, 8), (5120, 17408, 8, 16)])
def test_gemv_matrix_cores_full_layers(rows, cols, seed, batch):
    """The full layers; the down layer splits K over workgroups (fp32
    partials in the workspace, added in split order)."""
    inp, packed = case(rows, cols, seed)
    w = weights(rows, cols, seed)
    assert (fqm.workspace_size(w, batch) > 0) == (rows == 5120)  # batch 8, 16: the matrix-core kernel's K split
    x = synth.activations(batch, cols, 11)
    y = fqm.gemv(w, bf16_dev(x))
    ref = oracle.lut4.gemv(packed, inp.lut, x, cols)
    assert_close(to_f64(y), ref, "bf16", f"b{batch}")
    y2 = fqm.gemv(w, bf16_dev(x))
    assert torch.equal(y, y2)  # fixed-order sums: bitwise repeatable


def test_gemv_mirror_negates():
    """Mirror-symmetric tables: codes c -> 15 - c give -y (fp32 output; the
    kernel's fp32 sums need not negate bit for bit, so within rounding)."""
    inp, packed = case(300, 2048, 12)
    x = bf16_dev(synth.activations(1, 2048, 12))
    w = fqm.Lut4Weights.from_codes(inp.codes, inp.lut, device=DEV)
    wm = fqm.Lut4Weights.from_codes(15 - inp.codes, inp.lut, device=DEV)
    y = to_f64(fqm.gemv(w, x, out_dtype=torch.float32))
    ym = to_f64(fqm.gemv(wm, x, out_dtype=torch.float32))
    assert np.allclose(ym, -y, rtol=1e-5, atol=1e-6 * np.abs(y).max())


@pytest.mark.parametrize("M", [17, 64, 100, 300])
def test_gemm_ragged(M):
    """Prefill GEMM on the matrix cores: 64-row tiles up to 64 rows, 256-row
    tiles above; rows not a multiple of the 256-row N tile."""
    rows, cols, seed = 600, 1536, 16
    inp, packed = case(rows, cols, seed)
    w = weights(rows, cols, seed)
    X = synth.activations(M, cols, seed)
    buf, Y = guarded((M, rows), torch.bfloat16)
    fqm.gemm(w, bf16_dev(X), Y=Y)
    torch.cuda.synchronize()
    assert canaries_intact(buf)
    assert_close(to_f64(Y), oracle.lut4.gemv(packed, inp.lut, X, cols), "bf16", f"M={M}")


@pytest.mark.parametrize("M", [1, 5, 16])
def test_gemm_small_m_is_the_gemv(M):
    rows, cols, seed = 17408, 5120, 7
    w = weights(rows, cols, seed)
    X = bf16_dev(synth.activations(M, cols, 17))
    assert torch.equal(fqm.gemm(w, X), fqm.gemv(w, X))


def test_gemm_prefill_full_layer_sampled():
    """M = 2048 on the up layer (17408 x 5120), checked on 48 sampled rows of
    X against the oracle (the whole product is too slow for the oracle)."""
    rows, cols, seed = 17408, 5120, 7
    inp, packed = case(rows, cols, seed)
    w = weights(rows, cols, seed)
    X = synth.activations(2048, cols, 18)
    Y = fqm.gemm(w, bf16_dev(X))
    pick = np.random.default_rng(0).choice(2048, size=48, replace=False)
    pick[:2] = [0, 2047]
    assert_close(to_f64(Y)[pick], oracle.lut4.gemv(packed, inp.lut, X[pick], cols), "bf16", "prefill")
    assert torch.equal(Y, fqm.gemm(w, bf16_dev(X)))  # fixed-order sums: bitwise repeatable
