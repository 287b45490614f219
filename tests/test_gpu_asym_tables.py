"""GPU parity on per-row tables that are sorted but NOT mirror-symmetric.

The default generator places levels at shell centres, so its tables satisfy
lut[63 - j] = -lut[j]; a kernel that stored 32 magnitudes and applied the
sign bit would pass every test built on them.  Real tables are Lloyd-refined
("Qwen3.8-27B - BenQ 6-bit", "Reconstruction error"), and the decode is a
plain gather of the stored entry ("What BenQ stores").  Here every level is
moved on its own by up to 0.3 of a shell width, and each LUT path (6- and
4-bit: batch-1 cells, generic widths, batch 2-16 on the matrix cores with and
without the K split, the prefill GEMM with its big, small and K-split tiles,
and small-M routing) is compared with the oracle; dequantisation bit-exactly.
"""
import functools

import numpy as np
import pytest
import torch

import dequant_matmul_amd as fqm
import oracle
import synth
from gpu_common import DEV, assert_close, bf16_dev, canaries_intact, guarded, to_f64

pytestmark = pytest.mark.gpu

JITTER = 0.3
FMT = {
    6: (synth.lut6_input, fqm.Lut6Weights, oracle.lut6),
    4: (synth.lut4_input, fqm.Lut4Weights, oracle.lut4),
}


@functools.lru_cache(maxsize=None)
def case(bits, rows, cols, seed):
    gen, _, orc = FMT[bits]
    inp = gen(rows, cols, seed, level_jitter=JITTER)
    lv = oracle.numerics.bf16_to_f64(inp.lut)
    assert np.all(np.any(lv[:, ::-1] != -lv, axis=1)), "generator gave a mirror table"
    return inp, orc.pack_codes(inp.codes)


def weights(bits, rows, cols, seed):
    inp, _ = case(bits, rows, cols, seed)
    return FMT[bits][1].from_codes(inp.codes, inp.lut, device=DEV)


def reference(bits, rows, cols, seed, x):
    inp, packed = case(bits, rows, cols, seed)
    return FMT[bits][2].gemv(packed, inp.lut, x, cols)


@pytest.mark.parametrize("bits", [6, 4])
def test_dequant_bit_exact(bits):
    rows, cols, seed = 1000, 3072, 31
    inp, _ = case(bits, rows, cols, seed)
    W = fqm.dequant(weights(bits, rows, cols, seed)).view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(W, inp.lut[np.arange(rows)[:, None], inp.codes])


# (rows, cols, batch, seed): batch-1 cells (4- and 10-wave groups, the full
# layers), generic widths (1088 is not whole cells), batch 2-16 on the matrix
# cores with the K split (300 x 4096, the down layer) and without it (the up
# layer, 1088 row blocks), and batch 2 on whole cells (the one-row-per-wave
# kernel for 6-bit codes).
GEMV_CASES = [(1000, 3072, 1, 32), (5120, 17408, 1, 33), (17408, 5120, 1, 34),
              (1000, 1088, 1, 35), (1000, 1088, 3, 35), (300, 4096, 8, 36),
              (300, 4096, 16, 36), (17408, 5120, 8, 34), (5120, 17408, 8, 33), (1000, 3072, 2, 32)]


@pytest.mark.parametrize("bits", [6, 4])
@pytest.mark.parametrize("rows,cols,batch,seed", GEMV_CASES)
def test_gemv_paths(bits, rows, cols, batch, seed):
    w = weights(bits, rows, cols, seed)
    x = synth.activations(batch, cols, seed + 1)
    out = "f32" if rows * cols < 10_000_000 else "bf16"
    dt = torch.float32 if out == "f32" else torch.bfloat16
    buf, y = guarded((batch, rows), dt)
    need = fqm.workspace_size(w, batch)
    wsp = torch.empty(need, dtype=torch.uint8, device=DEV) if need else None
    print(f"asym lut{bits} gemv {rows}x{cols} batch {batch} {out} workspace {need}", flush=True)
    fqm.gemv(w, bf16_dev(x), y=y, workspace=wsp)
    torch.cuda.synchronize()
    assert canaries_intact(buf)
    assert_close(to_f64(y), reference(bits, rows, cols, seed, x), out,
                 f"lut{bits} {rows}x{cols} b{batch}")


def test_mirror_codes_do_not_negate():
    """With these tables, mirrored codes give a different product (a
    symmetry shortcut in a kernel would make them negate y)."""
    rows, cols, seed = 1000, 3072, 32
    inp, packed = case(6, rows, cols, seed)
    x = synth.activations(1, cols, 40)
    wm = fqm.Lut6Weights.from_codes(63 - inp.codes, inp.lut, device=DEV)
    ym = to_f64(fqm.gemv(wm, bf16_dev(x), out_dtype=torch.float32))
    ref_m = oracle.lut6.gemv(oracle.lut6.pack_codes(63 - inp.codes), inp.lut, x, cols)
    assert_close(ym, ref_m, "f32", "mirrored codes")
    y = reference(6, rows, cols, seed, x)
    assert np.linalg.norm(ym + y) > 1e-3 * np.linalg.norm(y)


# (rows, cols, M, seed): the 64-row tiles (M 17-64), the 256-row tiles with the
# K-split last round (520 x 1088 at M 300: six tiles, all split), and small-M
# routing to the GEMV kernels (M 8).
@pytest.mark.parametrize("bits", [6, 4])
@pytest.mark.parametrize("rows,cols,M,seed", [(520, 1088, 40, 41), (520, 1088, 300, 41),
                                              (600, 1536, 257, 42), (520, 2048, 8, 43)])
def test_gemm_tiles(bits, rows, cols, M, seed):
    w = weights(bits, rows, cols, seed)
    X = synth.activations(M, cols, seed + 1)
    buf, Y = guarded((M, rows), torch.bfloat16)
    print(f"asym lut{bits} gemm {rows}x{cols} M={M}", flush=True)
    fqm.gemm(w, bf16_dev(X), Y=Y)
    torch.cuda.synchronize()
    assert canaries_intact(buf)
    assert_close(to_f64(Y), reference(bits, rows, cols, seed, X), "bf16", f"lut{bits} M={M}")


@pytest.mark.parametrize("bits", [6, 4])
def test_gemm_prefill_shape_sampled(bits):
    """M = 2048 on the up layer: 512 tiles in whole rounds plus a K-split last
    round; 40 sampled rows of X against the oracle."""
    rows, cols, seed, M = 17408, 5120, 34, 2048
    w = weights(bits, rows, cols, seed)
    X = synth.activations(M, cols, 44)
    print(f"asym lut{bits} prefill {M}x{rows}x{cols}", flush=True)
    Y = fqm.gemm(w, bf16_dev(X))
    pick = np.random.default_rng(bits).choice(M, size=40, replace=False)
    pick[:2] = [0, M - 1]
    assert_close(to_f64(Y)[pick], reference(bits, rows, cols, seed, X[pick]), "bf16", f"lut{bits} prefill")
