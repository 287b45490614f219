"""GPU parity for the per-row LUT 6-bit prefill GEMM (bf16 MFMA)."""
import numpy as np
import pytest
import torch

import dequant_matmul_amd as fqm
import oracle
import synth
from gpu_common import DEV, assert_close, bf16_dev, canaries_intact, guarded, lut6_case, lut6_weights, to_f64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M", [1, 17, 128, 300])
def test_gemm_ragged(M):
    rows, cols, seed = 520, 1088, 9
    inp, packed = lut6_case(rows, cols, seed)
    w = lut6_weights(rows, cols, seed)
    X = synth.activations(M, cols, seed + 100)
    buf, Y = guarded((M, rows), torch.bfloat16)
    fqm.gemm(w, bf16_dev(X), Y=Y)
    torch.cuda.synchronize()
    assert canaries_intact(buf)
    assert_close(to_f64(Y), oracle.lut6.gemm(packed, inp.lut, X, cols), "bf16", f"M={M}")


@pytest.mark.parametrize("M", [2047, 2048])
def test_gemm_prefill_shape_sampled(M):
    rows, cols, seed = 17408, 5120, 2
    inp, packed = lut6_case(rows, cols, seed)
    w = lut6_weights(rows, cols, seed)
    X = synth.activations(M, cols, 4)
    Y = fqm.gemm(w, bf16_dev(X))
    rng = np.random.default_rng(M)
    ms = np.unique(np.concatenate([rng.choice(M, 48, replace=False), [0, M - 1]]))
    W = oracle.lut6.decode(inp.codes, inp.lut)
    yo = oracle.numerics.bf16_to_f64(X[ms]) @ W.T
    assert_close(to_f64(Y[torch.from_numpy(ms).to(DEV)]), yo, "bf16", f"M={M}")


def test_gemm_matches_gemv_rows():
    rows, cols, seed = 520, 1088, 9
    w = lut6_weights(rows, cols, seed)
    X = bf16_dev(synth.activations(16, cols, 3))
    Y = fqm.gemm(w, X)
    y = fqm.gemv(w, X, out_dtype=torch.float32)
    # both follow the same definition; they differ only by summation order
    assert_close(to_f64(Y), to_f64(y), "bf16")
