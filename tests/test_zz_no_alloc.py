"""fqm_gemv_static (no workspace argument, for callers that cannot allocate)
against fqm_gemv with a caller workspace, on the paths that use scratch: the
K-split matrix-core LUT GEMV (batch 2-16 where it runs), FABQ with vector centroids and MDBF.  Two calls in a row share the library's
static scratch, the second with a smaller input, so a kernel reading scratch
it did not write in the same call would show up as a mismatch."""
import numpy as np
import pytest
import torch

import dequant_matmul_amd as fqm
import oracle
import synth
from gpu_common import DEV, assert_close, bf16_dev, canaries_intact, guarded, lut6_case, lut6_weights, to_f64

pytestmark = pytest.mark.gpu


def _both(w, x, out_dtype):
    need = fqm.workspace_size(w, x.shape[0])
    assert 0 < need <= fqm.STATIC_SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    y_ws = fqm.gemv(w, x, out_dtype=out_dtype, workspace=ws)
    buf, y_st = guarded((x.shape[0], w.rows), out_dtype)
    fqm.gemv_static(w, x, y=y_st)
    torch.cuda.synchronize()
    assert canaries_intact(buf)
    return y_ws, y_st


def test_lut6_two_calls_second_smaller():
    for rows, cols, seed, batch in ((5120, 17408, 3, 8), (300, 4096, 21, 5)):
        inp, packed = lut6_case(rows, cols, seed)
        w = lut6_weights(rows, cols, seed)
        x = synth.activations(batch, cols, seed + 7)
        print(f"gemv_static lut6 {rows}x{cols} batch {batch}", flush=True)
        y_ws, y_st = _both(w, bf16_dev(x), torch.float32)
        assert torch.equal(y_st, y_ws)
        assert_close(to_f64(y_st), oracle.lut6.gemv(packed, inp.lut, x, cols), "f32", f"{rows}x{cols}")


def test_lut4_two_calls_second_smaller():
    for rows, cols, seed, batch in ((5120, 17408, 8, 16), (70, 1536, 13, 5)):
        inp = synth.lut4_input(rows, cols, seed)
        packed = oracle.lut4.pack_codes(inp.codes)
        w = fqm.Lut4Weights.from_codes(inp.codes, inp.lut, device=DEV)
        x = synth.activations(batch, cols, seed + 7)
        print(f"gemv_static lut4 {rows}x{cols} batch {batch}", flush=True)
        y_ws, y_st = _both(w, bf16_dev(x), torch.bfloat16)
        assert torch.equal(y_st.view(torch.int16), y_ws.view(torch.int16))
        assert_close(to_f64(y_st), oracle.lut4.gemv(packed, inp.lut, x, cols), "bf16", f"{rows}x{cols}")


def test_fabq_vector_two_calls_second_smaller():
    for rows, cols, seed, batch, bs in ((301, 1536, 61, 3, 16), (5120, 5120, 5, 8, 512)):
        inp = synth.fabq_input(rows, cols, seed, blocksize=bs, cb_mode=2)
        p = oracle.fabq.pack(inp)
        w = fqm.FabqWeights.from_arrays(inp.rows, inp.cols, inp.blocksize, inp.n_hi, inp.row_of, inp.q4,
                                        inp.s_hi, inp.signs, inp.s_blk, inp.idx, inp.codebook, device=DEV,
                                        hi_bits=inp.hi_bits, cb_mode=inp.cb_mode, cb_base=inp.cb_base,
                                        tier=inp.tier, vcodebook=inp.vcodebook)
        x = synth.activations(batch, cols, seed + 7)
        print(f"gemv_static fabq vector {rows}x{cols} block {bs} batch {batch}", flush=True)
        y_ws, y_st = _both(w, bf16_dev(x), torch.float32)
        assert torch.equal(y_st, y_ws)
        assert_close(to_f64(y_st), oracle.fabq.gemv(p, x, rows, cols, bs, inp.n_hi), "f32", f"fabq {rows}x{cols}")


def test_mdbf_two_calls_second_smaller():
    for n, m, r, l, P, seed, batch in ((4096, 4096, 2000, 2, 1, 6, 16), (333, 544, 300, 3, 2, 75, 7)):
        inp = synth.mdbf_input(n, m, r, l, P, seed)
        paths = oracle.mdbf.pack(inp)
        w = fqm.MdbfWeights.from_arrays(inp.n, inp.m, inp.r, inp.l, inp.S_A, inp.S_B, inp.A_amp,
                                        inp.B_amp, inp.Q_U, inp.Q_V, device=DEV)
        x = synth.activations(batch, m, seed + 7)
        print(f"gemv_static mdbf {n}x{m} r={r} l={l} P={P} batch {batch}", flush=True)
        y_ws, y_st = _both(w, bf16_dev(x), torch.float32)
        assert torch.equal(y_st, y_ws)
        assert_close(to_f64(y_st), oracle.mdbf.gemv_factored(paths, x, n, m, r), "f32", f"mdbf {n}x{m}")


def test_no_scratch_needed_paths_and_the_limit():
    # batch 1 needs no scratch: the static entry point takes the same route
    inp, packed = lut6_case(1000, 3072, 8)
    w = lut6_weights(1000, 3072, 8)
    x = bf16_dev(synth.activations(1, 3072, 8))
    assert fqm.workspace_size(w, 1) == 0
    assert torch.equal(fqm.gemv_static(w, x, out_dtype=torch.float32), fqm.gemv(w, x, out_dtype=torch.float32))
    # a request past the static maximum is refused with FQM_E_SCRATCH
    big = synth.mdbf_input(5120, 17408, 64, 16, 2, 77)
    wb = fqm.MdbfWeights.from_arrays(big.n, big.m, big.r, big.l, big.S_A, big.S_B, big.A_amp,
                                     big.B_amp, big.Q_U, big.Q_V, device=DEV)
    assert fqm.workspace_size(wb, 16) > fqm.STATIC_SCRATCH_BYTES
    with pytest.raises(fqm.FqmError) as err:
        fqm.gemv_static(wb, bf16_dev(synth.activations(16, 17408, 1)))
    assert err.value.status == 8
