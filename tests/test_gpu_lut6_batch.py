"""GPU parity for the batch 2..16 per-row LUT 6-bit GEMV on the matrix cores
("Qwen3.8-27B - BenQ 6-bit", "What BenQ stores"): cols a multiple of 512,
row counts that leave a partial 16-row block, and K split over workgroups
(evenly, unevenly, one chunk per split)."""
import numpy as np
import pytest
import torch

import dequant_matmul_amd as fqm
import oracle
import synth
from gpu_common import (DEV, assert_close, bf16_dev, canaries_intact, guarded, lut6_case,
                        lut6_weights, to_f64)

pytestmark = pytest.mark.gpu

# (rows, cols, seed, batches), K in 512-wide chunks split into
# ceil(chunks / ceil(chunks / ceil(1024 / row blocks))) parts:
# 2 chunks in 2 splits with a partial row block; 8 in 8; 6 in 6; 34 in 34;
# 10 in 10; 34 in splits of 9, 9, 9, 7.
CASES = [(77, 1024, 9, (2, 16)), (300, 4096, 21, (3, 8)), (1000, 3072, 8, (5, 13)),
         (600, 17408, 10, (2, 8)), (2000, 5120, 5, (16,)), (4100, 17408, 4, (4,))]


@pytest.mark.parametrize("rows,cols,seed,batches", CASES)
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_gemv_mfma_cases(rows, cols, seed, batches, out):
    inp, packed = lut6_case(rows, cols, seed)
    w = lut6_weights(rows, cols, seed)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    for b in batches:
        x = synth.activations(b, cols, seed + b)
        buf, y = guarded((b, rows), dt)
        need = fqm.workspace_size(w, b)
        wsp = torch.empty(need, dtype=torch.uint8, device=DEV) if need else None
        print(f"lut6 mfma gemv {rows}x{cols} batch {b} {out} workspace {need}", flush=True)
        fqm.gemv(w, bf16_dev(x), y=y, workspace=wsp)
        torch.cuda.synchronize()
        assert canaries_intact(buf)
        assert_close(to_f64(y), oracle.lut6.gemv(packed, inp.lut, x, cols), out, f"{rows}x{cols} b{b} {out}")


# Batches 2 and 3 on whole 1024-column cells (2: 1-19, 3: 1-12) take the
# one-row-per-wave kernel (every batch row's x block in LDS, one decode per
# weight for all rows): 4-wave groups up to 8 cells, 10-wave groups past
# that, last groups partly past the end, the largest cell counts, and the
# two MLP layers.
@pytest.mark.parametrize("rows,cols,seed,batch", [(1, 1024, 39, 2), (1, 9216, 39, 3), (5, 1024, 40, 2),
                                                  (77, 3072, 41, 3), (130, 8192, 42, 2),
                                                  (23, 9216, 44, 2), (41, 12288, 45, 3), (11, 19456, 46, 2),
                                                  (17408, 5120, 43, 2), (17408, 5120, 43, 3), (5120, 17408, 47, 2)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_gemv_batch_rows_kernel(rows, cols, seed, batch, out):
    inp, packed = lut6_case(rows, cols, seed)
    w = lut6_weights(rows, cols, seed)
    assert fqm.workspace_size(w, batch) == 0
    x = synth.activations(batch, cols, seed + 1)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    buf, y = guarded((batch, rows), dt)
    print(f"lut6 batch-{batch} rows kernel {rows}x{cols} {out}", flush=True)
    fqm.gemv(w, bf16_dev(x), y=y)
    torch.cuda.synchronize()
    assert canaries_intact(buf)
    assert_close(to_f64(y), oracle.lut6.gemv(packed, inp.lut, x, cols), out, f"{rows}x{cols} b{batch} {out}")
    if out == "f32" and rows < 1000:
        # each batch row as its own batch-1 call: the same decode, the same sums
        y1 = torch.stack([fqm.gemv(w, bf16_dev(x[b:b + 1]), out_dtype=torch.float32)[0] for b in range(batch)])
        assert torch.allclose(y, y1, rtol=1e-6, atol=0)


def test_gemv_mfma_workspace_rule():
    # K is split while there are fewer than 1024 row blocks of 16
    assert fqm.workspace_size(lut6_weights(300, 4096, 21), 8) == 8 * 8 * 300 * 4
    assert fqm.workspace_size(lut6_weights(4100, 17408, 4), 8) == 4 * 8 * 4100 * 4
    assert fqm.workspace_size(lut6_weights(16384, 1024, 4), 8) == 0
    assert fqm.workspace_size(lut6_weights(300, 4096, 21), 1) == 0
    # a too-small workspace is refused
    w = lut6_weights(300, 4096, 21)
    x = bf16_dev(synth.activations(8, 4096, 1))
    with pytest.raises(RuntimeError):
        fqm.gemv(w, x, workspace=torch.empty(16, dtype=torch.uint8, device=DEV))


def test_gemv_mfma_exact_invariants():
    rows, cols, seed = 300, 4096, 21
    inp, _ = lut6_case(rows, cols, seed)
    w = lut6_weights(rows, cols, seed)
    lv = oracle.numerics.bf16_to_f64(inp.lut)
    # one-hot x rows return decoded columns exactly (each batch row its own k)
    ks = [0, 1023, 1024, 2047 + 17, 3000, cols - 1]
    x = np.zeros((len(ks), cols), np.uint16)
    for b, k in enumerate(ks):
        x[b, k] = 0x3F80
    y = to_f64(fqm.gemv(w, bf16_dev(x), out_dtype=torch.float32))
    for b, k in enumerate(ks):
        assert np.array_equal(y[b], lv[np.arange(rows), inp.codes[:, k]]), k
    # scaling x by 4 scales y by 4 exactly; the same call twice gives the same bits
    x = synth.activations(6, cols, seed)
    y = to_f64(fqm.gemv(w, bf16_dev(x), out_dtype=torch.float32))
    x4 = x.astype(np.uint32) + (2 << 7)
    x4 = np.where((x & 0x7FFF) == 0, x, x4).astype(np.uint16)
    assert np.array_equal(to_f64(fqm.gemv(w, bf16_dev(x4), out_dtype=torch.float32)), 4 * y)
    assert np.array_equal(to_f64(fqm.gemv(w, bf16_dev(x), out_dtype=torch.float32)), y)
    # each batch row is independent of the others: row b alone equals row b of the batch
    y1 = to_f64(fqm.gemv(w, bf16_dev(np.repeat(x[2:3], 2, axis=0)), out_dtype=torch.float32))
    assert np.array_equal(y1[0], y1[1])
    assert np.linalg.norm(y1[0] - y[2]) <= 1e-6 * np.linalg.norm(y[2])


@pytest.mark.parametrize("batch", [1, 2, 3, 8])
def test_graph_replays_match_eager(batch):
    """The down layer (17 cells: batches 1-2 on the one-row-per-wave kernels,
    3 and 8 on the matrix cores with their K split and sum in the workspace),
    captured in a HIP graph and replayed with new x, with eager work in
    between: every replay gives the eager result bit for bit."""
    rows, cols, seed = 5120, 17408, 3
    w = lut6_weights(rows, cols, seed)
    xs = [bf16_dev(synth.activations(batch, cols, 80 + i)) for i in range(3)]
    x = xs[0].clone()
    need = fqm.workspace_size(w, batch)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV) if need else None
    y = torch.empty((batch, rows), dtype=torch.float32, device=DEV)
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
        eager = fqm.gemv(w, xi, out_dtype=torch.float32, workspace=ws)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(got, eager)
