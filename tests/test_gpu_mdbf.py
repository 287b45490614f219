"""GPU parity for the MDBF two-pass double-binary GEMV."""
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
def case(n, m, r, l, P, seed):
    inp = synth.mdbf_input(n, m, r, l, P, seed)
    return inp, oracle.mdbf.pack(inp)


def weights(inp):
    return fqm.MdbfWeights.from_arrays(inp.n, inp.m, inp.r, inp.l, inp.S_A, inp.S_B, inp.A_amp,
                                       inp.B_amp, inp.Q_U, inp.Q_V, device=DEV)


@pytest.mark.parametrize("batch", [1, 16])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_config_shape(batch, out):
    inp, paths = case(4096, 4096, 2000, 2, 1, 6)
    x = synth.activations(batch, 4096, 6)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    buf, y = guarded((batch, 4096), dt)
    fqm.gemv(weights(inp), bf16_dev(x), y=y)
    torch.cuda.synchronize()
    assert canaries_intact(buf)
    yo = oracle.mdbf.gemv_factored(paths, x, 4096, 4096, 2000)
    assert_close(to_f64(y), yo, out, f"b{batch}")


@pytest.mark.parametrize("l,P", [(1, 1), (1, 2), (3, 1), (4, 2), (16, 1)])
def test_variants(l, P):
    n, m, r = 300, 512, 77
    inp, paths = case(n, m, r, l, P, 60 + l + P)
    x = synth.activations(5, m, 61)
    y = fqm.gemv(weights(inp), bf16_dev(x), out_dtype=torch.float32)
    assert_close(to_f64(y), oracle.mdbf.gemv_dense(paths, x, n, m, r), "f32", f"l={l} P={P}")


# A batch slice is floor(64 / (3 l)) rows, at least 1 (three bf16 parts of
# each of l envelopes per row fill at most four 16-column operand blocks):
# l = 16 splits a batch of 16 into sixteen slices of one row, l = 3 into
# slices of 7, 7 and 2 (a partly empty last slice); m = 544 and r = 300 are
# not multiples of the 512-column K block.
@pytest.mark.parametrize("l,P,batch", [(16, 1, 16), (3, 2, 16), (2, 1, 7), (1, 2, 1)])
def test_batch_slices_and_padding(l, P, batch):
    n, m, r = 333, 544, 300
    inp, paths = case(n, m, r, l, P, 70 + l + P)
    x = synth.activations(batch, m, 71)
    buf, y = guarded((batch, n), torch.float32)
    print(f"mdbf n={n} m={m} r={r} l={l} P={P} batch {batch}", flush=True)
    fqm.gemv(weights(inp), bf16_dev(x), y=y)
    torch.cuda.synchronize()
    assert canaries_intact(buf)
    assert_close(to_f64(y), oracle.mdbf.gemv_dense(paths, x, n, m, r), "f32", f"l={l} P={P} b={batch}")


# The smallest shapes: m = 32 inputs (one 512-wide K block, 480 of its
# columns padding), r = 5 (one sign byte per row of S_A, 3 of its bits
# padding), two paths.  At batch 1 pass 1 forms its dense operand in LDS
# itself; at batch 2 it reads the one that the prep launch wrote.
@pytest.mark.parametrize("batch", [1, 2])
def test_smallest_shapes(batch):
    n, m, r, l, P = 40, 32, 5, 2, 2
    inp, paths = case(n, m, r, l, P, 90)
    x = synth.activations(batch, m, 91)
    buf, y = guarded((batch, n), torch.float32)
    print(f"mdbf n={n} m={m} r={r} l={l} P={P} batch {batch}", flush=True)
    fqm.gemv(weights(inp), bf16_dev(x), y=y)
    torch.cuda.synchronize()
    assert canaries_intact(buf)
    assert_close(to_f64(y), oracle.mdbf.gemv_dense(paths, x, n, m, r), "f32", f"smallest b={batch}")


def test_deterministic_and_batch_independent():
    inp, paths = case(4096, 4096, 2000, 2, 1, 6)
    w = weights(inp)
    x = synth.activations(16, 4096, 9)
    y1 = to_f64(fqm.gemv(w, bf16_dev(x), out_dtype=torch.float32))
    y2 = to_f64(fqm.gemv(w, bf16_dev(x), out_dtype=torch.float32))
    assert np.array_equal(y1, y2)
    # a batch row computed alone matches its row of the batch
    y3 = to_f64(fqm.gemv(w, bf16_dev(x[5:6]), out_dtype=torch.float32))
    assert np.linalg.norm(y3[0] - y1[5]) <= 1e-6 * np.linalg.norm(y1[5])


# Rectangular MLP shapes of a 27B-class layer (up 17408 x 5120, down
# 5120 x 17408), the rank taken from the page's bit accounting at 2 bits per
# weight (clamped to the shape's reachable maximum), with more envelopes (l)
# and two paths (P).
@pytest.mark.parametrize("n,m,l,P,batch", [(17408, 5120, 4, 2, 1), (5120, 17408, 4, 2, 16),
                                           (17408, 5120, 16, 1, 8), (5120, 17408, 1, 2, 1)])
def test_mlp_shapes_more_envelopes_and_paths(n, m, l, P, batch):
    r = oracle.mdbf.rank(2.0, n, m, l, P)
    assert 1 <= r <= min(n, m)
    inp, paths = case(n, m, r, l, P, 80 + l + P)
    x = synth.activations(batch, m, 81)
    print(f"mdbf n={n} m={m} r={r} l={l} P={P} batch {batch}", flush=True)
    buf, y = guarded((batch, n), torch.float32)
    fqm.gemv(weights(inp), bf16_dev(x), y=y)
    torch.cuda.synchronize()
    assert canaries_intact(buf)
    assert_close(to_f64(y), oracle.mdbf.gemv_factored(paths, x, n, m, r), "f32", f"{n}x{m} l={l} P={P}")


def test_workspace_contents_and_repeated_calls():
    """The workspace's contents on entry do not matter: a workspace full of
    0xFF bytes, and the same workspace reused call after call, give the same
    bits (every operand word is written before it is read)."""
    inp, paths = case(4096, 4096, 2000, 2, 1, 6)
    w = weights(inp)
    x = bf16_dev(synth.activations(16, 4096, 12))
    need = fqm.workspace_size(w, 16)
    ws = torch.full((need,), 255, dtype=torch.uint8, device=DEV)
    y0 = fqm.gemv(w, x, out_dtype=torch.float32, workspace=ws)
    for _ in range(3):
        y1 = fqm.gemv(w, x, out_dtype=torch.float32, workspace=ws)
        assert torch.equal(y0, y1)
    yo = oracle.mdbf.gemv_factored(paths, synth.activations(16, 4096, 12), 4096, 4096, 2000)
    assert_close(to_f64(y0), yo, "f32", "garbage workspace")


def test_graph_replays_match_eager():
    """Captured in a HIP graph and replayed several times, with eager work in
    between, every replay gives the eager result."""
    inp, paths = case(4096, 4096, 2000, 2, 1, 6)
    w = weights(inp)
    xs = [bf16_dev(synth.activations(1, 4096, 20 + i)) for i in range(3)]
    x = xs[0].clone()
    need = fqm.workspace_size(w, 1)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    y = torch.empty((1, 4096), dtype=torch.float32, device=DEV)
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
