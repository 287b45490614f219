"""GPU parity for the per-row LUT 6-bit prefill GEMM (bf16 MFMA)."""
import numpy as np
import pytest
import torch

import dequant_matmul_amd as fqm
import oracle
import synth
from gpu_common import DEV, assert_close, bf16_dev, canaries_intact, guarded, lut6_case, lut6_weights, to_f64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M", [1, 17, 64, 128, 255, 256, 257, 300])
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


def test_gemm_prefill_shape_every_output():
    """The prefill configuration (X 2048 x 5120, the up layer 17408 x 5120):
    all 35.7 M outputs against the fp64 product (one BLAS matmul on the host)."""
    rows, cols, seed, M = 17408, 5120, 2, 2048
    inp, packed = lut6_case(rows, cols, seed)
    w = lut6_weights(rows, cols, seed)
    X = synth.activations(M, cols, 4)
    Y = fqm.gemm(w, bf16_dev(X))
    W = oracle.lut6.decode(inp.codes, inp.lut)
    yo = oracle.numerics.bf16_to_f64(X) @ W.T
    del W
    assert_close(to_f64(Y), yo, "bf16", f"M={M}")


@pytest.mark.parametrize("M", [100, 256, 2047, 2048])
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



def _plan_ws(rows, cols, M):
    """Workspace rule of the tile plan: tiles are 256 rows of X tall (64 when
    M <= 64) and 256 columns wide; whole rounds of tiles (one per compute unit,
    two per compute unit for 64-row tiles) run directly; the N tiles of a
    last partial round split K into the k parts (2 <= k <= steps // 8, at most
    4 for 64-row tiles, partials at most 256 MB) that minimise
    ceil(tail k / slots) * ceil(steps / k), fewer parts on ties, and only when
    that beats ceil(tail / slots) * steps; fp32 partial tiles."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    small = M <= 64
    bm = 64 if small else 256
    mt, nt = -(-M // bm), -(-rows // 256)
    tiles = mt * nt
    slots = cus * (2 if small else 1)
    if tiles % slots == 0:
        return 0
    nt_main = (tiles // slots) * slots // mt
    tail = (nt - nt_main) * mt
    steps = cols // 64
    kmax = min(steps // 8, 4) if small else steps // 8
    best_k, best = 1, -(-tail // slots) * steps
    for k in range(2, kmax + 1):
        if tail * k * bm * 256 * 4 > 256 << 20:
            break
        length = -(-tail * k // slots) * -(-steps // k)
        if length < best:
            best_k, best = k, length
    return tail * best_k * bm * 256 * 4 if best_k >= 2 else 0


@pytest.mark.parametrize("M", [1, 2, 8, 16])
@pytest.mark.parametrize("rows,cols", [(520, 2048), (300, 17408)])
def test_gemm_small_m_runs_the_gemv_kernels(rows, cols, M):
    """Up to 16 rows on a shape the GEMV kernels cover: the same workspace and
    the same bits as fqm_gemv, and the oracle's product."""
    inp, packed = lut6_case(rows, cols, 21)
    w = lut6_weights(rows, cols, 21)
    assert fqm.gemm_workspace_size(w, M) == fqm.workspace_size(w, M)
    X = synth.activations(M, cols, 22)
    buf, Y = guarded((M, rows), torch.bfloat16)
    fqm.gemm(w, bf16_dev(X), Y=Y)
    y = fqm.gemv(w, bf16_dev(X))
    torch.cuda.synchronize()
    assert canaries_intact(buf)
    assert torch.equal(Y.view(torch.int16), y.view(torch.int16))
    assert_close(to_f64(Y), oracle.lut6.gemm(packed, inp.lut, X, cols), "bf16", f"M={M}")


def test_gemm_small_m_missing_workspace_is_an_error():
    rows, cols, M = 300, 17408, 8  # the GEMV kernel splits K here: fp32 partials in the workspace
    w = lut6_weights(rows, cols, 21)
    assert fqm.gemm_workspace_size(w, M) > 0
    X = bf16_dev(synth.activations(M, cols, 1))
    Y = torch.empty((M, rows), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(fqm.FqmError) as err:
        fqm.gemm(w, X, Y=Y, workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
    assert err.value.status == 5  # FQM_E_WORKSPACE


@pytest.mark.parametrize("rows,cols,M", [(520, 1088, 300), (17408, 5120, 2048), (300, 128, 50),
                                         (5120, 17408, 77), (17408, 5120, 64), (5120, 17408, 33),
                                         (5120, 17408, 2048), (2560, 17408, 1024)])
def test_gemm_workspace_rule(rows, cols, M):
    w = lut6_weights(256, cols, 1)
    w.desc.rows = rows  # the rule reads the shape only (no launch)
    assert fqm.gemm_workspace_size(w, M) == _plan_ws(rows, cols, M)


def test_gemm_missing_workspace_is_an_error():
    rows, cols, M = 520, 1088, 64
    w = lut6_weights(rows, cols, 9)
    assert fqm.gemm_workspace_size(w, M) > 0
    X = bf16_dev(synth.activations(M, cols, 1))
    Y = torch.empty((M, rows), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(fqm.FqmError) as err:
        fqm.gemm(w, X, Y=Y, workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
    assert err.value.status == 5  # FQM_E_WORKSPACE


@pytest.mark.parametrize("rows,cols,M", [(300, 128, 50), (700, 192, 257)])
def test_gemm_unsplit_short_k(rows, cols, M):
    """K too short to split (fewer than 16 steps of 64): every tile in the
    direct launch, no workspace."""
    inp, packed = lut6_case(rows, cols, 5)
    w = lut6_weights(rows, cols, 5)
    assert fqm.gemm_workspace_size(w, M) == 0
    X = synth.activations(M, cols, 6)
    buf, Y = guarded((M, rows), torch.bfloat16)
    fqm.gemm(w, bf16_dev(X), Y=Y)
    torch.cuda.synchronize()
    assert canaries_intact(buf)
    assert_close(to_f64(Y), oracle.lut6.gemm(packed, inp.lut, X, cols), "bf16", f"rows={rows}")


@pytest.mark.parametrize("M", [2048, 1500])
def test_gemm_down_shape_sampled(M):
    """The down layer (5120 x 17408, K = 17408) at a prefill's 2048 rows (and a
    ragged 1500): 8 x 20 tiles of 256 x 256, fewer than the compute units, so
    every tile is split along K (three parts at 2048 rows) and reduced; 40
    sampled rows of X against the oracle."""
    rows, cols, seed = 5120, 17408, 3
    inp, packed = lut6_case(rows, cols, seed)
    w = lut6_weights(rows, cols, seed)
    need = fqm.gemm_workspace_size(w, M)
    assert need == _plan_ws(rows, cols, M) > 0
    X = synth.activations(M, cols, 44)
    print(f"gemm down shape {M}x{rows}x{cols} workspace {need}", flush=True)
    buf, Y = guarded((M, rows), torch.bfloat16)
    fqm.gemm(w, bf16_dev(X), Y=Y)
    torch.cuda.synchronize()
    assert canaries_intact(buf)
    pick = np.random.default_rng(M).choice(M, size=40, replace=False)
    pick[:2] = [0, M - 1]
    W = oracle.lut6.decode(inp.codes, inp.lut)
    yo = oracle.numerics.bf16_to_f64(X[pick]) @ W.T
    assert_close(to_f64(Y)[pick], yo, "bf16", f"down M={M}")


# K of 1 to 7 steps of 64 columns.  The main loop runs in groups of three
# steps and the prologue requests its first tiles and codes at clamped step
# indices, so every remainder of steps / 3 and the shortest K appear, for the
# 64-row tiles (M = 40) and the 256-row tiles (M = 300), both code widths.
SHORT_K_FMT = {6: (synth.lut6_input, fqm.Lut6Weights, oracle.lut6),
               4: (synth.lut4_input, fqm.Lut4Weights, oracle.lut4)}


@pytest.mark.parametrize("bits", [6, 4])
@pytest.mark.parametrize("cols", [64, 128, 192, 256, 320, 448])
@pytest.mark.parametrize("M", [40, 300])
def test_gemm_short_k(bits, cols, M):
    gen, W, orc = SHORT_K_FMT[bits]
    rows, seed = 300, 50 + cols // 64
    inp = gen(rows, cols, seed)
    w = W.from_codes(inp.codes, inp.lut, device=DEV)
    X = synth.activations(M, cols, seed + 1)
    buf, Y = guarded((M, rows), torch.bfloat16)
    print(f"lut{bits} gemm {rows}x{cols} M={M}", flush=True)
    fqm.gemm(w, bf16_dev(X), Y=Y)
    torch.cuda.synchronize()
    assert canaries_intact(buf)
    assert_close(to_f64(Y), orc.gemv(orc.pack_codes(inp.codes), inp.lut, X, cols), "bf16", f"lut{bits} K={cols} M={M}")
