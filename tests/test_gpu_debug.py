"""GPU tests of the debug checks (fqm_set_debug / FQM_DEBUG): correct calls
still match the oracle and return FQM_OK after waiting for their kernels;
buffers shorter than their shapes, host memory and short workspaces are
refused with FQM_E_BOUNDS before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import dequant_matmul_amd as fqm
import oracle
import synth
from gpu_common import DEV, assert_close, bf16_dev, lut6_case, lut6_weights, to_f64

pytestmark = pytest.mark.gpu

BOUNDS = 9


def hip_runtime():
    """The HIP runtime this process already uses (torch's copy), by path."""
    torch.zeros(1, device=DEV)
    for line in open("/proc/self/maps"):
        if "libamdhip64.so" in line:
            return ctypes.CDLL(line.split()[-1])
    raise RuntimeError("libamdhip64.so is not loaded")


@pytest.fixture
def debug():
    prev = fqm.set_debug(True)
    yield
    fqm.set_debug(prev)


@pytest.fixture(scope="module")
def hip():
    h = hip_runtime()
    h.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
    h.hipFree.argtypes = [ctypes.c_void_p]
    return h


def hip_alloc(hip, n):
    p = ctypes.c_void_p()
    assert hip.hipMalloc(ctypes.byref(p), n) == 0
    return p.value


def test_correct_calls_pass(debug):
    rows, cols, seed = 1000, 3072, 8
    inp, packed = lut6_case(rows, cols, seed)
    w = lut6_weights(rows, cols, seed)
    x = synth.activations(1, cols, seed)
    y = fqm.gemv(w, bf16_dev(x), out_dtype=torch.float32)
    assert_close(to_f64(y), oracle.lut6.gemv(packed, inp.lut, x, cols), "f32", "debug gemv")
    X = synth.activations(40, cols, seed + 1)
    Y = fqm.gemm(w, bf16_dev(X))
    assert_close(to_f64(Y), oracle.lut6.gemv(packed, inp.lut, X, cols), "bf16", "debug gemm")
    W = fqm.dequant(w).view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(W, inp.lut[np.arange(rows)[:, None], inp.codes])


def test_short_and_host_buffers_refused(debug, hip):
    lib = fqm.load()
    rows, cols = 64, 262144  # x needs 512 KB
    w = fqm.Lut6Weights(torch.zeros((rows, cols * 3 // 4), dtype=torch.uint8, device=DEV),
                        torch.zeros((rows, 64), dtype=torch.bfloat16, device=DEV), rows, cols)
    d = w.desc
    y = torch.empty((1, rows), dtype=torch.float32, device=DEV)
    short = hip_alloc(hip, 64 * 1024)
    try:
        print("debug: short x", flush=True)
        assert lib.fqm_gemv(ctypes.byref(d), short, y.data_ptr(), 1, 1, None, 0, None) == BOUNDS
        x_ok = torch.zeros((1, cols), dtype=torch.bfloat16, device=DEV)
        host_y = np.zeros(rows, np.float32)
        assert lib.fqm_gemv(ctypes.byref(d), x_ok.data_ptr(), host_y.ctypes.data, 1, 1, None, 0, None) == BOUNDS
        # a descriptor whose packed rows reach past their allocation
        d.lut6.packed = short
        assert lib.fqm_gemv(ctypes.byref(d), x_ok.data_ptr(), y.data_ptr(), 1, 1, None, 0, None) == BOUNDS
        assert lib.fqm_dequant(ctypes.byref(d), x_ok.data_ptr(), None) == BOUNDS
    finally:
        hip.hipFree(short)
    torch.cuda.synchronize()


def test_short_workspace_refused(debug, hip):
    """ws_bytes claims enough, the allocation holds less."""
    lib = fqm.load()
    rows, cols, seed = 300, 4096, 36
    w = lut6_weights(rows, cols, seed)
    need = fqm.workspace_size(w, 8)
    assert need > 64 * 1024
    x = torch.zeros((8, cols), dtype=torch.bfloat16, device=DEV)
    y = torch.empty((8, rows), dtype=torch.bfloat16, device=DEV)
    short = hip_alloc(hip, 16 * 1024)
    try:
        print("debug: short workspace", flush=True)
        d = w.desc
        assert lib.fqm_gemv(ctypes.byref(d), x.data_ptr(), y.data_ptr(), 0, 8, short, need, None) == BOUNDS
    finally:
        hip.hipFree(short)
    torch.cuda.synchronize()
