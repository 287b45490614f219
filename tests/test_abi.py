"""The C ABI on the CPU: the library loads, exports every declared symbol,
and rejects bad arguments on the host before anything touches a GPU.

The buffers here are fake addresses.  A call whose arguments are meant to
pass the host checks runs through refused_before_launch, with the debug
checks on: the fake addresses are no device allocations, so the call stops
with FQM_E_BOUNDS before anything is enqueued, on a machine with a GPU as
well as without one."""
import ctypes
import os
import re

import pytest

import dequant_matmul_amd as fqm
from conftest import ROOT

E = dict(OK=0, NULL=1, ALIGN=2, SHAPE=3, FORMAT=4, WORKSPACE=5, UNSUPPORTED=6, HIP=7, SCRATCH=8, BOUNDS=9)
FAKE = 0x7f0000000000  # a 16-byte-aligned address the host never dereferences


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fqm.LIB_PATH):
        from dequant_matmul_amd import build
        build.build()
    return fqm.load()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "fqm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(fqm_[a-z_]+)\s*\(", text))


def test_exports_every_declared_symbol(lib):
    decl = declared_functions()
    assert decl == set(fqm.SYMBOLS)
    for name in decl:
        assert hasattr(lib, name), name
    assert lib.fqm_version() == 5


def test_bench_library_exports_its_references():
    """libfqm_bench.so (the benchmark's streaming-read and GEMM-mix reference
    kernels) loads and exports both entry points; they reject bad arguments
    on the host."""
    from dequant_matmul_amd import build
    if not os.path.exists(build.BENCH_LIB):
        build.build()
    blib = ctypes.CDLL(build.BENCH_LIB)
    blib.fqm_bench_stream_read.restype = ctypes.c_int
    blib.fqm_bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_uint32, ctypes.c_void_p]
    blib.fqm_bench_gemm_mix.restype = ctypes.c_int
    blib.fqm_bench_gemm_mix.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_float, ctypes.c_void_p]
    assert hasattr(blib, "fqm_bench_wall_clock_khz")
    assert blib.fqm_bench_stream_read(None, 1024, FAKE, None, 0, None) == 1
    assert blib.fqm_bench_stream_read(FAKE + 4, 1024, FAKE, None, 0, None) == 1
    assert blib.fqm_bench_gemm_mix(None, None, 256, 10, -1.0, None) == 1
    assert blib.fqm_bench_gemm_mix(FAKE, None, 0, 10, -1.0, None) == 1
    assert blib.fqm_bench_gemm_mix(FAKE, None, 256, 0, -1.0, None) == 1


def test_status_strings(lib):
    for code in E.values():
        assert lib.fqm_status_str(code)
    assert lib.fqm_status_str(99) == b"unknown status"


def lut6(rows=64, cols=128, ld=96, packed=FAKE, lut=FAKE):
    w = fqm._Weights()
    w.format, w.rows, w.cols = fqm.FQM_LUT6, rows, cols
    w.lut6.packed, w.lut6.lut, w.lut6.ld = packed, lut, ld
    return w


def gemv(lib, w, x=FAKE, y=FAKE, dt=0, batch=1, ws=None, wsb=0):
    return lib.fqm_gemv(ctypes.byref(w), x, y, dt, batch, ws, wsb, None)


def refused_before_launch(lib, call):
    """call() with the debug checks on.  Argument errors still come first;
    arguments that pass them stop at the allocation checks (FQM_E_BOUNDS), so
    no kernel ever reads or writes a fake address."""
    prev = lib.fqm_set_debug(1)
    try:
        return call()
    finally:
        lib.fqm_set_debug(prev)


def gemm(lib, w, X=FAKE, Y=FAKE, M=4, ws=None, wsb=0):
    return lib.fqm_gemm(ctypes.byref(w), X, Y, M, ws, wsb, None)


def test_lut6_argument_errors(lib):
    assert lib.fqm_gemv(None, FAKE, FAKE, 0, 1, None, 0, None) == E["NULL"]
    assert gemv(lib, lut6(cols=100)) == E["SHAPE"]            # cols % 64
    assert gemv(lib, lut6(ld=80)) == E["SHAPE"]               # ld < cols*3/4
    assert gemv(lib, lut6(ld=104)) == E["ALIGN"]              # ld % 16
    assert gemv(lib, lut6(packed=FAKE + 4)) == E["ALIGN"]
    assert gemv(lib, lut6(lut=None)) == E["NULL"]
    assert gemv(lib, lut6(), batch=0) == E["SHAPE"]
    assert gemv(lib, lut6(), batch=17) == E["SHAPE"]
    assert gemv(lib, lut6(), dt=5) == E["FORMAT"]
    assert gemv(lib, lut6(), x=None) == E["NULL"]
    assert gemv(lib, lut6(), y=FAKE + 2) == E["ALIGN"]
    bad = lut6()
    bad.format = 9
    assert gemv(lib, bad) == E["FORMAT"]
    assert gemv(lib, lut6(rows=-1)) == E["SHAPE"]
    # empty work returns before any launch
    assert gemv(lib, lut6(rows=0, packed=None, lut=None)) == E["OK"]
    assert gemm(lib, lut6(), M=0) == E["OK"]
    assert gemm(lib, lut6(), M=-1) == E["SHAPE"]
    assert gemm(lib, lut6(), X=None) == E["NULL"]
    assert gemm(lib, lut6(), Y=FAKE + 2) == E["ALIGN"]
    # X must stay below 2 GiB (buffer addressing): M * cols * 2 < 2^31
    assert gemm(lib, lut6(cols=65536, ld=49152), M=16384) == E["SHAPE"]
    assert lib.fqm_gemm_workspace_size(ctypes.byref(lut6()), 0) == 0
    assert lib.fqm_gemm_workspace_size(ctypes.byref(lut6()), -3) == 0
    assert lib.fqm_gemm_workspace_size(None, 4) == 0


def lut4(rows=64, cols=128, ld=64, packed=FAKE, lut=FAKE):
    w = fqm._Weights()
    w.format, w.rows, w.cols = fqm.FQM_LUT4, rows, cols
    w.lut4.packed, w.lut4.lut, w.lut4.ld = packed, lut, ld
    return w


def test_lut4_argument_errors(lib):
    assert gemv(lib, lut4(cols=96)) == E["SHAPE"]             # cols % 64
    assert gemv(lib, lut4(ld=48)) == E["SHAPE"]               # ld < cols/2
    assert gemv(lib, lut4(ld=72)) == E["ALIGN"]               # ld % 16
    assert gemv(lib, lut4(packed=FAKE + 4)) == E["ALIGN"]
    assert gemv(lib, lut4(lut=None)) == E["NULL"]
    assert gemv(lib, lut4(), batch=17) == E["SHAPE"]
    assert gemv(lib, lut4(rows=0, packed=None, lut=None)) == E["OK"]
    assert gemm(lib, lut4(), M=-1) == E["SHAPE"]
    assert gemm(lib, lut4(cols=96)) == E["SHAPE"]
    assert gemm(lib, lut4(), X=None) == E["NULL"]
    assert gemm(lib, lut4(), Y=FAKE + 2) == E["ALIGN"]
    assert gemm(lib, lut4(rows=0, packed=None, lut=None)) == E["OK"]
    assert lib.fqm_workspace_size(ctypes.byref(lut4()), 8) == 0
    for M in (1, 8, 17, 300):  # the GEMM's tile plan does not depend on the code width
        assert (lib.fqm_gemm_workspace_size(ctypes.byref(lut4(5120, 17408, ld=8704)), M)
                == lib.fqm_gemm_workspace_size(ctypes.byref(lut6(5120, 17408, ld=13056)), M))


def test_lut4_batch_workspace_follows_the_lut6_rule(lib):
    """Batches 2..16 of both LUT formats share the matrix-core kernel's K
    split, so the workspace depends on the shape and batch only."""
    for rows, cols, batch in ((5120, 17408, 8), (5120, 17408, 16), (17408, 5120, 8), (300, 4096, 4),
                              (5120, 17408, 1), (64, 1088, 4), (300, 20480, 2)):
        a = lib.fqm_workspace_size(ctypes.byref(lut4(rows, cols, ld=cols // 2)), batch)
        b = lib.fqm_workspace_size(ctypes.byref(lut6(rows, cols, ld=cols * 3 // 4)), batch)
        assert a == b, (rows, cols, batch)
    # batch 2 (3) on 1-19 (1-12) whole 1024-column cells runs one row per wave in
    # both formats: no K split, no workspace
    for batch, cols in ((2, 4096), (2, 17408), (3, 12288)):
        assert lib.fqm_workspace_size(ctypes.byref(lut4(300, cols, ld=cols // 2)), batch) == 0
        assert lib.fqm_workspace_size(ctypes.byref(lut6(300, cols, ld=cols * 3 // 4)), batch) == 0
    need = lib.fqm_workspace_size(ctypes.byref(lut4(5120, 17408, ld=8704)), 8)
    assert need > 0
    w = lut4(5120, 17408, ld=8704)
    assert gemv(lib, w, batch=8) == E["WORKSPACE"]
    assert gemv(lib, w, batch=8, ws=FAKE, wsb=need - 16) == E["WORKSPACE"]
    assert gemv(lib, w, batch=8, ws=FAKE + 8, wsb=need + 16) == E["ALIGN"]


def test_descriptor_layout_matches_the_header():
    """The LUT4 member sits after the others, so their offsets are unchanged."""
    W = fqm._Weights
    assert W.lut4.offset > W.mdbf.offset > W.fabq.offset > W.lut6.offset
    assert ctypes.sizeof(fqm._Lut4) == 24


def test_lut6_workspace_rule(lib):
    # batch >= 2 with cols % 512 == 0 splits K (512-wide chunks) while there
    # are fewer than 1024 row blocks of 16: ceil(1024 / blocks) splits, capped
    # at the chunk count, evened out over the chunks; S*batch*rows fp32
    assert lib.fqm_workspace_size(ctypes.byref(lut6(rows=300, cols=4096, ld=3072)), 8) == 8 * 8 * 300 * 4
    assert lib.fqm_workspace_size(ctypes.byref(lut6(rows=5120, cols=17408, ld=13056)), 8) == 4 * 8 * 5120 * 4
    assert lib.fqm_workspace_size(ctypes.byref(lut6(rows=17408, cols=5120, ld=3840)), 8) == 0
    assert lib.fqm_workspace_size(ctypes.byref(lut6(rows=16384, cols=1024, ld=768)), 8) == 0
    assert lib.fqm_workspace_size(ctypes.byref(lut6(rows=16368, cols=1024, ld=768)), 8) == 2 * 8 * 16368 * 4
    assert lib.fqm_workspace_size(ctypes.byref(lut6(rows=300, cols=4096, ld=3072)), 1) == 0
    assert lib.fqm_workspace_size(ctypes.byref(lut6(rows=300, cols=4032, ld=3024)), 8) == 0
    # batch 2 on 1-19 and batch 3 on 1-12 whole 1024-column cells run one row
    # per wave: no workspace; past that the matrix-core kernel splits K
    assert lib.fqm_workspace_size(ctypes.byref(lut6(rows=300, cols=4096, ld=3072)), 2) == 0
    assert lib.fqm_workspace_size(ctypes.byref(lut6(rows=300, cols=17408, ld=13056)), 2) == 0
    assert lib.fqm_workspace_size(ctypes.byref(lut6(rows=300, cols=20480, ld=15360)), 2) > 0
    assert lib.fqm_workspace_size(ctypes.byref(lut6(rows=300, cols=12288, ld=9216)), 3) == 0
    assert lib.fqm_workspace_size(ctypes.byref(lut6(rows=300, cols=13312, ld=9984)), 3) > 0
    assert lib.fqm_workspace_size(ctypes.byref(lut6(rows=300, cols=4096, ld=3072)), 4) > 0
    # a missing workspace is refused before anything is enqueued
    assert gemv(lib, lut6(rows=300, cols=4096, ld=3072), batch=8) == E["WORKSPACE"]


def test_pack_argument_errors(lib):
    assert lib.fqm_pack_bits(FAKE, FAKE, 4, 64, 3, 64, None, None) == E["FORMAT"]
    assert lib.fqm_pack_bits(FAKE, FAKE, 4, 64, 6, 32, None, None) == E["SHAPE"]   # ld < 48
    assert lib.fqm_pack_bits(FAKE, FAKE, 4, 64, 6, 56, None, None) == E["ALIGN"]
    assert lib.fqm_pack_bits(FAKE, FAKE + 8, 4, 64, 6, 48, None, None) == E["ALIGN"]
    assert lib.fqm_pack_bits(FAKE, None, 4, 64, 6, 48, None, None) == E["NULL"]
    assert lib.fqm_pack_bits(FAKE, FAKE, 0, 64, 6, 48, None, None) == E["OK"]
    assert lib.fqm_pack(FAKE, FAKE, -2, 64, 48, None, None) == E["SHAPE"]
    assert lib.fqm_unpack(FAKE, FAKE, 4, 66, 64, None) == E["SHAPE"]


def fabq(bs=128, n_hi=4, rows=64, cols=512):
    w = fqm._Weights()
    w.format, w.rows, w.cols = fqm.FQM_FABQ, rows, cols
    f = w.fabq
    f.blocksize, f.n_hi = bs, n_hi
    f.row_of = f.q4 = f.s_hi = f.signs = f.s_blk = f.idx = f.codebook = FAKE
    f.ld_q4, f.ld_signs, f.ld_idx = 256, 64, 16
    return w


def test_fabq_argument_errors(lib):
    # sanity: the base descriptor passes the argument checks
    assert refused_before_launch(lib, lambda: gemv(lib, fabq())) == E["BOUNDS"]
    assert gemv(lib, fabq(bs=96)) == E["FORMAT"]
    assert gemv(lib, fabq(bs=512, cols=768)) == E["SHAPE"]   # bs does not divide cols
    assert gemv(lib, fabq(n_hi=65)) == E["SHAPE"]
    w = fabq()
    w.fabq.ld_signs = 48
    assert gemv(lib, w) == E["SHAPE"]
    w = fabq()
    w.fabq.codebook = None
    assert gemv(lib, w) == E["NULL"]
    w = fabq(n_hi=64)  # no binary rows: their pointers are not needed
    w.fabq.codebook = w.fabq.signs = None
    assert gemm(lib, w, M=1) == E["UNSUPPORTED"]
    assert lib.fqm_gemm_workspace_size(ctypes.byref(w), 1) == 0
    assert lib.fqm_workspace_size(ctypes.byref(fabq()), 4) == 0


def test_fabq_vector_workspace(lib):
    """Vector centroids fold x into one fp32 term per batch row, block and
    active centroid (4 tiers x 16) before the GEMV: batch x blocks x 64 x 4
    bytes of workspace, none without binary rows; a missing or short
    workspace is refused before anything is enqueued."""
    w = fabq()
    w.fabq.cb_mode, w.fabq.tier, w.fabq.vcodebook = 2, FAKE, FAKE
    assert lib.fqm_workspace_size(ctypes.byref(w), 1) == 4 * 64 * 4
    assert lib.fqm_workspace_size(ctypes.byref(w), 5) == 5 * 4 * 64 * 4
    w16 = fabq(bs=16, cols=1040)
    w16.fabq.cb_mode, w16.fabq.tier, w16.fabq.vcodebook = 2, FAKE, FAKE
    w16.fabq.ld_q4, w16.fabq.ld_signs, w16.fabq.ld_idx = 528, 144, 48
    assert lib.fqm_workspace_size(ctypes.byref(w16), 3) == 3 * 65 * 64 * 4
    hi = fabq(n_hi=64)
    hi.fabq.cb_mode, hi.fabq.tier, hi.fabq.vcodebook = 2, FAKE, FAKE
    assert lib.fqm_workspace_size(ctypes.byref(hi), 4) == 0
    for mode in (0, 1):
        t = fabq()
        t.fabq.cb_mode, t.fabq.tier = mode, FAKE
        assert lib.fqm_workspace_size(ctypes.byref(t), 8) == 0
    need = lib.fqm_workspace_size(ctypes.byref(w), 2)
    assert gemv(lib, w, batch=2) == E["WORKSPACE"]
    assert gemv(lib, w, batch=2, ws=FAKE, wsb=need - 16) == E["WORKSPACE"]
    assert gemv(lib, w, batch=2, ws=FAKE + 8, wsb=need) == E["ALIGN"]
    assert refused_before_launch(lib, lambda: gemv(lib, w, batch=2, ws=FAKE, wsb=need)) == E["BOUNDS"]


def mdbf(r=2000, l=2, P=1, n=4096, m=4096):
    w = fqm._Weights()
    w.format, w.rows, w.cols = fqm.FQM_MDBF, n, m
    md = w.mdbf
    md.r, md.l, md.P = r, l, P
    for p in range(2):
        q = md.path[p]
        q.S_A = q.S_B = q.A_amp = q.B_amp = q.Q_U = q.Q_V = FAKE
        q.ld_A, q.ld_B = 256, 512
    return w


def test_mdbf_argument_errors_and_workspace(lib):
    w = mdbf()
    need = lib.fqm_workspace_size(ctypes.byref(w), 16)
    # both passes' dense operands: batch slices of 64 // (3 l) = 10 batch
    # rows (2 slices), each with the first slice's 3 l x 10 = 60 columns in
    # 16-column blocks (64), K padded to 512; 2 bytes each
    assert need == 2 * 1 * 2 * 64 * (4096 + 2048)
    assert gemv(lib, w, batch=16, ws=None, wsb=0) == E["WORKSPACE"]
    assert gemv(lib, w, batch=16, ws=FAKE, wsb=need - 4) == E["WORKSPACE"]
    assert gemv(lib, mdbf(l=0)) == E["FORMAT"]
    assert gemv(lib, mdbf(l=17)) == E["FORMAT"]
    assert gemv(lib, mdbf(P=3)) == E["FORMAT"]
    assert gemv(lib, mdbf(m=4100)) == E["SHAPE"]
    w = mdbf()
    w.mdbf.path[0].ld_A = 240   # < ceil(2000/8)
    assert gemv(lib, w) == E["SHAPE"]
    # batch 3: one slice of 18 columns -> two 16-column blocks, per path
    assert lib.fqm_workspace_size(ctypes.byref(mdbf(P=2)), 3) == 2 * 2 * 1 * 32 * (4096 + 2048)
    # batch 1: one 16-column block
    assert lib.fqm_workspace_size(ctypes.byref(mdbf()), 1) == 2 * 1 * 1 * 16 * (4096 + 2048)
    assert lib.fqm_dequant(ctypes.byref(mdbf()), FAKE, None) == E["UNSUPPORTED"]
    assert gemm(lib, mdbf(), M=1) == E["UNSUPPORTED"]


def test_zero_cols_needs_no_x_and_no_workspace(lib):
    """cols == 0 is an empty sum: y (or Y) is zero-filled by a kernel, x / X
    may be NULL, and no K parts need a workspace.  The argument checks let
    such a call through (the fill itself runs in the GPU tests)."""
    w = lut6(cols=0, ld=16)
    assert lib.fqm_gemm_workspace_size(ctypes.byref(w), 300) == 0
    assert refused_before_launch(lib, lambda: gemm(lib, w, X=None, M=300)) == E["BOUNDS"]
    assert refused_before_launch(lib, lambda: gemv(lib, w, x=None, batch=3)) == E["BOUNDS"]
    assert gemm(lib, w, X=None, Y=None, M=300) == E["NULL"]


# ---- the Python binding refuses operands the C ABI cannot check -------------
import numpy as np  # noqa: E402
import torch  # noqa: E402


def _host_lut6(rows=4, cols=64):
    return fqm.Lut6Weights(torch.zeros((rows, 48), dtype=torch.uint8),
                           torch.zeros((rows, 64), dtype=torch.bfloat16), rows, cols)


@pytest.mark.parametrize("bad", ["dtype", "cols", "strided", "host", "ndim"])
def test_binding_rejects_bad_x(bad):
    w = _host_lut6()
    x = {"dtype": torch.zeros((1, 64), dtype=torch.float32),
         "cols": torch.zeros((1, 60), dtype=torch.bfloat16),
         "strided": torch.zeros((64, 2), dtype=torch.bfloat16).t(),
         "host": torch.zeros((1, 64), dtype=torch.bfloat16),
         "ndim": torch.zeros((1, 1, 64), dtype=torch.bfloat16)}[bad]
    with pytest.raises(ValueError):
        fqm.gemv(w, x)
    if x.dim() == 2:
        with pytest.raises(ValueError):
            fqm.gemm(w, x)


@pytest.mark.parametrize("bad", ["shape", "dtype", "strided"])
def test_binding_rejects_bad_y(bad):
    w = _host_lut6()
    y = {"shape": torch.zeros((2, 4), dtype=torch.bfloat16),
         "dtype": torch.zeros((1, 4), dtype=torch.float16),
         "strided": torch.zeros((4, 1), dtype=torch.float32).t()[:, :]}[bad]
    if bad == "strided":
        y = torch.zeros((4, 2), dtype=torch.float32)[:, :1].t()
    with pytest.raises(ValueError):
        fqm.gemv(w, torch.zeros((1, 64), dtype=torch.bfloat16), y=y)


def test_binding_rejects_bad_gemm_output():
    w = _host_lut6()
    X = torch.zeros((3, 64), dtype=torch.bfloat16)
    for Y in (torch.zeros((3, 5), dtype=torch.bfloat16), torch.zeros((3, 4), dtype=torch.float32)):
        with pytest.raises(ValueError):
            fqm.gemm(w, X, Y=Y)


@pytest.mark.parametrize("row_of", [[0, 1, 1, 3], [0, 1, 2], [0, 1, 2, 4]])
def test_fabq_row_map_must_be_a_permutation(row_of):
    """A repeated or out-of-range output row would make the kernels write one
    output twice or outside y: refused on the host before any upload."""
    rows, cols, bs = 4, 64, 64
    with pytest.raises(ValueError):
        fqm.FabqWeights.from_arrays(rows, cols, bs, 1, np.asarray(row_of, np.int32),
                                    np.zeros((1, cols), np.int8), np.zeros(1, np.uint16),
                                    np.zeros((3, cols), np.uint8), np.zeros((3, 1), np.uint16),
                                    np.zeros((3, 1), np.uint8), np.zeros(16, np.uint16),
                                    device="cpu")


def test_gemv_static_rejects_more_than_its_scratch(lib):
    """fqm_gemv_static refuses, before any device call, a request whose
    workspace exceeds the static array (16 MiB): MDBF with 16 envelopes and
    two paths at batch 16 on the 5120 x 17408 shape needs 66 MB (16 slices
    of one batch row, 48 columns each)."""
    w = fqm._Weights()
    w.format, w.rows, w.cols = fqm.FQM_MDBF, 5120, 17408
    w.mdbf.r, w.mdbf.l, w.mdbf.P = 4096, 16, 2
    for p in range(2):
        q = w.mdbf.path[p]
        q.S_A, q.ld_A, q.S_B, q.ld_B = FAKE, 512, FAKE, 2176
        q.A_amp = q.B_amp = q.Q_U = q.Q_V = FAKE
    need = lib.fqm_workspace_size(ctypes.byref(w), 16)
    assert need == 2 * 2 * 16 * 48 * (17408 + 4096) > fqm.STATIC_SCRATCH_BYTES
    rc = lib.fqm_gemv_static(ctypes.byref(w), FAKE, FAKE, 0, 16, None)
    assert rc == 8 and lib.fqm_status_str(rc).startswith(b"needs more scratch")
    assert lib.fqm_gemv_static(ctypes.byref(w), FAKE, FAKE, 0, 17, None) == E["SHAPE"]
    assert lib.fqm_gemv_static(None, FAKE, FAKE, 0, 1, None) == E["NULL"]


def test_fabq_variant_argument_errors(lib):
    """The descriptor's variant fields are checked on the host: blocksizes 16
    and 32 pass, other widths, high-row widths, codebook modes and windows are
    refused; the tiered modes need the tier array, the vector mode its
    vector codebook; int8 rows need cols bytes per row."""
    for bs in (16, 32):
        assert refused_before_launch(lib, lambda: gemv(lib, fabq(bs=bs))) == E["BOUNDS"]
    assert gemv(lib, fabq(bs=8)) == E["FORMAT"]
    for field, bad in (("hi_bits", 6), ("cb_mode", 3), ("cb_mode", -1)):
        w = fabq()
        setattr(w.fabq, field, bad)
        assert gemv(lib, w) == E["FORMAT"], field
    for mode in (1, 2):
        w = fabq()
        w.fabq.cb_mode, w.fabq.cb_base = mode, 8  # not a multiple of 16
        assert gemv(lib, w) == E["FORMAT"]
        w.fabq.cb_base = 48
        w.fabq.tier = None
        assert gemv(lib, w) == E["NULL"]
    w = fabq()
    w.fabq.cb_mode, w.fabq.tier, w.fabq.vcodebook = 2, FAKE, None
    assert gemv(lib, w) == E["NULL"]
    w.fabq.vcodebook, w.fabq.codebook = FAKE, None  # the vector mode needs no fp16 codebook
    assert refused_before_launch(lib, lambda: gemv(lib, w)) == E["BOUNDS"]
    w = fabq()
    w.fabq.hi_bits = 8  # int8 rows: ld_q4 >= cols = 512 bytes
    assert gemv(lib, w) == E["SHAPE"]
    w.fabq.ld_q4 = 512
    assert refused_before_launch(lib, lambda: gemv(lib, w)) == E["BOUNDS"]
    assert lib.fqm_pack_bits(FAKE, FAKE, 0, 64, 8, 64, None, None) == E["OK"]  # 8-bit fields


def test_debug_switch_and_host_pointers(lib):
    """fqm_set_debug returns the previous setting; with the checks on, a call
    whose buffers are not device allocations (host addresses here) returns
    FQM_E_BOUNDS before anything is enqueued, where the same call with the
    checks off would have been accepted by the argument checks."""
    prev = lib.fqm_set_debug(1)
    try:
        assert lib.fqm_set_debug(1) == 1
        w = lut6()
        assert gemv(lib, w) == E["BOUNDS"]
        assert gemm(lib, w, M=64) == E["BOUNDS"]
        assert lib.fqm_dequant(ctypes.byref(w), FAKE, None) == E["BOUNDS"]
        assert lib.fqm_unpack(FAKE, FAKE, 4, 64, 48, None) == E["BOUNDS"]
        assert lib.fqm_pack(FAKE, FAKE, 4, 64, 48, None, None) == E["BOUNDS"]
        # argument errors still come first
        assert gemv(lib, w, batch=0) == E["SHAPE"]
        assert lib.fqm_status_str(E["BOUNDS"]).startswith(b"debug checks")
    finally:
        lib.fqm_set_debug(prev)
    assert lib.fqm_set_debug(prev) == prev


@pytest.mark.parametrize("env,expect", [("1", 1), ("0", 0), ("", 0), (None, 0)])
def test_debug_setting_starts_from_the_environment(lib, env, expect):
    """The first fqm_set_debug call returns the setting FQM_DEBUG gave
    (a fresh process, so the variable is read on first use)."""
    import subprocess
    import sys
    code = ("import ctypes, sys; sys.path.insert(0, %r); import dequant_matmul_amd as f; "
            "l = f.load(); print(l.fqm_set_debug(0))" % ROOT)
    e = dict(os.environ)
    e.pop("FQM_DEBUG", None)
    if env is not None:
        e["FQM_DEBUG"] = env
    out = subprocess.run([sys.executable, "-c", code], env=e, capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip().splitlines()[-1] == str(expect)
