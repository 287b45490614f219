"""The C ABI on the CPU: the library loads, exports every declared symbol,
and rejects bad arguments on the host before anything touches a GPU."""
import ctypes
import os
import re

import pytest

import dequant_matmul_amd as fqm
from conftest import ROOT

E = dict(OK=0, NULL=1, ALIGN=2, SHAPE=3, FORMAT=4, WORKSPACE=5, UNSUPPORTED=6, HIP=7)
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
    assert lib.fqm_version() == 2


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
    for rows, cols, batch in ((5120, 17408, 8), (5120, 17408, 16), (17408, 5120, 8), (300, 4096, 2),
                              (5120, 17408, 1), (64, 1088, 4)):
        a = lib.fqm_workspace_size(ctypes.byref(lut4(rows, cols, ld=cols // 2)), batch)
        b = lib.fqm_workspace_size(ctypes.byref(lut6(rows, cols, ld=cols * 3 // 4)), batch)
        assert a == b, (rows, cols, batch)
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
    assert gemv(lib, fabq()) != E["FORMAT"]  # sanity: the base descriptor is valid
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
    # both passes' dense operands, 64 bf16 columns per batch slice (slices of
    # 64 // (3 l) = 10 batch rows -> 2 slices), K padded to 256
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
    assert lib.fqm_workspace_size(ctypes.byref(mdbf(P=2)), 3) == 2 * 2 * 1 * 64 * (4096 + 2048)
    assert lib.fqm_dequant(ctypes.byref(mdbf()), FAKE, None) == E["UNSUPPORTED"]
    assert gemm(lib, mdbf(), M=1) == E["UNSUPPORTED"]
