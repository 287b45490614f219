"""Python binding for ``libfqm.so`` (fused low-bit dequant-matmul on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/fqm.h``.  PyTorch supplies
device memory and the current HIP stream; the functions take and return
``torch`` tensors on a ROCm device.  There is no CPU fallback: if the library
is not built, importing works but every call raises ``FqmNotBuilt``.

Functions mirror the C ABI names: ``pack_bits``, ``pack``, ``unpack``,
``dequant``, ``workspace_size``, ``gemv``, ``gemv_static``, ``gemm_workspace_size``, ``gemm``,
``version``, ``set_debug``,
``status_str``.  Weight descriptors are built with ``Lut6Weights``,
``FabqWeights`` and ``MdbfWeights``; their ``from_*`` constructors upload
unpacked host arrays and pack them on the GPU with ``fqm_pack_bits``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfqm.so")

FQM_LUT6, FQM_FABQ, FQM_MDBF, FQM_LUT4 = 1, 2, 3, 4
FQM_CB_SCALAR16, FQM_CB_TIERED, FQM_CB_VECTOR = 0, 1, 2
FQM_BF16, FQM_F32 = 0, 1

__all__ = [
    "FqmError", "FqmNotBuilt", "load", "version", "set_debug", "status_str", "pack_bits", "pack",
    "unpack", "dequant", "workspace_size", "gemv", "gemv_static", "gemm_workspace_size", "gemm", "Lut6Weights", "Lut4Weights", "FabqWeights",
    "MdbfWeights", "SYMBOLS",
]

# Every symbol include/fqm.h declares.
SYMBOLS = ("fqm_version", "fqm_set_debug", "fqm_status_str", "fqm_pack_bits", "fqm_pack", "fqm_unpack",
           "fqm_dequant", "fqm_workspace_size", "fqm_gemv", "fqm_gemv_static",
           "fqm_gemm_workspace_size", "fqm_gemm")
STATIC_SCRATCH_BYTES = 16 << 20  # FQM_STATIC_SCRATCH_BYTES


class FqmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} (status {status})")


class FqmNotBuilt(RuntimeError):
    pass


# ---------------------------------------------------------------------------
# ctypes mirrors of the descriptor structs
# ---------------------------------------------------------------------------
c_void_p, c_int32, c_int64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64


class _Lut6(ctypes.Structure):
    _fields_ = [("packed", c_void_p), ("lut", c_void_p), ("ld", c_int64)]


class _Fabq(ctypes.Structure):
    _fields_ = [("blocksize", c_int32), ("n_hi", c_int32), ("row_of", c_void_p),
                ("q4", c_void_p), ("ld_q4", c_int64), ("s_hi", c_void_p),
                ("signs", c_void_p), ("ld_signs", c_int64), ("s_blk", c_void_p),
                ("idx", c_void_p), ("ld_idx", c_int64), ("codebook", c_void_p),
                ("hi_bits", c_int32), ("cb_mode", c_int32), ("cb_base", c_int32),
                ("tier", c_void_p), ("vcodebook", c_void_p)]


class _MdbfPath(ctypes.Structure):
    _fields_ = [("S_A", c_void_p), ("ld_A", c_int64), ("S_B", c_void_p), ("ld_B", c_int64),
                ("A_amp", c_void_p), ("B_amp", c_void_p), ("Q_U", c_void_p), ("Q_V", c_void_p)]


class _Mdbf(ctypes.Structure):
    _fields_ = [("r", c_int32), ("l", c_int32), ("P", c_int32), ("path", _MdbfPath * 2)]


class _Lut4(ctypes.Structure):
    _fields_ = [("packed", c_void_p), ("lut", c_void_p), ("ld", c_int64)]


class _Weights(ctypes.Structure):
    _fields_ = [("format", c_int32), ("rows", c_int64), ("cols", c_int64), ("lut6", _Lut6),
                ("fabq", _Fabq), ("mdbf", _Mdbf), ("lut4", _Lut4)]


_lib = None


def load():
    """Load ``libfqm.so`` (once).  Raises ``FqmNotBuilt`` if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise FqmNotBuilt(f"{LIB_PATH} is missing; build it with `python -m dequant_matmul_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    lib.fqm_version.restype = c_int32
    lib.fqm_set_debug.restype = c_int32
    lib.fqm_set_debug.argtypes = [c_int32]
    lib.fqm_status_str.restype = ctypes.c_char_p
    lib.fqm_status_str.argtypes = [c_int32]
    lib.fqm_pack_bits.restype = c_int32
    lib.fqm_pack_bits.argtypes = [c_void_p, c_void_p, c_int64, c_int64, c_int32, c_int64, c_void_p, c_void_p]
    lib.fqm_pack.restype = c_int32
    lib.fqm_pack.argtypes = [c_void_p, c_void_p, c_int64, c_int64, c_int64, c_void_p, c_void_p]
    lib.fqm_unpack.restype = c_int32
    lib.fqm_unpack.argtypes = [c_void_p, c_void_p, c_int64, c_int64, c_int64, c_void_p]
    lib.fqm_dequant.restype = c_int32
    lib.fqm_dequant.argtypes = [P(_Weights), c_void_p, c_void_p]
    lib.fqm_workspace_size.restype = ctypes.c_size_t
    lib.fqm_workspace_size.argtypes = [P(_Weights), c_int32]
    lib.fqm_gemv.restype = c_int32
    lib.fqm_gemv.argtypes = [P(_Weights), c_void_p, c_void_p, c_int32, c_int32, c_void_p,
                             ctypes.c_size_t, c_void_p]
    lib.fqm_gemv_static.restype = c_int32
    lib.fqm_gemv_static.argtypes = [P(_Weights), c_void_p, c_void_p, c_int32, c_int32, c_void_p]
    lib.fqm_gemm.restype = c_int32
    lib.fqm_gemm.argtypes = [P(_Weights), c_void_p, c_void_p, c_int64, c_void_p, ctypes.c_size_t, c_void_p]
    lib.fqm_gemm_workspace_size.restype = ctypes.c_size_t
    lib.fqm_gemm_workspace_size.argtypes = [P(_Weights), c_int64]
    _lib = lib
    return lib


def version() -> int:
    return load().fqm_version()


def set_debug(on: bool) -> bool:
    """Turn the library's debug checks on or off (``fqm_set_debug``): every
    call then checks that each buffer lies inside one device allocation of
    its size and waits for its kernels.  Returns the previous setting; the
    first setting comes from the environment variable ``FQM_DEBUG``."""
    return bool(load().fqm_set_debug(1 if on else 0))


def status_str(status: int) -> str:
    try:
        return load().fqm_status_str(status).decode()
    except FqmNotBuilt:
        return f"status {status}"


def _check(status: int, where: str):
    if status != 0:
        raise FqmError(status, where)


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else c_void_p(t.data_ptr())


def _dev(a, dtype, device):
    """Host array (numpy) or tensor -> contiguous device tensor of ``dtype``."""
    if isinstance(a, np.ndarray):
        a = torch.from_numpy(np.ascontiguousarray(a))
    return a.to(device=device).contiguous().view(dtype) if a.dtype.itemsize == dtype.itemsize \
        else a.to(device=device, dtype=dtype).contiguous()


def _round16(n: int) -> int:
    return (n + 15) // 16 * 16


# ---------------------------------------------------------------------------
# packing
# ---------------------------------------------------------------------------
def pack_bits(vals: torch.Tensor, bits: int, ld: int | None = None, err: torch.Tensor | None = None,
              stream=None) -> torch.Tensor:
    """Pack uint8 fields [rows][cols] into [rows][ld] bytes on the GPU."""
    rows, cols = vals.shape
    ld = _round16((cols * bits + 7) // 8) if ld is None else ld
    out = torch.empty((rows, ld), dtype=torch.uint8, device=vals.device)
    _check(load().fqm_pack_bits(_ptr(vals.contiguous()), _ptr(out), rows, cols, bits, ld,
                                _ptr(err), _stream(stream)), "fqm_pack_bits")
    return out


def pack(codes: torch.Tensor, ld: int | None = None, err: torch.Tensor | None = None,
         stream=None) -> torch.Tensor:
    """Pack 6-bit LUT codes, four per three bytes."""
    rows, cols = codes.shape
    ld = _round16(cols * 3 // 4) if ld is None else ld
    out = torch.empty((rows, ld), dtype=torch.uint8, device=codes.device)
    _check(load().fqm_pack(_ptr(codes.contiguous()), _ptr(out), rows, cols, ld, _ptr(err),
                           _stream(stream)), "fqm_pack")
    return out


def unpack(packed: torch.Tensor, cols: int, stream=None) -> torch.Tensor:
    rows, ld = packed.shape
    out = torch.empty((rows, cols), dtype=torch.uint8, device=packed.device)
    _check(load().fqm_unpack(_ptr(packed), _ptr(out), rows, cols, ld, _stream(stream)), "fqm_unpack")
    return out


# ---------------------------------------------------------------------------
# weight descriptors
# ---------------------------------------------------------------------------
class _WeightsBase:
    fmt = 0

    def __init__(self, rows: int, cols: int):
        self.rows, self.cols = int(rows), int(cols)
        self.desc = _Weights()
        self.desc.format = self.fmt
        self.desc.rows = self.rows
        self.desc.cols = self.cols
        self._keep = []

    def _hold(self, t):
        self._keep.append(t)
        return _ptr(t)

    @property
    def ref(self):
        return ctypes.byref(self.desc)


class Lut6Weights(_WeightsBase):
    """Per-row LUT 6-bit weights: packed [rows][ld] uint8, lut [rows][64] bf16."""
    fmt = FQM_LUT6

    def __init__(self, packed: torch.Tensor, lut: torch.Tensor, rows: int, cols: int):
        super().__init__(rows, cols)
        self.packed, self.lut = packed, lut
        self.desc.lut6.packed = self._hold(packed)
        self.desc.lut6.lut = self._hold(lut)
        self.desc.lut6.ld = packed.shape[1] if packed.dim() == 2 else 0

    @classmethod
    def from_codes(cls, codes, lut_bits, device="cuda", ld: int | None = None):
        codes_d = _dev(codes, torch.uint8, device)
        lut_d = _dev(lut_bits, torch.int16, device).view(torch.bfloat16)
        rows, cols = codes_d.shape
        packed = pack(codes_d, ld=ld)
        return cls(packed, lut_d, rows, cols)

    def clone(self):
        return Lut6Weights(self.packed.clone(), self.lut.clone(), self.rows, self.cols)

    def nbytes(self) -> int:
        """Algorithmic bytes: packed codes (unpadded) + tables."""
        return self.rows * self.cols * 3 // 4 + self.rows * 128


class Lut4Weights(_WeightsBase):
    """Per-row LUT 4-bit weights: packed [rows][ld] uint8 (two codes per byte),
    lut [rows][16] bf16."""
    fmt = FQM_LUT4

    def __init__(self, packed: torch.Tensor, lut: torch.Tensor, rows: int, cols: int):
        super().__init__(rows, cols)
        self.packed, self.lut = packed, lut
        self.desc.lut4.packed = self._hold(packed)
        self.desc.lut4.lut = self._hold(lut)
        self.desc.lut4.ld = packed.shape[1] if packed.dim() == 2 else 0

    @classmethod
    def from_codes(cls, codes, lut_bits, device="cuda", ld: int | None = None):
        codes_d = _dev(codes, torch.uint8, device)
        lut_d = _dev(lut_bits, torch.int16, device).view(torch.bfloat16)
        rows, cols = codes_d.shape
        packed = pack_bits(codes_d, 4, ld=ld)
        return cls(packed, lut_d, rows, cols)

    def clone(self):
        return Lut4Weights(self.packed.clone(), self.lut.clone(), self.rows, self.cols)

    def nbytes(self) -> int:
        """Algorithmic bytes: packed codes (unpadded) + tables."""
        return self.rows * self.cols // 2 + self.rows * 32


class FabqWeights(_WeightsBase):
    """FABQ-RC-style weights; see ``fqm_fabq`` in include/fqm.h for the layout."""
    fmt = FQM_FABQ

    def __init__(self, rows, cols, blocksize, n_hi, row_of, q4, s_hi, signs, s_blk, idx, codebook,
                 hi_bits=4, cb_mode=FQM_CB_SCALAR16, cb_base=0, tier=None, vcodebook=None):
        super().__init__(rows, cols)
        self.blocksize, self.n_hi = int(blocksize), int(n_hi)
        self.hi_bits, self.cb_mode, self.cb_base = int(hi_bits), int(cb_mode), int(cb_base)
        self.tensors = dict(row_of=row_of, q4=q4, s_hi=s_hi, signs=signs, s_blk=s_blk, idx=idx,
                            codebook=codebook, tier=tier, vcodebook=vcodebook)
        f = self.desc.fabq
        f.blocksize, f.n_hi = self.blocksize, self.n_hi
        f.row_of = self._hold(row_of)
        f.q4, f.ld_q4 = self._hold(q4), q4.shape[1]
        f.s_hi = self._hold(s_hi)
        f.signs, f.ld_signs = self._hold(signs), signs.shape[1]
        f.s_blk = self._hold(s_blk)
        f.idx, f.ld_idx = self._hold(idx), idx.shape[1]
        f.codebook = self._hold(codebook)
        f.hi_bits, f.cb_mode, f.cb_base = self.hi_bits, self.cb_mode, self.cb_base
        f.tier = self._hold(tier) if tier is not None else None
        f.vcodebook = self._hold(vcodebook) if vcodebook is not None else None

    @classmethod
    def from_arrays(cls, rows, cols, blocksize, n_hi, row_of, q4, s_hi, signs, s_blk, idx,
                    codebook, device="cuda", hi_bits=4, cb_mode=FQM_CB_SCALAR16, cb_base=0,
                    tier=None, vcodebook=None):
        """Unpacked host arrays (as the synthetic generator returns them) ->
        device tensors, with the high rows (hi_bits-wide fields), signs and
        indices packed on the GPU.  codebook: [16] fp16 bits (scalar mode) or
        [4][64] (tiered); tier: [rows - n_hi] 0..3 (tiered and vector modes);
        vcodebook: [4][64][128] float32 (vector mode)."""
        n_lo = rows - n_hi
        nb = cols // blocksize
        ro = np.asarray(row_of).reshape(-1)
        if ro.shape != (rows,) or not np.array_equal(np.sort(ro), np.arange(rows)):
            raise ValueError("row_of must be a permutation of range(rows): each output row is "
                             "written by exactly one stored row")
        if hi_bits not in (4, 8) or cb_mode not in (0, 1, 2):
            raise ValueError("hi_bits must be 4 or 8 and cb_mode 0, 1 or 2")
        if cb_mode and (tier is None or np.asarray(tier).shape != (n_lo,)):
            raise ValueError("the tiered codebook modes need one tier per binary row")
        if cb_mode == FQM_CB_VECTOR and (vcodebook is None or np.asarray(vcodebook).size != 4 * 64 * 128):
            raise ValueError("the vector codebook mode needs a [4][64][128] float32 vcodebook")
        mask = (1 << hi_bits) - 1
        q_d = _dev((np.asarray(q4).astype(np.int16) & mask).astype(np.uint8).reshape(n_hi, cols),
                   torch.uint8, device)
        signs_d = _dev(np.asarray(signs, dtype=np.uint8).reshape(n_lo, cols), torch.uint8, device)
        idx_d = _dev(np.asarray(idx, dtype=np.uint8).reshape(n_lo, nb), torch.uint8, device)
        q_p = pack_bits(q_d, hi_bits, ld=max(16, _round16(cols * hi_bits // 8)))
        signs_p = pack_bits(signs_d, 1, ld=max(16, _round16(cols // 8)))
        idx_p = pack_bits(idx_d, 4, ld=max(16, _round16((nb + 1) // 2)))

        def t16(a):
            return _dev(np.asarray(a, dtype=np.uint16).view(np.int16), torch.int16, device)

        cb = np.asarray(codebook, dtype=np.uint16).reshape(-1)
        tier_d = _dev(np.asarray(tier, dtype=np.uint8), torch.uint8, device) if cb_mode else None
        v_d = (_dev(np.asarray(vcodebook, dtype=np.float32).reshape(4, 64, 128), torch.float32, device)
               if cb_mode == FQM_CB_VECTOR else None)
        return cls(rows, cols, blocksize, n_hi,
                   _dev(np.asarray(row_of, dtype=np.int32), torch.int32, device),
                   q_p, t16(s_hi).view(torch.float16), signs_p,
                   t16(np.asarray(s_blk).reshape(n_lo, nb)).view(torch.float16), idx_p,
                   t16(cb).view(torch.float16), hi_bits=hi_bits, cb_mode=cb_mode, cb_base=cb_base,
                   tier=tier_d, vcodebook=v_d)

    def clone(self):
        t = {k: (v.clone() if v is not None else None) for k, v in self.tensors.items()}
        return FabqWeights(self.rows, self.cols, self.blocksize, self.n_hi, t["row_of"], t["q4"],
                           t["s_hi"], t["signs"], t["s_blk"], t["idx"], t["codebook"],
                           hi_bits=self.hi_bits, cb_mode=self.cb_mode, cb_base=self.cb_base,
                           tier=t["tier"], vcodebook=t["vcodebook"])

    def nbytes(self) -> int:
        """Algorithmic bytes: high rows + scales, sign bits + block scales +
        4-bit indices, the codebook (16 or 4 x 64 fp16, or 4 x 64 x 128
        fp32), tier bytes and the row map (all unpadded)."""
        n_lo = self.rows - self.n_hi
        nb = self.cols // self.blocksize
        cb = {FQM_CB_SCALAR16: 32, FQM_CB_TIERED: 4 * 64 * 2, FQM_CB_VECTOR: 4 * 64 * 128 * 4}[self.cb_mode]
        tier = n_lo if self.cb_mode else 0
        return (self.n_hi * self.cols * self.hi_bits // 8 + 2 * self.n_hi + n_lo * self.cols // 8
                + n_lo * nb * 2 + (n_lo * nb + 1) // 2 + cb + tier + 4 * self.rows)


class MdbfWeights(_WeightsBase):
    """MDBF weights (rows = n, cols = m), P paths of sign matrices + envelopes."""
    fmt = FQM_MDBF

    def __init__(self, n, m, r, l, paths):
        super().__init__(n, m)
        self.r, self.l, self.P = int(r), int(l), len(paths)
        self.paths = paths
        md = self.desc.mdbf
        md.r, md.l, md.P = self.r, self.l, self.P
        for p, t in enumerate(paths):
            q = md.path[p]
            q.S_A, q.ld_A = self._hold(t["S_A"]), t["S_A"].shape[1]
            q.S_B, q.ld_B = self._hold(t["S_B"]), t["S_B"].shape[1]
            q.A_amp, q.B_amp = self._hold(t["A_amp"]), self._hold(t["B_amp"])
            q.Q_U, q.Q_V = self._hold(t["Q_U"]), self._hold(t["Q_V"])

    @classmethod
    def from_arrays(cls, n, m, r, l, S_A, S_B, A_amp, B_amp, Q_U, Q_V, device="cuda"):
        """Lists (one entry per path) of unpacked host arrays -> device tensors,
        sign matrices packed on the GPU (rows padded to 16 bytes)."""
        paths = []

        def t16(a):
            return _dev(np.asarray(a, dtype=np.uint16).view(np.int16), torch.int16, device).view(torch.float16)

        for p in range(len(S_A)):
            sa = pack_bits(_dev(np.asarray(S_A[p], np.uint8), torch.uint8, device), 1,
                           ld=_round16((r + 7) // 8))
            sb = pack_bits(_dev(np.asarray(S_B[p], np.uint8), torch.uint8, device), 1,
                           ld=_round16((m + 7) // 8))
            paths.append(dict(S_A=sa, S_B=sb, A_amp=t16(A_amp[p]), B_amp=t16(B_amp[p]),
                              Q_U=t16(Q_U[p]), Q_V=t16(Q_V[p])))
        return cls(n, m, r, l, paths)

    def clone(self):
        return MdbfWeights(self.rows, self.cols, self.r, self.l,
                           [{k: v.clone() for k, v in t.items()} for t in self.paths])

    def nbytes(self) -> int:
        """Algorithmic bytes: sign bits (unpadded) + fp16 envelopes, all paths."""
        n, m, r, l = self.rows, self.cols, self.r, self.l
        return self.P * ((n * r + r * m + 7) // 8 + 2 * l * (n + m + 2 * r))


# ---------------------------------------------------------------------------
# compute
# ---------------------------------------------------------------------------
def dequant(w: _WeightsBase, stream=None) -> torch.Tensor:
    """Test helper: decoded W [rows][cols] as bf16."""
    dev = next(t.device for t in w._keep)
    out = torch.empty((w.rows, w.cols), dtype=torch.bfloat16, device=dev)
    _check(load().fqm_dequant(w.ref, _ptr(out), _stream(stream)), "fqm_dequant")
    return out


def _weights_device(w: _WeightsBase):
    return next((t.device for t in w._keep if isinstance(t, torch.Tensor)), None)


def _check_operand(t: torch.Tensor, name: str, shape: tuple, dtypes: tuple, device):
    """The C ABI sees only a pointer, so a wrong dtype, shape, layout or
    device would read or write past the tensor: refuse it here."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}; expected one of {dtypes}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}; expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major)")
    if t.device.type != "cuda":
        raise ValueError(f"{name} is on {t.device}; the library takes GPU tensors")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device} but the weights are on {device}")


def _check_workspace(ws, device):
    if ws is None:
        return
    if not isinstance(ws, torch.Tensor) or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous torch.Tensor")
    if ws.device.type != "cuda" or (device is not None and ws.device != device):
        raise ValueError(f"workspace is on {ws.device}; expected the weights' device {device}")


def workspace_size(w: _WeightsBase, batch: int) -> int:
    return int(load().fqm_workspace_size(w.ref, batch))


def gemv(w: _WeightsBase, x: torch.Tensor, y: torch.Tensor | None = None,
         out_dtype: torch.dtype = torch.bfloat16, workspace: torch.Tensor | None = None,
         stream=None) -> torch.Tensor:
    """y[batch][rows] = x[batch][cols] W^T (batch 1..16), decoded in-kernel."""
    if not isinstance(x, torch.Tensor):
        raise ValueError("x must be a torch.Tensor")
    if x.dim() == 1:
        x = x[None]
    if x.dim() != 2:
        raise ValueError(f"x must be [batch][cols]; got shape {tuple(x.shape)}")
    batch = x.shape[0]
    dev = _weights_device(w)
    _check_operand(x, "x", (batch, w.cols), (torch.bfloat16,), dev)
    if y is None:
        if out_dtype not in (torch.bfloat16, torch.float32):
            raise ValueError(f"out_dtype must be bfloat16 or float32, not {out_dtype}")
        y = torch.empty((batch, w.rows), dtype=out_dtype, device=x.device)
    _check_operand(y, "y", (batch, w.rows), (torch.bfloat16, torch.float32), dev)
    _check_workspace(workspace, dev)
    ydt = FQM_F32 if y.dtype == torch.float32 else FQM_BF16
    need = workspace_size(w, batch)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().fqm_gemv(w.ref, _ptr(x), _ptr(y), ydt, batch, _ptr(workspace), ws_bytes,
                           _stream(stream)), "fqm_gemv")
    return y


def gemv_static(w: _WeightsBase, x: torch.Tensor, y: torch.Tensor | None = None,
                out_dtype: torch.dtype = torch.bfloat16, stream=None) -> torch.Tensor:
    """``gemv`` through ``fqm_gemv_static``: no workspace; the library's
    per-GPU static scratch stands in for it (calls overlapping on one GPU
    race).  With ``y`` given, nothing is allocated."""
    if not isinstance(x, torch.Tensor):
        raise ValueError("x must be a torch.Tensor")
    if x.dim() == 1:
        x = x[None]
    if x.dim() != 2:
        raise ValueError(f"x must be [batch][cols]; got shape {tuple(x.shape)}")
    batch = x.shape[0]
    dev = _weights_device(w)
    _check_operand(x, "x", (batch, w.cols), (torch.bfloat16,), dev)
    if y is None:
        if out_dtype not in (torch.bfloat16, torch.float32):
            raise ValueError(f"out_dtype must be bfloat16 or float32, not {out_dtype}")
        y = torch.empty((batch, w.rows), dtype=out_dtype, device=x.device)
    _check_operand(y, "y", (batch, w.rows), (torch.bfloat16, torch.float32), dev)
    ydt = FQM_F32 if y.dtype == torch.float32 else FQM_BF16
    _check(load().fqm_gemv_static(w.ref, _ptr(x), _ptr(y), ydt, batch, _stream(stream)),
           "fqm_gemv_static")
    return y


def gemm_workspace_size(w: _WeightsBase, M: int) -> int:
    return int(load().fqm_gemm_workspace_size(w.ref, M))


def gemm(w: _WeightsBase, X: torch.Tensor, Y: torch.Tensor | None = None,
         workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Y[M][rows] = X[M][cols] W^T in bf16 with fp32 accumulation (LUT6 or LUT4 weights)."""
    if not isinstance(X, torch.Tensor) or X.dim() != 2:
        raise ValueError("X must be a 2-D torch.Tensor [M][cols]")
    M = X.shape[0]
    dev = _weights_device(w)
    _check_operand(X, "X", (M, w.cols), (torch.bfloat16,), dev)
    if Y is None:
        Y = torch.empty((M, w.rows), dtype=torch.bfloat16, device=X.device)
    _check_operand(Y, "Y", (M, w.rows), (torch.bfloat16,), dev)
    _check_workspace(workspace, dev)
    need = gemm_workspace_size(w, M)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().fqm_gemm(w.ref, _ptr(X), _ptr(Y), M, _ptr(workspace), ws_bytes, _stream(stream)),
           "fqm_gemm")
    return Y
