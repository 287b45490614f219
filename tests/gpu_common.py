"""Helpers shared by the GPU parity tests (inputs from the seeded generators,
expected values from the oracle only)."""
import functools

import numpy as np
import torch

import dequant_matmul_amd as fqm
import oracle
import synth

DEV = "cuda"


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


@functools.lru_cache(maxsize=None)
def lut6_case(rows, cols, seed):
    inp = synth.lut6_input(rows, cols, seed)
    return inp, oracle.lut6.pack_codes(inp.codes)


def lut6_weights(rows, cols, seed):
    inp, _ = lut6_case(rows, cols, seed)
    return fqm.Lut6Weights.from_codes(inp.codes, inp.lut, device=DEV)


def assert_close(y, yo, out_dtype, what=""):
    ok, m = oracle.compare.check(y, yo, out_dtype)
    assert ok, f"{what}: {m}"
    return m


def guarded(shape, dtype, guard=64, fill=-12345.0):
    """A tensor view with canary elements before and after it."""
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * guard,), fill, dtype=dtype, device=DEV)
    return buf, buf[guard:guard + n].view(shape)


def canaries_intact(buf, guard=64, fill=-12345.0):
    f = torch.tensor(fill, dtype=buf.dtype)
    return bool((buf[:guard].cpu() == f).all() and (buf[-guard:].cpu() == f).all())
