"""Comparison rule between a GPU result and the fp64 oracle.

Test infrastructure only.

fp32 outputs:  rel-L2 = ||y - yo|| / ||yo|| <= 1e-3 and
               max_i |y_i - yo_i| / max(|yo_i|, 1e-3 * rms(yo)) <= 5e-3.
bf16 outputs:  rel-L2 against yo rounded to bf16 (RNE) <= 1e-3, and the same
               floored elementwise bound against the unrounded yo <= 5e-3.

Rounding a result to bf16 alone costs about 1.6e-3 rel-L2 against the
unrounded value, so a literal 1e-3 gate on bf16 outputs would reject every
implementation; the elementwise bound stays against the unrounded value
because a one-ulp flip of the rounded oracle is up to 2^-7 relative.  The
floor 1e-3 * rms keeps the elementwise ratio meaningful near zero outputs,
where fp32 reassociation error (about u * sqrt(K) * rms) dominates.
"""
import numpy as np

from .numerics import f64_to_bf16_rne

REL_L2 = 1e-3
MAX_REL = 5e-3


def metrics(y, yo, out_dtype: str):
    y = np.asarray(y, dtype=np.float64)
    yo = np.asarray(yo, dtype=np.float64)
    ref_l2 = f64_to_bf16_rne(yo) if out_dtype == "bf16" else yo
    denom = np.linalg.norm(ref_l2)
    rel_l2 = float(np.linalg.norm(y - ref_l2) / denom) if denom > 0 else float(np.linalg.norm(y))
    rms = float(np.sqrt(np.mean(yo ** 2))) if yo.size else 0.0
    floor = max(1e-3 * rms, np.finfo(np.float64).tiny)
    err = np.abs(y - yo)
    max_rel = float((err / np.maximum(np.abs(yo), floor)).max()) if yo.size else 0.0
    nz = np.abs(yo) > 0
    literal_max_rel = float((err[nz] / np.abs(yo[nz])).max()) if nz.any() else 0.0
    literal_rel_l2 = float(np.linalg.norm(y - yo) / np.linalg.norm(yo)) if yo.size and np.linalg.norm(yo) > 0 else 0.0
    return dict(rel_l2=rel_l2, max_rel=max_rel, literal_rel_l2=literal_rel_l2,
                literal_max_rel=literal_max_rel)


def check(y, yo, out_dtype: str, rel_l2: float = REL_L2, max_rel: float = MAX_REL):
    m = metrics(y, yo, out_dtype)
    ok = m["rel_l2"] <= rel_l2 and m["max_rel"] <= max_rel
    return ok, m
