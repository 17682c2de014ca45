"""Tolerance check of a GPU result against the oracle (test infrastructure).

The bar: over the whole output tensor O (bf16 from the GPU, fp64 from the
oracle), max |O_gpu - O_ref| <= 1e-2 and ||O_gpu - O_ref||_2 / ||O_ref||_2
<= 5e-3; LSE within 1e-3 (absolute) wherever the oracle's LSE is finite; the
entries where the oracle gives LSE = -inf (empty selection) must be -inf on
the GPU with O == 0 exactly; no NaN anywhere.
"""
from __future__ import annotations

import numpy as np

MAX_ABS = 1e-2
REL_L2 = 5e-3
LSE_ABS = 1e-3


def check(out_gpu, lse_gpu, out_ref, lse_ref, max_abs=MAX_ABS, rel_l2=REL_L2, lse_abs=LSE_ABS):
    """Return (ok, metrics dict).  Arrays: out [..., H, 512], lse [..., H]."""
    o = np.asarray(out_gpu, np.float64)
    r = np.asarray(out_ref, np.float64)
    lg = np.asarray(lse_gpu, np.float64)
    lr = np.asarray(lse_ref, np.float64)
    assert o.shape == r.shape and lg.shape == lr.shape, (o.shape, r.shape, lg.shape, lr.shape)
    m = {"n": int(o.size)}
    reasons = []
    if np.isnan(o).any() or np.isnan(lg).any():
        reasons.append("NaN in GPU output")
    diff = np.abs(o - r)
    m["max_abs"] = float(np.nanmax(diff)) if diff.size else 0.0
    nr = float(np.linalg.norm(r))
    m["rel_l2"] = float(np.linalg.norm(np.nan_to_num(o - r)) / nr) if nr > 0 else float(np.linalg.norm(o))
    empty = np.isneginf(lr)
    m["empty"] = int(empty.sum())
    if (~np.isneginf(lg[empty])).any():
        reasons.append("LSE must be -inf where the selection is empty")
    if empty.any() and np.any(o[empty] != 0.0):
        reasons.append("O must be 0 where the selection is empty")
    fin = ~empty
    if (~np.isfinite(lg[fin])).any():
        reasons.append("non-finite GPU LSE where the oracle's is finite")
    m["lse_max_abs"] = float(np.max(np.abs(lg[fin] - lr[fin]))) if fin.any() else 0.0
    if m["max_abs"] > max_abs:
        reasons.append(f"max_abs {m['max_abs']:.3g} > {max_abs}")
    if m["rel_l2"] > rel_l2:
        reasons.append(f"rel_l2 {m['rel_l2']:.3g} > {rel_l2}")
    if m["lse_max_abs"] > lse_abs:
        reasons.append(f"lse_max_abs {m['lse_max_abs']:.3g} > {lse_abs}")
    m["reasons"] = reasons
    return not reasons, m
