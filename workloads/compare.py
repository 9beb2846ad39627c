"""Error metric used to compare a result with the fp64 oracle.

err = max_i |g_i - r_i| / max(|r_i|, rms(r)), with rms over the whole tensor.

A pure element-wise relative error is ill-posed where r_i is near zero by
cancellation in the readout sum; the rms floor measures error relative to the
data's own scale there.  Mismatched NaN/Inf positions give err = inf.
"""
from __future__ import annotations

import math
from typing import Dict

import numpy as np


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):
        import torch

        a = a.detach().to("cpu")
        if a.dtype in (torch.bfloat16, torch.float16):
            a = a.to(torch.float32)
        a = a.numpy()
    return np.asarray(a, dtype=np.float64)


def max_rel_err(got, ref) -> float:
    g = _f64(got).ravel()
    r = _f64(ref).ravel()
    if g.shape != r.shape:
        raise ValueError(f"shape mismatch {g.shape} vs {r.shape}")
    if g.size == 0:
        return 0.0
    fin_g, fin_r = np.isfinite(g), np.isfinite(r)
    if not np.array_equal(fin_g, fin_r):
        return math.inf
    if not fin_r.all():
        # non-finite values must agree exactly (same NaN/Inf pattern and sign of Inf)
        nf = ~fin_r
        if not np.array_equal(np.isnan(g[nf]), np.isnan(r[nf])):
            return math.inf
        inf_mask = np.isinf(r[nf])
        if not np.array_equal(g[nf][inf_mask], r[nf][inf_mask]):
            return math.inf
        g, r = g[fin_r], r[fin_r]
        if g.size == 0:
            return 0.0
    rms = math.sqrt(float(np.mean(r * r)))
    diff = np.abs(g - r)
    if rms == 0.0:
        return float(diff.max())
    return float((diff / np.maximum(np.abs(r), rms)).max())


def err_report(got, ref) -> Dict[str, float]:
    g = _f64(got).ravel()
    r = _f64(ref).ravel()
    out = {"max_rel": max_rel_err(g, r)}
    fin = np.isfinite(g) & np.isfinite(r)
    g, r = g[fin], r[fin]
    if r.size:
        rms = math.sqrt(float(np.mean(r * r)))
        nr = float(np.linalg.norm(r))
        out["normwise"] = float(np.linalg.norm(g - r) / nr) if nr > 0 else float(np.linalg.norm(g - r))
        big = np.abs(r) >= rms
        out["elementwise_big"] = float((np.abs(g - r)[big] / np.abs(r[big])).max()) if big.any() else 0.0
        out["rms_ref"] = rms
    return out
