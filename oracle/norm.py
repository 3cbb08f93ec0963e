"""RMSNorm ahead of MX quantization (CPU oracle, test infrastructure only).

What the pages fix ([News], contributions paragraph): a fused RMSNorm +
Quantize producer emits the FP8 payload and its scale layouts in one pass.
They give no formula.  The reading taken (listed in the design notes):

  * RMSNorm is the usual root-mean-square normalization with a gain vector,
    applied per (token, head) row over the D features of that head:
        y_d = x_d / sqrt(mean_d(x_d^2) + eps) * gamma_d
  * Precision, step by step:
        ss   = sum_d x_d^2, exactly, rounded once to float64
        v    = fl64(ss / D + eps)            (ss / D is exact: D is 64 or 128)
        rstd = fl32(fl64(1 / fl64(sqrt(v))))
        y_d  = fl32(fl32(x_d * rstd) * gamma_d)
    x_d is a bf16 or fp32 value, so x_d^2 is exact in float64.
  * y is then quantized exactly as the quantizer quantizes x (mx.py).
"""
from __future__ import annotations

import math

import numpy as np

from . import mx


def _fl32(a):
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def rstd_rows(x, eps: float) -> np.ndarray:
    """Per-row 1/sqrt(mean(x^2) + eps) as fp32 values, rows along the last axis."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    flat = x.reshape(-1, D)
    out = np.empty(flat.shape[0])
    for i in range(flat.shape[0]):
        ss = math.fsum(float(t) * float(t) for t in flat[i])   # exact sum, rounded once
        v = ss / D + float(np.float32(eps))
        out[i] = 1.0 / math.sqrt(v)
    return _fl32(out).reshape(x.shape[:-1])


def rmsnorm(x, gamma, eps: float) -> np.ndarray:
    """y = fl32(fl32(x * rstd) * gamma) over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    g = _fl32(gamma)
    r = rstd_rows(x, eps)[..., None]
    return _fl32(_fl32(x * r) * g)


def rmsnorm_quantize(x, gamma, eps: float, layouts=("row32", "col32", "sq32")):
    """[B, S, H, D] -> {layout: (codes, scale codes)} of the normalized tensor,
    in the quantizer's layouts (tokens along axis 1)."""
    y = rmsnorm(x, gamma, eps)
    out = {}
    if "row32" in layouts:
        out["row32"] = mx.quantize_row32(y)
    if "col32" in layouts:
        out["col32"] = mx.quantize_col32(y, axis=1)
    if "sq32" in layouts:
        out["sq32"] = mx.quantize_sq32(y, axis_pos=1)
    return out
