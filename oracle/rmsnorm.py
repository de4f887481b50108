"""Float64 CPU oracle for RMS layer normalisation, forward and backward.

TEST INFRASTRUCTURE ONLY.  Only the tests and the benchmark's ``cpu_baseline``
leg may import this module; the GPU library never does, and the two share no
code.

What is computed.  The pages list "Fast RMS LayerNorm" among the kernels of the
package (PyPI page "fms-acceleration-foak 0.7.4", kernel list) and patch it in
for a model's RMSNorm class (same page, the model-patcher rule that replaces
GraniteRMSNorm's forward with fast_rms_layernorm; fms-hf-tuning PR #280, "Notes
on FastKernels": FastRMSLayerNorm).  The plain reading is the RMSNorm of those
models, per row x[0..H) with weight w and epsilon eps:

    rstd = 1 / sqrt(mean_j x_j^2 + eps)
    y_j  = w_j x_j rstd

and its gradient for an upstream dy (x^_j = x_j rstd):

    dx_j = rstd (w_j dy_j - x^_j mean_k(x^_k w_k dy_k))
    dw_j = sum over rows of dy_j x^_j

float64 throughout (inputs widened exactly from their storage format), one
rounding to the storage format at the end with the pinned ``oracle.round_to``.
"""
from __future__ import annotations

import numpy as np

from . import round_to, widen


def forward64(x: np.ndarray, w: np.ndarray, eps: float):
    """(y, rstd) in float64 for float64 rows x [N, H] and weight w [H]."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    rstd = 1.0 / np.sqrt(np.mean(x * x, axis=1) + eps)
    return x * rstd[:, None] * w[None, :], rstd


def backward64(dy: np.ndarray, x: np.ndarray, w: np.ndarray, eps: float):
    """(dx, dw) in float64."""
    dy = np.asarray(dy, np.float64)
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    _, rstd = forward64(x, w, eps)
    xh = x * rstd[:, None]
    wdy = w[None, :] * dy
    c = np.mean(xh * wdy, axis=1)
    dx = rstd[:, None] * (wdy - xh * c[:, None])
    dw = np.sum(dy * xh, axis=0)
    return dx, dw


def rmsnorm(x: np.ndarray, w: np.ndarray, dtype: str, eps: float, dy: np.ndarray | None = None) -> dict:
    """Forward (and, with dy, backward) on storage arrays ('f32' float32,
    'bf16' / 'f16' uint16 bit patterns): y, rstd, and dx, dw with their float64
    values (y64, dx64, dw64)."""
    x64, w64 = widen(x, dtype), widen(w, dtype)
    y64, rstd = forward64(x64, w64, eps)
    out = {"y64": y64, "y": round_to(y64, dtype), "rstd": rstd}
    if dy is not None:
        dy64 = widen(dy, dtype)
        dx64, dw64 = backward64(dy64, x64, w64, eps)
        out.update(dx64=dx64, dw64=dw64, dx=round_to(dx64, dtype), dw=round_to(dw64, dtype))
    return out
