"""Float64 CPU oracle for rotary position embedding (RoPE) with per-token
position ids, forward and backward.

TEST INFRASTRUCTURE ONLY.  Only the tests and the benchmark's ``cpu_baseline``
leg may import this module; the GPU library never does, and the two share no
code.

What is computed.  The pages list "Fast RoPE" among the package's kernels
(PyPI page "fms-acceleration-foak 0.7.4", kernel list) and say twice that it
does not take position ids (same page, known issues; fms-hf-tuning PR #280,
"Notes on FastKernels"), which padding-free packed batches need: positions
restart at each packed sequence.  The plain reading is the rotary embedding of
the Llama / Mistral models the pages patch: head_dim D, P = D/2 pairs, pair i
made of elements i and i + P of a head, rotated by the angle

    theta(t, i) = position[t] * base^(-2 i / D)

    y_i     = x_i cos(theta) - x_{i+P} sin(theta)
    y_{i+P} = x_{i+P} cos(theta) + x_i sin(theta)

the same for every head of the token.  The map is a rotation, so its gradient
is the rotation by -theta (``inverse=True``).  float64 throughout (inputs
widened exactly from their storage format), one rounding to the storage format
at the end with the pinned ``oracle.round_to``.
"""
from __future__ import annotations

import numpy as np

from . import round_to, widen


def inv_freq64(head_dim: int, base: float) -> np.ndarray:
    """base^(-2 i / D) for the P = D/2 pairs."""
    return np.power(float(base), -(2.0 * np.arange(head_dim // 2)) / head_dim)


def angles64(positions: np.ndarray, head_dim: int, base: float) -> np.ndarray:
    """theta [T, P] in float64 (positions are integers, exact in float64)."""
    p = np.asarray(positions, dtype=np.int64).astype(np.float64)
    return p[:, None] * inv_freq64(head_dim, base)[None, :]


def rope64(x: np.ndarray, positions: np.ndarray, base: float, inverse: bool = False) -> np.ndarray:
    """Rotate x [T, H, D] (float64) by the angles of its tokens' positions."""
    x = np.asarray(x, np.float64)
    T, H, D = x.shape
    th = angles64(positions, D, base)
    c = np.cos(th)[:, None, :]
    s = np.sin(th)[:, None, :]
    if inverse:
        s = -s
    P = D // 2
    x1, x2 = x[..., :P], x[..., P:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rope(x: np.ndarray, dtype: str, positions: np.ndarray, base: float, inverse: bool = False) -> dict:
    """Storage arrays ('f32' float32, 'bf16' / 'f16' uint16 bit patterns) of
    shape [T, H, D]: the rotated tensor y and its float64 value y64."""
    y64 = rope64(widen(x, dtype), positions, base, inverse)
    return {"y64": y64, "y": round_to(y64, dtype)}
