"""Float64 CPU oracle for the LM-head projection followed by softmax cross-entropy.

TEST INFRASTRUCTURE ONLY.  Only the tests and the benchmark's ``cpu_baseline``
leg may import this module; the GPU library never does, and the two share no
code.

What is computed.  The pages compare the plain "Fast Cross Entropy" kernel with
a fused linear cross-entropy (PyPI page "fms-acceleration-foak 0.7.4", section
"Running Liger Kernel Benchmarks": the fused LigerFusedLinearCrossEntropy runs
against the triton cross-entropy), list fused cross-entropy among the kernels
to come (fms-hf-tuning PR #280, "Notes on FastKernels") and leave a chunked
loss as a to-do (fms-acceleration PR #79, "TODO").  The plain reading: the
language-model head turns hidden states h [N, H] into logits with the weight
W [V, H] of a bias-free linear layer, logits = h W^T, and the token-mean
cross-entropy of the rest of this package is taken on those logits.  With
g = dL/dlogits = (dloss / n_valid) (softmax - onehot) on valid rows (0 on
ignored rows):

    dL/dh = g W          [N, H]
    dL/dW = g^T h        [V, H]

Everything here is float64: the inputs are widened exactly from their storage
format, the products use numpy's float64 matrix product (a library primitive,
as the definition allows), and rounding to a storage format happens once, at
the end, with the pinned ``oracle.round_to``.  Chunking over tokens does not
enter the definition.
"""
from __future__ import annotations

import numpy as np

from . import round_to, widen


def forward64(h: np.ndarray, w: np.ndarray, labels: np.ndarray, ignore_index: int = -100):
    """Per-row loss and softmax of logits = h w^T (float64 in, float64 out).

    Returns (loss_rows, p, logits, valid, bad): loss 0 on ignored rows, NaN on
    rows whose label is outside [0, V) and not ignore_index.
    """
    h = np.asarray(h, np.float64)
    w = np.asarray(w, np.float64)
    y = np.asarray(labels, np.int64).reshape(-1)
    logits = h @ w.T
    N, V = logits.shape
    valid = y != ignore_index
    bad = valid & ((y < 0) | (y >= V))
    good = valid & ~bad
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    s = e.sum(axis=1, keepdims=True)
    lse = (m + np.log(s)).reshape(-1)
    p = e / s
    loss = np.zeros(N, np.float64)
    rows = np.nonzero(good)[0]
    loss[rows] = lse[rows] - logits[rows, y[rows]]
    loss[bad] = np.nan
    return loss, p, logits, valid, bad


def loss_mean64(h, w, labels, ignore_index: int = -100) -> float:
    """Token mean of the per-row losses (NaN when no row is valid)."""
    loss, _, _, valid, _ = forward64(h, w, labels, ignore_index)
    n = int(valid.sum())
    return float(np.sum(loss[valid]) / n) if n else float("nan")


def linear_cross_entropy(hidden: np.ndarray, weight: np.ndarray, labels: np.ndarray, dtype: str,
                         ignore_index: int = -100, dloss: float = 1.0) -> dict:
    """Forward and backward of loss = CE(hidden weight^T) in float64.

    ``hidden`` [N, H] and ``weight`` [V, H] are storage arrays ('f32' float32,
    'bf16' / 'f16' uint16 bit patterns).  Returns loss_mean, loss_rows, n_valid,
    grad_logits64, grad_hidden64 / grad_weight64 and their roundings to dtype
    (grad_hidden, grad_weight), and the count of bad labels.
    """
    h = widen(hidden, dtype)
    w = widen(weight, dtype)
    y = np.asarray(labels, np.int64).reshape(-1)
    loss, p, _, valid, bad = forward64(h, w, y, ignore_index)
    n = int(valid.sum())
    scale = dloss / n if n else float("nan")
    g = np.zeros_like(p)
    good = valid & ~bad
    rows = np.nonzero(good)[0]
    g[rows] = scale * p[rows]
    g[rows, y[rows]] -= scale
    g[bad] = np.nan
    gh = g @ w
    gw = g.T @ h
    L = float(np.sum(loss[valid]) / n) if n else float("nan")
    return {"loss_mean": L, "loss_rows": loss, "n_valid": n, "bad": int(bad.sum()), "scale": scale,
            "grad_logits64": g, "grad_hidden64": gh, "grad_weight64": gw,
            "grad_hidden": round_to(gh, dtype), "grad_weight": round_to(gw, dtype)}


def linear_sampled(hidden: np.ndarray, weight: np.ndarray, labels: np.ndarray, dtype: str, rows, cols,
                   ignore_index: int = -100, dloss: float = 1.0, row_block: int = 512) -> dict:
    """The same definition as ``linear_cross_entropy`` for shapes whose full
    [N, V] float64 arrays do not fit: the rows are taken ``row_block`` at a
    time (each row's softmax depends on its own logits only), and only the
    requested outputs are kept -- every row's loss, dL/dh for the rows in
    ``rows`` and dL/dW for the vocabulary rows in ``cols``, whose sums over the
    tokens are accumulated block by block (float64; only the order of that sum
    differs from ``linear_cross_entropy``), and the softmax's columns ``cols``
    for every row.
    """
    h = widen(hidden, dtype)
    w = widen(weight, dtype)
    y = np.asarray(labels, np.int64).reshape(-1)
    N, V = h.shape[0], w.shape[0]
    rows = np.asarray(rows, np.int64)
    cols = np.asarray(cols, np.int64)
    valid = y != ignore_index
    n = int(valid.sum())
    scale = dloss / n if n else float("nan")
    loss = np.zeros(N, np.float64)
    gh = np.zeros((len(rows), h.shape[1]), np.float64)
    gw = np.zeros((len(cols), h.shape[1]), np.float64)
    pc = np.zeros((N, len(cols)), np.float64)
    for r0 in range(0, N, row_block):
        r1 = min(N, r0 + row_block)
        lb, p, _, vb, bad = forward64(h[r0:r1], w, y[r0:r1], ignore_index)
        loss[r0:r1] = lb
        pc[r0:r1] = p[:, cols]
        g = np.zeros_like(p)
        good = vb & ~bad
        rr = np.nonzero(good)[0]
        g[rr] = scale * p[rr]
        g[rr, y[r0:r1][rr]] -= scale
        g[bad] = np.nan
        sel = np.nonzero((rows >= r0) & (rows < r1))[0]
        if len(sel):
            gh[sel] = g[rows[sel] - r0] @ w
        gw += g[:, cols].T @ h[r0:r1]
    L = float(np.sum(loss[valid]) / n) if n else float("nan")
    return {"loss_mean": L, "loss_rows": loss, "n_valid": n, "scale": scale, "grad_hidden64": gh,
            "grad_weight64": gw, "softmax_cols": pc}
