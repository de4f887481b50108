"""Float64 CPU oracle for token-level softmax cross-entropy (forward + backward).

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  The GPU library never
imports it, and the two share no code: this wrapper loads ``ce_oracle.c``
(compiled with gcc, plain C, double precision) and nothing else.

What is computed, and why, is stated in the header of ``ce_oracle.c``: the
textbook softmax cross-entropy that the pages' "Fast Cross Entropy" kernel
(PyPI page "fms-acceleration-foak 0.7.4", kernel list) stands in for as a
drop-in replacement of the model's loss (fms-acceleration PR #79, "Bug Fix to
Model Patcher"), with the token mean of fms-hf-tuning PR #280 ("Early Version Of
This Plugin": per-token averaging).

Storage formats are named 'f32', 'bf16', 'f16'.  16-bit formats are passed and
returned as numpy uint16 bit patterns; 'f32' as numpy float32.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ce_oracle.c")
_BUILD = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD, "libce_oracle.so")

DTYPES = {"f32": 0, "bf16": 1, "f16": 2}
_lock = threading.Lock()
_lib = None


def build(force: bool = False, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the C oracle with gcc (no fast-math, no FP contraction)."""
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _bind(lib):
    c_i64, c_int, c_dbl, c_vp = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
    lib.ceo_widen.argtypes = [c_vp, c_int, c_i64, c_vp]
    lib.ceo_widen.restype = None
    lib.ceo_round.argtypes = [c_vp, c_i64, c_int, c_vp]
    lib.ceo_round.restype = None
    lib.ceo_count_valid.argtypes = [c_vp, c_i64, c_i64]
    lib.ceo_count_valid.restype = c_i64
    lib.ceo_rows.argtypes = [c_vp, c_i64, c_int, c_vp, c_i64, c_i64, c_i64, c_dbl,
                             c_vp, c_vp, c_vp, c_vp, c_int]
    lib.ceo_rows.restype = c_i64
    lib.ceo_mean.argtypes = [c_vp, c_vp, c_i64, c_i64]
    lib.ceo_mean.restype = c_dbl
    lib.ceo_chunked_lse.argtypes = [c_vp, c_int, c_i64, c_i64]
    lib.ceo_chunked_lse.restype = c_dbl
    return lib


def load(path: str | None = None):
    """Load (building first if needed) the oracle library."""
    global _lib
    with _lock:
        if path is not None:
            return _bind(ctypes.CDLL(path))
        if _lib is None:
            _lib = _bind(ctypes.CDLL(build()))
        return _lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _storage(dtype: str):
    return np.float32 if dtype == "f32" else np.uint16


def widen(x: np.ndarray, dtype: str, lib=None) -> np.ndarray:
    """Exact float64 value of each stored element."""
    lib = lib or load()
    x = np.ascontiguousarray(x, dtype=_storage(dtype))
    out = np.empty(x.shape, np.float64)
    lib.ceo_widen(_ptr(x), DTYPES[dtype], x.size, _ptr(out))
    return out


def round_to(x64: np.ndarray, dtype: str, lib=None) -> np.ndarray:
    """Round float64 values to the storage format, nearest-even, subnormals kept."""
    lib = lib or load()
    x64 = np.ascontiguousarray(x64, dtype=np.float64)
    out = np.empty(x64.shape, _storage(dtype))
    lib.ceo_round(_ptr(x64), x64.size, DTYPES[dtype], _ptr(out))
    return out


def count_valid(labels: np.ndarray, ignore_index: int = -100, lib=None) -> int:
    lib = lib or load()
    labels = np.ascontiguousarray(labels, dtype=np.int64)
    return int(lib.ceo_count_valid(_ptr(labels), labels.size, ignore_index))


class LabelError(ValueError):
    """A label outside [0, V) that is not ignore_index."""


def rows(logits: np.ndarray, labels: np.ndarray, dtype: str, scale: float,
         ignore_index: int = -100, want_grad: bool = True, want_grad64: bool = False,
         threads: int = 1, allow_bad: bool = False, lib=None) -> dict:
    """Per-row lse, loss and (optionally) gradient rows with a given dloss/n_valid.

    ``logits`` is [R, V] (or [R, ld] with only the first V columns used when
    ``V`` is passed through a view; here the array's last dimension is V).
    """
    lib = lib or load()
    x = np.ascontiguousarray(logits, dtype=_storage(dtype))
    if x.ndim != 2:
        raise ValueError("logits must be 2-D")
    R, V = x.shape
    y = np.ascontiguousarray(labels, dtype=np.int64).reshape(-1)
    if y.size != R:
        raise ValueError("labels must have one entry per row")
    lse = np.empty(R, np.float64)
    loss = np.empty(R, np.float64)
    grad = np.empty((R, V), _storage(dtype)) if want_grad else None
    grad64 = np.empty((R, V), np.float64) if want_grad64 else None
    bad = lib.ceo_rows(_ptr(x), V, DTYPES[dtype], _ptr(y), R, V, ignore_index, float(scale),
                       _ptr(lse), _ptr(loss), _ptr(grad), _ptr(grad64), int(threads))
    if bad and not allow_bad:
        raise LabelError(f"{bad} label(s) outside [0, {V}) and not ignore_index")
    return {"lse": lse, "loss": loss, "grad": grad, "grad64": grad64, "bad": int(bad)}


def mean(loss: np.ndarray, labels: np.ndarray, ignore_index: int = -100, lib=None) -> float:
    lib = lib or load()
    loss = np.ascontiguousarray(loss, dtype=np.float64)
    y = np.ascontiguousarray(labels, dtype=np.int64)
    return float(lib.ceo_mean(_ptr(loss), _ptr(y), y.size, ignore_index))


def cross_entropy(logits: np.ndarray, labels: np.ndarray, dtype: str, ignore_index: int = -100,
                  dloss: float = 1.0, want_grad: bool = True, want_grad64: bool = False,
                  threads: int = 1, allow_bad: bool = False, lib=None) -> dict:
    """Whole-batch forward + backward: token-mean loss and dloss-scaled gradient.

    Returns dict(loss_mean, loss_rows, lse, n_valid, grad, grad64, scale).
    ``loss_mean`` is NaN when no row is valid; the gradient is then all +0
    (``scale`` is NaN but every row is ignored, so no element uses it).
    """
    lib = lib or load()
    n = count_valid(labels, ignore_index, lib)
    scale = dloss / n if n > 0 else float("nan")
    r = rows(logits, labels, dtype, scale, ignore_index, want_grad, want_grad64, threads,
             allow_bad, lib)
    L = mean(r["loss"], labels, ignore_index, lib)
    return {"loss_mean": L, "loss_rows": r["loss"], "lse": r["lse"], "n_valid": n,
            "grad": r["grad"], "grad64": r["grad64"], "scale": scale, "bad": r["bad"]}


def chunked_lse(row: np.ndarray, dtype: str, chunk: int, lib=None) -> float:
    """Log-sum-exp of one row computed per vocabulary chunk and merged."""
    lib = lib or load()
    x = np.ascontiguousarray(row, dtype=_storage(dtype)).reshape(-1)
    return float(lib.ceo_chunked_lse(_ptr(x), DTYPES[dtype], x.size, int(chunk)))
