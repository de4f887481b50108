"""Shared helpers for the GPU parity tests: moving seeded inputs to the device,
calling the library, and comparing with the oracle element by element.

Tolerances (stated once, used everywhere):
  * loss mean, per-row loss and lse: relative 1e-5 for fp32 logits, 2e-3 for
    bf16/fp16 logits (plus an absolute floor of 1e-6 for near-zero losses);
  * gradient: every element within 1 unit in the last place of the oracle's
    value rounded to the logits' format (distance between the monotone integer
    images of the bit patterns, +0 and -0 equal);
  * n_valid and the status word: exact.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from oracle_pins import _ordered

REL = {"f32": 1e-5, "bf16": 2e-3, "f16": 2e-3}
TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def to_device(bits: np.ndarray, dtype: str, ld: int | None = None, offset: int = 0) -> torch.Tensor:
    """[N, V] storage array -> device tensor view [N, V] with row stride ld and
    the base `offset` elements past a 256-byte aligned allocation."""
    N, V = bits.shape
    ld = ld or V
    raw = bits.view(np.int32) if dtype == "f32" else bits.view(np.int16)
    host = torch.from_numpy(np.ascontiguousarray(raw))
    buf = torch.zeros(offset + N * ld + 8, dtype=host.dtype, device="cuda")
    view = buf[offset: offset + N * ld].view(N, ld)[:, :V]
    view.copy_(host.cuda())
    return view.view(TORCH[dtype]) if dtype != "f32" else view.view(torch.float32)


def to_host_bits(t: torch.Tensor, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return t.detach().contiguous().cpu().numpy().astype(np.float32)
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray, dtype: str) -> np.ndarray:
    return np.abs(_ordered(a_bits, dtype) - _ordered(b_bits, dtype))


def assert_grad_close(got_bits, want_bits, dtype, what=""):
    d = ulp_distance(got_bits, want_bits, dtype)
    bad = np.argwhere(d > 1)
    assert bad.size == 0, f"{what}: {bad.shape[0]} gradient elements beyond 1 ulp, first {bad[:5].tolist()}, " \
                          f"max {int(d.max())}"


def assert_rel(got, want, dtype, what=""):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    tol = REL[dtype] * np.abs(want) + 1e-6
    bad = np.flatnonzero(~(np.abs(got - want) <= tol))
    assert bad.size == 0, f"{what}: {bad.size} values outside tolerance, first {bad[:5].tolist()} " \
                          f"got {got.reshape(-1)[bad[:3]]} want {want.reshape(-1)[bad[:3]]}"
