"""Pins of the float64 RMSNorm oracle (CPU only): closed forms, invariances
and central finite differences of the backward, plus planted mistakes that a
pin must reject."""
import math

import numpy as np
import pytest

from oracle import rmsnorm as rn
from workloads import to_storage

_ORIGINAL_BWD = rn.backward64


def test_constant_row_closed_form():
    # x_j = a for all j: mean x^2 = a^2, y_j = w_j a / sqrt(a^2 + eps)
    a, eps, H = -1.75, 1e-5, 12
    w = np.linspace(0.5, 2.0, H)
    y, rstd = rn.forward64(np.full((1, H), a), w, eps)
    assert rstd[0] == pytest.approx(1 / math.sqrt(a * a + eps), rel=1e-15)
    np.testing.assert_allclose(y[0], w * a / math.sqrt(a * a + eps), rtol=1e-15)


def test_two_level_row_closed_form():
    # half the row at a, half at b: mean x^2 = (a^2 + b^2) / 2
    a, b, eps = 3.0, -1.0, 0.25
    x = np.array([[a, b, a, b]])
    y, rstd = rn.forward64(x, np.ones(4), eps)
    r = 1 / math.sqrt((a * a + b * b) / 2 + eps)
    assert rstd[0] == pytest.approx(r, rel=1e-15)
    np.testing.assert_allclose(y[0], x[0] * r, rtol=1e-15)


def test_scale_invariance_without_eps():
    rng = np.random.default_rng(1)
    x, w = rng.standard_normal((5, 16)), rng.standard_normal(16)
    y1, _ = rn.forward64(x, w, 0.0)
    y2, _ = rn.forward64(-3.5 * x, w, 0.0)
    np.testing.assert_allclose(y2, -y1, rtol=1e-13)
    # hence the gradient has no component along x: sum_j x_j dx_j = 0
    dy = rng.standard_normal((5, 16))
    dx, _ = rn.backward64(dy, x, w, 0.0)
    assert np.abs(np.sum(x * dx, axis=1)).max() <= 1e-12


def _fd_check(seed, N, H, eps):
    rng = np.random.default_rng(seed)
    x, w, dy = rng.standard_normal((N, H)), rng.standard_normal(H), rng.standard_normal((N, H))
    dx, dw = rn.backward64(dy, x, w, eps)
    loss = lambda xx, ww: float(np.sum(dy * rn.forward64(xx, ww, eps)[0]))  # noqa: E731
    h = 1e-6
    for idx in np.ndindex(N, H):
        a, b = x.copy(), x.copy()
        a[idx] += h
        b[idx] -= h
        fd = (loss(a, w) - loss(b, w)) / (2 * h)
        assert abs(fd - dx[idx]) <= 1e-6 * max(1.0, abs(dx[idx])), ("dx", idx, fd, dx[idx])
    for j in range(H):
        a, b = w.copy(), w.copy()
        a[j] += h
        b[j] -= h
        fd = (loss(x, a) - loss(x, b)) / (2 * h)
        assert abs(fd - dw[j]) <= 1e-6 * max(1.0, abs(dw[j])), ("dw", j, fd, dw[j])


def test_finite_differences():
    _fd_check(2, 3, 7, 1e-5)
    _fd_check(3, 2, 5, 0.5)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_storage_round_trip(dtype):
    rng = np.random.default_rng(4)
    x = to_storage(rng.standard_normal((6, 32)), dtype)
    w = to_storage(1 + 0.1 * rng.standard_normal(32), dtype)
    dy = to_storage(rng.standard_normal((6, 32)), dtype)
    r = rn.rmsnorm(x, w, dtype, 1e-6, dy)
    assert r["y"].dtype == x.dtype and r["dx"].dtype == x.dtype and r["dw"].shape == (32,)
    # the storage path widens exactly and rounds once
    import oracle
    y64, rstd = rn.forward64(oracle.widen(x, dtype), oracle.widen(w, dtype), 1e-6)
    np.testing.assert_array_equal(r["y64"], y64)
    np.testing.assert_array_equal(r["y"], oracle.round_to(y64, dtype))
    np.testing.assert_array_equal(r["rstd"], rstd)


def _mutant(kind):
    def f(dy, x, w, eps):
        dx, dw = _ORIGINAL_BWD(dy, x, w, eps)
        x = np.asarray(x, np.float64)
        _, rstd = rn.forward64(x, w, eps)
        if kind == "no_projection":
            dx = rstd[:, None] * (np.asarray(w)[None, :] * dy)
        elif kind == "dw_without_rstd":
            dw = np.sum(dy * x, axis=0)
        elif kind == "sum_not_mean":
            xh = x * rstd[:, None]
            wdy = np.asarray(w)[None, :] * dy
            dx = rstd[:, None] * (wdy - xh * np.sum(xh * wdy, axis=1)[:, None])
        return dx, dw
    return f


@pytest.mark.parametrize("kind", ["no_projection", "dw_without_rstd", "sum_not_mean"])
def test_mutations_are_caught(kind, monkeypatch):
    monkeypatch.setattr(rn, "backward64", _mutant(kind))
    with pytest.raises(AssertionError):
        _fd_check(2, 3, 7, 1e-5)
