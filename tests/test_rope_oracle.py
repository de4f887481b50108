"""Pins of the float64 RoPE oracle (CPU only).  Each pin checks a property the
mathematics fixes, measured on the output rather than restated: the map is a
rotation of each (i, i + D/2) pair (norms kept, pairs not mixed), it turns
counter-clockwise by exactly position * base^(-2i/D) (angle read back with
atan2), position 0 is the identity, angles add, the inverse undoes it, it is
orthogonal (backward = transpose), and the attention score of two rotated
vectors depends only on the difference of their positions (the property rotary
embeddings are built for).  Planted mistakes must each fail a pin."""
import math

import numpy as np
import pytest

from oracle import rope as ro
from workloads import to_storage

_ORIGINAL = ro.rope64


def _x(seed, T, H, D):
    return np.random.default_rng(seed).standard_normal((T, H, D))


def pin_pairs_and_norms(D=8):
    x = _x(1, 5, 3, D)
    pos = np.array([0, 1, 7, 100, 12345])
    y = ro.rope64(x, pos, 10000.0)
    P = D // 2
    nx = x[..., :P] ** 2 + x[..., P:] ** 2
    ny = y[..., :P] ** 2 + y[..., P:] ** 2
    np.testing.assert_allclose(ny, nx, rtol=1e-13)
    # a single nonzero pair stays in its own pair
    z = np.zeros((1, 1, D))
    z[0, 0, 1] = 1.0
    yz = ro.rope64(z, np.array([3]), 10000.0)
    mask = np.zeros(D, bool)
    mask[[1, 1 + P]] = True
    assert np.abs(yz[0, 0, ~mask]).max() == 0.0


def pin_angles(D=8, base=100.0):
    # the angle from (x_i, x_{i+P}) to (y_i, y_{i+P}) is p * base^(-2i/D) modulo 2 pi, counter-clockwise
    P = D // 2
    x = _x(2, 4, 2, D)
    pos = np.array([1, 2, 5, 40])
    y = ro.rope64(x, pos, base)
    a_in = np.arctan2(x[..., P:], x[..., :P])
    a_out = np.arctan2(y[..., P:], y[..., :P])
    for t, p in enumerate(pos):
        for i in range(P):
            want = p * base ** (-2.0 * i / D)
            got = a_out[t, :, i] - a_in[t, :, i]
            d = np.angle(np.exp(1j * (got - want)))  # difference modulo 2 pi
            assert np.abs(d).max() < 1e-12, (t, i, got, want)


def pin_identity_composition_inverse(D=16):
    x = _x(3, 6, 4, D)
    a = np.array([0, 3, 9, 511, 2047, 70000])
    b = np.array([5, 0, 17, 2, 1000, 3])
    np.testing.assert_array_equal(ro.rope64(x, np.zeros(6, int), 500000.0), x)
    ab = ro.rope64(ro.rope64(x, a, 10000.0), b, 10000.0)
    np.testing.assert_allclose(ab, ro.rope64(x, a + b, 10000.0), rtol=1e-9, atol=1e-9)
    back = ro.rope64(ro.rope64(x, a, 10000.0), a, 10000.0, inverse=True)
    np.testing.assert_allclose(back, x, rtol=1e-12, atol=1e-12)


def pin_orthogonal(D=12):
    # backward = transpose: <R x, g> = <x, R^-1 g>, checked on the explicit matrix of one token
    pos = np.array([37])
    M = np.stack([ro.rope64(np.eye(D)[k][None, None, :], pos, 10000.0)[0, 0] for k in range(D)], axis=1)
    Minv = np.stack([ro.rope64(np.eye(D)[k][None, None, :], pos, 10000.0, inverse=True)[0, 0] for k in range(D)],
                    axis=1)
    np.testing.assert_allclose(M.T @ M, np.eye(D), atol=1e-14)
    np.testing.assert_allclose(Minv, M.T, atol=1e-14)


def pin_relative_position(D=32):
    rng = np.random.default_rng(4)
    q, k = rng.standard_normal((1, 1, D)), rng.standard_normal((1, 1, D))
    for m, n in ((5, 2), (103, 100), (1003, 1000), (3, 0)):
        s = float(np.sum(ro.rope64(q, np.array([m]), 10000.0) * ro.rope64(k, np.array([n]), 10000.0)))
        s0 = float(np.sum(ro.rope64(q, np.array([m - n]), 10000.0) * k))
        assert abs(s - s0) < 1e-10, (m, n, s, s0)


PINS = [pin_pairs_and_norms, pin_angles, pin_identity_composition_inverse, pin_orthogonal, pin_relative_position]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


def test_storage_round_trip():
    import oracle
    rng = np.random.default_rng(5)
    for dtype in ("f32", "bf16", "f16"):
        x = to_storage(rng.standard_normal((3, 2, 16)), dtype)
        r = ro.rope(x, dtype, np.array([0, 1, 2]), 10000.0)
        np.testing.assert_array_equal(r["y64"], ro.rope64(oracle.widen(x, dtype), np.array([0, 1, 2]), 10000.0))
        np.testing.assert_array_equal(r["y"], oracle.round_to(r["y64"], dtype))
        np.testing.assert_array_equal(r["y"][0], x[0])  # position 0: the identity, bit for bit


def _mutant(kind):
    def f(x, positions, base, inverse=False):
        x = np.asarray(x, np.float64)
        T, H, D = x.shape
        P = D // 2
        if kind == "interleaved":  # GPT-J pairs (2i, 2i+1) instead of (i, i+P)
            xi = x.reshape(T, H, P, 2).transpose(0, 1, 3, 2).reshape(T, H, D)
            y = _ORIGINAL(xi, positions, base, inverse)
            return y.reshape(T, H, 2, P).transpose(0, 1, 3, 2).reshape(T, H, D)
        if kind == "exponent":  # base^(-i/D)
            th = np.asarray(positions, float)[:, None] * float(base) ** (-np.arange(P) / D)[None, :]
        else:
            th = ro.angles64(positions, D, base)
        c, s = np.cos(th)[:, None, :], np.sin(th)[:, None, :]
        if kind == "clockwise":
            s = -s
        if inverse and kind != "inverse_not_negated":
            s = -s
        x1, x2 = x[..., :P], x[..., P:]
        return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)
    return f


@pytest.mark.parametrize("kind", ["interleaved", "exponent", "clockwise", "inverse_not_negated"])
def test_mutations_are_caught(kind, monkeypatch):
    monkeypatch.setattr(ro, "rope64", _mutant(kind))
    failed = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1, f"no pin rejects the planted '{kind}' mistake"


def test_unmutated_control(monkeypatch):
    monkeypatch.setattr(ro, "rope64", _mutant("none"))
    for pin in PINS:
        pin()
    assert math.isclose(ro.inv_freq64(4, 100.0)[1], 0.1)
