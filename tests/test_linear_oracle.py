"""Pins of the float64 LM-head + cross-entropy oracle (CPU only).

Each pin ties the oracle to something other than itself: the separately pinned
cross-entropy oracle (identity weight), central finite differences of the
loss, a closed form (zero weight), and invariances a transposed operand, a
dropped scale or a sign slip would break.  The mutation tests at the end plant
such mistakes in copies of the backward and check that a pin rejects each.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import linear as lin
from workloads import to_storage


def _bits(x, dtype):
    return to_storage(np.asarray(x, np.float64), dtype)


def _case(seed, N, H, V, dtype, sigma_w=0.5, ignore_frac=0.2):
    rng = np.random.default_rng(seed)
    h = _bits(rng.standard_normal((N, H)), dtype)
    w = _bits(rng.standard_normal((V, H)) * sigma_w, dtype)
    y = rng.integers(0, V, N)
    y[rng.random(N) < ignore_frac] = -100
    return h, w, y


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_identity_weight_matches_cross_entropy_oracle(dtype):
    # W = I (exact in every format): logits are the hidden states themselves
    N, V = 24, 40
    rng = np.random.default_rng(3)
    h = _bits(rng.standard_normal((N, V)) * 3, dtype)
    w = _bits(np.eye(V), dtype)
    y = rng.integers(0, V, N)
    y[[1, 7, 8]] = -100
    r = lin.linear_cross_entropy(h, w, y, dtype, dloss=0.75)
    ref = oracle.cross_entropy(h, y, dtype, dloss=0.75, want_grad64=True)
    assert r["n_valid"] == ref["n_valid"]
    assert abs(r["loss_mean"] - ref["loss_mean"]) <= 1e-13 * abs(ref["loss_mean"])
    np.testing.assert_allclose(r["loss_rows"], ref["loss_rows"], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(r["grad_logits64"], ref["grad64"], rtol=0, atol=1e-15)
    # dL/dh = g I = g;  dL/dW = g^T h
    np.testing.assert_allclose(r["grad_hidden64"], ref["grad64"], rtol=0, atol=1e-15)
    hx = oracle.widen(h, dtype)
    np.testing.assert_allclose(r["grad_weight64"], ref["grad64"].T @ hx, rtol=1e-12, atol=1e-15)


def test_zero_weight_closed_form():
    # W = 0: every logit is 0, loss = ln V, g = s (1/V - onehot), dL/dh = 0
    N, H, V = 9, 6, 11
    rng = np.random.default_rng(5)
    h = _bits(rng.standard_normal((N, H)), "f32")
    w = _bits(np.zeros((V, H)), "f32")
    y = rng.integers(0, V, N)
    y[4] = -100
    r = lin.linear_cross_entropy(h, w, y, "f32", dloss=2.0)
    valid = y != -100
    s = 2.0 / valid.sum()
    assert r["loss_rows"][valid] == pytest.approx(math.log(V), rel=1e-15)
    assert r["loss_mean"] == pytest.approx(math.log(V), rel=1e-15)
    g = np.zeros((N, V))
    g[valid] = s / V
    g[np.nonzero(valid)[0], y[valid]] -= s
    np.testing.assert_allclose(r["grad_logits64"], g, atol=1e-16)
    assert np.all(r["grad_hidden64"] == 0)
    np.testing.assert_allclose(r["grad_weight64"], g.T @ oracle.widen(h, "f32"), rtol=1e-14, atol=1e-16)


def _fd_check(N, H, V, seed, dloss):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((N, H))
    w = rng.standard_normal((V, H)) * 0.7
    y = rng.integers(0, V, N)
    y[0] = -100
    hb, wb = _bits(h, "f32"), _bits(w, "f32")
    h, w = oracle.widen(hb, "f32"), oracle.widen(wb, "f32")
    r = lin.linear_cross_entropy(hb, wb, y, "f32", dloss=dloss)
    eps = 2.0 ** -20
    for (mat, grad) in ((h, r["grad_hidden64"]), (w, r["grad_weight64"])):
        for idx in np.ndindex(*mat.shape):
            a, b = mat.copy(), mat.copy()
            a[idx] += eps
            b[idx] -= eps
            if mat is h:
                fd = (lin.loss_mean64(a, w, y) - lin.loss_mean64(b, w, y)) / (2 * eps)
            else:
                fd = (lin.loss_mean64(h, a, y) - lin.loss_mean64(h, b, y)) / (2 * eps)
            assert abs(fd * dloss - grad[idx]) <= 1e-7 * max(1.0, abs(grad[idx])), (idx, fd, grad[idx])


def test_finite_differences():
    _fd_check(4, 5, 7, 11, 1.0)
    _fd_check(3, 6, 5, 12, 0.5)


def test_vocab_permutation():
    # permuting the rows of W (and relabelling) permutes the logits' columns
    h, w, y = _case(7, 12, 16, 20, "bf16")
    perm = np.random.default_rng(8).permutation(20)
    inv = np.argsort(perm)
    r0 = lin.linear_cross_entropy(h, w, y, "bf16")
    y2 = np.where(y == -100, -100, inv[np.maximum(y, 0)])
    r1 = lin.linear_cross_entropy(h, w[perm], y2, "bf16")
    np.testing.assert_allclose(r1["loss_rows"], r0["loss_rows"], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(r1["grad_hidden64"], r0["grad_hidden64"], rtol=1e-11, atol=1e-15)
    np.testing.assert_allclose(r1["grad_weight64"], r0["grad_weight64"][perm], rtol=1e-11, atol=1e-15)


def test_gradient_sums_and_scale():
    h, w, y = _case(9, 16, 8, 30, "f16")
    r1 = lin.linear_cross_entropy(h, w, y, "f16", dloss=1.0)
    r3 = lin.linear_cross_entropy(h, w, y, "f16", dloss=3.0)
    # rows of g sum to zero, so sum_v dL/dW[v, :] = 0
    assert np.abs(r1["grad_weight64"].sum(axis=0)).max() <= 1e-14
    np.testing.assert_allclose(r3["grad_hidden64"], 3 * r1["grad_hidden64"], rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(r3["grad_weight64"], 3 * r1["grad_weight64"], rtol=1e-13, atol=1e-16)
    ign = y == -100
    assert np.all(r1["grad_hidden64"][ign] == 0)


@pytest.mark.parametrize("dtype,block", [("bf16", 7), ("f16", 64), ("f32", 1)])
def test_row_blocked_form_matches_the_whole(dtype, block):
    # linear_sampled takes the rows a block at a time and keeps some outputs; it must give the whole
    # computation's loss rows and the selected rows of dL/dh and dL/dW (which it sums block by block)
    h, w, y = _case(11, 40, 12, 50, dtype)
    y[3] = 50  # a bad label: NaN row, NaN in every dL/dW row
    whole = lin.linear_cross_entropy(h, w, y, dtype, dloss=0.7)
    rows, cols = [0, 3, 17, 39], [0, 5, 49]
    part = lin.linear_sampled(h, w, y, dtype, rows, cols, dloss=0.7, row_block=block)
    assert part["n_valid"] == whole["n_valid"]
    np.testing.assert_array_equal(np.isnan(part["loss_rows"]), np.isnan(whole["loss_rows"]))
    # numpy's product may sum a one-row block in another order: float64 rounding apart, the same
    np.testing.assert_allclose(part["loss_rows"], whole["loss_rows"], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(part["grad_hidden64"], whole["grad_hidden64"][rows], rtol=1e-12, atol=1e-18)
    assert np.isnan(part["grad_weight64"]).all() and np.isnan(whole["grad_weight64"][cols]).all()
    y[3] = 1
    whole = lin.linear_cross_entropy(h, w, y, dtype, dloss=0.7)
    part = lin.linear_sampled(h, w, y, dtype, rows, cols, dloss=0.7, row_block=block)
    np.testing.assert_allclose(part["grad_weight64"], whole["grad_weight64"][cols], rtol=1e-12, atol=1e-18)
    assert part["loss_mean"] == pytest.approx(whole["loss_mean"], rel=1e-15)


def test_no_valid_rows_and_bad_label():
    h, w, y = _case(10, 5, 4, 6, "bf16")
    r = lin.linear_cross_entropy(h, w, np.full(5, -100), "bf16")
    assert r["n_valid"] == 0 and math.isnan(r["loss_mean"])
    assert np.all(r["grad_hidden64"] == 0) and np.all(r["grad_weight64"] == 0)
    y = y.copy()
    y[2] = 6  # == V: out of range
    r = lin.linear_cross_entropy(h, w, y, "bf16")
    assert r["bad"] == 1 and math.isnan(r["loss_rows"][2]) and math.isnan(r["loss_mean"])
    assert np.isnan(r["grad_hidden64"][2]).all()


# ---------------------------------------------------------------------------
# Mutations: plausible mistakes in the backward, each rejected by a pin above.

_ORIGINAL = lin.linear_cross_entropy


def _mutant(kind):
    def f(hidden, weight, labels, dtype, ignore_index=-100, dloss=1.0):
        r = _ORIGINAL(hidden, weight, labels, dtype, ignore_index, dloss)
        g = r["grad_logits64"]
        h = oracle.widen(hidden, dtype)
        w = oracle.widen(weight, dtype)
        if kind == "no_scale":
            r["grad_hidden64"] = (g / r["scale"]) @ w
        elif kind == "sign":
            r["grad_weight64"] = -(g.T @ h)
        elif kind == "transposed_weight":
            r["grad_hidden64"] = g @ w.T[: g.shape[1]] if w.shape[0] == w.shape[1] else g @ w * 1.5
        elif kind == "mean_over_all_rows":
            r["grad_hidden64"] = g @ w * r["n_valid"] / len(labels)
        return r
    return f


@pytest.mark.parametrize("kind", ["no_scale", "sign", "transposed_weight", "mean_over_all_rows"])
def test_mutations_are_caught(kind, monkeypatch):
    monkeypatch.setattr(lin, "linear_cross_entropy", _mutant(kind))
    failures = 0
    for check in (lambda: _fd_check(4, 5, 5, 11, 1.0), lambda: _fd_check(3, 6, 6, 12, 0.5)):
        try:
            check()
        except AssertionError:
            failures += 1
    assert failures > 0, f"mutation {kind} not caught"
