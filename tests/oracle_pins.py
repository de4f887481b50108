"""Pins that tie the float64 oracle to facts other than itself.

Each ``pin_*`` function takes a loaded oracle library (``oracle.load()`` or a
deliberately broken copy built by the mutation test) and raises
AssertionError (or any exception) when the oracle disagrees with:

  * exhaustive format facts (every bf16/fp16 bit pattern; round-to-nearest-even
    midpoints and overflow);
  * a 50-digit ``decimal`` brute force of the definition on tiny inputs;
  * closed forms: constant rows (loss = ln V), two-level rows, V = 2
    (softplus / logistic), V = 1;
  * invariants: shift and permutation invariance, zero row sums, ignored rows,
    batch duplication, linearity in dloss;
  * central finite differences of the loss;
  * torch's float64 cross_entropy + autograd (a library special case);
  * the per-chunk log-sum-exp merge.

The definition pinned is the textbook softmax cross-entropy behind the pages'
"Fast Cross Entropy" kernel (PyPI page "fms-acceleration-foak 0.7.4", kernel
list), with the token mean of fms-hf-tuning PR #280 ("Early Version Of This
Plugin", per-token averaging) and ignore_index = -100.
"""
from __future__ import annotations

import decimal
import math

import numpy as np

import oracle
import workloads as wl

D = decimal.Decimal
CTX = decimal.Context(prec=50)


# ---------------------------------------------------------------------------
# helpers that do not use the oracle
# ---------------------------------------------------------------------------

def _np_value(bits: np.ndarray, dtype: str) -> np.ndarray:
    """float64 value of stored elements, via numpy's own types."""
    if dtype == "f32":
        return np.asarray(bits, np.float32).astype(np.float64)
    if dtype == "bf16":
        return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def _ordered(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Monotone integer image of the bit patterns (-0 and +0 both map to 0)."""
    if dtype == "f32":
        u = np.asarray(bits, np.float32).view(np.uint32).astype(np.int64)
        mag, sign = u & 0x7FFFFFFF, (u >> 31) & 1
    else:
        u = np.asarray(bits, np.uint16).astype(np.int64)
        mag, sign = u & 0x7FFF, (u >> 15) & 1
    return np.where(sign == 1, -mag, mag)


def _from_ordered(o: int, dtype: str) -> float:
    if dtype == "f32":
        u = np.array([abs(o) | ((1 << 31) if o < 0 else 0)], np.uint32)
        return float(u.view(np.float32)[0])
    u = np.array([abs(o) | (0x8000 if o < 0 else 0)], np.uint16)
    return float(_np_value(u, dtype)[0])


def _brute(x64: np.ndarray, y: np.ndarray, dloss: float, ignore: int = -100):
    """50-digit evaluation of the definition, straight from its formulas."""
    with decimal.localcontext(CTX):
        return _brute_inner(x64, y, dloss, ignore)


def _brute_inner(x64, y, dloss, ignore):
    N, V = x64.shape
    valid = [i for i in range(N) if y[i] != ignore]
    n = len(valid)
    out_lse, out_loss, out_g = [], [], []
    for i in range(N):
        xs = [D(float(v)) for v in x64[i]]
        Z = sum((CTX.exp(v) for v in xs), D(0))
        lse = CTX.ln(Z)
        out_lse.append(lse)
        if y[i] == ignore:
            out_loss.append(D(0))
            out_g.append([D(0)] * V)
            continue
        out_loss.append(CTX.subtract(lse, xs[y[i]]))
        s = CTX.divide(D(dloss), D(n))
        g = []
        for j in range(V):
            p = CTX.divide(CTX.exp(xs[j]), Z)
            g.append(CTX.multiply(s, p - (1 if j == y[i] else 0)))
        out_g.append(g)
    L = CTX.divide(sum((out_loss[i] for i in valid), D(0)), D(n)) if n else None
    return out_lse, out_loss, out_g, L, n


def _rel_close(a: float, b: D, rel: float, abs_floor: float = 0.0) -> bool:
    b = float(b)
    return abs(a - b) <= rel * abs(b) + abs_floor


# ---------------------------------------------------------------------------
# format pins
# ---------------------------------------------------------------------------

def pin_widen_exhaustive(lib):
    for dt in ("bf16", "f16"):
        bits = np.arange(65536, dtype=np.uint16)
        got = oracle.widen(bits, dt, lib)
        ref = _np_value(bits, dt)
        same = (got == ref) | (np.isnan(got) & np.isnan(ref))
        assert same.all(), (dt, int(np.flatnonzero(~same)[0]))


def pin_round_bf16_midpoints(lib):
    # every finite positive bf16 value, its upper neighbour and their midpoint
    b = np.arange(0, 0x7F7F, dtype=np.uint16)          # below the largest finite
    lo, hi = _np_value(b, "bf16"), _np_value(b + 1, "bf16")
    mid = (lo + hi) / 2                                  # exact in float64
    even = np.where((b & 1) == 0, b, b + 1).astype(np.uint16)
    assert (oracle.round_to(lo, "bf16", lib) == b).all()
    assert (oracle.round_to(mid, "bf16", lib) == even).all()
    below = np.nextafter(mid, -np.inf)
    above = np.nextafter(mid, np.inf)
    assert (oracle.round_to(below, "bf16", lib) == b).all()
    assert (oracle.round_to(above, "bf16", lib) == b + 1).all()
    # negative side mirrors, and overflow goes to infinity at the midpoint
    assert (oracle.round_to(-mid, "bf16", lib) == (even | 0x8000)).all()
    top, inf_mid = _np_value(np.array([0x7F7F], np.uint16), "bf16")[0], None
    inf_mid = top + (top - _np_value(np.array([0x7F7E], np.uint16), "bf16")[0]) / 2
    r = oracle.round_to(np.array([inf_mid, np.nextafter(inf_mid, 0)]), "bf16", lib)
    assert r[0] == 0x7F80 and r[1] == 0x7F7F


def pin_round_f16_midpoints(lib):
    b = np.arange(0, 0x7BFF, dtype=np.uint16)
    lo, hi = _np_value(b, "f16"), _np_value(b + 1, "f16")
    mid = (lo + hi) / 2
    even = np.where((b & 1) == 0, b, b + 1).astype(np.uint16)
    assert (oracle.round_to(lo, "f16", lib) == b).all()
    assert (oracle.round_to(mid, "f16", lib) == even).all()
    assert (oracle.round_to(np.nextafter(mid, -np.inf), "f16", lib) == b).all()
    assert (oracle.round_to(np.nextafter(mid, np.inf), "f16", lib) == b + 1).all()
    # overflow threshold 65520 = 65504 + half an ulp (32/2)
    r = oracle.round_to(np.array([65520.0, np.nextafter(65520.0, 0), -65520.0]), "f16", lib)
    assert list(r) == [0x7C00, 0x7BFF, 0xFC00]


def pin_round_random_vs_numpy(lib):
    rng = np.random.default_rng(7)
    e = rng.uniform(-30, 17, 200000)
    x = rng.choice([-1.0, 1.0], e.size) * 2.0 ** e
    # numpy converts float64 -> float16 and float64 -> float32 with one rounding
    assert (oracle.round_to(x, "f16", lib) == x.astype(np.float16).view(np.uint16)).all()
    e = rng.uniform(-150, 127, 200000)
    x = rng.choice([-1.0, 1.0], e.size) * 2.0 ** e
    assert (oracle.round_to(x, "f32", lib).view(np.uint32) == x.astype(np.float32).view(np.uint32)).all()


# ---------------------------------------------------------------------------
# brute force on tiny inputs
# ---------------------------------------------------------------------------

def _tiny_cases():
    rng = np.random.default_rng(11)
    cases = []
    for dt in ("f32", "bf16", "f16"):
        for V in (1, 2, 3, 5, 16):
            N = 6
            x64 = rng.normal(0, 3, (N, V))
            if V > 1:
                x64[0, :] = 0.0
                x64[1, 0] = 12.0                       # confident row when label 0
            bits = wl.to_storage(x64, dt)
            y = rng.integers(0, V, N).astype(np.int64)
            y[1] = 0
            y[4] = -100
            cases.append((dt, bits, y, float(rng.choice([1.0, 0.5, 3.0]))))
    return cases


def pin_brute_force(lib):
    for dt, bits, y, dloss in _tiny_cases():
        x64 = _np_value(bits, dt)
        lse, loss, g, L, n = _brute(x64, y, dloss)
        r = oracle.cross_entropy(bits, y, dt, dloss=dloss, want_grad64=True, lib=lib)
        assert r["n_valid"] == n
        N, V = x64.shape
        for i in range(N):
            assert _rel_close(r["lse"][i], lse[i], 1e-14, 1e-15), (dt, V, i, "lse")
            assert _rel_close(r["loss_rows"][i], loss[i], 1e-13, 1e-15), (dt, V, i, "loss")
            for j in range(V):
                assert _rel_close(r["grad64"][i, j], g[i][j], 1e-13, 1e-300), (dt, V, i, j, "g64")
                # the stored gradient is the nearest (ties to even) representable value
                got = int(_ordered(r["grad"][i:i + 1, j], dt)[0])
                exact = g[i][j]
                cand = [(abs(D(_from_ordered(k, dt)) - exact), k) for k in (got - 1, got, got + 1)]
                best = min(cand)
                if best[1] != got:
                    # allow only a near-tie (double rounding of a value within 1e-12 of a midpoint)
                    dist_got = abs(D(_from_ordered(got, dt)) - exact)
                    assert abs(dist_got - best[0]) <= D("1e-12") * abs(exact), (dt, V, i, j, "round")
        assert _rel_close(r["loss_mean"], L, 1e-13, 1e-15), (dt, V, "mean")


def pin_confident_rows(lib):
    # p_y -> 1: loss and g_y must keep their relative precision
    for A in (8.0, 20.0, 36.0):
        V = 7
        x64 = np.zeros((2, V))
        x64[:, 2] = A
        bits = wl.to_storage(x64, "f32")
        y = np.array([2, 2], np.int64)
        r = oracle.cross_entropy(bits, y, "f32", want_grad64=True, lib=lib)
        q = (V - 1) * math.exp(-A) / (1 + (V - 1) * math.exp(-A))   # 1 - p_y
        loss = math.log1p((V - 1) * math.exp(-A))
        assert abs(r["loss_rows"][0] - loss) <= 1e-14 * loss
        assert abs(r["grad64"][0, 2] - (-0.5 * q)) <= 1e-14 * 0.5 * q


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def pin_constant_rows(lib):
    for V, dt in ((1000, "f32"), (32000, "bf16"), (49152, "f16"), (128256, "bf16"), (7, "f32")):
        x = wl.to_storage(np.full((3, V), 1.75), dt)
        y = np.array([0, V - 1, -100], np.int64)
        r = oracle.cross_entropy(x, y, dt, dloss=2.0, want_grad64=True, lib=lib)
        assert abs(r["loss_rows"][0] - math.log(V)) <= 1e-14 * math.log(V)
        assert abs(r["loss_mean"] - math.log(V)) <= 1e-14 * math.log(V)
        assert abs(r["lse"][0] - (1.75 + math.log(V))) <= 1e-14 * 12
        s = 2.0 / 2
        g = r["grad64"]
        assert np.allclose(g[0, 1:], s / V, rtol=1e-13, atol=0)
        assert abs(g[0, 0] - s * (1 / V - 1)) <= 1e-13
        assert abs(g[1, V - 1] - s * (1 / V - 1)) <= 1e-13
        assert (g[2] == 0).all()


def pin_two_level_rows(lib):
    # k entries at A, V-k at 0: lse = ln(k e^A + V - k)
    for V, k, A, lab_in_A in ((10, 1, 3.0, True), (10, 1, 3.0, False), (50, 4, -2.5, True),
                              (33, 5, 40.0, False), (4, 1, 1000.0, False), (4, 1, 1000.0, True)):
        x64 = np.zeros((1, V))
        x64[0, :k] = A
        y = np.array([0 if lab_in_A else V - 1], np.int64)
        r = oracle.cross_entropy(wl.to_storage(x64, "f32"), y, "f32", want_grad64=True, lib=lib)
        if A < 700:
            lse = math.log(k * math.exp(A) + V - k)
        else:
            lse = A + math.log(k)                      # e^-A underflows below double precision
        loss = lse - (A if lab_in_A else 0.0)
        assert abs(r["lse"][0] - lse) <= 1e-13 * abs(lse) + 1e-300
        assert abs(r["loss_rows"][0] - loss) <= 1e-13 * max(abs(loss), 1e-300) + 1e-15
        pA, p0 = math.exp(A - lse), math.exp(-lse)
        g = r["grad64"][0]
        for j in range(V):
            want = (pA if j < k else p0) - (1.0 if j == y[0] else 0.0)
            assert abs(g[j] - want) <= 1e-13, (V, k, A, j)


def pin_v2_logistic(lib):
    # V = 2: loss = softplus(x_other - x_y) = ln(1 + e^d);  g_other = sigmoid(d) = -g_y
    rng = np.random.default_rng(3)
    x64 = np.round(rng.normal(0, 4, (64, 2)) * 64) / 64
    y = rng.integers(0, 2, 64).astype(np.int64)
    r = oracle.cross_entropy(wl.to_storage(x64, "f32"), y, "f32", want_grad64=True, lib=lib)
    for i in range(64):
        d = x64[i, 1 - y[i]] - x64[i, y[i]]
        sp = max(d, 0.0) + math.log1p(math.exp(-abs(d)))
        sig = 1.0 / (1.0 + math.exp(-d))
        assert abs(r["loss_rows"][i] - sp) <= 1e-14 * sp + 1e-300
        s = 1.0 / 64
        assert abs(r["grad64"][i, 1 - y[i]] - s * sig) <= 1e-14 * s
        assert abs(r["grad64"][i, y[i]] + s * sig) <= 1e-14 * s


def pin_v1(lib):
    x = wl.to_storage(np.array([[3.0], [-7.0]]), "bf16")
    r = oracle.cross_entropy(x, np.array([0, 0], np.int64), "bf16", want_grad64=True, lib=lib)
    assert r["loss_mean"] == 0.0 and (r["grad64"] == 0).all()
    assert list(r["lse"]) == [3.0, -7.0]


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

def pin_shift_and_permutation(lib):
    rng = np.random.default_rng(5)
    N, V = 12, 40
    x64 = rng.integers(-64, 65, (N, V)).astype(np.float64)
    y = rng.integers(0, V, N).astype(np.int64)
    y[3] = -100
    for dt in ("bf16", "f16", "f32"):
        a = oracle.cross_entropy(wl.to_storage(x64, dt), y, dt, want_grad64=True, lib=lib)
        b = oracle.cross_entropy(wl.to_storage(x64 + 64.0, dt), y, dt, want_grad64=True, lib=lib)
        assert np.allclose(a["loss_rows"], b["loss_rows"], rtol=1e-13, atol=1e-13)
        assert np.allclose(a["grad64"], b["grad64"], rtol=1e-12, atol=1e-18)
        perm = rng.permutation(V)
        inv = np.argsort(perm)
        yp = np.where(y == -100, -100, inv[np.clip(y, 0, V - 1)])
        c = oracle.cross_entropy(wl.to_storage(x64[:, perm], dt), yp, dt, want_grad64=True, lib=lib)
        assert np.allclose(c["loss_rows"], a["loss_rows"], rtol=1e-13, atol=1e-13)
        assert np.allclose(c["grad64"], a["grad64"][:, perm], rtol=1e-12, atol=1e-18)
        rp = rng.permutation(N)
        d = oracle.cross_entropy(wl.to_storage(x64[rp], dt), y[rp], dt, lib=lib)
        assert abs(d["loss_mean"] - a["loss_mean"]) <= 1e-13 * abs(a["loss_mean"])


def pin_row_sums_and_signs(lib):
    rng = np.random.default_rng(6)
    x64 = rng.normal(0, 2, (20, 300))
    y = rng.integers(0, 300, 20).astype(np.int64)
    y[::5] = -100
    r = oracle.cross_entropy(wl.to_storage(x64, "f32"), y, "f32", dloss=1.5, want_grad64=True, lib=lib)
    g, s = r["grad64"], 1.5 / 16
    assert r["n_valid"] == 16
    assert np.abs(g.sum(1)).max() <= 300 * 2 ** -52 * s * 4
    for i in range(20):
        if y[i] == -100:
            assert (g[i] == 0).all() and r["loss_rows"][i] == 0.0
            assert (r["grad"][i].view(np.uint32) == 0).all()
        else:
            assert -s <= g[i, y[i]] <= 0
            others = np.delete(g[i], y[i])
            assert (others >= 0).all() and (others <= s).all()


def pin_duplicate_and_dloss(lib):
    rng = np.random.default_rng(8)
    x64 = rng.normal(0, 2, (10, 50))
    y = rng.integers(0, 50, 10).astype(np.int64)
    y[2] = -100
    bits = wl.to_storage(x64, "f32")
    a = oracle.cross_entropy(bits, y, "f32", want_grad64=True, lib=lib)
    b = oracle.cross_entropy(np.concatenate([bits, bits]), np.concatenate([y, y]), "f32",
                             want_grad64=True, lib=lib)
    assert abs(a["loss_mean"] - b["loss_mean"]) <= 1e-14 * a["loss_mean"]
    assert np.allclose(b["grad64"][:10], a["grad64"] / 2, rtol=1e-14, atol=0)
    c = oracle.cross_entropy(bits, y, "f32", dloss=-3.0, want_grad64=True, lib=lib)
    assert np.allclose(c["grad64"], -3.0 * a["grad64"], rtol=1e-14, atol=0)
    z = oracle.cross_entropy(bits, y, "f32", dloss=0.0, want_grad64=True, lib=lib)
    assert (z["grad64"] == 0).all()


def pin_no_valid_rows(lib):
    bits = wl.to_storage(np.ones((3, 5)), "bf16")
    r = oracle.cross_entropy(bits, np.full(3, -100, np.int64), "bf16", lib=lib)
    assert r["n_valid"] == 0 and math.isnan(r["loss_mean"])
    assert (r["grad"] == 0).all()


def pin_bad_label(lib):
    bits = wl.to_storage(np.ones((3, 5)), "bf16")
    for bad in (5, -1, 1 << 40):
        try:
            oracle.cross_entropy(bits, np.array([0, bad, 1], np.int64), "bf16", lib=lib)
        except oracle.LabelError:
            pass
        else:
            raise AssertionError("label %d accepted" % bad)
    r = oracle.cross_entropy(bits, np.array([0, 7, 1], np.int64), "bf16", allow_bad=True, lib=lib)
    assert r["bad"] == 1 and math.isnan(r["loss_rows"][1]) and not math.isnan(r["loss_rows"][0])


def pin_ignore_index_inside_range(lib):
    # an ignore_index inside [0, V) masks exactly the rows whose label equals it
    rng = np.random.default_rng(9)
    x64 = rng.normal(0, 1, (6, 8))
    y = np.array([3, 1, 3, 0, 7, 3], np.int64)
    r = oracle.cross_entropy(wl.to_storage(x64, "f32"), y, "f32", ignore_index=3, lib=lib)
    assert r["n_valid"] == 3
    assert (r["loss_rows"][[0, 2, 5]] == 0).all() and (r["loss_rows"][[1, 3, 4]] > 0).all()


# ---------------------------------------------------------------------------
# finite differences and the library special case
# ---------------------------------------------------------------------------

def pin_finite_differences(lib):
    rng = np.random.default_rng(12)
    N, V = 4, 9
    x64 = np.round(rng.normal(0, 1.5, (N, V)) * 256) / 256
    y = np.array([1, -100, 8, 0], np.int64)
    h = 2.0 ** -9
    base = oracle.cross_entropy(wl.to_storage(x64, "f32"), y, "f32", want_grad64=True, lib=lib)

    def L(xx):
        return oracle.cross_entropy(wl.to_storage(xx, "f32"), y, "f32", want_grad=False, lib=lib)["loss_mean"]

    for i in range(N):
        for j in range(V):
            # fourth-order central difference; every x + k h is exact in float32
            xs = []
            for k in (-2, -1, 1, 2):
                xx = x64.copy()
                xx[i, j] += k * h
                xs.append(L(xx))
            fd = (xs[0] - 8 * xs[1] + 8 * xs[2] - xs[3]) / (12 * h)
            assert abs(fd - base["grad64"][i, j]) <= 1e-8, (i, j, fd, base["grad64"][i, j])


def pin_torch_float64(lib):
    import torch
    import torch.nn.functional as F
    for k in (1, 2, 3, 4, 5):
        w = wl.WORKLOADS[k]
        p = wl.plan(w)
        rows = np.arange(0, min(w.N, 48), dtype=np.int64) if k == 1 else \
            np.sort(np.random.default_rng(k).choice(w.N, 24, replace=False))
        if p.spike_rows.size:
            rows = np.unique(np.concatenate([rows, p.spike_rows[:4], p.spike_rows[-4:]]))
        bits = wl.logits(w, rows, p)
        y = p.labels[rows]
        n_full = int((p.labels != -100).sum())
        scale = w.dloss / n_full
        r = oracle.rows(bits, y, w.dtype, scale, want_grad64=True, lib=lib)
        xt = torch.tensor(_np_value(bits, w.dtype), dtype=torch.float64, requires_grad=True)
        yt = torch.tensor(y)
        lt = F.cross_entropy(xt, yt, ignore_index=-100, reduction="none")
        (lt.sum() * scale).backward()
        assert np.allclose(r["loss"], lt.detach().numpy(), rtol=1e-12, atol=1e-12), k
        lse_t = torch.logsumexp(xt.detach(), dim=1).numpy()
        assert np.allclose(r["lse"], lse_t, rtol=1e-13, atol=1e-13), k
        assert np.allclose(r["grad64"], xt.grad.numpy(), rtol=1e-10, atol=1e-18), k


def pin_chunk_merge(lib):
    rng = np.random.default_rng(13)
    for V, dt in ((1000, "f32"), (4097, "bf16"), (70000, "bf16"), (3000, "f16")):
        row = wl.to_storage(rng.normal(0, 3, V), dt)
        x64 = _np_value(row, dt)
        m = x64.max()
        ref = m + math.log(math.fsum(np.exp(x64 - m)))
        for chunk in (0, 1, 7, 128, 999, V - 1, V, V + 5, 65536):
            got = oracle.chunked_lse(row, dt, chunk, lib)
            assert abs(got - ref) <= 1e-13 * abs(ref), (V, chunk)


def pin_threads_independent(lib):
    w = wl.custom("thr", 21, 37, 513, "bf16", 2.0, 0.1)
    bits, p = wl.make(w)
    a = oracle.cross_entropy(bits, p.labels, "bf16", threads=1, want_grad64=True, lib=lib)
    b = oracle.cross_entropy(bits, p.labels, "bf16", threads=4, want_grad64=True, lib=lib)
    assert a["loss_mean"] == b["loss_mean"]
    assert (a["grad"] == b["grad"]).all() and (a["grad64"] == b["grad64"]).all()


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
