"""GPU parity of the RMSNorm entry points against the float64 oracle
(oracle/rmsnorm.py), through the C ABI.

Tolerance, from the arithmetic (u_d: unit roundoff of the storage format,
2^-8 bf16, 2^-11 fp16, 2^-24 fp32; u: unit roundoff of the kernel's working
precision, 2^-24 for the 16-bit formats, 2^-53 for fp32 rows; the sum of
squares and the dot product run over at most H terms):
  rstd   relative error <= (H/2 + 2) 2^-24 (fp32 sum of squares, one rounding
         of the result to fp32); fp32 rows: 2^-24 + H 2^-53
  y      |y~ - y| <= (u_d + d)(1 + d) |y| + tiny,  d = (H/2 + 3) u + 2^-24
  dx     with r~ = r (1 + e_r), |e_r| <= d_r (the rstd handed in), A = |w dy|,
         B = |x^ c|, S = sum_k |x^_k w_k dy_k| and E = (d_r + (H + 3) u) S:
         |dx~ - dx| <= u_d |dx| + 1.1 [r (A + B)(d_r + 4u) + r |x^| E / H
                                       + (d_r + 2 2^-24) |dx|] + tiny
  dw     |dw~ - dw| <= u_d |dw| + 1.1 (d_r + (N + 6) 2^-24) sum_rows |dy x^| + tiny
(first-order bounds with a 10% margin for the second-order terms; fp32 dw
sums run in fp32 within a workgroup and in fp64 across workgroups).
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import cross_entropy_loss_amd as ce
import oracle
from oracle import rmsnorm as rn
from workloads import to_storage

pytestmark = pytest.mark.gpu

U_D = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "f32": 2.0 ** -24}
TINY = {"bf16": 2.0 ** -133, "f16": 2.0 ** -24, "f32": 2.0 ** -149}
TORCH = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this machine")
    ce._lib.load()


def _say(msg):
    print(msg, flush=True)


def make(seed, N, H, dtype, scale=1.0):
    rng = np.random.default_rng(seed)
    x = to_storage(rng.standard_normal((N, H)) * scale, dtype)
    w = to_storage(1.0 + 0.25 * rng.standard_normal(H), dtype)
    dy = to_storage(rng.standard_normal((N, H)), dtype)
    return x, w, dy


def to_dev(bits, dtype, ld=None):
    bits = np.atleast_2d(bits) if bits.ndim == 1 else bits
    rows, cols = bits.shape
    ld = ld or cols
    raw = torch.from_numpy(np.ascontiguousarray(bits.view(np.int32) if dtype == "f32" else bits.view(np.int16)))
    buf = torch.zeros(rows * ld + 16, dtype=raw.dtype, device="cuda")
    view = buf[: rows * ld].view(rows, ld)[:, :cols]
    view.copy_(raw.cuda())
    return view.view(TORCH[dtype])


def host_bits(t, dtype):
    t = t.detach().contiguous().cpu()
    return t.view(torch.int32).numpy().view(np.float32) if dtype == "f32" else t.view(torch.int16).numpy().view(np.uint16)


def wide(t, dtype):
    return oracle.widen(host_bits(t, dtype), dtype)


def u_work(dtype):
    return 2.0 ** -53 if dtype == "f32" else 2.0 ** -24


def rstd_bound(H, dtype):
    return 2.0 ** -24 + H * 2.0 ** -53 if dtype == "f32" else (H / 2 + 2) * 2.0 ** -24


def check_forward(y_t, rstd_t, x, w, dtype, eps):
    H = x.shape[1]
    ref = rn.rmsnorm(x, w, dtype, eps)
    r = rstd_t.cpu().numpy().astype(np.float64)
    rel = np.abs(r - ref["rstd"]) / ref["rstd"]
    assert (rel <= rstd_bound(H, dtype)).all(), f"rstd: worst relative error {rel.max():.3e}"
    y = wide(y_t, dtype)
    d = (H / 2 + 3) * u_work(dtype) + 2.0 ** -24
    bound = (U_D[dtype] + d) * (1 + d) * np.abs(ref["y64"]) + TINY[dtype]
    err = np.abs(y - ref["y64"])
    assert (err <= bound).all(), f"y: {int((err > bound).sum())} beyond the bound, worst {np.max(err / bound):.3f}"
    exact = np.mean(host_bits(y_t, dtype) == ref["y"])
    _say(f"  y: worst err/bound {np.max(err / bound):.3f}, {100 * exact:.2f}% equal to the rounded oracle")
    return ref


def check_backward(dx_t, dw_t, dy, x, w, dtype, eps, d_r):
    """dx, dw against the oracle's float64 gradient; d_r bounds the relative
    error of the fp32 rstd the kernel was given."""
    N, H = x.shape
    x64, w64, dy64 = oracle.widen(x, dtype), oracle.widen(w, dtype), oracle.widen(dy, dtype)
    dx64, dw64 = rn.backward64(dy64, x64, w64, eps)
    _, r = rn.forward64(x64, w64, eps)
    u = u_work(dtype)
    xh = x64 * r[:, None]
    S = np.sum(np.abs(xh * w64[None, :] * dy64), axis=1)
    c = np.sum(xh * w64[None, :] * dy64, axis=1) / H
    A = np.abs(w64[None, :] * dy64)
    B = np.abs(xh * c[:, None])
    E = (d_r + (H + 3) * u) * S
    bound = (U_D[dtype] * np.abs(dx64) + 1.1 * (r[:, None] * (A + B) * (d_r + 4 * u)
                                              + r[:, None] * np.abs(xh) * (E / H)[:, None]
                                              + (d_r + 2 * 2.0 ** -24) * np.abs(dx64)) + TINY[dtype])
    got = wide(dx_t, dtype)
    err = np.abs(got - dx64)
    assert (err <= bound).all(), f"dx: {int((err > bound).sum())} beyond the bound, worst {np.max(err / bound):.3f}"
    gw = wide(dw_t, dtype).reshape(-1)
    bw = U_D[dtype] * np.abs(dw64) + 1.1 * (d_r + (N + 6) * 2.0 ** -24) * np.sum(np.abs(dy64 * xh), axis=0) \
        + TINY[dtype]
    ew = np.abs(gw - dw64)
    assert (ew <= bw).all(), f"dw: {int((ew > bw).sum())} beyond the bound, worst {np.max(ew / bw):.3f}"
    _say(f"  dx: worst err/bound {np.max(err / bound):.3f}; dw: worst err/bound {np.max(ew / bw):.3f}")


def oracle_rstd32(x, w, dtype, eps):
    _, r = rn.forward64(oracle.widen(x, dtype), oracle.widen(w, dtype), eps)
    return torch.from_numpy(r.astype(np.float32)).cuda()


# (dtype, N, H, ld): one wave per row, 1..32 vectors per lane, ragged last vector slots, strided rows
FWD_CASES = [("bf16", 37, 8, None), ("bf16", 64, 512, None), ("bf16", 130, 4096, None), ("f16", 129, 4096, None),
             ("f32", 131, 4096, None), ("bf16", 33, 4104, None), ("bf16", 17, 16384, None), ("f32", 9, 8192, None),
             ("f16", 50, 1000, 1024), ("f32", 41, 252, 260), ("bf16", 5, 2056, None), ("f16", 3, 16384, 16392)]


@pytest.mark.parametrize("dtype,N,H,ld", FWD_CASES, ids=[f"{d}-N{n}-H{h}-ld{l}" for d, n, h, l in FWD_CASES])
def test_rmsnorm_forward_parity(dtype, N, H, ld):
    _say(f"[rmsnorm fwd] dtype={dtype} N={N} H={H} ld={ld}")
    x, w, _ = make(N * 7 + H, N, H, dtype)
    eps = 1e-6
    y, rstd = ce.ce_rmsnorm_forward(to_dev(x, dtype, ld), to_dev(w, dtype)[0], eps)
    torch.cuda.synchronize()
    check_forward(y, rstd, x, w, dtype, eps)


# rows split over 2 or 4 waves past 4096 (16-bit) / 2048 (fp32) elements: 4104, 8192, 12296, 16384; 4096, 8192
BWD_CASES = [("bf16", 37, 8), ("bf16", 64, 512), ("bf16", 1031, 4096), ("f16", 700, 4096), ("f32", 301, 2048),
             ("bf16", 5, 2056), ("f16", 2000, 1000), ("f32", 64, 252), ("bf16", 3, 64),
             ("bf16", 37, 4104), ("bf16", 515, 8192), ("f16", 21, 12296), ("bf16", 130, 16384), ("f32", 77, 4096),
             ("f32", 9, 8192), ("bf16", 2500, 8192)]


@pytest.mark.parametrize("dtype,N,H", BWD_CASES, ids=[f"{d}-N{n}-H{h}" for d, n, h in BWD_CASES])
def test_rmsnorm_backward_parity(dtype, N, H):
    _say(f"[rmsnorm bwd] dtype={dtype} N={N} H={H}")
    x, w, dy = make(N * 11 + H, N, H, dtype)
    eps = 1e-5
    r32 = oracle_rstd32(x, w, dtype, eps)
    dx, dw = ce.ce_rmsnorm_backward(to_dev(dy, dtype), to_dev(x, dtype), to_dev(w, dtype)[0], r32)
    torch.cuda.synchronize()
    check_backward(dx, dw, dy, x, w, dtype, eps, 2.0 ** -24)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_rmsnorm_forward_then_backward(dtype):
    # the backward on the forward's own rstd, strided inputs, dx written over dy
    N, H = 257, 2048
    _say(f"[rmsnorm chain] dtype={dtype} N={N} H={H}")
    x, w, dy = make(31, N, H, dtype, scale=3.0)
    eps = 1e-6
    xd, wd = to_dev(x, dtype, H + 64), to_dev(w, dtype)[0]
    y, rstd = ce.ce_rmsnorm_forward(xd, wd, eps)
    check_forward(y, rstd, x, w, dtype, eps)
    dyd = to_dev(dy, dtype, H + 8 * (4 if dtype != "f32" else 2))
    dx, dw = ce.ce_rmsnorm_backward(dyd, xd, wd, rstd, inplace=True)
    torch.cuda.synchronize()
    assert dx.data_ptr() == dyd.data_ptr()
    check_backward(dx, dw, dy, x, w, dtype, eps, rstd_bound(H, dtype))


def test_rmsnorm_forward_in_place():
    x, w, _ = make(41, 90, 1024, "bf16")
    xd, wd = to_dev(x, "bf16"), to_dev(w, "bf16")[0]
    rstd = torch.empty(90, dtype=torch.float32, device="cuda")  # every buffer held for the whole call
    ref_y, ref_r = ce.ce_rmsnorm_forward(xd.clone(), wd)
    rc = ce._lib.load().ce_rmsnorm_forward(ce._ptr(xd), 1024, ce._ptr(wd), 90, 1024, ce._lib.CE_DTYPE_BF16, 1e-6,
                                           ce._ptr(xd), 1024, ce._ptr(rstd), ce._stream(xd.device))
    ce._lib.check(rc, "ce_rmsnorm_forward")
    torch.cuda.synchronize()
    assert torch.equal(xd, ref_y) and torch.equal(rstd, ref_r)


def test_rmsnorm_extreme_ranges():
    # bf16 rows beyond fp32's square range, and rows of subnormal-sized squares with eps = 0:
    # the fp32 sum of squares would overflow / lose its digits; the kernel redoes it in fp64
    rng = np.random.default_rng(5)
    H = 1024
    big = rng.standard_normal((4, H)) * 2.0 ** 100
    small = rng.standard_normal((4, H)) * 2.0 ** -70
    fp16_max = np.clip(rng.standard_normal((4, H)) * 30000, -65504, 65504)
    for dtype, rows, eps in (("bf16", big, 1e-6), ("bf16", small, 0.0), ("f16", fp16_max, 1e-6)):
        _say(f"[rmsnorm range] dtype={dtype} eps={eps} max|x|={np.abs(rows).max():.3e}")
        x = to_storage(rows, dtype)
        w = to_storage(np.ones(H), dtype)
        y, rstd = ce.ce_rmsnorm_forward(to_dev(x, dtype), to_dev(w, dtype)[0], eps)
        torch.cuda.synchronize()
        assert torch.isfinite(rstd).all()
        check_forward(y, rstd, x, w, dtype, eps)


def test_rmsnorm_zero_rows():
    w = to_storage(np.ones(64), "bf16")
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    y, rstd = ce.ce_rmsnorm_forward(x, to_dev(w, "bf16")[0])
    assert y.shape == (0, 64) and rstd.numel() == 0
    dx, dw = ce.ce_rmsnorm_backward(x, x, to_dev(w, "bf16")[0], rstd)
    torch.cuda.synchronize()
    assert dx.shape == (0, 64) and (dw.float() == 0).all()


def test_rmsnorm_zero_row_eps0_is_nan():
    # a row of zeros with eps = 0: rstd = 1/0 = inf and y = 0 * inf = NaN in the float64 definition too
    x = np.zeros((2, 64))
    x[1] = 1.0
    xs, ws = to_storage(x, "bf16"), to_storage(np.ones(64), "bf16")
    ref = rn.rmsnorm(xs, ws, "bf16", 0.0)
    y, rstd = ce.ce_rmsnorm_forward(to_dev(xs, "bf16"), to_dev(ws, "bf16")[0], 0.0)
    torch.cuda.synchronize()
    assert math.isinf(float(rstd[0])) and math.isinf(ref["rstd"][0])
    assert torch.isnan(y[0].float()).all() and np.isnan(ref["y64"][0]).all()
    assert (y[1].float() == 1.0).all() and float(rstd[1]) == 1.0


def test_rmsnorm_backward_deterministic_and_repeatable():
    x, w, dy = make(51, 3001, 4096, "bf16")
    r32 = oracle_rstd32(x, w, "bf16", 1e-6)
    args = (to_dev(dy, "bf16"), to_dev(x, "bf16"), to_dev(w, "bf16")[0], r32)
    a = ce.ce_rmsnorm_backward(*args)
    for _ in range(3):
        b = ce.ce_rmsnorm_backward(*args)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    # a smaller call through the same cached workspace, then the large one again
    small = ce.ce_rmsnorm_backward(args[0][:10], args[1][:10], args[2], r32[:10])
    c = ce.ce_rmsnorm_backward(*args)
    torch.cuda.synchronize()
    assert torch.equal(a[1], c[1])
    check_backward(small[0], small[1], dy[:10], x[:10], w, "bf16", 1e-6, 2.0 ** -24)


def test_rmsnorm_autograd_module():
    torch.manual_seed(0)
    m = ce.FastRMSNorm(512, eps=1e-6, dtype=torch.float32, device="cuda")
    with torch.no_grad():
        m.weight.copy_(1 + 0.1 * torch.randn(512))
    x = torch.randn(3, 40, 512, device="cuda", requires_grad=True)
    y = m(x)
    g = torch.randn_like(y)
    y.backward(g)
    torch.cuda.synchronize()
    xs = x.detach().reshape(-1, 512).cpu().numpy()
    ws = m.weight.detach().cpu().numpy()
    gs = g.reshape(-1, 512).cpu().numpy()
    ref = rn.rmsnorm(xs, ws, "f32", 1e-6)
    np.testing.assert_allclose(y.detach().reshape(-1, 512).cpu().numpy(), ref["y64"], rtol=2.0 ** -23, atol=0)
    check_backward(x.grad.reshape(-1, 512), m.weight.grad, gs, xs, ws, "f32", 1e-6, rstd_bound(512, "f32"))
