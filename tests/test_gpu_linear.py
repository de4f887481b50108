"""GPU parity of the LM-head + cross-entropy entry point against the float64
oracle (oracle/linear.py), through the C ABI.

Tolerance, from the arithmetic (u_d: unit roundoff of the storage format,
2^-8 bf16, 2^-11 fp16, 2^-24 fp32; gamma_K = K 2^-24 for an fp32 sum of K
exact products):
  logits   |x~ - x| <= E_i = gamma_H max_v sum_k |h_ik| |W_vk|        (row i)
  loss     |loss~ - loss| <= 2 E_i + 2^-23 |loss|   (lse and x_y each move by
           at most E_i; the fp32 loss is rounded once)
  g        16-bit: off the label g~ = RN_d(RN_d(e~) f~), e~ the exponential relative to
           its 256-column tile's max (stored in the format before the row's
           log-sum-exp is known) and f~ = s 2^(c - lse log2 e) the tile's factor;
           on the label g~ = RN_d(-s (1 - p_y)).  So
           |g~ - g| <= (2 u_d + u_d^2) |g| + s p (e^{2E} - 1)
           (fp16: e is stored times 2^14 and g times 2^k, s 2^k in [2^14, 2^15),
           so elements below fp16's normal range add at most s 2^-39 each, twice)
           fp32: g~ = RN(s (p~ - onehot)), u_d |g| in place of (2 u_d + u_d^2) |g|
  dh       |dh~ - dh| <= (r_d + gamma_V) (|g| |W|) + 2.1 E_i s (p |W|) + u_d |dh| + tiny
  dW       |dW~ - dW| <= (r_d + gamma_N) (|g|^T |h|) + 2.1 (E s p)^T |h| + u_d |dW| + tiny
           (r_d: the relative bound on g above)
(products of absolute values in float64; "tiny" is the format's smallest
subnormal).  The bounds are worst cases: the typical error is reported and is
far below them.
"""
from __future__ import annotations

import ctypes
import math

import numpy as np
import pytest
import torch

import cross_entropy_loss_amd as ce
import oracle
from oracle import linear as lin
from workloads import to_storage

pytestmark = pytest.mark.gpu

U = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "f32": 2.0 ** -24}
TINY = {"bf16": 2.0 ** -133, "f16": 2.0 ** -24, "f32": 2.0 ** -149}
TORCH = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this machine")
    ce._lib.load()


def _say(msg):
    print(msg, flush=True)


def make(seed, N, H, V, dtype, sigma_w=None, ignore_frac=0.1):
    rng = np.random.default_rng(seed)
    sigma_w = sigma_w if sigma_w is not None else 2.0 / math.sqrt(H)  # logits of spread ~2
    h = to_storage(rng.standard_normal((N, H)), dtype)
    w = to_storage(rng.standard_normal((V, H)) * sigma_w, dtype)
    y = rng.integers(0, V, N)
    y[rng.random(N) < ignore_frac] = -100
    return h, w, y


def to_dev(bits, dtype, ld=None):
    rows, cols = bits.shape
    ld = ld or cols
    raw = torch.from_numpy(np.ascontiguousarray(bits.view(np.int32) if dtype == "f32" else bits.view(np.int16)))
    buf = torch.zeros(rows * ld + 8, dtype=raw.dtype, device="cuda")
    view = buf[: rows * ld].view(rows, ld)[:, :cols]
    view.copy_(raw.cuda())
    return view.view(TORCH[dtype])


def host_bits(t, dtype):
    t = t.detach().contiguous().cpu()
    return t.view(torch.int32).numpy().view(np.float32) if dtype == "f32" else t.view(torch.int16).numpy().view(np.uint16)


def run(h, w, y, dtype, dloss=1.0, chunk_rows=0, ldh=None, ldw=None, **kw):
    _say(f"[linear] dtype={dtype} N,H,V={h.shape[0]},{h.shape[1]},{w.shape[0]} chunk_rows={chunk_rows} "
         f"ldh={ldh} ldw={ldw} dloss={dloss}")
    hd, wd = to_dev(h, dtype, ldh), to_dev(w, dtype, ldw)
    yd = torch.from_numpy(np.ascontiguousarray(y)).cuda()
    dl = torch.tensor([dloss], dtype=torch.float32, device="cuda")
    out = ce.ce_linear_fwd_bwd(hd, wd, yd, chunk_rows=chunk_rows, dloss=dl, **kw)
    torch.cuda.synchronize()
    return out


def check(out, h, w, y, dtype, dloss=1.0, expect_status=0):
    ref = lin.linear_cross_entropy(h, w, y, dtype, dloss=dloss)
    hx, wx = oracle.widen(h, dtype), oracle.widen(w, dtype)
    N, H = hx.shape
    V = wx.shape[0]
    assert int(out["n_valid"].item()) == ref["n_valid"]
    assert int(out["status"].item()) == expect_status
    valid = y != -100
    bad = valid & ((y < 0) | (y >= V))
    good = valid & ~bad
    g16 = 2.0 ** -24
    E = H * g16 * (np.abs(hx) @ np.abs(wx).T).max(axis=1)  # per row
    lr = out["loss_rows"].cpu().numpy().astype(np.float64)
    tol = 2 * E + 2.0 ** -23 * np.abs(ref["loss_rows"]) + 1e-30
    err = np.abs(lr - ref["loss_rows"])
    assert (err[good] <= tol[good]).all(), f"loss rows: max err/tol {np.max(err[good] / tol[good])}"
    assert (lr[~valid] == 0).all()
    assert np.isnan(lr[bad]).all()
    L = float(out["loss_mean"].item())
    if ref["n_valid"] == 0 or bad.any():
        assert math.isnan(L)
    else:
        tolL = np.sum(2 * E[valid]) / ref["n_valid"] + 2.0 ** -22 * abs(ref["loss_mean"])
        assert abs(L - ref["loss_mean"]) <= tolL, (L, ref["loss_mean"], tolL)
    if bad.any() or ref["n_valid"] == 0:
        return ref
    u = U[dtype]
    g = ref["grad_logits64"]
    s = ref["scale"]
    _, p, _, _, _ = lin.forward64(hx, wx, y)
    sp = np.where(valid[:, None], s * p, 0.0)
    for name, got_t, want, A, B, K in (
            ("grad_hidden", out["grad_hidden"], ref["grad_hidden64"], np.abs(g) @ np.abs(wx),
             (2.1 * E[:, None] * sp) @ np.abs(wx), V),
            ("grad_weight", out["grad_weight"], ref["grad_weight64"], np.abs(g).T @ np.abs(hx),
             (2.1 * E[:, None] * sp).T @ np.abs(hx), N)):
        if got_t is None:
            continue
        got = oracle.widen(host_bits(got_t, dtype), dtype)
        # g's relative rounding: two roundings to the format in the 16-bit path (the tile's exponential,
        # then its product with the tile's factor), one in the fp32 path
        rg = u if dtype == "f32" else 2 * u + u * u
        bound = (rg + K * g16) * A + B + u * np.abs(want) + TINY[dtype]
        if dtype == "f16":
            # e is stored times 2^14 and g times 2^k (s 2^k in [2^14, 2^15)): an element below fp16's
            # normal range keeps an absolute error of at most s 2^-39 in each of the two roundings
            other = wx if name == "grad_hidden" else hx
            bound = bound + abs(s) * 2.0 ** -38 * np.abs(other).sum(axis=0)[None, :]
        d = np.abs(got - want)
        ratio = d / bound
        assert (d <= bound).all(), f"{name}: {int((d > bound).sum())} beyond the bound, worst ratio {ratio.max():.3f}"
        nz = np.abs(want) > 0
        rel = np.linalg.norm((got - want)[nz]) / max(np.linalg.norm(want[nz]), 1e-300)
        _say(f"  {name}: worst err/bound {ratio.max():.3f}, relative Frobenius error {rel:.2e}")
    ign = ~valid
    if out["grad_hidden"] is not None:
        gh = host_bits(out["grad_hidden"], dtype)
        assert (oracle.widen(gh[ign], dtype) == 0).all(), "ignored rows of grad_hidden must be 0"
    return ref


# 16-bit cases run the matrix-core path (logits tiles with the tile statistics in the epilogue, the
# per-row merge and rescale, then dh and dW); vocab 3001 / 2999 leave a partial 16-byte chunk at the end of
# g's rows and a partial last vocabulary tile; N = 1100 and 600 leave a ragged last row tile; chunk_rows
# only matters for fp32.
CASES = [("bf16", 256, 384, 3000, 0), ("bf16", 300, 256, 5000, 128), ("f16", 200, 320, 4000, 64),
         ("f32", 130, 192, 2500, 64), ("bf16", 64, 128, 32000, 0), ("bf16", 513, 512, 1000, 256),
         ("bf16", 150, 192, 3001, 64), ("f16", 140, 160, 2999, 64),
         ("bf16", 256, 256, 4096, 0), ("bf16", 320, 192, 2048, 128), ("f16", 192, 256, 3072, 64),
         ("bf16", 1100, 128, 32000, 0), ("f16", 600, 64, 40000, 0)]


@pytest.mark.parametrize("dtype,N,H,V,chunk", CASES, ids=[f"{d}-N{n}-H{h}-V{v}-c{c}" for d, n, h, v, c in CASES])
def test_linear_parity(dtype, N, H, V, chunk):
    h, w, y = make(N + H + V, N, H, V, dtype)
    out = run(h, w, y, dtype, chunk_rows=chunk)
    check(out, h, w, y, dtype)


def test_linear_strided_and_dloss():
    h, w, y = make(21, 190, 160, 2100, "bf16")
    out = run(h, w, y, "bf16", dloss=0.37, chunk_rows=64, ldh=168, ldw=163)
    check(out, h, w, y, "bf16", dloss=0.37)


@pytest.mark.parametrize("ldh", [136, 131])
def test_linear_tn_strided_hidden(ldh):
    # a hidden row stride that keeps 16-byte rows takes the direct-to-LDS operand loads; one that does not
    # (131 elements) takes the element-wise loads of the same kernels
    h, w, y = make(26, 128, 128, 2048, "bf16")
    check(run(h, w, y, "bf16", chunk_rows=64, ldh=ldh), h, w, y, "bf16")


def test_linear_one_gradient_only():
    h, w, y = make(22, 100, 128, 1500, "bf16")
    a = run(h, w, y, "bf16", chunk_rows=64, want_grad_weight=False)
    assert a["grad_weight"] is None
    check(a, h, w, y, "bf16")
    b = run(h, w, y, "bf16", chunk_rows=64, want_grad_hidden=False)
    assert b["grad_hidden"] is None
    check(b, h, w, y, "bf16")


@pytest.mark.parametrize("chunk", [64, 128, 192, 0])
def test_linear_chunk_sizes(chunk):
    # one row per chunk boundary case: ragged last chunk, a single chunk
    h, w, y = make(23, 320, 128, 3000, "bf16")
    check(run(h, w, y, "bf16", chunk_rows=chunk), h, w, y, "bf16")


def test_linear_no_valid_rows_and_bad_label():
    h, w, y = make(24, 70, 64, 500, "bf16")
    out = run(h, w, np.full(70, -100), "bf16", chunk_rows=64)
    assert int(out["n_valid"].item()) == 0 and math.isnan(float(out["loss_mean"].item()))
    assert (oracle.widen(host_bits(out["grad_hidden"], "bf16"), "bf16") == 0).all()
    assert (oracle.widen(host_bits(out["grad_weight"], "bf16"), "bf16") == 0).all()
    y2 = y.copy()
    y2[5] = 500
    out = run(h, w, y2, "bf16", chunk_rows=64)
    check(out, h, w, y2, "bf16", expect_status=ce.CE_STATUS_LABEL_RANGE)


def test_linear_deterministic():
    h, w, y = make(25, 200, 256, 2000, "bf16")
    a = run(h, w, y, "bf16", chunk_rows=64)
    b = run(h, w, y, "bf16", chunk_rows=64)
    for k in ("loss_rows", "grad_hidden", "grad_weight"):
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("dtype,N,H,V", [("bf16", 40, 64, 65537), ("bf16", 64, 64, 128256), ("f16", 48, 64, 70001)])
def test_linear_wide_vocab(dtype, N, H, V):
    # vocabularies of hundreds of 256-column tiles (128256: the large-vocabulary shape), the last one ragged
    h, w, y = make(27 + V, N, H, V, dtype)
    check(run(h, w, y, dtype), h, w, y, dtype)


def test_linear_many_row_tiles():
    # 17 row tiles: two full groups of 8 in the tile order and a group of one, ragged
    h, w, y = make(28, 4100, 64, 1000, "bf16")
    check(run(h, w, y, "bf16"), h, w, y, "bf16")


def test_linear_llama3_vocab_full_size():
    # the 128k-vocabulary head at the benchmark's full size (8192 x 4096 x 128256 bf16; g alone is 2.1 GB):
    # every row's loss, 24 rows of dL/dh and 24 vocabulary rows of dL/dW against the row-blocked oracle,
    # with the bounds of check() (the logits' error E_i bounded through Cauchy-Schwarz,
    # gamma_H |h_i|_2 max_v |W_v|_2, which needs no [N, V] product)
    import workloads as wl
    lw = wl.LINEAR_WORKLOADS[4]
    h, w, y = wl.linear_inputs(lw)
    out = run(h, w, y, lw.dtype, dloss=lw.dloss)
    assert int(out["status"].item()) == 0
    rng = np.random.default_rng(29)
    N, V = len(y), w.shape[0]
    rows = np.sort(rng.choice(N, 24, replace=False))
    cols = np.unique(np.concatenate([y[rows[:12]][y[rows[:12]] >= 0], rng.choice(V, 12, replace=False)]))
    _say(f"  oracle over {N} rows in blocks (rows {rows[:4]}..., {len(cols)} vocabulary rows)")
    ref = lin.linear_sampled(h, w, y, lw.dtype, rows, cols, dloss=lw.dloss)
    assert int(out["n_valid"].item()) == ref["n_valid"]
    hx, wx = oracle.widen(h, lw.dtype), oracle.widen(w, lw.dtype)
    g16, u = 2.0 ** -24, U[lw.dtype]
    E = lw.H * g16 * np.linalg.norm(hx, axis=1) * np.linalg.norm(wx, axis=1).max()
    valid = y != -100
    lr = out["loss_rows"].cpu().numpy().astype(np.float64)
    tol = 2 * E + 2.0 ** -23 * np.abs(ref["loss_rows"]) + 1e-30
    err = np.abs(lr - ref["loss_rows"])
    assert (err[valid] <= tol[valid]).all(), f"loss rows: max err/tol {np.max(err[valid] / tol[valid])}"
    assert (lr[~valid] == 0).all()
    L = float(out["loss_mean"].item())
    assert abs(L - ref["loss_mean"]) <= np.sum(2 * E[valid]) / ref["n_valid"] + 2.0 ** -22 * abs(ref["loss_mean"])
    s, rg = ref["scale"], 2 * u + u * u
    # |g| <= s (p + onehot) on valid rows
    _, p_rows, _, _, _ = lin.forward64(hx[rows], wx, y[rows])
    aw = np.abs(wx)
    onehot_w = np.where((valid[rows] & (y[rows] >= 0))[:, None], aw[np.clip(y[rows], 0, V - 1)], 0.0)
    sp_rows = np.where(valid[rows][:, None], s * p_rows, 0.0)
    A = sp_rows @ aw + s * onehot_w
    B = (2.1 * E[rows][:, None] * sp_rows) @ aw
    got = oracle.widen(host_bits(out["grad_hidden"][torch.from_numpy(rows).cuda()], lw.dtype), lw.dtype)
    want = ref["grad_hidden64"]
    bound = (rg + V * g16) * A + B + u * np.abs(want) + TINY[lw.dtype]
    d = np.abs(got - want)
    assert (d <= bound).all(), f"grad_hidden rows: worst err/bound {(d / bound).max():.3f}"
    _say(f"  grad_hidden rows: worst err/bound {(d / bound).max():.3f}")
    pc = np.where(valid[:, None], ref["softmax_cols"], 0.0)
    hit = (y[:, None] == cols[None, :]) & valid[:, None]
    ah = np.abs(hx)
    A = s * (pc + hit).T @ ah
    B = (2.1 * s * E[:, None] * pc).T @ ah
    got = oracle.widen(host_bits(out["grad_weight"][torch.from_numpy(cols).cuda()], lw.dtype), lw.dtype)
    want = ref["grad_weight64"]
    bound = (rg + N * g16) * A + B + u * np.abs(want) + TINY[lw.dtype]
    d = np.abs(got - want)
    assert (d <= bound).all(), f"grad_weight rows: worst err/bound {(d / bound).max():.3f}"
    _say(f"  grad_weight rows: worst err/bound {(d / bound).max():.3f}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_linear_wide_logit_range(dtype):
    # logits spread ~25 (weights 12x the default): within a tile the exponentials relative to its max span
    # fp16's subnormals (e is stored times 2^14) and far below, and the tiles' shifts differ widely
    h, w, y = make(31, 300, 64, 5000, dtype, sigma_w=25.0 / math.sqrt(64))
    check(run(h, w, y, dtype, dloss=2.0), h, w, y, dtype, dloss=2.0)


@pytest.mark.parametrize("N,V", [(256, 3000), (4096, 1500)])
def test_linear_unaligned_grad_outputs(N, V):
    # through the C ABI: grad_hidden and grad_weight one element past a 16-byte boundary with an odd row
    # stride, so the products (and, with vocabulary 3000, dL/dh's sum over its two ranges) store element by
    # element; the values must be those of the aligned call, bit for bit
    H = 128
    h, w, y = make(33 + N, N, H, V, "bf16")
    ref = run(h, w, y, "bf16")
    hd, wd = to_dev(h, "bf16"), to_dev(w, "bf16")
    yd = torch.from_numpy(np.ascontiguousarray(y)).cuda()
    ld = H + 3
    gh_buf = torch.zeros(N * ld + 16, dtype=torch.bfloat16, device="cuda")
    gw_buf = torch.zeros(V * ld + 16, dtype=torch.bfloat16, device="cuda")
    lib = ce._lib.load()
    nbytes = lib.ce_linear_workspace_bytes(N, H, V, 0, ce._lib.CE_DTYPE_BF16)
    ws = torch.zeros(nbytes + 256, dtype=torch.uint8, device="cuda")
    off = (-ws.data_ptr()) % 256
    outs = [torch.empty(1, dtype=torch.float32, device="cuda"), torch.empty(N, dtype=torch.float32, device="cuda"),
            torch.empty(1, dtype=torch.int32, device="cuda"), torch.empty(1, dtype=torch.int32, device="cuda")]
    P = lambda t, k=0: ctypes.c_void_p(t.data_ptr() + k)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = lib.ce_linear_fwd_bwd(P(hd), H, P(wd), H, P(yd), N, H, V, ce._lib.CE_DTYPE_BF16, -100, 0, None,
                               P(outs[0]), P(outs[1]), P(outs[2]), P(outs[3]), P(gh_buf, 2), ld, P(gw_buf, 2), ld,
                               P(ws, off), nbytes, st)
    assert rc == 0
    torch.cuda.synchronize()
    gh = gh_buf[1:1 + N * ld].view(N, ld)[:, :H]
    gw = gw_buf[1:1 + V * ld].view(V, ld)[:, :H]
    assert torch.equal(gh.view(torch.int16), ref["grad_hidden"].view(torch.int16))
    assert torch.equal(gw.view(torch.int16), ref["grad_weight"].view(torch.int16))
    assert torch.equal(outs[1], ref["loss_rows"])
