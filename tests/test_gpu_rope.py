"""GPU parity of the RoPE entry point (ce_rope) against the float64 oracle
(oracle/rope.py), through the C ABI.

Tolerance, from the arithmetic, per element j of pair (i, i + D/2), with
X = |x_i| + |x_{i+D/2}| and u_d the storage format's unit roundoff:
  angle   theta = p base^(-2i/D) in fp64 via exp2 (the oracle uses pow): the two
          differ by at most |theta| 2^-47, moving y by at most that times X
  16-bit  cos and sin rounded to fp32 (2^-25 each), one fp32 product and one
          fp32 fma (2^-24 each, relative to X):
          |y~ - y| <= u_d |y| + (1 + u_d)(5 2^-24 + |theta| 2^-47) X + tiny
  fp32    cos, sin and the rotation in fp64, one rounding to fp32:
          |y~ - y| <= 2^-24 |y| + (6 2^-53 + |theta| 2^-47) X + tiny
Position 0 is the identity and must come back bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import cross_entropy_loss_amd as ce
import oracle
from oracle import rope as ro
from workloads import packed_positions, to_storage

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


def to_dev(bits, dtype, ld_head=None, ld_tok=None):
    """[T, H, D] storage array into a (possibly padded) device view."""
    T, H, D = bits.shape
    ld_head = ld_head or D
    ld_tok = ld_tok or H * ld_head
    raw = torch.from_numpy(np.ascontiguousarray(bits.view(np.int32) if dtype == "f32" else bits.view(np.int16)))
    buf = torch.zeros(T * ld_tok + 64, dtype=raw.dtype, device="cuda")
    view = torch.as_strided(buf, (T, H, D), (ld_tok, ld_head, 1))
    view.copy_(raw.cuda())
    return view.view(TORCH[dtype])


def host(t, dtype):
    t = t.detach().contiguous().cpu()
    return t.view(torch.int32).numpy().view(np.float32) if dtype == "f32" else t.view(torch.int16).numpy().view(np.uint16)


def check(y_t, x, dtype, pos, base, inverse=False, label=""):
    ref = ro.rope(x, dtype, pos, base, inverse)
    x64 = oracle.widen(x, dtype)
    T, H, D = x.shape
    P = D // 2
    th = np.abs(ro.angles64(pos, D, base))                     # [T, P]
    X = np.abs(x64[..., :P]) + np.abs(x64[..., P:])              # [T, H, P]
    A = np.concatenate([X, X], axis=-1)
    TH = np.concatenate([th, th], axis=-1)[:, None, :]
    if dtype == "f32":
        bound = 2.0 ** -24 * np.abs(ref["y64"]) + (6 * 2.0 ** -53 + TH * 2.0 ** -47) * A + TINY[dtype]
    else:
        u = U_D[dtype]
        bound = u * np.abs(ref["y64"]) + (1 + u) * (5 * 2.0 ** -24 + TH * 2.0 ** -47) * A + TINY[dtype]
    got_bits = host(y_t, dtype)
    got = oracle.widen(got_bits, dtype)
    err = np.abs(got - ref["y64"])
    assert (err <= bound).all(), f"{label}: {int((err > bound).sum())} beyond the bound, worst {np.max(err / bound):.3f}"
    z = pos == 0
    if z.any():
        np.testing.assert_array_equal(got_bits[z], x[z])  # the identity, bit for bit
    _say(f"  {label}: worst err/bound {np.max(err / bound):.3f}, "
         f"{100 * np.mean(got_bits == ref['y']):.2f}% equal to the rounded oracle")


def make(seed, T, H, D, dtype, scale=1.0):
    return to_storage(np.random.default_rng(seed).standard_normal((T, H, D)) * scale, dtype)


CASES = [  # dtype, T, Hq, Hk, D, base, max position
    ("bf16", 300, 32, 8, 128, 10000.0, None), ("f16", 200, 4, 2, 64, 10000.0, None),
    ("f32", 130, 5, 1, 128, 10000.0, None), ("bf16", 77, 3, 3, 256, 500000.0, None),
    ("bf16", 65, 70, 0, 16, 10000.0, None), ("f32", 50, 9, 3, 8, 10000.0, None),
    ("f16", 40, 12, 4, 80, 10000.0, None), ("bf16", 64, 8, 8, 128, 1000000.0, 600000),
    ("f32", 64, 4, 4, 64, 10000.0, 131071)]


@pytest.mark.parametrize("dtype,T,Hq,Hk,D,base,pmax", CASES,
                         ids=[f"{c[0]}-T{c[1]}-H{c[2]}x{c[3]}-D{c[4]}" for c in CASES])
def test_rope_parity(dtype, T, Hq, Hk, D, base, pmax):
    _say(f"[rope] dtype={dtype} T={T} Hq={Hq} Hk={Hk} D={D} base={base} pmax={pmax}")
    q = make(T + D, T, Hq, D, dtype)
    k = make(T + D + 1, T, max(Hk, 1), D, dtype)
    if pmax is None:
        pos = packed_positions(T, T, 1, 60)
    else:
        pos = np.random.default_rng(T).integers(0, pmax + 1, T)
        pos[0] = 0
    pd = torch.from_numpy(pos).cuda()
    qd = to_dev(q, dtype)
    kd = to_dev(k, dtype) if Hk else None
    for inverse in (False, True):
        qo, ko = ce.ce_rope(qd, kd, pd, base, inverse)
        torch.cuda.synchronize()
        check(qo, q, dtype, pos, base, inverse, f"q inverse={inverse}")
        if Hk:
            check(ko, k, dtype, pos, base, inverse, f"k inverse={inverse}")


def test_rope_strided_and_in_place():
    T, H, D = 90, 6, 128
    q = make(1, T, H, D, "bf16")
    pos = packed_positions(2, T, 5, 40)
    qd = to_dev(q, "bf16", ld_head=D + 64, ld_tok=H * (D + 64) + 256)  # padded heads and tokens
    pad = qd.as_strided((T * (H * (D + 64) + 256),), (1,)).clone()
    qo, _ = ce.ce_rope(qd, None, torch.from_numpy(pos).cuda(), 10000.0, inplace=True)
    torch.cuda.synchronize()
    assert qo.data_ptr() == qd.data_ptr()
    check(qo, q, "bf16", pos, 10000.0, label="in place, padded")
    # the padding between heads and tokens is untouched
    flat = qd.as_strided((T * (H * (D + 64) + 256),), (1,))
    mask = torch.ones_like(flat, dtype=torch.bool)
    mask.as_strided((T, H, D), (H * (D + 64) + 256, D + 64, 1)).fill_(False)
    assert torch.equal(flat[mask], pad[mask])


def test_rope_heads_major_layout_and_autograd():
    # [batch, heads, seq, D] (the attention layout after the head transpose), positions [batch, seq]
    B, H, S, D = 3, 4, 50, 64
    rng = np.random.default_rng(7)
    x = torch.from_numpy(rng.standard_normal((B, H, S, D)).astype(np.float32)).cuda().requires_grad_(True)
    pos = torch.from_numpy(np.stack([packed_positions(10 + b, S, 3, 30) for b in range(B)])).cuda()
    y = ce.rope(x, pos, 10000.0)
    g = torch.from_numpy(rng.standard_normal((B, H, S, D)).astype(np.float32)).cuda()
    y.backward(g)
    torch.cuda.synchronize()
    for b in range(B):
        xb = x[b].detach().transpose(0, 1).contiguous().cpu().numpy()   # [S, H, D]
        pb = pos[b].cpu().numpy()
        check(y[b].detach().transpose(0, 1), xb, "f32", pb, 10000.0, label=f"forward b={b}")
        check(x.grad[b].transpose(0, 1), g[b].transpose(0, 1).contiguous().cpu().numpy(), "f32", pb, 10000.0,
              inverse=True, label=f"gradient b={b}")


def test_rope_round_trip_and_repeatability():
    T, H, D = 257, 8, 128
    q = make(3, T, H, D, "f32")
    pos = torch.from_numpy(packed_positions(4, T, 10, 100)).cuda()
    qd = to_dev(q, "f32")
    a, _ = ce.ce_rope(qd, None, pos)
    b, _ = ce.ce_rope(qd, None, pos)
    back, _ = ce.ce_rope(a, None, pos, inverse=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.allclose(back, qd, rtol=0, atol=1e-5)


def test_rope_zero_tokens():
    q = torch.empty((0, 4, 64), dtype=torch.bfloat16, device="cuda")
    qo, ko = ce.ce_rope(q, None, torch.empty(0, dtype=torch.int64, device="cuda"))
    assert qo.shape == (0, 4, 64) and ko is None
