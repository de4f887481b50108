"""The allocation-free fused entry point (ce_fwd_bwd_inplace_noalloc) against
ce_fwd_bwd_inplace through the C ABI: two calls in a row, the second on a
smaller batch, each bit for bit equal to the workspace entry point's outputs
and within the oracle's tolerances."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import cross_entropy_loss_amd as ce
import oracle
import workloads as wl
from parity import assert_grad_close, assert_rel, to_device, to_host_bits

pytestmark = pytest.mark.gpu


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _noalloc(lib, x, y, dloss, chunk=0):
    N, V = x.shape
    out = ce._outputs(N, x.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream(x.device).cuda_stream)
    rc = lib.ce_fwd_bwd_inplace_noalloc(
        _p(x), x.stride(0) if N > 1 else V, _p(y), N, V, ce._dtype_code(x), -100, chunk, _p(dloss),
        _p(out["loss_mean"]), _p(out["loss_rows"]), _p(out["lse_rows"]), _p(out["pcomp_rows"]), _p(out["n_valid"]),
        _p(out["status"]), stream)
    assert rc == 0, ce._lib.error_string(rc)
    return out


CASES = [("bf16", 600, 32000, 0, 200, 7), ("f16", 96, 49152, 0, 40, 0), ("f32", 64, 1000, 0, 7, 1000),
         ("bf16", 24, 150001, 65536, 6, 5000)]


@pytest.mark.parametrize("dtype,N1,V1,chunk,N2,V2", CASES, ids=[f"{c[0]}-{c[1]}x{c[2]}-then-{c[4]}x{c[5]}"
                                                                 for c in CASES])
def test_noalloc_matches_workspace_entry(dtype, N1, V1, chunk, N2, V2):
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this machine")
    lib = ce._lib.load()
    for k, (N, V) in enumerate(((N1, V1), (N2, V2 or V1))):
        print(f"[noalloc] {dtype} call {k}: {N}x{V} chunk={chunk if k == 0 else 0}", flush=True)
        ck = chunk if k == 0 else 0
        w = wl.custom(f"noalloc-{dtype}-{k}", 301 + k, N, V, dtype, 30.0 if dtype == "f16" else 2.0, 0.1)
        bits, p = wl.make(w)
        y = torch.from_numpy(p.labels).cuda()
        dl = torch.tensor([0.5], dtype=torch.float32, device="cuda")
        xa = to_device(bits, dtype)
        a = _noalloc(lib, xa, y, dl, ck)
        xb = to_device(bits, dtype)
        b = ce.ce_fwd_bwd_inplace(xb, y, chunk=ck, dloss=dl)
        torch.cuda.synchronize()
        ga, gb = to_host_bits(xa, dtype), to_host_bits(xb, dtype)
        assert (ga == gb).all(), "gradient differs from ce_fwd_bwd_inplace"
        for key in ("loss_mean", "loss_rows", "lse_rows", "pcomp_rows", "n_valid", "status"):
            assert torch.equal(a[key], b[key]) or (key == "loss_mean" and torch.isnan(a[key]).all()
                                                   and torch.isnan(b[key]).all()), key
        assert int(a["status"].item()) == 0
        ref = oracle.cross_entropy(bits, p.labels, dtype, dloss=0.5, threads=8)
        assert int(a["n_valid"].item()) == ref["n_valid"]
        assert_rel(float(a["loss_mean"].item()), ref["loss_mean"], dtype, "loss_mean")
        assert_grad_close(ga, ref["grad"], dtype, "noalloc grad")


