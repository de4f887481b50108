"""MI355X (gfx950) token-level softmax cross-entropy: forward, backward and the
fused forward + in-place backward, as hand-written HIP kernels behind a C ABI
(include/ce_mi355x.h).

This module only marshals torch tensors (device memory and the current HIP
stream) into the C calls of the same names; every step of the computation runs
in the library's kernels.  The operation is the "Fast Cross Entropy" loss of
the pages (PyPI page "fms-acceleration-foak 0.7.4", kernel list) used as a
drop-in replacement of a causal LM's cross-entropy (fms-acceleration PR #79,
"Bug Fix to Model Patcher"): mean over valid tokens (fms-hf-tuning PR #280,
"Early Version Of This Plugin"), ignore_index -100.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import (CE_STATUS_LABEL_RANGE, CE_STATUS_SYNC_TIMEOUT, CeError)  # noqa: F401

__all__ = [
    "ce_workspace_bytes", "ce_workspace_init", "Workspace", "ce_forward", "ce_backward",
    "ce_fwd_bwd_inplace", "ce_fwd_bwd_inplace_noalloc", "cross_entropy", "FastCrossEntropyLoss", "CeError",
    "ce_linear_workspace_bytes", "ce_linear_fwd_bwd", "ce_rmsnorm_workspace_bytes", "ce_rmsnorm_forward",
    "ce_rmsnorm_backward", "rms_norm", "FastRMSNorm", "ce_rope", "rope", "FastRoPE",
]

_DTYPES = {torch.float32: _lib.CE_DTYPE_F32, torch.bfloat16: _lib.CE_DTYPE_BF16,
           torch.float16: _lib.CE_DTYPE_F16}


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"logits dtype {t.dtype} is not float32, bfloat16 or float16") from None


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _rows(logits: torch.Tensor):
    if logits.dim() != 2:
        raise ValueError("logits must be 2-D [rows, vocab]")
    if logits.stride(1) != 1:
        raise ValueError("logits rows must be contiguous (stride(1) == 1)")
    if not logits.is_cuda:
        raise ValueError("logits must be on a GPU")
    N, V = logits.shape
    ld = logits.stride(0) if N > 1 else V
    return N, V, ld


def _labels(labels: torch.Tensor, N: int, device) -> torch.Tensor:
    if labels.dtype != torch.int64 or labels.dim() != 1 or labels.numel() != N:
        raise ValueError("labels must be a 1-D int64 tensor with one entry per row")
    if labels.device != device or not labels.is_contiguous():
        raise ValueError("labels must be contiguous on the logits' device")
    return labels


def ce_workspace_bytes(n_rows: int, vocab: int, chunk: int, dtype: torch.dtype) -> int:
    n = _lib.load().ce_workspace_bytes(n_rows, vocab, chunk, _DTYPES[dtype])
    if n == 0:
        raise ValueError("no workspace size for these arguments")
    return int(n)


def ce_workspace_init(ws: torch.Tensor) -> None:
    _lib.check(_lib.load().ce_workspace_init(_ptr(ws), ws.numel(), _stream(ws.device)), "ce_workspace_init")


class Workspace:
    """A device workspace that grows on demand; calls that share one must be
    ordered on one stream."""

    def __init__(self, device=None, nbytes: int = 0):
        self.device = torch.device(device or "cuda")
        self.buf = None
        if nbytes:
            self.reserve(nbytes)

    def reserve(self, nbytes: int) -> torch.Tensor:
        if self.buf is None or self.buf.numel() < nbytes:
            nbytes = max(nbytes, 4096)
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
            ce_workspace_init(self.buf)
        return self.buf


_default_ws: dict = {}


def _workspace(device, nbytes: int, ws: Workspace | None) -> torch.Tensor:
    if ws is None:
        key = (device, torch.cuda.current_stream(device).cuda_stream)
        ws = _default_ws.get(key)
        if ws is None:
            ws = _default_ws[key] = Workspace(device)
    return ws.reserve(nbytes)


def _outputs(N: int, device):
    f32 = dict(dtype=torch.float32, device=device)
    f64 = dict(dtype=torch.float64, device=device)
    return {
        "loss_mean": torch.empty(1, **f32),
        "loss_rows": torch.empty(max(N, 1), **f32)[:N],
        "lse_rows": torch.empty(max(N, 1), **f64)[:N],
        "pcomp_rows": torch.empty(max(N, 1), **f64)[:N],
        "n_valid": torch.empty(1, dtype=torch.int32, device=device),
        "status": torch.empty(1, dtype=torch.int32, device=device),
    }


def check_status(out: dict) -> None:
    """Synchronises and raises when the kernels flagged bad labels or a timeout."""
    st = int(out["status"].item())
    if st & CE_STATUS_SYNC_TIMEOUT:
        raise RuntimeError("cross-entropy kernel: inter-workgroup wait timed out")
    if st & CE_STATUS_LABEL_RANGE:
        raise ValueError("a label is outside [0, vocab) and not ignore_index")


def ce_forward(logits: torch.Tensor, labels: torch.Tensor, ignore_index: int = -100, chunk: int = 0,
               workspace: Workspace | None = None, out: dict | None = None) -> dict:
    """Loss mean, per-row loss / lse / (1 - p_label), n_valid and status."""
    N, V, ld = _rows(logits)
    dt = _dtype_code(logits)
    labels = _labels(labels, N, logits.device)
    out = out or _outputs(N, logits.device)
    ws = _workspace(logits.device, ce_workspace_bytes(N, V, chunk, logits.dtype), workspace)
    rc = _lib.load().ce_forward(
        _ptr(logits), ld, _ptr(labels), N, V, dt, ignore_index, chunk, _ptr(out["loss_mean"]),
        _ptr(out["loss_rows"]), _ptr(out["lse_rows"]), _ptr(out["pcomp_rows"]), _ptr(out["n_valid"]),
        _ptr(out["status"]), _ptr(ws), ws.numel(), _stream(logits.device))
    _lib.check(rc, "ce_forward")
    return out


def ce_backward(logits: torch.Tensor, labels: torch.Tensor, lse_rows: torch.Tensor, pcomp_rows: torch.Tensor,
                n_valid: torch.Tensor, dloss: torch.Tensor | None = None, ignore_index: int = -100,
                grad: torch.Tensor | None = None) -> torch.Tensor:
    """Gradient of dloss * L with respect to the logits (out of place unless
    grad is the logits tensor itself)."""
    N, V, ld = _rows(logits)
    dt = _dtype_code(logits)
    labels = _labels(labels, N, logits.device)
    if grad is None:
        grad = torch.empty_like(logits, memory_format=torch.contiguous_format)
    if grad.shape != logits.shape or grad.dtype != logits.dtype or grad.stride(1) != 1:
        raise ValueError("grad must match the logits' shape and dtype with contiguous rows")
    for t, d in ((lse_rows, torch.float64), (pcomp_rows, torch.float64), (n_valid, torch.int32)):
        if t.dtype != d or not t.is_contiguous() or t.device != logits.device:
            raise ValueError("saved statistics must be contiguous fp64 rows and an int32 count")
    if dloss is not None and (dloss.dtype != torch.float32 or dloss.numel() != 1):
        raise ValueError("dloss must be a one-element float32 tensor")
    gld = grad.stride(0) if N > 1 else V
    rc = _lib.load().ce_backward(
        _ptr(logits), ld, _ptr(labels), _ptr(lse_rows), _ptr(pcomp_rows), _ptr(n_valid), _ptr(dloss), N, V, dt,
        ignore_index, _ptr(grad), gld, _stream(logits.device))
    _lib.check(rc, "ce_backward")
    return grad


def ce_fwd_bwd_inplace(logits: torch.Tensor, labels: torch.Tensor, ignore_index: int = -100, chunk: int = 0,
                       dloss: torch.Tensor | None = None, workspace: Workspace | None = None,
                       out: dict | None = None) -> dict:
    """Forward outputs, with the gradient of dloss * L written over `logits`."""
    N, V, ld = _rows(logits)
    dt = _dtype_code(logits)
    labels = _labels(labels, N, logits.device)
    if dloss is not None and (dloss.dtype != torch.float32 or dloss.numel() != 1):
        raise ValueError("dloss must be a one-element float32 tensor")
    out = out or _outputs(N, logits.device)
    ws = _workspace(logits.device, ce_workspace_bytes(N, V, chunk, logits.dtype), workspace)
    rc = _lib.load().ce_fwd_bwd_inplace(
        _ptr(logits), ld, _ptr(labels), N, V, dt, ignore_index, chunk, _ptr(dloss), _ptr(out["loss_mean"]),
        _ptr(out["loss_rows"]), _ptr(out["lse_rows"]), _ptr(out["pcomp_rows"]), _ptr(out["n_valid"]),
        _ptr(out["status"]), _ptr(ws), ws.numel(), _stream(logits.device))
    _lib.check(rc, "ce_fwd_bwd_inplace")
    return out


def ce_fwd_bwd_inplace_noalloc(logits: torch.Tensor, labels: torch.Tensor, out: dict, ignore_index: int = -100,
                               chunk: int = 0, dloss: torch.Tensor | None = None) -> dict:
    """ce_fwd_bwd_inplace on the library's static per-GPU scratch: no
    workspace, and nothing allocated here either (the caller passes `out`,
    as made by _outputs(rows, device)).  Calls on one GPU must be ordered."""
    N, V, ld = _rows(logits)
    dt = _dtype_code(logits)
    labels = _labels(labels, N, logits.device)
    if dloss is not None and (dloss.dtype != torch.float32 or dloss.numel() != 1):
        raise ValueError("dloss must be a one-element float32 tensor")
    rc = _lib.load().ce_fwd_bwd_inplace_noalloc(
        _ptr(logits), ld, _ptr(labels), N, V, dt, ignore_index, chunk, _ptr(dloss), _ptr(out["loss_mean"]),
        _ptr(out["loss_rows"]), _ptr(out["lse_rows"]), _ptr(out["pcomp_rows"]), _ptr(out["n_valid"]),
        _ptr(out["status"]), _stream(logits.device))
    _lib.check(rc, "ce_fwd_bwd_inplace_noalloc")
    return out


def ce_linear_workspace_bytes(n_rows: int, hidden: int, vocab: int, chunk_rows: int, dtype: torch.dtype) -> int:
    n = _lib.load().ce_linear_workspace_bytes(n_rows, hidden, vocab, chunk_rows, _DTYPES[dtype])
    if n == 0:
        raise ValueError("no LM-head workspace size for these arguments")
    return int(n)


def _matrix(t: torch.Tensor, name: str):
    if t.dim() != 2 or t.stride(1) != 1 or not t.is_cuda:
        raise ValueError(f"{name} must be a 2-D GPU tensor with contiguous rows")
    return t.shape[0], t.shape[1], (t.stride(0) if t.shape[0] > 1 else t.shape[1])


def ce_linear_fwd_bwd(hidden: torch.Tensor, weight: torch.Tensor, labels: torch.Tensor, ignore_index: int = -100,
                      chunk_rows: int = 0, dloss: torch.Tensor | None = None, workspace: Workspace | None = None,
                      want_grad_hidden: bool = True, want_grad_weight: bool = True) -> dict:
    """LM-head projection + cross-entropy, forward and backward (logits =
    hidden weight^T, never stored for bf16 / fp16; fp32 goes chunk_rows rows
    at a time): loss_mean, loss_rows, n_valid, status and (when asked for)
    grad_hidden, grad_weight of dloss * L."""
    N, H, ldh = _matrix(hidden, "hidden")
    V, H2, ldw = _matrix(weight, "weight")
    if H2 != H or weight.dtype != hidden.dtype or weight.device != hidden.device:
        raise ValueError("weight must be [vocab, hidden] of the hidden states' dtype and device")
    dt = _dtype_code(hidden)
    labels = _labels(labels, N, hidden.device)
    if dloss is not None and (dloss.dtype != torch.float32 or dloss.numel() != 1):
        raise ValueError("dloss must be a one-element float32 tensor")
    dev = hidden.device
    out = {
        "loss_mean": torch.empty(1, dtype=torch.float32, device=dev),
        "loss_rows": torch.empty(max(N, 1), dtype=torch.float32, device=dev)[:N],
        "n_valid": torch.empty(1, dtype=torch.int32, device=dev),
        "status": torch.empty(1, dtype=torch.int32, device=dev),
        "grad_hidden": torch.empty_like(hidden, memory_format=torch.contiguous_format) if want_grad_hidden else None,
        "grad_weight": torch.empty_like(weight, memory_format=torch.contiguous_format) if want_grad_weight else None,
    }
    gh, gw = out["grad_hidden"], out["grad_weight"]
    if workspace is None:  # its own: the cross-entropy workspaces carry their own state from call to call
        key = (dev, torch.cuda.current_stream(dev).cuda_stream)
        workspace = _lin_ws.get(key)
        if workspace is None:
            workspace = _lin_ws[key] = Workspace(dev)
    ws = _workspace(dev, ce_linear_workspace_bytes(N, H, V, chunk_rows, hidden.dtype), workspace)
    rc = _lib.load().ce_linear_fwd_bwd(
        _ptr(hidden), ldh, _ptr(weight), ldw, _ptr(labels), N, H, V, dt, ignore_index, chunk_rows, _ptr(dloss),
        _ptr(out["loss_mean"]), _ptr(out["loss_rows"]), _ptr(out["n_valid"]), _ptr(out["status"]), _ptr(gh),
        H if gh is None else (gh.stride(0) if N > 1 else H), _ptr(gw), H if gw is None else (gw.stride(0) if V > 1 else H),
        _ptr(ws), ws.numel(), _stream(dev))
    _lib.check(rc, "ce_linear_fwd_bwd")
    return out


_norm_ws: dict = {}
_lin_ws: dict = {}


def ce_rmsnorm_workspace_bytes(n_rows: int, hidden: int, dtype: torch.dtype) -> int:
    n = _lib.load().ce_rmsnorm_workspace_bytes(n_rows, hidden, _DTYPES[dtype])
    if n == 0:
        raise ValueError("no RMSNorm workspace size for these arguments")
    return int(n)


def _norm_weight(weight: torch.Tensor, x: torch.Tensor):
    if weight.dim() != 1 or weight.numel() != x.shape[1] or weight.dtype != x.dtype or weight.device != x.device \
            or (weight.numel() > 1 and weight.stride(0) != 1):
        raise ValueError("weight must be a contiguous [hidden] tensor of x's dtype and device")


def ce_rmsnorm_forward(x: torch.Tensor, weight: torch.Tensor, eps: float = 1e-6) -> tuple:
    """RMS layer normalisation of the rows of x [rows, hidden]: (y, rstd)."""
    N, H, ldx = _matrix(x, "x")
    _norm_weight(weight, x)
    y = torch.empty((N, H), dtype=x.dtype, device=x.device)
    rstd = torch.empty(max(N, 1), dtype=torch.float32, device=x.device)[:N]
    rc = _lib.load().ce_rmsnorm_forward(_ptr(x), ldx, _ptr(weight), N, H, _dtype_code(x), eps, _ptr(y), H,
                                        _ptr(rstd), _stream(x.device))
    _lib.check(rc, "ce_rmsnorm_forward")
    return y, rstd


def ce_rmsnorm_backward(dy: torch.Tensor, x: torch.Tensor, weight: torch.Tensor, rstd: torch.Tensor,
                        inplace: bool = False, workspace: torch.Tensor | None = None) -> tuple:
    """Gradients (dx, dweight) of RMSNorm for the upstream dy; with inplace,
    dx is written over dy."""
    N, H, ldx = _matrix(x, "x")
    N2, H2, lddy = _matrix(dy, "dy")
    if (N2, H2) != (N, H) or dy.dtype != x.dtype or dy.device != x.device:
        raise ValueError("dy must match x in shape, dtype and device")
    _norm_weight(weight, x)
    if rstd.dtype != torch.float32 or rstd.numel() != N or (N > 1 and rstd.stride(0) != 1) or rstd.device != x.device:
        raise ValueError("rstd must be a contiguous float32 [rows] tensor on x's device")
    dx = dy if inplace else torch.empty((N, H), dtype=x.dtype, device=x.device)
    lddx = lddy if inplace else H
    dw = torch.empty(H, dtype=x.dtype, device=x.device)
    # its own scratch: the cross-entropy workspaces carry state from call to call
    nbytes = ce_rmsnorm_workspace_bytes(N, H, x.dtype)
    if workspace is None:
        key = (x.device, torch.cuda.current_stream(x.device).cuda_stream)
        ws = _norm_ws.get(key)
        if ws is None or ws.numel() < nbytes:
            ws = _norm_ws[key] = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    else:
        ws = workspace
        if ws.dtype != torch.uint8 or ws.numel() < nbytes or not ws.is_cuda:
            raise ValueError(f"workspace must be a uint8 GPU tensor of at least {nbytes} bytes")
    rc = _lib.load().ce_rmsnorm_backward(_ptr(dy), lddy, _ptr(x), ldx, _ptr(weight), _ptr(rstd), N, H,
                                         _dtype_code(x), _ptr(dx), lddx, _ptr(dw), _ptr(ws), ws.numel(),
                                         _stream(x.device))
    _lib.check(rc, "ce_rmsnorm_backward")
    return dx, dw


class _RMSNorm(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, weight, eps):
        y, rstd = ce_rmsnorm_forward(x, weight, eps)
        ctx.save_for_backward(x, weight, rstd)
        return y

    @staticmethod
    def backward(ctx, dy):
        x, weight, rstd = ctx.saved_tensors
        dx, dw = ce_rmsnorm_backward(dy.contiguous(), x, weight, rstd)
        return dx, dw, None


def rms_norm(x: torch.Tensor, weight: torch.Tensor, eps: float = 1e-6) -> torch.Tensor:
    """RMSNorm over the last dimension with autograd (x [..., hidden])."""
    H = x.shape[-1]
    return _RMSNorm.apply(x.reshape(-1, H), weight, eps).reshape(x.shape)


class FastRMSNorm(torch.nn.Module):
    """RMSNorm layer (weight initialised to ones) on the library's kernels."""

    def __init__(self, hidden: int, eps: float = 1e-6, dtype: torch.dtype = torch.bfloat16, device=None):
        super().__init__()
        self.weight = torch.nn.Parameter(torch.ones(hidden, dtype=dtype, device=device))
        self.eps = eps

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return rms_norm(x, self.weight, self.eps)


def _heads_view(t: torch.Tensor, name: str):
    """(tokens, heads, ld_token, ld_head) of a [tokens, heads, head_dim] view."""
    if t.dim() != 3 or t.stride(2) != 1 or not t.is_cuda:
        raise ValueError(f"{name} must be a [tokens, heads, head_dim] GPU tensor with contiguous head_dim")
    return t.shape[0], t.shape[1], t.stride(0), t.stride(1)


def ce_rope(q: torch.Tensor, k: torch.Tensor | None, positions: torch.Tensor, base: float = 10000.0,
            inverse: bool = False, inplace: bool = False) -> tuple:
    """Rotary embedding of q and k ([tokens, heads, head_dim] views) at the
    tokens' positions (int64 [tokens]); returns (q_out, k_out), written over
    q and k when inplace."""
    T, Hq, ltq, lhq = _heads_view(q, "q")
    D = q.shape[2]
    if k is not None:
        Tk, Hk, ltk, lhk = _heads_view(k, "k")
        if Tk != T or k.shape[2] != D or k.dtype != q.dtype or k.device != q.device:
            raise ValueError("k must match q in tokens, head_dim, dtype and device")
    else:
        Hk, ltk, lhk = 0, 0, 0
    if positions.dtype != torch.int64 or positions.numel() != T or positions.device != q.device \
            or (T > 1 and positions.stride(0) != 1):
        raise ValueError("positions must be a contiguous int64 [tokens] tensor on q's device")

    def out_like(t):
        return t if inplace else torch.empty_strided(t.shape, t.stride(), dtype=t.dtype, device=t.device)

    qo = out_like(q)
    ko = out_like(k) if k is not None else None
    rc = _lib.load().ce_rope(_ptr(q), _ptr(qo), ltq, lhq, Hq, _ptr(k), _ptr(ko), ltk, lhk, Hk, _ptr(positions), T, D,
                             float(base), int(inverse), _dtype_code(q), _stream(q.device))
    _lib.check(rc, "ce_rope")
    return qo, ko


def _rope_any(x: torch.Tensor, positions: torch.Tensor, base: float, inverse: bool) -> torch.Tensor:
    """x as [tokens, heads, D] or [batch, heads, seq, D] (positions [tokens] or
    [batch, seq]); the 4-D layout runs one call per batch row, each writing
    its slice of the output (same strides as x)."""
    if x.dim() == 3:
        return ce_rope(x, None, positions.reshape(-1), base, inverse)[0]
    if x.dim() != 4:
        raise ValueError("x must be [tokens, heads, head_dim] or [batch, heads, seq, head_dim]")
    out = torch.empty_strided(x.shape, x.stride(), dtype=x.dtype, device=x.device)
    pos = positions.reshape(x.shape[0], x.shape[2])
    lib = _lib.load()
    for b in range(x.shape[0]):
        xb, ob = x[b].transpose(0, 1), out[b].transpose(0, 1)  # [seq, heads, D] views
        T, H, lt, lh = _heads_view(xb, "x")
        pb = pos[b].contiguous()
        rc = lib.ce_rope(_ptr(xb), _ptr(ob), lt, lh, H, None, None, 0, 0, 0, _ptr(pb), T, x.shape[3], float(base),
                         int(inverse), _dtype_code(x), _stream(x.device))
        _lib.check(rc, "ce_rope")
    return out


class _RoPE(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, positions, base):
        ctx.save_for_backward(positions)
        ctx.base = base
        return _rope_any(x, positions, base, False)

    @staticmethod
    def backward(ctx, dy):
        (positions,) = ctx.saved_tensors
        return _rope_any(dy.contiguous(), positions, ctx.base, True), None, None


def rope(x: torch.Tensor, positions: torch.Tensor, base: float = 10000.0) -> torch.Tensor:
    """Rotary embedding with autograd: x [tokens, heads, D] with positions
    [tokens], or [batch, heads, seq, D] with positions [batch, seq]."""
    return _RoPE.apply(x, positions, base)


class FastRoPE(torch.nn.Module):
    """Applies the rotary embedding to q and k at explicit position ids."""

    def __init__(self, base: float = 10000.0):
        super().__init__()
        self.base = base

    def forward(self, q: torch.Tensor, k: torch.Tensor, positions: torch.Tensor):
        return rope(q, positions, self.base), rope(k, positions, self.base)


class _CrossEntropy(torch.autograd.Function):
    @staticmethod
    def forward(ctx, logits, labels, ignore_index, chunk, inplace_backward):
        out = ce_forward(logits, labels, ignore_index, chunk)
        ctx.save_for_backward(logits, labels, out["lse_rows"], out["pcomp_rows"], out["n_valid"])
        ctx.ignore_index = ignore_index
        ctx.inplace_backward = inplace_backward
        return out["loss_mean"][0].to(logits.dtype)

    @staticmethod
    def backward(ctx, g):
        logits, labels, lse, pcomp, n = ctx.saved_tensors
        dloss = g.reshape(1).to(torch.float32)
        grad = ce_backward(logits, labels, lse, pcomp, n, dloss, ctx.ignore_index,
                           grad=logits if ctx.inplace_backward else None)
        return grad, None, None, None, None


def cross_entropy(logits: torch.Tensor, labels: torch.Tensor, ignore_index: int = -100,
                  chunk: int = 0, inplace_backward: bool = False) -> torch.Tensor:
    """Token-mean softmax cross-entropy with autograd (logits [rows, vocab]).

    inplace_backward: the backward writes the gradient over the logits'
    storage instead of a new tensor (no second [rows, vocab] buffer; the
    logits must not be read after the backward)."""
    return _CrossEntropy.apply(logits, labels, ignore_index, chunk, inplace_backward)


class FastCrossEntropyLoss(torch.nn.Module):
    """Drop-in for torch.nn.CrossEntropyLoss(ignore_index, reduction='mean')
    over [..., vocab] logits and [...] int64 labels."""

    def __init__(self, ignore_index: int = -100, reduction: str = "mean", chunk: int = 0,
                 weight=None, label_smoothing: float = 0.0, inplace_backward: bool = False):
        super().__init__()
        if reduction != "mean" or weight is not None or label_smoothing != 0.0:
            raise NotImplementedError("only reduction='mean' without weights or label smoothing")
        self.ignore_index = ignore_index
        self.chunk = chunk
        self.inplace_backward = inplace_backward

    def forward(self, logits: torch.Tensor, labels: torch.Tensor) -> torch.Tensor:
        V = logits.shape[-1]
        return cross_entropy(logits.reshape(-1, V), labels.reshape(-1), self.ignore_index, self.chunk,
                             self.inplace_backward)
