"""GPU parity: the HIP library against the float64 oracle, element by element,
on seeded inputs (tolerances in tests/parity.py).  Every call goes through the
C ABI (the ctypes binding only marshals pointers)."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import cross_entropy_loss_amd as ce
import oracle
import workloads as wl
from parity import REL, assert_grad_close, assert_rel, to_device, to_host_bits, ulp_distance

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this machine")
    ce._lib.load()  # raises when the library is missing


def _say(msg):
    print(msg, flush=True)


def run_fused(bits, labels, dtype, dloss=1.0, chunk=0, ld=None, offset=0, ignore=-100):
    _say(f"[fused] dtype={dtype} shape={bits.shape} ld={ld} offset={offset} chunk={chunk} dloss={dloss}")
    x = to_device(bits, dtype, ld, offset)
    y = torch.from_numpy(np.ascontiguousarray(labels)).cuda()
    dl = torch.tensor([dloss], dtype=torch.float32, device="cuda")
    out = ce.ce_fwd_bwd_inplace(x, y, ignore, chunk, dl)
    torch.cuda.synchronize()
    return out, x


def check_against_oracle(out, grad_t, bits, labels, dtype, dloss=1.0, ignore=-100, expect_status=0):
    ref = oracle.cross_entropy(bits, labels, dtype, ignore_index=ignore, dloss=dloss, allow_bad=True, threads=8)
    valid = labels != ignore
    n = int(out["n_valid"].item())
    assert n == ref["n_valid"]
    assert int(out["status"].item()) == expect_status
    L = float(out["loss_mean"].item())
    if ref["n_valid"] == 0 or ref["bad"]:
        assert math.isnan(L)
    else:
        assert_rel(L, ref["loss_mean"], dtype, "loss_mean")
    good = valid & ~np.isnan(ref["loss_rows"])
    loss_rows = out["loss_rows"].cpu().numpy()
    lse_rows = out["lse_rows"].cpu().numpy()
    pcomp = out["pcomp_rows"].cpu().numpy()
    assert_rel(loss_rows[good], ref["loss_rows"][good], dtype, "loss_rows")
    assert_rel(lse_rows[good], ref["lse"][good], dtype, "lse_rows")
    pc_ref = -np.expm1(-ref["loss_rows"][good])  # 1 - p_y from the oracle's loss
    assert_rel(pcomp[good], pc_ref, dtype, "pcomp_rows")
    assert (loss_rows[~valid] == 0).all() and (lse_rows[~valid] == 0).all()
    bad_rows = valid & np.isnan(ref["loss_rows"])
    assert np.isnan(loss_rows[bad_rows]).all()
    g = to_host_bits(grad_t, dtype)
    if bad_rows.any():
        gv = g[bad_rows].view(np.float32) if dtype == "f32" else g[bad_rows]
        if dtype == "f32":
            assert np.isnan(gv).all()
        else:
            assert ((gv & 0x7FFF) > (0x7F80 if dtype == "bf16" else 0x7C00)).all()
    rows_ok = ~bad_rows
    assert_grad_close(g[rows_ok], ref["grad"][rows_ok], dtype, "grad")
    zero = g[~valid].view(np.uint32 if dtype == "f32" else np.uint16)
    assert (zero == 0).all(), "ignored rows must be +0"
    return ref


# ---------------------------------------------------------------------------

def test_config1_tiny():
    w = wl.WORKLOADS[1]
    bits, p = wl.make(w)
    out, g = run_fused(bits, p.labels, w.dtype)
    check_against_oracle(out, g, bits, p.labels, w.dtype)


RAGGED = [(d, V) for d in ("bf16", "f16") for V in (1, 2, 3, 7, 8, 9, 17, 1000, 1023, 2049, 4097, 32001)] + \
         [("f32", V) for V in (1, 3, 4, 5, 999, 4097, 16385, 24001, 32000, 49999, 65536)]


@pytest.mark.parametrize("dtype,V", RAGGED, ids=[f"{d}-V{v}" for d, v in RAGGED])
def test_ragged_rows(dtype, V):
    w = wl.custom(f"ragged-{dtype}-{V}", 100 + V, 37, V, dtype, 30.0 if dtype == "f16" else 2.0, 0.1)
    bits, p = wl.make(w)
    out, g = run_fused(bits, p.labels, dtype)
    check_against_oracle(out, g, bits, p.labels, dtype)


@pytest.mark.parametrize("V", [32000, 32005, 49152, 65536, 98304, 128256])
def test_tiles_and_tails_bf16(V):
    # the whole-row kernel at several capacities, with a ragged last vector
    w = wl.custom(f"tiles-{V}", 7 + V, 24, V, "bf16", 3.0, 0.1)
    bits, p = wl.make(w)
    out, g = run_fused(bits, p.labels, "bf16")
    check_against_oracle(out, g, bits, p.labels, "bf16")


@pytest.mark.parametrize("k", [2, 3, 4, 5])
def test_config_rows(k):
    # the first 96 rows of each workload at its real vocabulary, chunking and dloss
    w = wl.WORKLOADS[k]
    p = wl.plan(w)
    rows = np.arange(96)
    bits = wl.logits(w, rows, p)
    labels = p.labels[rows]
    out, g = run_fused(bits, labels, w.dtype, dloss=w.dloss, chunk=w.chunk)
    check_against_oracle(out, g, bits, labels, w.dtype, dloss=w.dloss)


@pytest.mark.parametrize("dtype,ld,offset", [("bf16", 1003, 1), ("bf16", 1000, 3), ("f16", 1007, 5),
                                             ("f32", 1001, 1), ("f32", 1000, 2)])
def test_strided_and_unaligned(dtype, ld, offset):
    w = wl.custom(f"strided-{dtype}", 17, 29, 1000, dtype, 2.0, 0.1)
    bits, p = wl.make(w)
    out, g = run_fused(bits, p.labels, dtype, ld=ld, offset=offset)
    check_against_oracle(out, g, bits, p.labels, dtype)


@pytest.mark.parametrize("dtype,V,ld,offset", [("bf16", 32001, 32003, 1), ("bf16", 5000, 5000, 3),
                                               ("f16", 32001, 32011, 5), ("f16", 70001, 70001, 7)])
def test_split_rows_strided_and_unaligned(dtype, V, ld, offset):
    # rows cut into pieces whose 16-byte phase differs from piece to piece
    w = wl.custom(f"split-strided-{dtype}-{V}", 23, 21, V, dtype, 30.0 if dtype == "f16" else 2.0, 0.1)
    bits, p = wl.make(w)
    out, g = run_fused(bits, p.labels, dtype, ld=ld, offset=offset)
    check_against_oracle(out, g, bits, p.labels, dtype)
    st = g.untyped_storage()
    buf = torch.empty(0, dtype=torch.int16, device=g.device).set_(st, 0, (st.nbytes() // 2,), (1,))
    rows = buf[offset: offset + bits.shape[0] * ld].view(bits.shape[0], ld)
    assert (rows[:, V:] == 0).all() and (buf[:offset] == 0).all() and (buf[offset + bits.shape[0] * ld:] == 0).all(), \
        "elements outside the rows were written"


# rows that fit on chip are reduced whole whatever the chunk; wider rows
# (beyond 131072 16-bit or 65536 fp32 elements) are cut into slabs of width
# chunk (0: 65536 / 32768) whose partials are merged
CHUNKS = [("f32", 1000, c) for c in (1, 7, 128, 999, 1000)] + \
         [("bf16", 4097, c) for c in (1, 64, 1000, 4096, 4097)] + [("f16", 3000, 1024), ("bf16", 70000, 65536)] + \
         [("bf16", 140000, 0), ("bf16", 140001, 50000), ("f16", 200003, 65536), ("f16", 131073, 1),
          ("f32", 70001, 0), ("f32", 65537, 20000)]


@pytest.mark.parametrize("dtype,V,chunk", CHUNKS, ids=[f"{d}-V{v}-c{c}" for d, v, c in CHUNKS])
def test_chunked(dtype, V, chunk):
    N = 64 if V <= 1000 else (12 if V <= 70000 else 6)
    w = wl.custom(f"chunk-{dtype}-{V}", 5, N, V, dtype, 1.0 if dtype == "f32" else 2.0, 0.1)
    bits, p = wl.make(w)
    out, g = run_fused(bits, p.labels, dtype, chunk=chunk)
    check_against_oracle(out, g, bits, p.labels, dtype)


def test_slab_calls_leave_no_stale_status():
    # the slab path's second launch has workgroups the finisher does not wait
    # for; none of them may leave a status bit behind for the next call
    w = wl.custom("slab-status", 9, 6, 131073, "f16", 2.0, 0.1)
    bits, p = wl.make(w)
    small = wl.custom("slab-status-small", 10, 8, 1000, "f32", 1.0, 0.1)
    sbits, sp = wl.make(small)
    for i in range(4):
        out, g = run_fused(bits, p.labels, "f16", chunk=1)
        assert int(out["status"].item()) == 0, f"call {i}"
        out, g = run_fused(sbits, sp.labels, "f32")
        assert int(out["status"].item()) == 0, f"call {i} (small)"
    check_against_oracle(out, g, sbits, sp.labels, "f32")


def test_no_valid_rows():
    bits = wl.to_storage(np.random.default_rng(1).normal(0, 2, (9, 500)), "bf16")
    labels = np.full(9, -100, np.int64)
    out, g = run_fused(bits, labels, "bf16")
    assert int(out["n_valid"].item()) == 0 and math.isnan(float(out["loss_mean"].item()))
    assert (to_host_bits(g, "bf16") == 0).all()


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_zero_and_one_rows(dtype):
    # an empty batch: L = NaN (0/0), n_valid 0, status 0, through all three
    # entry points; then a batch of one row against the oracle
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    _say(f"[zero rows] {dtype}")
    x = torch.empty((0, 1000), dtype=tdt, device="cuda")
    y = torch.empty(0, dtype=torch.int64, device="cuda")
    fused = ce.ce_fwd_bwd_inplace(x, y)
    f = ce.ce_forward(x, y)
    g = ce.ce_backward(x, y, f["lse_rows"], f["pcomp_rows"], f["n_valid"])
    torch.cuda.synchronize()
    for o in (fused, f):
        assert int(o["n_valid"].item()) == 0 and int(o["status"].item()) == 0
        assert math.isnan(float(o["loss_mean"].item()))
    assert g.shape == (0, 1000)
    w = wl.custom(f"one-{dtype}", 81, 1, 1000, dtype, 2.0, 0.0)
    bits, p = wl.make(w)
    out, gg = run_fused(bits, p.labels, dtype)
    check_against_oracle(out, gg, bits, p.labels, dtype)


@pytest.mark.parametrize("dloss", [0.0, -1.0, 0.5, 65536.0])
def test_dloss_values(dloss):
    w = wl.custom("dloss", 23, 40, 1000, "bf16", 2.0, 0.1)
    bits, p = wl.make(w)
    out, g = run_fused(bits, p.labels, "bf16", dloss=dloss)
    check_against_oracle(out, g, bits, p.labels, "bf16", dloss=dloss)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_bad_label(dtype):
    w = wl.custom("badlabel", 29, 16, 300, dtype, 2.0, 0.1)
    bits, p = wl.make(w)
    labels = p.labels.copy()
    labels[3] = 300
    labels[7] = -5
    out, g = run_fused(bits, labels, dtype)
    check_against_oracle(out, g, bits, labels, dtype, expect_status=ce.CE_STATUS_LABEL_RANGE)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_ignore_index_inside_range(dtype):
    w = wl.custom("ign3", 31, 40, 50, dtype, 2.0, 0.0)
    bits, p = wl.make(w)
    labels = p.labels.copy()
    labels[::4] = 3
    out, g = run_fused(bits, labels, dtype, ignore=3)
    check_against_oracle(out, g, bits, labels, dtype, ignore=3)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_confident_rows(dtype):
    rng = np.random.default_rng(4)
    V = 3000
    x = rng.normal(0, 1, (12, V))
    y = rng.integers(0, V, 12).astype(np.int64)
    for i, A in enumerate((6.0, 12.0, 20.0, 30.0, 40.0, 60.0)):
        x[i, y[i]] = A                     # label dominates: p_y -> 1
        x[i + 6, (y[i + 6] + 1) % V] = A   # another column dominates: p_y -> 0
    bits = wl.to_storage(x, dtype)
    out, g = run_fused(bits, y, dtype)
    check_against_oracle(out, g, bits, y, dtype)


@pytest.mark.parametrize("dtype,sigma,n", [("bf16", 40.0, 5), ("bf16", 60.0, 3), ("f16", 30.0, 16),
                                           ("f32", 40.0, 5)])
def test_wide_rows_subnormal_outputs(dtype, sigma, n):
    # few rows (large dloss / n) and wide logit spread: outputs reach the
    # format's subnormal range, where a flushed exponential would show
    w = wl.custom("wide", 41, n, 2000, dtype, sigma, 0.0)
    bits, p = wl.make(w)
    out, g = run_fused(bits, p.labels, dtype, dloss=1.0)
    check_against_oracle(out, g, bits, p.labels, dtype)


# every pass-2 arithmetic (folded scale, scaled power of two for outputs in
# the subnormal range, plain product) through every kernel family: whole rows,
# the persistent kernel for wide aligned rows, slabs, and the split backward
MODES = [("bf16", 2000, 40.0, 5, 1.0), ("bf16", 2000, 40.0, 5, -3.0), ("bf16", 2000, 2.0, 5, -3.0),
         ("bf16", 128000, 40.0, 3, 1.0), ("bf16", 128000, 40.0, 3, -3.0), ("bf16", 140000, 40.0, 3, -3.0),
         ("f16", 3000, 30.0, 8, -1e32), ("f16", 3000, 30.0, 8, 1e32), ("f16", 130000, 30.0, 3, -1e32)]


@pytest.mark.parametrize("dtype,V,sigma,n,dloss", MODES, ids=[f"{d}-V{v}-s{s:g}-dl{dl:g}" for d, v, s, n, dl in MODES])
def test_gradient_modes(dtype, V, sigma, n, dloss):
    w = wl.custom("modes", 43, n, V, dtype, sigma, 0.0)
    bits, p = wl.make(w)
    out, g = run_fused(bits, p.labels, dtype, dloss=dloss)
    check_against_oracle(out, g, bits, p.labels, dtype, dloss=dloss)
    x = to_device(bits, dtype)
    y = torch.from_numpy(p.labels).cuda()
    dl = torch.tensor([dloss], dtype=torch.float32, device="cuda")
    f = ce.ce_forward(x, y)
    grad = ce.ce_backward(x, y, f["lse_rows"], f["pcomp_rows"], f["n_valid"], dl)
    torch.cuda.synchronize()
    check_against_oracle(f, grad, bits, p.labels, dtype, dloss=dloss)


@pytest.mark.parametrize("chunk", [0, 65536])
def test_wide_rows_repeated_calls(chunk):
    # the persistent buffer-store kernel (rows of 128256 bf16 elements, whole
    # or as two 65536-wide chunks): every call must reproduce the oracle and
    # the first call bit for bit (its store data registers are rewritten
    # right after each store)
    w = wl.WORKLOADS[4]
    p = wl.plan(w)
    rows = np.arange(96)
    bits = wl.logits(w, rows, p)
    labels = p.labels[rows]
    first = None
    for i in range(6):
        out, g = run_fused(bits, labels, w.dtype, dloss=w.dloss, chunk=chunk)
        gb = to_host_bits(g, w.dtype)
        if first is None:
            check_against_oracle(out, g, bits, labels, w.dtype, dloss=w.dloss)
            first = gb
        else:
            assert (gb == first).all(), f"call {i} differs from call 0"


def test_deterministic():
    # ten calls on the same input: every output bit for bit the same
    w = wl.custom("det", 43, 300, 32000, "bf16", 2.0, 0.05)
    bits, p = wl.make(w)
    a, ga = run_fused(bits, p.labels, "bf16")
    g0 = to_host_bits(ga, "bf16")
    for _ in range(9):
        b, gb = run_fused(bits, p.labels, "bf16")
        assert (to_host_bits(gb, "bf16") == g0).all()
        for k in ("loss_mean", "loss_rows", "lse_rows", "pcomp_rows", "n_valid"):
            assert torch.equal(a[k], b[k]), k


NEG_INF_BITS = {"bf16": 0xFF80, "f16": 0xFC00, "f32": 0xFF800000}
MASKED = [("bf16", 1000, 0), ("bf16", 32000, 0), ("f16", 49152, 0), ("f32", 1000, 0), ("f32", 32000, 0),
          ("bf16", 128256, 0), ("bf16", 128256, 65536), ("f16", 128256, 65536), ("bf16", 150001, 65536),
          ("f32", 70001, 0)]


@pytest.mark.parametrize("dtype,V,chunk", MASKED, ids=[f"{d}-V{v}-c{c}" for d, v, c in MASKED])
def test_masked_vocabulary(dtype, V, chunk):
    # -inf logits (a masked vocabulary, and whole masked ranges of a row):
    # they take no probability and get a +0 gradient; labels stay unmasked
    N = 24 if V <= 32000 else 8
    w = wl.custom(f"masked-{dtype}-{V}", 71, N, V, dtype, 2.0, 0.1)
    bits, p = wl.make(w)
    rng = np.random.default_rng(72)
    mask = rng.random(bits.shape) < 0.3
    mask[1, : V // 2] = True           # the first half of a row masked
    mask[2, V // 2:] = True            # the second half of another
    mask[3, : min(V, 65536)] = True    # a whole first vocabulary chunk
    rows = np.arange(N)
    valid = p.labels != -100
    mask[rows[valid], p.labels[valid]] = False
    bits = bits.copy()
    bits.view(np.uint32 if dtype == "f32" else np.uint16)[mask] = NEG_INF_BITS[dtype]
    out, g = run_fused(bits, p.labels, dtype, chunk=chunk)
    check_against_oracle(out, g, bits, p.labels, dtype)
    gb = to_host_bits(g, dtype)
    assert (gb[mask & valid[:, None]] == 0).all(), "masked logits must get a +0 gradient"


def test_concurrent_host_threads():
    # two host threads, each with its own stream and (through the binding)
    # its own workspace, call the fused entry point at the same time: one on
    # the persistent wide-row kernel, one on the row-per-workgroup kernel;
    # every call must reproduce the single-threaded result bit for bit
    import threading

    cases = []
    for seed, V in ((61, 128256), (62, 32000)):
        w = wl.custom("threads", seed, 48, V, "bf16", 2.0, 0.05)
        bits, p = wl.make(w)
        out, g = run_fused(bits, p.labels, "bf16")
        check_against_oracle(out, g, bits, p.labels, "bf16")
        cases.append((bits, p.labels, to_host_bits(g, "bf16"), float(out["loss_mean"].item())))
    errors = []

    def worker(i):
        try:
            bits, labels, g_ref, L_ref = cases[i]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                y = torch.from_numpy(np.ascontiguousarray(labels)).cuda()
                for it in range(12):
                    x = to_device(bits, "bf16")
                    out = ce.ce_fwd_bwd_inplace(x, y)
                    s.synchronize()
                    if float(out["loss_mean"].item()) != L_ref or not (to_host_bits(x, "bf16") == g_ref).all():
                        errors.append(f"thread {i}, call {it}: result differs from the single-threaded call")
                        return
        except Exception as e:  # reported below, in the main thread
            errors.append(f"thread {i}: {e!r}")

    _say("[threads] bf16 48x128256 and 48x32000 on two host threads")
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors


@pytest.mark.parametrize("dtype,V,chunk", [("bf16", 32000, 0), ("f16", 5000, 0), ("f32", 1000, 0),
                                           ("bf16", 70000, 32768), ("f32", 3000, 1000), ("bf16", 150001, 65536),
                                           ("f32", 70001, 0)])
def test_split_forward_backward(dtype, V, chunk):
    w = wl.custom("split", 47, 20 if V <= 70000 else 6, V, dtype, 2.0, 0.1)
    bits, p = wl.make(w)
    _say(f"[split] dtype={dtype} V={V} chunk={chunk}")
    x = to_device(bits, dtype)
    y = torch.from_numpy(p.labels).cuda()
    dl = torch.tensor([0.75], dtype=torch.float32, device="cuda")
    f = ce.ce_forward(x, y, chunk=chunk)
    grad = ce.ce_backward(x, y, f["lse_rows"], f["pcomp_rows"], f["n_valid"], dl)
    torch.cuda.synchronize()
    assert (to_host_bits(x, dtype) == bits).all(), "ce_forward must not modify the logits"
    check_against_oracle(f, grad, bits, p.labels, dtype, dloss=0.75)
    # in place through the same entry point
    ce.ce_backward(x, y, f["lse_rows"], f["pcomp_rows"], f["n_valid"], dl, grad=x)
    torch.cuda.synchronize()
    assert (to_host_bits(x, dtype) == to_host_bits(grad, dtype)).all()


def test_autograd_module():
    w = wl.custom("autograd", 53, 2 * 33, 1000, "bf16", 2.0, 0.1)
    bits, p = wl.make(w)
    _say("[autograd] bf16 66x1000")
    x = to_device(bits, "bf16").clone().requires_grad_(True)
    y = torch.from_numpy(p.labels).cuda()
    loss_fn = ce.FastCrossEntropyLoss()
    L = loss_fn(x.view(2, 33, 1000), y.view(2, 33))
    (L * 3.0).backward()
    ref = oracle.cross_entropy(bits, p.labels, "bf16", dloss=3.0)
    assert abs(float(L) - ref["loss_mean"]) <= REL["bf16"] * ref["loss_mean"]
    assert_grad_close(to_host_bits(x.grad, "bf16"), ref["grad"], "bf16", "autograd grad")


def test_autograd_inplace_backward():
    # the module's backward written over the logits' storage: the same
    # gradient as the out-of-place backward, and no second buffer
    w = wl.custom("autograd-inplace", 57, 2 * 40, 5000, "bf16", 2.0, 0.1)
    bits, p = wl.make(w)
    _say("[autograd in place] bf16 80x5000")
    y = torch.from_numpy(p.labels).cuda()
    x0 = to_device(bits, "bf16").clone().requires_grad_(True)
    ce.FastCrossEntropyLoss()(x0.view(2, 40, 5000), y.view(2, 40)).mul(2.0).backward()
    logits = to_device(bits, "bf16").clone()
    h = torch.nn.Parameter(torch.zeros(1, device="cuda"))  # a non-leaf logits tensor: logits + 0 * h
    z = logits + (h * 0).to(torch.bfloat16)
    z.retain_grad()
    L = ce.FastCrossEntropyLoss(inplace_backward=True)(z.view(2, 40, 5000), y.view(2, 40))
    (L * 2.0).backward()
    torch.cuda.synchronize()
    # the logits' own storage now holds the gradient (z.grad itself is a copy
    # autograd keeps for retain_grad)
    assert torch.equal(z.detach(), x0.grad), "the gradient must be written over the logits"
    assert torch.equal(z.grad, x0.grad)
    ref = oracle.cross_entropy(bits, p.labels, "bf16", dloss=2.0)
    assert_grad_close(to_host_bits(z.grad, "bf16"), ref["grad"], "bf16", "in-place autograd grad")


# ---------------------------------------------------------------------------
# Full-size workloads, in the launch configuration the benchmark times: the
# mean and n_valid against the oracle, the loss of every row, and the
# gradient of every row element by element (in row blocks, so the host holds
# one block of the oracle's gradient at a time).
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("k", [2, 3, 4, 5])
def test_full_size(k):
    w = wl.WORKLOADS[k]
    p = wl.plan(w)
    _say(f"[full] generating workload {k} {w.name} N={w.N} V={w.V}")
    bits = wl.logits(w, None, p, threads=16)
    out, g = run_fused(bits, p.labels, w.dtype, dloss=w.dloss, chunk=w.chunk)
    n_full = int((p.labels != -100).sum())
    assert int(out["n_valid"].item()) == n_full and int(out["status"].item()) == 0
    _say("[full] oracle forward over every row")
    fwd = oracle.rows(bits, p.labels, w.dtype, w.dloss / n_full, want_grad=False, threads=16)
    L_ref = oracle.mean(fwd["loss"], p.labels)
    assert_rel(float(out["loss_mean"].item()), L_ref, w.dtype, "loss_mean")
    valid = p.labels != -100
    assert_rel(out["loss_rows"].cpu().numpy()[valid], fwd["loss"][valid], w.dtype, "loss_rows")
    _say("[full] every row's gradient against the oracle")
    B = 1024
    for r0 in range(0, w.N, B):
        r1 = min(w.N, r0 + B)
        ref = oracle.rows(bits[r0:r1], p.labels[r0:r1], w.dtype, w.dloss / n_full, threads=16)
        got = to_host_bits(g[r0:r1], w.dtype)
        assert_grad_close(got, ref["grad"], w.dtype, f"rows {r0}..{r1 - 1}")
        ign = ~valid[r0:r1]
        assert (got[ign] == 0).all(), "ignored rows must be +0"


# ---------------------------------------------------------------------------
# The backward into a gradient buffer laid out differently from the logits
# (another 16-byte phase, another row stride), through the C ABI and through
# the autograd module on strided and offset views.
# ---------------------------------------------------------------------------

PHASES = [("bf16", 1000, 1000, 0, 1003, 3), ("bf16", 32001, 32003, 1, 32001, 0), ("bf16", 4100, 4100, 0, 4100, 5),
          ("f16", 5003, 5010, 2, 5003, 7), ("f32", 1001, 1001, 1, 1003, 0), ("f32", 4000, 4000, 0, 4002, 3),
          ("bf16", 70001, 70001, 1, 70001, 6)]


@pytest.mark.parametrize("dtype,V,ld,off,gld,goff", PHASES,
                         ids=[f"{d}-V{v}-ld{a}+{b}-gld{c}+{e}" for d, v, a, b, c, e in PHASES])
def test_backward_other_layout(dtype, V, ld, off, gld, goff):
    w = wl.custom(f"phase-{dtype}-{V}", 91, 13, V, dtype, 30.0 if dtype == "f16" else 2.0, 0.1)
    bits, p = wl.make(w)
    _say(f"[backward layout] {dtype} V={V} logits ld={ld}+{off} grad ld={gld}+{goff}")
    x = to_device(bits, dtype, ld, off)
    y = torch.from_numpy(p.labels).cuda()
    dl = torch.tensor([1.5], dtype=torch.float32, device="cuda")
    f = ce.ce_forward(x, y)
    grad = to_device(np.zeros_like(bits), dtype, gld, goff)
    ce.ce_backward(x, y, f["lse_rows"], f["pcomp_rows"], f["n_valid"], dl, grad=grad)
    torch.cuda.synchronize()
    assert (to_host_bits(x, dtype) == bits).all(), "the logits must not change"
    check_against_oracle(f, grad, bits, p.labels, dtype, dloss=1.5)
    # nothing outside the gradient rows was written
    st = grad.untyped_storage()
    wd = torch.int32 if dtype == "f32" else torch.int16
    es = 4 if dtype == "f32" else 2
    buf = torch.empty(0, dtype=wd, device=grad.device).set_(st, 0, (st.nbytes() // es,), (1,))
    N = bits.shape[0]
    rows = buf[goff: goff + N * gld].view(N, gld)
    assert (rows[:, V:] == 0).all() and (buf[:goff] == 0).all() and (buf[goff + N * gld:] == 0).all()


@pytest.mark.parametrize("dtype,ld,off", [("bf16", 1001, 0), ("bf16", 1000, 3), ("f32", 1003, 0), ("f32", 1000, 1),
                                          ("f16", 1005, 1)])
def test_autograd_views(dtype, ld, off):
    # the drop-in module on a padded view (row stride above the vocabulary)
    # and on a view whose base is not 16-byte aligned: forward and backward
    # against the oracle (the backward allocates a contiguous gradient)
    V = 1000
    w = wl.custom(f"autograd-view-{dtype}", 93, 2 * 21, V, dtype, 2.0, 0.1)
    bits, p = wl.make(w)
    _say(f"[autograd view] {dtype} ld={ld} offset={off}")
    x = to_device(bits, dtype, ld, off).requires_grad_(True)
    y = torch.from_numpy(p.labels).cuda()
    L = ce.FastCrossEntropyLoss()(x, y)
    (L * 2.0).backward()
    ref = oracle.cross_entropy(bits, p.labels, dtype, dloss=2.0)
    assert abs(float(L) - ref["loss_mean"]) <= REL[dtype] * abs(ref["loss_mean"]) + (
        2.0 ** -8 * abs(ref["loss_mean"]) if dtype != "f32" else 0.0)  # L is returned in the logits' format
    assert_grad_close(to_host_bits(x.grad, dtype), ref["grad"], dtype, "autograd grad on a view")


# ---------------------------------------------------------------------------
# The bounded wait of the single-launch kernels: forced to expire from the
# host (extra partial-count words that nobody publishes, a short spin limit),
# every workgroup still exits; the call reports CE_STATUS_SYNC_TIMEOUT with a
# NaN mean and NaN gradients, and after ce_workspace_init the next call
# matches the oracle.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,V", [("bf16", 1000), ("f32", 1000), ("bf16", 128256)])
def test_sync_timeout_contract(dtype, V):
    lib = ce._lib.load()
    w = wl.custom(f"timeout-{dtype}-{V}", 95, 40 if V <= 32000 else 8, V, dtype, 2.0, 0.1)
    bits, p = wl.make(w)
    y = torch.from_numpy(p.labels).cuda()
    ws = ce.Workspace("cuda")
    _say(f"[timeout] {dtype} V={V}: forced expiry")
    assert lib.ce_debug_sync_override(64, 1) == 0
    try:
        x = to_device(bits, dtype)
        out = ce.ce_fwd_bwd_inplace(x, y, workspace=ws)
        torch.cuda.synchronize()
    finally:
        assert lib.ce_debug_sync_override(0, 0) == 0
    assert int(out["status"].item()) & ce.CE_STATUS_SYNC_TIMEOUT
    assert math.isnan(float(out["loss_mean"].item()))
    g = x.float()
    valid = torch.from_numpy(p.labels != -100).cuda()
    assert torch.isnan(g[valid]).all(), "an expired wait must leave NaN gradients"
    assert (g[~valid] == 0).all()
    with pytest.raises(RuntimeError):
        ce.check_status(out)
    _say(f"[timeout] {dtype} V={V}: recovery")
    ce.ce_workspace_init(ws.buf)
    for _ in range(2):
        x = to_device(bits, dtype)
        out = ce.ce_fwd_bwd_inplace(x, y, workspace=ws)
        torch.cuda.synchronize()
        check_against_oracle(out, x, bits, p.labels, dtype)
