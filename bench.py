"""Benchmark: fused softmax cross-entropy forward + in-place backward on MI355X.

One step = one ce_fwd_bwd_inplace call over the whole batch (every step of the
path: label count, row max / log-sum-exp, loss, token mean, gradient written
over the logits).  Default workload: 4096 rows (batch 4 x sequence 1024) of a
32000-token vocabulary in bf16 (the Mistral-7B shape of the pages' "Improvements
to Full Finetuning" table), synthetic seeded logits resident in HBM.

Protocol per timed step (the restore and the flush are not timed):
  restore the logits from a pristine device copy (the call overwrites them);
  write a 1 GiB scratch buffer so neither the 4 MB L2s nor the 256 MB MALL
  hold any of the input;  then HIP events on the call's stream bracket the call.
The call is one kernel (rows fit on chip), so the same events time the
dominant kernel for the roofline figure.

    python bench.py [--steps K] [--warmup W] [--workload 2]

Profiling (rocprofv3 databases -> profiles/ summaries):
    rocprofv3 --kernel-trace --stats -d D -o trace -- python bench.py --steps 10 --no-cpu-baseline
    rocprofv3 --pmc FETCH_SIZE -d D -o fetch -- python bench.py --steps 5 --no-cpu-baseline --calibrate
    rocprofv3 --pmc WRITE_SIZE -d D -o write -- python bench.py --steps 5 --no-cpu-baseline --calibrate
    python bench.py --profile-summary D
Every run also times plain copies of the logits' size under the same protocol,
in several shapes (cross_entropy_loss_amd/csrc/calib_copy.hip), and reports the
fastest as roofline.copy_ceiling (the attainable read + write rate, with the
shape in copy_shape); the split forward also gets the fastest plain read
(read_ceiling).  Under the --calibrate runs only the first copy shape runs,
and the counters' reading of it gives the factor that turns FETCH_SIZE /
WRITE_SIZE into bytes.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD published peak
HEADLINE_METRIC = "CE fwd+bwd tokens/s and HBM GB/s (% of peak), N=4096 V=32000 bf16"
KERNEL_SOURCES = ["cross_entropy_loss_amd/csrc/ce_kernels.h", "cross_entropy_loss_amd/csrc/ce_buffer.h",
                  "cross_entropy_loss_amd/csrc/ce_api.hip"]


NORM_SOURCES = ["cross_entropy_loss_amd/csrc/rmsnorm.hip", "cross_entropy_loss_amd/csrc/ce_buffer.h",
                "cross_entropy_loss_amd/csrc/row_formats.h"]


def kernel_sha(sources=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for p in sources:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w, labels) -> int:
    """Minimum HBM traffic of one fused call: each valid row read once and
    written once, each ignored row written once (not read), plus per row the
    label (8 B) and the loss (4 B), lse (8 B) and 1 - p_label (8 B) outputs."""
    n_valid = int((labels != -100).sum())
    n_ign = w.N - n_valid
    return (2 * n_valid + n_ign) * w.V * w.elem_bytes + w.N * (8 + 4 + 8 + 8)


def measured_traffic(name: str, sources=KERNEL_SOURCES):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", f"{name}.counters.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        c = json.load(f)
    if c.get("kernel_sha") != kernel_sha(sources):
        return None
    return c.get("traffic_bytes")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, bits, labels, max_seconds=20.0, min_seconds=5.0):
    """The float64 oracle (forward + backward of every sampled row) on the host
    cores: a bounded sample of the workload's rows, repeated until at least
    min_seconds of work so the rate is stable; then the same on one thread
    (a smaller sample, about 2 s)."""
    import oracle
    threads = min(16, os.cpu_count() or 1)
    n = int((labels != -100).sum())

    def rate(nthreads, budget_max, budget_min):
        t0 = time.perf_counter()
        oracle.rows(bits[:16], labels[:16], w.dtype, w.dloss / n, threads=nthreads)
        per_row = (time.perf_counter() - t0) / 16
        rows = int(min(w.N, max(16, budget_max / 2 / max(per_row, 1e-9))))
        done, t0 = 0, time.perf_counter()
        while True:
            oracle.rows(bits[:rows], labels[:rows], w.dtype, w.dloss / n, threads=nthreads)
            done += rows
            dt = time.perf_counter() - t0
            if dt >= budget_min or dt >= budget_max:
                return done / dt, rows, done // rows, dt

    v, rows, passes, dt = rate(threads, max_seconds, min_seconds)
    v1, rows1, _, dt1 = rate(1, 4.0, 2.0)
    row_bytes = 2 * w.V * w.elem_bytes
    return {"value": v, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {rows} of {w.N} rows of {w.name}, {passes} passes: float64 forward + "
                      f"backward, {threads} threads, {dt:.2f} s; one thread: first {rows1} rows, {dt1:.2f} s",
            "value_1thread": v1, "gbs": v * row_bytes / 1e9, "cpu": cpu_model(), "nproc": os.cpu_count()}


def _db_rows(path, sql):
    import sqlite3
    con = sqlite3.connect(path)
    try:
        return con.execute(sql).fetchall()
    finally:
        con.close()


def profile_summary_linear(d: str, workload: int) -> None:
    """Kernel-trace summary of the LM-head path (bench.py --op linear) ->
    profiles/ce_linear_<workload>.txt: per kernel the time per call, and for
    the three matrix-product kernels (logits with the tile statistics, dh,
    dW) their rate over 2 N H V flops each.  The two backward launches of a
    call are told apart by their order (dh, then dW)."""
    import glob
    import workloads as wl
    workload = workload if workload in wl.LINEAR_WORKLOADS else 1
    lw = wl.LINEAR_WORKLOADS[workload]
    trace = (glob.glob(os.path.join(d, "**", "trace_results.db"), recursive=True) or [None])[0]
    if not trace:
        raise SystemExit(f"no trace_results.db under {d}")
    rows = _db_rows(trace, "select name, duration from kernels order by start")
    calls = sum(1 for n, _ in rows if "lin_prep_kernel" in n)
    per = {}
    bwd_seen = 0
    for name, dur in rows:
        if name.startswith(("void at::native", "__amd_rocclr", "cek::ws_fill")):
            continue  # the benchmark's own flush / copies, the workspace fill
        if "lin_prep_kernel" in name:
            bwd_seen = 0
            label = "lin_prep_kernel (labels, counts)"
        elif "lin_logits_kernel" in name:
            label = "lin_logits_kernel (logits = h W^T, tile statistics and exponentials)"
        elif "lin_rescale_kernel" in name:
            label = "lin_rescale_kernel (row log-sum-exp, loss, g over the exponentials)"
        elif "lin_bwd_kernel" in name:
            label = ("lin_bwd_kernel dh = g W" if bwd_seen == 0 else "lin_bwd_kernel dW = g^T h")
            bwd_seen += 1
        elif "lin_finish_kernel" in name:
            label = "lin_finish_kernel (token mean, status)"
        else:
            label = name[:72]
        n, s_ = per.get(label, (0, 0))
        per[label] = (n + 1, s_ + dur)
    flops_per_gemm = 2.0 * lw.N * lw.H * lw.V
    lines = [f"# rocprofv3 summary: LM-head projection + cross-entropy (ce_linear_fwd_bwd), workload {lw.name}",
             f"# N={lw.N} H={lw.H} V={lw.V} dtype={lw.dtype} chunk_rows={lw.chunk_rows or 'default'}",
             "# commands (from the repository root):",
             "#   rocprofv3 --kernel-trace --stats -d D -o trace -- "
             f"python bench.py --op linear --workload {workload} --steps 5 --warmup 2 --no-cpu-baseline",
             f"#   python bench.py --op linear --profile-summary D --workload {workload}", "",
             f"{calls} calls traced (the first ones warm-up); per call:",
             f"  {'kernel':76s} {'launches':>8s} {'ms/call':>9s} {'TFLOP/s':>8s}"]
    total = 0.0
    for label, (n, s_) in sorted(per.items(), key=lambda kv: -kv[1][1]):
        per_call = s_ / calls / 1e6
        total += per_call
        rate = ""
        if label.startswith(("lin_logits_kernel", "lin_bwd_kernel")):
            rate = f"{flops_per_gemm / (per_call * 1e-3) / 1e12:8.0f}"
        lines.append(f"  {label:76s} {n // calls:8d} {per_call:9.3f} {rate:>8s}")
    lines.append(f"  {'total':76s} {'':8s} {total:9.3f} {3 * flops_per_gemm / (total * 1e-3) / 1e12:8.0f}")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"ce_linear_{lw.name}.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def profile_summary(d: str, workload: int) -> None:
    """Reads rocprofv3 databases (trace_results.db, fetch_results.db,
    write_results.db under d) and writes profiles/<kernel>_<workload>.txt and
    the counters JSON that bench.py reads for roofline.traffic."""
    import glob
    import workloads as wl
    w = wl.WORKLOADS[workload]
    labels = wl.plan(w).labels
    find = lambda stem: (glob.glob(os.path.join(d, "**", f"{stem}_results.db"), recursive=True) or [None])[0]
    trace, fetch, write = find("trace"), find("fetch"), find("write")
    lines = [f"# rocprofv3 summary: fused cross-entropy forward+backward, workload {w.name}",
             f"# N={w.N} V={w.V} dtype={w.dtype} chunk={w.chunk}; kernel sources sha {kernel_sha()}",
             "# commands (from the repository root):",
             "#   rocprofv3 --kernel-trace --stats -d D -o trace -- "
             f"python bench.py --workload {workload} --steps 10 --no-cpu-baseline",
             "#   rocprofv3 --pmc FETCH_SIZE -d D -o fetch -- "
             f"python bench.py --workload {workload} --steps 5 --no-cpu-baseline --calibrate",
             "#   rocprofv3 --pmc WRITE_SIZE -d D -o write -- "
             f"python bench.py --workload {workload} --steps 5 --no-cpu-baseline --calibrate",
             f"#   python bench.py --profile-summary D --workload {workload}", ""]
    ce_names = ("row_kernel", "row_fused", "slab_", "grad_kernel")
    dominant = None
    if trace:
        rows = _db_rows(trace, "select name, count(*), avg(duration), min(duration), max(duration) from kernels "
                               "group by name order by sum(duration) desc")
        lines.append("kernel-trace (durations in us; the first calls of a run are cold):")
        lines.append(f"  {'kernel':70s} {'calls':>5s} {'avg':>9s} {'median':>9s} {'min':>9s} {'max':>9s}")
        for name, n, avg, mn, mx in rows:
            durs = sorted(r[0] for r in _db_rows(trace, "select duration from kernels where name = '%s'"
                                                       % name.replace("'", "''")))
            med = durs[len(durs) // 2]
            lines.append(f"  {name[:70]:70s} {n:5d} {avg / 1e3:9.2f} {med / 1e3:9.2f} {mn / 1e3:9.2f} {mx / 1e3:9.2f}")
            if dominant is None and any(c in name for c in ce_names):
                dominant = (name, med / 1e3)
        lines.append("")
    abytes = algorithmic_bytes(w, labels)
    logits_bytes = w.N * w.V * w.elem_bytes
    rec = {"kernel_sha": kernel_sha(), "workload": w.name, "algorithmic_bytes": abytes}
    for tag, db, counter in (("read", fetch, "FETCH_SIZE"), ("write", write, "WRITE_SIZE")):
        if not db:
            continue
        rows = _db_rows(db, f"select kernel_name, avg(value), count(*) from counters_collection "
                            f"where counter_name = '{counter}' group by kernel_name")
        calib = [r for r in rows if "calib_copy" in r[0]]
        ce = [r for r in rows if any(c in r[0] for c in ce_names)]
        lines.append(f"{counter} (KiB per dispatch, as reported):")
        for name, val, n in rows:
            lines.append(f"  {name[:70]:70s} {val:14.1f}  ({n} dispatches)")
        if calib and ce:
            factor = (logits_bytes / 1024.0) / calib[0][1]
            kib = sum(r[1] for r in ce)
            rec[f"{tag}_kib_raw"] = kib
            rec[f"{tag}_factor"] = factor
            rec[f"{tag}_bytes"] = kib * 1024.0 * factor
            lines.append(f"  calibration: copy of {logits_bytes} B reads as {calib[0][1]:.1f} KiB -> factor {factor:.4f}")
            lines.append(f"  cross-entropy kernels: {kib:.1f} KiB x {factor:.4f} = {kib * 1024 * factor / 1e6:.2f} MB")
        lines.append("")
    if "read_bytes" in rec and "write_bytes" in rec:
        rec["traffic_bytes"] = rec["read_bytes"] + rec["write_bytes"]
        lines.append(f"HBM traffic per call: {rec['traffic_bytes'] / 1e6:.2f} MB "
                     f"(algorithmic minimum {abytes / 1e6:.2f} MB, ratio {rec['traffic_bytes'] / abytes:.3f})")
    if dominant:
        rec["dominant_kernel"], rec["avg_us"] = dominant
        lines.append(f"dominant kernel: {dominant[0]}  median {dominant[1]:.2f} us  "
                     f"-> {abytes / (dominant[1] * 1e-6) / 1e9:.0f} GB/s algorithmic "
                     f"({abytes / (dominant[1] * 1e-6) / 1e9 / HBM_PEAK_GBS * 100:.1f}% of {HBM_PEAK_GBS:.0f} GB/s)")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"ce_fused_{w.name}.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(os.path.join(ROOT, "profiles", f"ce_fused_{w.name}.counters.json"), "w") as f:
        json.dump(rec, f, indent=1)
    print("\n".join(lines))


MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}  # MI355X dense, AMD published


def bench_linear(args) -> None:
    """LM-head projection + cross-entropy, forward and backward (ce_linear_fwd_bwd):
    one step = one call over the whole batch with the hidden states and weight
    resident in HBM; L2 and MALL flushed before each step.  Roofline: the call
    is dominated by its three GEMMs (6 N H V flops), priced against the MFMA
    peak of the input format."""
    import torch
    import cross_entropy_loss_amd as ce
    import workloads as wl
    lw = wl.LINEAR_WORKLOADS[args.workload if args.workload in wl.LINEAR_WORKLOADS else 1]
    if args.chunk_rows is not None:
        import dataclasses
        lw = dataclasses.replace(lw, chunk_rows=args.chunk_rows)
    h, w, y = wl.linear_inputs(lw)
    dev = torch.device("cuda:0")
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[lw.dtype]

    def to_dev(a):
        return torch.from_numpy(a.view(np.int16) if lw.elem_bytes == 2 else a.view(np.int32)).to(dev).view(tdt)

    hd, wd = to_dev(h), to_dev(w)
    yd = torch.from_numpy(y).to(dev)
    dl = torch.tensor([lw.dloss], dtype=torch.float32, device=dev)
    ws = ce.Workspace(dev, ce.ce_linear_workspace_bytes(lw.N, lw.H, lw.V, lw.chunk_rows, tdt))
    flush = torch.empty(1 << 28, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    out = None
    for i in range(args.warmup):
        flush.fill_(i)
        out = ce.ce_linear_fwd_bwd(hd, wd, yd, chunk_rows=lw.chunk_rows, dloss=dl, workspace=ws)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        flush.fill_(args.warmup + i)
        ev[i][0].record(stream)
        out = ce.ce_linear_fwd_bwd(hd, wd, yd, chunk_rows=lw.chunk_rows, dloss=dl, workspace=ws)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st = int(out["status"].item())
    if st != 0:
        raise SystemExit(f"kernel status {st:#x}")
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    ms_mean = float(ms.mean())
    flops = 6.0 * lw.N * lw.H * lw.V
    tf = flops / (ms_mean * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS[lw.dtype]
    rec = {
        "metric": f"LM-head + CE fwd+bwd tokens/s, N={lw.N} H={lw.H} V={lw.V} {lw.dtype}",
        "value": lw.N / (ms_mean * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_mean, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": lw.dtype, "data": "synthetic",
        "config": {"workload": lw.name, "rows": lw.N, "hidden": lw.H, "vocab": lw.V, "chunk_rows": lw.chunk_rows,
                   "n_valid": int((y != -100).sum()), "parallelism": "none"},
        "roofline": {"bound": "mfma", "achieved": tf, "peak": peak, "unit": "TFLOP/s", "frac": tf / peak,
                     "traffic": None},
        "timing": {"ms_p10": float(np.percentile(ms, 10)), "ms_median": float(np.median(ms)),
                   "ms_p90": float(np.percentile(ms, 90)), "flops": flops,
                   "wall_ms_per_step_incl_flush": wall / args.steps * 1e3},
    }
    if not args.no_cpu_baseline:
        from oracle import linear as olin
        rows, done, t0 = 16, 0, time.perf_counter()
        while time.perf_counter() - t0 < 5.0:
            olin.linear_cross_entropy(h[:rows], w, y[:rows], lw.dtype, dloss=lw.dloss)
            done += rows
        dt = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": done / dt, "unit": "tokens/s", "cores": min(16, os.cpu_count() or 1),
                               "kind": "oracle",
                               "sample": f"first {rows} rows of {lw.name} against the whole weight, float64 "
                                         f"forward + both gradients (numpy BLAS), {done // rows} passes, {dt:.2f} s"}
    print(json.dumps(rec), flush=True)


def norm_bytes(nw) -> dict:
    """Algorithmic HBM bytes of the two RMSNorm calls: the forward reads x and
    the weight and writes y and rstd; the backward reads dy, x, the weight and
    rstd and writes dx and dweight (the workgroups' partial sums of dweight are
    the implementation's, not the algorithm's)."""
    e, N, H = nw.elem_bytes, nw.N, nw.H
    return {"forward": 2 * N * H * e + H * e + 4 * N, "backward": 3 * N * H * e + 2 * H * e + 4 * N}


def _summarize(d: str, stem: str, header: list, parts: dict, calib_bytes: int, sha: str) -> dict:
    """rocprofv3 databases under d (trace_results.db, fetch_results.db,
    write_results.db) -> profiles/<stem>.txt and, with counters, the
    <stem>.counters.json that bench.py reads for roofline.traffic.
    parts: name -> (kernel-name substrings, algorithmic bytes of that call)."""
    import glob
    find = lambda tag: (glob.glob(os.path.join(d, "**", f"{tag}_results.db"), recursive=True) or [None])[0]
    trace, fetch, write = find("trace"), find("fetch"), find("write")
    lines = list(header)
    rec = {"kernel_sha": sha, "algorithmic_bytes": {k: v[1] for k, v in parts.items()}}
    med = {}
    if trace:
        rows = _db_rows(trace, "select name, count(*), avg(duration), min(duration), max(duration) from kernels "
                               "group by name order by sum(duration) desc")
        lines.append("kernel-trace (durations in us; the first calls of a run are cold):")
        lines.append(f"  {'kernel':70s} {'calls':>5s} {'avg':>9s} {'median':>9s} {'min':>9s} {'max':>9s}")
        for name, n, avg, mn, mx in rows:
            durs = sorted(r[0] for r in _db_rows(trace, "select duration from kernels where name = '%s'"
                                                       % name.replace("'", "''")))
            m = durs[len(durs) // 2] / 1e3
            lines.append(f"  {name[:70]:70s} {n:5d} {avg / 1e3:9.2f} {m:9.2f} {mn / 1e3:9.2f} {mx / 1e3:9.2f}")
            for part, (keys, _) in parts.items():
                if any(k in name for k in keys):
                    med[part] = med.get(part, 0.0) + m
        lines.append("")
    for tag, db, counter in (("read", fetch, "FETCH_SIZE"), ("write", write, "WRITE_SIZE")):
        if not db:
            continue
        rows = _db_rows(db, f"select kernel_name, avg(value), count(*) from counters_collection "
                            f"where counter_name = '{counter}' group by kernel_name")
        calib = [r for r in rows if "calib_copy" in r[0]]
        lines.append(f"{counter} (KiB per dispatch, as reported):")
        for name, val, n in rows:
            lines.append(f"  {name[:70]:70s} {val:14.1f}  ({n} dispatches)")
        if calib:
            factor = (calib_bytes / 1024.0) / calib[0][1]
            rec[f"{tag}_factor"] = factor
            for part, (keys, _) in parts.items():
                kib = sum(r[1] for r in rows if any(k in r[0] for k in keys))
                rec[f"{part}_{tag}_bytes"] = kib * 1024.0 * factor
                lines.append(f"  {part}: {kib:.1f} KiB x {factor:.4f} = {kib * 1024 * factor / 1e6:.2f} MB")
            lines.append(f"  calibration: copy of {calib_bytes} B reads as {calib[0][1]:.1f} KiB -> factor {factor:.4f}")
        lines.append("")
    for part, (keys, ab) in parts.items():
        if f"{part}_read_bytes" in rec and f"{part}_write_bytes" in rec:
            t = rec[f"{part}_read_bytes"] + rec[f"{part}_write_bytes"]
            rec[f"{part}_traffic_bytes"] = t
            lines.append(f"HBM traffic, {part} call: {t / 1e6:.2f} MB (algorithmic {ab / 1e6:.2f} MB, "
                         f"ratio {t / ab:.3f})")
    for part, (keys, ab) in parts.items():
        if part in med:
            rec[f"{part}_us"] = med[part]
            lines.append(f"{part} call ({' + '.join(keys)}): {med[part]:.2f} us (kernel medians) -> "
                         f"{ab / (med[part] * 1e-6) / 1e9:.0f} GB/s algorithmic "
                         f"({ab / (med[part] * 1e-6) / 1e9 / HBM_PEAK_GBS * 100:.1f}% of {HBM_PEAK_GBS:.0f} GB/s)")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"{stem}.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    if fetch or write:
        with open(os.path.join(ROOT, "profiles", f"{stem}.counters.json"), "w") as f:
            json.dump(rec, f, indent=1)
    print("\n".join(lines))
    return rec


def _profile_header(title: str, shape: str, sha: str, op: str, workload: int) -> list:
    return [f"# rocprofv3 summary: {title}", f"# {shape}; kernel sources sha {sha}",
            "# commands (from the repository root):",
            "#   rocprofv3 --kernel-trace --stats -d D -o trace -- "
            f"python bench.py --op {op} --workload {workload} --steps 10 --no-cpu-baseline",
            "#   rocprofv3 --pmc FETCH_SIZE -d D -o fetch -- "
            f"python bench.py --op {op} --workload {workload} --steps 5 --no-cpu-baseline --calibrate",
            "#   rocprofv3 --pmc WRITE_SIZE -d D -o write -- "
            f"python bench.py --op {op} --workload {workload} --steps 5 --no-cpu-baseline --calibrate",
            f"#   python bench.py --op {op} --profile-summary D --workload {workload}", ""]


def profile_summary_norm(d: str, workload: int) -> None:
    """Summary of bench.py --op rmsnorm runs -> profiles/rmsnorm_<workload>.*
    (roofline.traffic: the backward call, rms_bwd* + rms_dw_reduce)."""
    import workloads as wl
    workload = workload if workload in wl.NORM_WORKLOADS else 1
    nw = wl.NORM_WORKLOADS[workload]
    ab = norm_bytes(nw)
    sha = kernel_sha(NORM_SOURCES)
    head = _profile_header(f"RMSNorm forward and backward, workload {nw.name}",
                           f"N={nw.N} H={nw.H} dtype={nw.dtype} eps={nw.eps}", sha, "rmsnorm", workload)
    _summarize(d, f"rmsnorm_{nw.name}", head,
               {"forward": (("rms_fwd",), ab["forward"]), "backward": (("rms_bwd", "rms_dw_reduce"), ab["backward"])},
               nw.N * nw.H * nw.elem_bytes, sha)


ROPE_SOURCES = ["cross_entropy_loss_amd/csrc/rope.hip", "cross_entropy_loss_amd/csrc/ce_buffer.h",
                "cross_entropy_loss_amd/csrc/row_formats.h"]


def rope_bytes(rw) -> int:
    """Algorithmic HBM bytes of one ce_rope call over q and k: every element
    read once and written once, plus the positions."""
    return 2 * rw.T * (rw.Hq + rw.Hk) * rw.D * rw.elem_bytes + 8 * rw.T


def profile_summary_rope(d: str, workload: int) -> None:
    """Summary of bench.py --op rope runs -> profiles/rope_<workload>.*"""
    import workloads as wl
    workload = workload if workload in wl.ROPE_WORKLOADS else 1
    rw = wl.ROPE_WORKLOADS[workload]
    sha = kernel_sha(ROPE_SOURCES)
    head = _profile_header(f"rotary embedding (ce_rope, forward and inverse), workload {rw.name}",
                           f"T={rw.T} Hq={rw.Hq} Hk={rw.Hk} D={rw.D} dtype={rw.dtype} base={rw.base}", sha, "rope",
                           workload)
    # both launches of a step run the same kernel: per-launch figures
    _summarize(d, f"rope_{rw.name}", head, {"launch": (("rope16", "rope32"), rope_bytes(rw))},
               rw.T * rw.Hq * rw.D * rw.elem_bytes, sha)


COPY_SHAPES = ["grid-stride 16384 workgroups", "1 vector/thread", "4 vectors/thread", "8 vectors/thread",
               "4 vectors/thread, cached", "persistent 8/CU, 4 vectors/thread"]


def _calib_lib():
    import ctypes
    calib = ctypes.CDLL(os.path.join(ROOT, "cross_entropy_loss_amd", "libce_calib.so"))
    calib.ce_calib_copy_shape.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                          ctypes.c_void_p]
    calib.ce_calib_read_shape.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                          ctypes.c_void_p]
    return calib


def _best_shape(launch, nbytes_moved, flush, stream, reps, shapes):
    """Median time of each shape over `reps` flushed runs (the first dropped);
    returns (best GB/s, shape index, {shape: GB/s})."""
    import torch
    rates = {}
    for sh in shapes:
        cms = []
        for i in range(reps):
            flush.fill_(i)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            rc = launch(sh)
            e1.record(stream)
            if rc:
                raise SystemExit(f"calibration kernel (shape {sh}) failed: {rc}")
            torch.cuda.synchronize()
            cms.append(e0.elapsed_time(e1))
        rates[sh] = nbytes_moved / (float(np.median(cms[1:])) * 1e-3) / 1e9
    best = max(rates, key=rates.get)
    return rates[best], best, rates


def _calib_copy(src, dst, nbytes, flush, stream, calibrate):
    """The attainable read + write rate for nbytes: the fastest copy shape
    (only shape 0, the counters' calibration copy, under --calibrate)."""
    import ctypes
    calib = _calib_lib()
    shapes = [0] if calibrate else list(range(calib.ce_calib_shapes()))
    launch = lambda sh: calib.ce_calib_copy_shape(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                                  nbytes, sh, ctypes.c_void_p(stream.cuda_stream))
    return _best_shape(launch, 2 * nbytes, flush, stream, 3 if calibrate else 5, shapes)


def _calib_read(src, nbytes, flush, stream):
    """The attainable read rate for nbytes: the fastest read shape."""
    import ctypes
    import torch
    calib = _calib_lib()
    sink = torch.zeros(4, dtype=torch.int32, device=src.device)
    launch = lambda sh: calib.ce_calib_read_shape(ctypes.c_void_p(src.data_ptr()), nbytes, sh,
                                                  ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
    return _best_shape(launch, nbytes, flush, stream, 5, list(range(calib.ce_calib_shapes())))


def bench_rmsnorm(args) -> None:
    """RMSNorm forward + backward (ce_rmsnorm_forward, ce_rmsnorm_backward):
    one step = one forward call and one backward call over the whole batch,
    inputs resident in HBM, L2 and MALL flushed before each call.  Roofline:
    the backward call (its two kernels) against HBM peak."""
    import torch
    import cross_entropy_loss_amd as ce
    import workloads as wl
    nw = wl.NORM_WORKLOADS[args.workload if args.workload in wl.NORM_WORKLOADS else 1]
    x, w, dy = wl.norm_inputs(nw)
    dev = torch.device("cuda:0")
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[nw.dtype]

    def to_dev(a):
        return torch.from_numpy(a.view(np.int16) if nw.elem_bytes == 2 else a.view(np.int32)).to(dev).view(tdt)

    xd, wd, dyd = to_dev(x), to_dev(w), to_dev(dy)
    ws = torch.empty(ce.ce_rmsnorm_workspace_bytes(nw.N, nw.H, tdt), dtype=torch.uint8, device=dev)
    flush = torch.empty(1 << 28, dtype=torch.int32, device=dev)  # 1 GiB
    stream = torch.cuda.current_stream(dev)

    def step(i, ev=None):
        flush.fill_(2 * i)
        if ev:
            ev[0].record(stream)
        y, rstd = ce.ce_rmsnorm_forward(xd, wd, nw.eps)
        if ev:
            ev[1].record(stream)
        flush.fill_(2 * i + 1)
        if ev:
            ev[2].record(stream)
        dx, dw = ce.ce_rmsnorm_backward(dyd, xd, wd, rstd, workspace=ws)
        if ev:
            ev[3].record(stream)
        return y, dx, dw

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd = np.array([e[0].elapsed_time(e[1]) for e in evs])
    bwd = np.array([e[2].elapsed_time(e[3]) for e in evs])
    copy_gbs, copy_shape, _ = _calib_copy(xd, torch.empty_like(xd), nw.N * nw.H * nw.elem_bytes, flush, stream,
                                          args.calibrate)
    ab = norm_bytes(nw)
    step_ms = float(fwd.mean() + bwd.mean())
    bw_gbs = ab["backward"] / (float(bwd.mean()) * 1e-3) / 1e9
    fw_gbs = ab["forward"] / (float(fwd.mean()) * 1e-3) / 1e9
    traffic = None
    p = os.path.join(ROOT, "profiles", f"rmsnorm_{nw.name}.counters.json")
    if os.path.exists(p):
        with open(p) as f:
            c = json.load(f)
        if c.get("kernel_sha") == kernel_sha(NORM_SOURCES):
            traffic = c.get("backward_traffic_bytes")
    rec = {
        "metric": f"RMSNorm fwd+bwd tokens/s and HBM GB/s (% of peak), N={nw.N} H={nw.H} {nw.dtype}",
        "value": nw.N / (step_ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": step_ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": nw.dtype, "data": "synthetic",
        "config": {"workload": nw.name, "rows": nw.N, "hidden": nw.H, "eps": nw.eps, "parallelism": "none"},
        "roofline": {"bound": "hbm", "kernel": "backward call: rms_bwd16 + rms_dw_reduce", "achieved": bw_gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": bw_gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "copy_ceiling": copy_gbs, "frac_of_copy": bw_gbs / copy_gbs, "copy_shape": COPY_SHAPES[copy_shape]},
        "timing": {"forward_ms_mean": float(fwd.mean()), "forward_ms_median": float(np.median(fwd)),
                   "forward_gbs": fw_gbs, "backward_ms_mean": float(bwd.mean()),
                   "backward_ms_median": float(np.median(bwd)), "algorithmic_bytes": ab,
                   "wall_ms_per_step_incl_flush": wall / args.steps * 1e3, "kernel_sha": kernel_sha(NORM_SOURCES)},
    }
    if not args.no_cpu_baseline:
        from oracle import rmsnorm as orn
        rows, done, t0 = 256, 0, time.perf_counter()
        while time.perf_counter() - t0 < 8.0:
            orn.rmsnorm(x[:rows], w, nw.dtype, nw.eps, dy[:rows])
            done += rows
        dt = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": done / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                               "sample": f"first {rows} rows of {nw.name}, float64 forward + backward (numpy, "
                                         f"one thread), {done // rows} passes, {dt:.2f} s"}
    print(json.dumps(rec), flush=True)


def bench_rope(args) -> None:
    """Rotary embedding (ce_rope) of one attention layer's q and k at packed
    position ids: one step = the forward call and the inverse (backward) call,
    inputs resident in HBM, L2 and MALL flushed before each call.  Roofline:
    one launch (both are the same kernel) against HBM peak."""
    import torch
    import cross_entropy_loss_amd as ce
    import workloads as wl
    workload = args.workload if args.workload in wl.ROPE_WORKLOADS else 1
    rw = wl.ROPE_WORKLOADS[workload]
    q, k, pos = wl.rope_inputs(rw)
    dev = torch.device("cuda:0")
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[rw.dtype]

    def to_dev(a):
        return torch.from_numpy(a.view(np.int16) if rw.elem_bytes == 2 else a.view(np.int32)).to(dev).view(tdt)

    qd, kd, pd = to_dev(q), to_dev(k), torch.from_numpy(pos).to(dev)
    flush = torch.empty(1 << 28, dtype=torch.int32, device=dev)  # 1 GiB
    stream = torch.cuda.current_stream(dev)

    def step(i, ev=None):
        flush.fill_(2 * i)
        if ev:
            ev[0].record(stream)
        qo, ko = ce.ce_rope(qd, kd, pd, rw.base)
        if ev:
            ev[1].record(stream)
        flush.fill_(2 * i + 1)
        if ev:
            ev[2].record(stream)
        ce.ce_rope(qo, ko, pd, rw.base, inverse=True)
        if ev:
            ev[3].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd = np.array([e[0].elapsed_time(e[1]) for e in evs])
    bwd = np.array([e[2].elapsed_time(e[3]) for e in evs])
    copy_gbs, copy_shape, _ = _calib_copy(qd, torch.empty_like(qd), qd.numel() * qd.element_size(), flush, stream,
                                          args.calibrate)
    ab = rope_bytes(rw)
    step_ms = float(fwd.mean() + bwd.mean())
    per_launch_ms = step_ms / 2
    gbs = ab / (per_launch_ms * 1e-3) / 1e9
    traffic = None
    p = os.path.join(ROOT, "profiles", f"rope_{rw.name}.counters.json")
    if os.path.exists(p):
        with open(p) as f:
            c = json.load(f)
        if c.get("kernel_sha") == kernel_sha(ROPE_SOURCES):
            traffic = c.get("launch_traffic_bytes")
    rec = {
        "metric": f"RoPE fwd+bwd tokens/s and HBM GB/s (% of peak), T={rw.T} q {rw.Hq}x{rw.D} k {rw.Hk}x{rw.D} "
                  f"{rw.dtype}",
        "value": rw.T / (step_ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": step_ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": rw.dtype, "data": "synthetic",
        "config": {"workload": rw.name, "tokens": rw.T, "q_heads": rw.Hq, "k_heads": rw.Hk, "head_dim": rw.D,
                   "base": rw.base, "sequences": int((pos == 0).sum()), "parallelism": "none"},
        "roofline": {"bound": "hbm", "kernel": "rope16 (one launch: q and k)", "achieved": gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS, "traffic": traffic, "copy_ceiling": copy_gbs,
                     "frac_of_copy": gbs / copy_gbs, "copy_shape": COPY_SHAPES[copy_shape]},
        "timing": {"forward_ms_mean": float(fwd.mean()), "forward_ms_median": float(np.median(fwd)),
                   "inverse_ms_mean": float(bwd.mean()), "inverse_ms_median": float(np.median(bwd)),
                   "algorithmic_bytes_per_launch": ab, "wall_ms_per_step_incl_flush": wall / args.steps * 1e3,
                   "kernel_sha": kernel_sha(ROPE_SOURCES)},
    }
    if not args.no_cpu_baseline:
        from oracle import rope as orope
        n, done, t0 = 128, 0, time.perf_counter()
        while time.perf_counter() - t0 < 8.0:
            yq = orope.rope(q[:n], rw.dtype, pos[:n], rw.base)["y"]
            yk = orope.rope(k[:n], rw.dtype, pos[:n], rw.base)["y"]
            orope.rope(yq, rw.dtype, pos[:n], rw.base, inverse=True)
            orope.rope(yk, rw.dtype, pos[:n], rw.base, inverse=True)
            done += n
        dt = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": done / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                               "sample": f"first {n} tokens of {rw.name}, float64 forward + inverse of q and k "
                                         f"(numpy, one thread), {done // n} passes, {dt:.2f} s"}
    print(json.dumps(rec), flush=True)


def split_bytes(w, labels) -> dict:
    """Algorithmic bytes of the split calls: ce_forward reads each valid row
    once (+ label, loss, lse, 1 - p_label per row); ce_backward reads each
    valid row and writes every row (+ label, lse, 1 - p_label per row)."""
    n_valid = int((labels != -100).sum())
    row = w.V * w.elem_bytes
    return {"forward": n_valid * row + 28 * w.N, "backward": (n_valid + w.N) * row + 24 * w.N}


def profile_summary_split(d: str, workload: int) -> None:
    """Summary of bench.py --op split runs -> profiles/ce_split_<workload>.*"""
    import workloads as wl
    w = wl.WORKLOADS[workload]
    sha = kernel_sha()
    head = _profile_header(f"split cross-entropy: ce_forward, then ce_backward in place, workload {w.name}",
                           f"N={w.N} V={w.V} dtype={w.dtype} chunk={w.chunk}", sha, "split", workload)
    b = split_bytes(w, wl.plan(w).labels)
    _summarize(d, f"ce_split_{w.name}", head,
               {"forward": (("row_kernel_16", "row_kernel_32", "slab_stats", "slab_merge"), b["forward"]),
                "backward": (("grad_kernel",), b["backward"])},
               w.N * w.V * w.elem_bytes, sha)


def bench_split(args) -> None:
    """ce_forward and ce_backward (in place, the split form of a8) timed
    separately on one workload: logits resident in HBM, restored before and
    L2 / MALL flushed before each call, events on the call's stream."""
    import torch
    import cross_entropy_loss_amd as ce
    import workloads as wl

    w = wl.WORKLOADS[args.workload]
    p = wl.plan(w)
    bits = wl.logits(w, None, p, threads=16)
    labels = p.labels
    dev = torch.device("cuda:0")
    raw = torch.from_numpy(bits.view(np.int16) if w.elem_bytes == 2 else bits.view(np.int32))
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[w.dtype]
    pristine = raw.to(dev).view(tdt)
    work = torch.empty_like(pristine)
    y = torch.from_numpy(labels).to(dev)
    dloss = torch.tensor([w.dloss], dtype=torch.float32, device=dev)
    flush = torch.empty(1 << 28, dtype=torch.int32, device=dev)  # 1 GiB
    ws = ce.Workspace(dev, ce.ce_workspace_bytes(w.N, w.V, w.chunk, tdt))
    out = ce._outputs(w.N, dev)
    stream = torch.cuda.current_stream(dev)

    def step(i, ev=None):
        work.copy_(pristine)
        flush.fill_(2 * i)
        if ev:
            ev[0].record(stream)
        ce.ce_forward(work, y, -100, w.chunk, ws, out)
        if ev:
            ev[1].record(stream)
        flush.fill_(2 * i + 1)
        if ev:
            ev[2].record(stream)
        ce.ce_backward(work, y, out["lse_rows"], out["pcomp_rows"], out["n_valid"], dloss, -100, grad=work)
        if ev:
            ev[3].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st = int(out["status"].item())
    if st != 0:
        raise SystemExit(f"kernel status {st:#x}")
    fms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    bms = np.array([e[2].elapsed_time(e[3]) for e in evs])
    nbytes = pristine.numel() * pristine.element_size()
    copy_gbs, copy_shape, _ = _calib_copy(pristine, work, nbytes, flush, stream, args.calibrate)
    # the forward only reads the logits: its ceiling is the fastest plain read
    read_gbs, read_shape, _ = _calib_read(pristine, nbytes, flush, stream)
    b = split_bytes(w, labels)
    traffic = None
    cpath = os.path.join(ROOT, "profiles", f"ce_split_{w.name}.counters.json")
    if os.path.exists(cpath):
        with open(cpath) as f:
            c = json.load(f)
        if c.get("kernel_sha") == kernel_sha():
            traffic = {"forward": c.get("forward_traffic_bytes"), "backward": c.get("backward_traffic_bytes")}

    def roof(part, ms_mean):
        a = b[part] / (ms_mean * 1e-3) / 1e9
        r = {"bound": "hbm", "achieved": a, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": a / HBM_PEAK_GBS,
             "traffic": traffic[part] if traffic else None}
        if part == "forward":
            r.update({"read_ceiling": read_gbs, "frac_of_read": a / read_gbs, "read_shape": COPY_SHAPES[read_shape]})
        else:
            r.update({"copy_ceiling": copy_gbs, "frac_of_copy": a / copy_gbs, "copy_shape": COPY_SHAPES[copy_shape]})
        return r

    f_mean, b_mean = float(fms.mean()), float(bms.mean())
    rec = {
        "metric": f"CE split forward + backward tokens/s, N={w.N} V={w.V} {w.dtype}",
        "value": w.N / ((f_mean + b_mean) * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": f_mean + b_mean, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "rows": w.N, "vocab": w.V, "logits_dtype": w.dtype, "chunk": w.chunk,
                   "n_valid": int((labels != -100).sum()), "calls": "ce_forward, then ce_backward in place"},
        "roofline": roof("backward", b_mean),
        "roofline_forward": roof("forward", f_mean),
        "timing": {"forward_ms_mean": f_mean, "forward_ms_median": float(np.median(fms)),
                   "backward_ms_mean": b_mean, "backward_ms_median": float(np.median(bms)),
                   "algorithmic_bytes": b, "wall_ms_per_step_incl_restore_and_flush": wall / args.steps * 1e3,
                   "kernel_sha": kernel_sha()},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, bits, labels)
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=2,
                    help="ce / split: 1-5 (default 2, 4096 x 32000 bf16); linear: 1 (4096 x 4096 x 32000, the "
                         "default) or 4 (8192 x 4096 x 128256); rmsnorm / rope: 1")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate", action="store_true")
    ap.add_argument("--profile-summary", metavar="DIR")
    ap.add_argument("--op", choices=["ce", "split", "linear", "rmsnorm", "rope"], default="ce",
                    help="ce: the fused cross-entropy call (default); split: ce_forward and ce_backward timed "
                         "separately; linear: LM-head projection + cross-entropy; rmsnorm: RMS layer "
                         "normalisation forward + backward; rope: rotary embedding of q and k")
    ap.add_argument("--chunk-rows", type=int, default=None, help="--op linear: rows per chunk")
    args = ap.parse_args()
    if args.profile_summary:
        if args.op == "linear":
            profile_summary_linear(args.profile_summary, args.workload)
        elif args.op == "rmsnorm":
            profile_summary_norm(args.profile_summary, args.workload)
        elif args.op == "rope":
            profile_summary_rope(args.profile_summary, args.workload)
        elif args.op == "split":
            profile_summary_split(args.profile_summary, args.workload)
        else:
            profile_summary(args.profile_summary, args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    if args.op == "linear":
        bench_linear(args)
        return
    if args.op == "rmsnorm":
        bench_rmsnorm(args)
        return
    if args.op == "rope":
        bench_rope(args)
        return
    if args.op == "split":
        bench_split(args)
        return

    import torch
    import cross_entropy_loss_amd as ce
    import workloads as wl

    w = wl.WORKLOADS[args.workload]
    p = wl.plan(w)
    bits = wl.logits(w, None, p, threads=16)
    labels = p.labels
    dev = torch.device("cuda:0")
    raw = torch.from_numpy(bits.view(np.int16) if w.elem_bytes == 2 else bits.view(np.int32))
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[w.dtype]
    pristine = raw.to(dev).view(tdt)
    work = torch.empty_like(pristine)
    y = torch.from_numpy(labels).to(dev)
    dloss = torch.tensor([w.dloss], dtype=torch.float32, device=dev)
    flush = torch.empty(1 << 28, dtype=torch.int32, device=dev)  # 1 GiB
    ws = ce.Workspace(dev, ce.ce_workspace_bytes(w.N, w.V, w.chunk, tdt))
    out = ce._outputs(w.N, dev)
    stream = torch.cuda.current_stream(dev)

    def step(i, events=None):
        work.copy_(pristine)
        flush.fill_(i)
        if events:
            events[0].record(stream)
        ce.ce_fwd_bwd_inplace(work, y, -100, w.chunk, dloss, ws, out)
        if events:
            events[1].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    # the measured ceiling: the fastest plain copy of the logits' size under
    # the same protocol; with --calibrate only the counters' calibration copy
    # runs, and its counter readings scale FETCH_SIZE / WRITE_SIZE
    nbytes = pristine.numel() * pristine.element_size()
    copy_gbs, copy_shape, copy_rates = _calib_copy(pristine, work, nbytes, flush, stream, args.calibrate)
    st = int(out["status"].item())
    if st != 0:
        raise SystemExit(f"kernel status {st:#x}")
    ms_mean = float(ms.mean())
    abytes = algorithmic_bytes(w, labels)
    achieved = abytes / (ms_mean * 1e-3) / 1e9
    traffic = measured_traffic(f"ce_fused_{w.name}")  # HBM bytes per call from the committed counters
    n_valid = int((labels != -100).sum())
    rec = {
        "metric": HEADLINE_METRIC,
        "value": w.N / (ms_mean * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_mean,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "rows": w.N, "vocab": w.V, "logits_dtype": w.dtype,
                   "chunk": w.chunk, "n_valid": n_valid, "parallelism": "none"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "counter_gbs": traffic / (ms_mean * 1e-3) / 1e9 if traffic else None,
                     "copy_ceiling": copy_gbs, "frac_of_copy": achieved / copy_gbs,
                     "copy_shape": COPY_SHAPES[copy_shape],
                     "copy_shapes_gbs": {COPY_SHAPES[k]: round(v, 1) for k, v in copy_rates.items()}},
        "timing": {"ms_p10": float(np.percentile(ms, 10)), "ms_median": float(np.median(ms)),
                   "ms_p90": float(np.percentile(ms, 90)), "algorithmic_bytes": abytes,
                   "valid_tokens_per_s": n_valid / (ms_mean * 1e-3),
                   "wall_ms_per_step_incl_restore_and_flush": wall / args.steps * 1e3,
                   "kernel_sha": kernel_sha(),
                   "inputs_sha256": {"logits": hashlib.sha256(bits.tobytes()).hexdigest(),
                                     "labels": hashlib.sha256(labels.tobytes()).hexdigest()}},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, bits, labels)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
