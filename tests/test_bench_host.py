"""Host-side checks of bench.py (no GPU): the one-GPU contract, the algorithmic
byte counts behind roofline.achieved, and the rocprofv3 summariser behind
roofline.traffic, run on a synthetic database with known counter values."""
import json
import os
import sqlite3
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import workloads as wl  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_cross_entropy_algorithmic_bytes():
    w = wl.WORKLOADS[2]
    labels = wl.plan(w).labels
    n_valid = int((labels != -100).sum())
    want = (2 * n_valid + (w.N - n_valid)) * w.V * 2 + 28 * w.N
    assert bench.algorithmic_bytes(w, labels) == want
    assert abs(want - 511.28e6) < 0.01e6  # the figure the measurement notes quote


def test_norm_and_rope_bytes():
    nw = wl.NORM_WORKLOADS[1]
    b = bench.norm_bytes(nw)
    assert b["forward"] == 2 * 4096 * 4096 * 2 + 4096 * 2 + 4 * 4096
    assert b["backward"] == 3 * 4096 * 4096 * 2 + 2 * 4096 * 2 + 4 * 4096
    rw = wl.ROPE_WORKLOADS[1]
    assert bench.rope_bytes(rw) == 2 * 4096 * (32 + 8) * 128 * 2 + 8 * 4096


def test_split_call_bytes():
    # ce_forward reads each valid row once; ce_backward reads each valid row
    # and writes every row (ignored rows get zeros); per-row labels and
    # statistics on top
    w = wl.WORKLOADS[2]
    labels = wl.plan(w).labels
    n_valid = int((labels != -100).sum())
    b = bench.split_bytes(w, labels)
    assert b["forward"] == n_valid * w.V * 2 + 28 * w.N
    assert b["backward"] == (n_valid + w.N) * w.V * 2 + 24 * w.N
    # the pair moves one row read more than the fused call
    assert b["forward"] + b["backward"] - bench.algorithmic_bytes(w, labels) == n_valid * w.V * 2 + 24 * w.N


def _fake_profile(d, kernel, calib_kib_read, calib_kib_write, k_read, k_write, durations_ns):
    os.makedirs(d, exist_ok=True)
    con = sqlite3.connect(os.path.join(d, "trace_results.db"))
    con.execute("create table kernels (name text, start integer, end integer, duration integer)")
    t = 0
    for dur in durations_ns:
        con.execute("insert into kernels values (?, ?, ?, ?)", (kernel, t, t + dur, dur))
        t += dur + 1000
    con.commit()
    con.close()
    for tag, counter, kib_c, kib_k in (("fetch", "FETCH_SIZE", calib_kib_read, k_read),
                                       ("write", "WRITE_SIZE", calib_kib_write, k_write)):
        con = sqlite3.connect(os.path.join(d, f"{tag}_results.db"))
        con.execute("create table counters_collection (kernel_name text, counter_name text, value real)")
        con.execute("insert into counters_collection values (?, ?, ?)", ("calib_copy_kernel(...)", counter, kib_c))
        con.execute("insert into counters_collection values (?, ?, ?)", (kernel, counter, kib_k))
        con.commit()
        con.close()


def test_summariser_scales_counters_by_the_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    d = str(tmp_path / "db")
    calib = 1 << 20  # a 1 MiB copy: reads as 512 KiB (factor 2), writes as 1024 KiB (factor 1)
    _fake_profile(d, "void rope16<BF16>(RopeArgs)", 512.0, 1024.0, 1000.0, 3000.0, [10_000, 12_000, 11_000])
    rec = bench._summarize(d, "unit", ["# test"], {"launch": (("rope16",), 4_000_000)}, calib, "abc")
    assert rec["read_factor"] == pytest.approx(2.0)
    assert rec["write_factor"] == pytest.approx(1.0)
    assert rec["launch_traffic_bytes"] == pytest.approx(1000 * 1024 * 2 + 3000 * 1024)
    assert rec["launch_us"] == pytest.approx(11.0)  # the median duration
    with open(tmp_path / "profiles" / "unit.counters.json") as f:
        assert json.load(f)["kernel_sha"] == "abc"
    text = (tmp_path / "profiles" / "unit.txt").read_text()
    assert "ratio" in text and "11.00 us" in text


def test_traffic_is_dropped_when_the_kernel_changed(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    src = tmp_path / "k.hip"
    src.write_text("kernel v1")
    os.makedirs(tmp_path / "profiles")
    sha = bench.kernel_sha([str(src)])
    with open(tmp_path / "profiles" / "x.counters.json", "w") as f:
        json.dump({"kernel_sha": sha, "traffic_bytes": 123.0}, f)
    assert bench.measured_traffic("x", [str(src)]) == 123.0
    src.write_text("kernel v2")
    assert bench.measured_traffic("x", [str(src)]) is None
    assert np.isfinite(bench.HBM_PEAK_GBS) and bench.HBM_PEAK_GBS == 8000.0


def test_split_summary_attributes_both_calls(tmp_path, monkeypatch):
    # the split leg's summary: forward-pass kernels and the backward kernel
    # are attributed to their own call, each scaled by the copy's counters
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_sha", lambda sources=None: "abc")
    d = tmp_path / "db"
    os.makedirs(d)
    fwd, bwd = "void cek::row_kernel_16<cek::BF16, 512, 8, 3, false>(cek::Args)", "void cek::grad_kernel<...>(cek::Args)"
    con = sqlite3.connect(str(d / "trace_results.db"))
    con.execute("create table kernels (name text, start integer, end integer, duration integer)")
    for name, dur in ((fwd, 50_000), (bwd, 90_000), (fwd, 52_000), (bwd, 91_000), (fwd, 51_000), (bwd, 89_000)):
        con.execute("insert into kernels values (?, 0, ?, ?)", (name, dur, dur))
    con.commit()
    con.close()
    for tag, counter, calib, kf, kb in (("fetch", "FETCH_SIZE", 128000.0, 120000.0, 121000.0),
                                        ("write", "WRITE_SIZE", 256000.0, 0.0, 256000.0)):
        con = sqlite3.connect(str(d / f"{tag}_results.db"))
        con.execute("create table counters_collection (kernel_name text, counter_name text, value real)")
        for name, v in (("calib_copy_kernel(...)", calib), (fwd, kf), (bwd, kb)):
            con.execute("insert into counters_collection values (?, ?, ?)", (name, counter, v))
        con.commit()
        con.close()
    bench.profile_summary_split(str(d), 2)
    with open(tmp_path / "profiles" / "ce_split_mistral7b-b4s1024-bf16.counters.json") as f:
        rec = json.load(f)
    nbytes = 4096 * 32000 * 2
    assert rec["read_factor"] == pytest.approx(nbytes / 1024 / 128000.0)
    assert rec["forward_traffic_bytes"] == pytest.approx(120000.0 * 1024 * rec["read_factor"])
    assert rec["backward_traffic_bytes"] == pytest.approx(121000.0 * 1024 * rec["read_factor"] +
                                                          256000.0 * 1024 * rec["write_factor"])
    assert rec["forward_us"] == pytest.approx(51.0) and rec["backward_us"] == pytest.approx(90.0)
