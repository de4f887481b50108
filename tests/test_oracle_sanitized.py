"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The oracle (oracle/ce_oracle.c) is built a second time with
``-fsanitize=address,undefined`` and driven, in a child process with the
sanitizer runtimes preloaded (the Python interpreter itself is not
instrumented), through every entry point on shapes that reach its edge paths:
one-element and ragged rows, every storage format, ignored and out-of-range
labels, no valid row, chunked log-sum-exp with chunks that do not divide the
row, subnormal and huge values.  Any report fails the test, and the sanitized
build must give the same bits as the plain one.
"""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = textwrap.dedent(r"""
    import sys
    import numpy as np
    sys.path.insert(0, sys.argv[2])
    import oracle
    from workloads import to_storage

    san = oracle.load(sys.argv[1])
    plain = oracle.load()
    rng = np.random.default_rng(5)
    cases = 0
    for dtype in ("f32", "bf16", "f16"):
        for R, V in ((1, 1), (3, 2), (7, 33), (16, 1000)):
            x = to_storage(rng.standard_normal((R, V)) * 4.0, dtype)
            y = rng.integers(0, V, R)
            if R > 2:
                y[0] = -100
                y[1] = V  # out of range: reported, not raised
            for dl in (1.0, 0.5):
                a = oracle.cross_entropy(x, y, dtype, dloss=dl, want_grad64=True, allow_bad=True, lib=san)
                b = oracle.cross_entropy(x, y, dtype, dloss=dl, want_grad64=True, allow_bad=True, lib=plain)
                for k in ("loss_rows", "lse", "grad", "grad64"):
                    assert np.array_equal(a[k], b[k], equal_nan=True), (dtype, R, V, k)
                cases += 1
            for chunk in (1, 7, V, V + 3):
                assert oracle.chunked_lse(x[-1], dtype, chunk, lib=san) == oracle.chunked_lse(x[-1], dtype, chunk,
                                                                                              lib=plain)
        # no valid row; extremes of the format (subnormals, the largest finite values)
        x = to_storage(np.array([[1e-40, -1e-40, 3e38, -3e38]] * 2), dtype)
        a = oracle.cross_entropy(x, np.array([-100, -100]), dtype, lib=san)
        assert np.isnan(a["loss_mean"]) and not np.any(oracle.widen(a["grad"], dtype, lib=san))
        big = to_storage(np.array([[60000.0, 1.0, -60000.0]]), dtype)
        oracle.cross_entropy(big, np.array([2]), dtype, lib=san)
        wide = np.linspace(-3.0e38, 3.0e38, 4099)
        assert np.array_equal(oracle.widen(oracle.round_to(wide, dtype, lib=san), dtype, lib=san),
                              oracle.widen(oracle.round_to(wide, dtype, lib=plain), dtype, lib=plain),
                              equal_nan=True)
        cases += 1
    print("sanitized cases", cases)
""")


def _runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


@pytest.mark.skipif(_runtime("libasan.so") is None or _runtime("libubsan.so") is None,
                    reason="gcc's sanitizer runtimes are not installed")
def test_oracle_under_sanitizers(tmp_path):
    lib = str(tmp_path / "libce_oracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-fno-fast-math", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", os.path.join(ROOT, "oracle", "ce_oracle.c"), "-o", lib, "-lm"],
                   check=True)
    env = dict(os.environ)
    env["LD_PRELOAD"] = _runtime("libasan.so") + ":" + _runtime("libubsan.so")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=23"  # the interpreter's own allocations
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "2"
    r = subprocess.run([sys.executable, "-c", CHILD, lib, ROOT], env=env, capture_output=True, text=True,
                       timeout=600)
    report = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, report
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, report
    assert "sanitized cases" in r.stdout


@pytest.mark.skipif(_runtime("libasan.so") is None or _runtime("libubsan.so") is None,
                    reason="gcc's sanitizer runtimes are not installed")
def test_sanitizer_harness_reports_a_planted_overflow(tmp_path):
    # the same build flags and child environment report a one-past-the-end heap read, so a clean run
    # of the oracle above means something
    src = tmp_path / "planted.c"
    src.write_text("#include <stdlib.h>\nint planted(int n) { int* a = malloc(4 * n); int s = a[n]; free(a); "
                   "return s; }\n")
    lib = str(tmp_path / "libplanted.so")
    subprocess.run(["gcc", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", str(src), "-o", lib], check=True)
    env = dict(os.environ)
    env["LD_PRELOAD"] = _runtime("libasan.so") + ":" + _runtime("libubsan.so")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=23"
    r = subprocess.run([sys.executable, "-c", f"import ctypes; ctypes.CDLL({lib!r}).planted(4)"], env=env,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 23 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]
