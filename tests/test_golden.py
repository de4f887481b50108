"""The oracle and the input generators still produce the frozen records
written by tests/golden/make_golden.py (CPU only)."""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))

import make_golden  # noqa: E402


def test_oracle_regression():
    with open(os.path.join(HERE, "golden", "oracle_regression.json")) as f:
        want = json.load(f)
    got = [make_golden.record(w) for w in make_golden.cases()]
    assert len(got) == len(want)
    for g, w in zip(got, want):
        assert g == w, g["workload"]
