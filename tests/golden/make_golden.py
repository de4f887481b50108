"""Writes tests/golden/oracle_regression.json from the float64 oracle only.

The stored values freeze the oracle's output on small seeded workloads, so any
later change to its arithmetic shows up as a test failure that the change's
commit message must justify.  Run:  python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads as wl  # noqa: E402


def cases():
    yield wl.WORKLOADS[1]
    yield wl.custom("ragged-bf16", 31, 40, 1031, "bf16", 2.0, 0.1)
    yield wl.custom("ragged-f16", 32, 40, 777, "f16", 30.0, 0.2, dloss=0.5, spike_frac=0.1)


def record(w):
    x, p = wl.make(w)
    r = oracle.cross_entropy(x, p.labels, w.dtype, dloss=w.dloss)
    return {
        "workload": w.name, "N": w.N, "V": w.V, "dtype": w.dtype, "seed": w.seed,
        "n_valid": r["n_valid"], "loss_mean": r["loss_mean"].hex(),
        "lse_first8": [v.hex() for v in r["lse"][:8]],
        "loss_first8": [v.hex() for v in r["loss_rows"][:8]],
        "grad_sha256": hashlib.sha256(r["grad"].tobytes()).hexdigest(),
        "logits_sha256": hashlib.sha256(x.tobytes()).hexdigest(),
    }


if __name__ == "__main__":
    out = [record(w) for w in cases()]
    with open(os.path.join(HERE, "oracle_regression.json"), "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", len(out), "records")
