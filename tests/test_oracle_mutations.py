"""Each plausible mistake planted in a copy of the oracle must fail a pin.

A mutant is the oracle's C source with one textual change (a dropped term, a
wrong sign, index or bias, the wrong rounding rule ...).  It is compiled into a
temporary directory and the whole pin battery runs against it in a child
process; the test passes when at least one pin rejects the mutant.  This runs
on the CPU only and never touches the real oracle build.
"""
import os
import subprocess
import sys
import textwrap

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ce_oracle.c")

# (name, original text, replacement); each original must occur in the source
MUTANTS = [
    ("no_max_shift", "kadd(&s, exp(x[j] - m));", "kadd(&s, exp(x[j]));"),
    ("loss_sign", "loss[i] = row_lse - x[y];", "loss[i] = x[y] - row_lse;"),
    ("onehot_sign", "g[y] = scale * (p_y - 1.0);", "g[y] = scale * (p_y + 1.0);"),
    ("label_off_by_one", "double p_y = exp(x[y] - row_lse);", "double p_y = exp(x[(y + 1) % V] - row_lse);"),
    ("count_all_rows", "n += (labels[i] != ignore_index);", "n += 1;"),
    ("ignored_rows_have_grad", "for (int64_t j = 0; j < V; ++j) g[j] = 0.0;",
     "for (int64_t j = 0; j < V; ++j) g[j] = scale * exp(x[j] - row_lse);"),
    ("mean_over_all_rows", "if (labels[i] == ignore_index) continue;", ""),
    ("confident_loss_sign", "loss[i] = -log1p(-kval(&q));", "loss[i] = log1p(-kval(&q));"),
    ("confident_includes_label", "if (j != y) kadd(&q, exp(x[j] - row_lse));", "kadd(&q, exp(x[j] - row_lse));"),
    ("round_truncates", "double r = nearbyint(x / quantum) * quantum;", "double r = trunc(x / quantum) * quantum;"),
    ("round_ties_away", "double r = nearbyint(x / quantum) * quantum;", "double r = round(x / quantum) * quantum;"),
    ("f16_bias", "v = ldexp((double)(1024 + man), ex - 25);", "v = ldexp((double)(1024 + man), ex - 24);"),
    ("f16_subnormal_scale", "v = ldexp((double)man, -24);", "v = ldexp((double)man, -25);"),
    ("bf16_shift", "uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;"),
    ("f16_no_subnormal_output", "if (lead < -14) return sign | (uint16_t)(a * 16777216.0);",
     "if (lead < -14) return sign;"),
    ("row_stride_dropped", "(size_t)i * (size_t)ld * esz;", "(size_t)i * esz;"),
    ("chunk_merge_no_shift", "kadd(&s, exp(part[c] - M));", "kadd(&s, exp(part[c]));"),
    ("chunk_last_slab_dropped", "int64_t C = (V + chunk - 1) / chunk;", "int64_t C = V / chunk;"),
    ("lse_log_base2", "return m + log(kval(&s));", "return m + log2(kval(&s));"),
    ("mean_divides_by_rows", "return kval(&s) / (double)n;", "return kval(&s) / (double)n_rows;"),
]

RUNNER = textwrap.dedent(
    """
    import sys
    sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
    import oracle, oracle_pins
    lib = oracle.load({lib!r})
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except Exception as e:
            print("CAUGHT_BY", pin.__name__, type(e).__name__)
            sys.exit(0)
    print("NOT_CAUGHT")
    """
)


def test_mutants_are_distinct_and_apply():
    src = open(SRC).read()
    for name, old, new in MUTANTS:
        assert src.count(old) >= 1, name


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_caught(name, old, new, tmp_path):
    src = open(SRC).read()
    mutated = src.replace(old, new, 1)
    assert mutated != src
    c_path = tmp_path / "mutant.c"
    c_path.write_text(mutated)
    lib_path = str(tmp_path / "libmutant.so")
    oracle.build(force=True, src=str(c_path), out=lib_path)
    code = RUNNER.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib_path)
    env = dict(os.environ, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600, env=env)
    # a crash of the child (signal) also means the mutant was caught
    assert "NOT_CAUGHT" not in r.stdout, (name, r.stdout[-2000:], r.stderr[-2000:])
    assert "CAUGHT_BY" in r.stdout or r.returncode != 0, (name, r.stdout, r.stderr[-2000:])
