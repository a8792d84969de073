"""Planted mistakes in the oracle must fail its pins.

Each case copies oracle.c, plants one plausible mistake (a dropped term, a wrong
comparison, sign or index), compiles the mutant on the CPU and runs the pin
tests against it; the pins pass on the real oracle and must fail on every mutant.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "hash-shift": ("z = (z ^ (z >> 27))", "z = (z ^ (z >> 26))"),
    "mod-32bit": ("% (uint64_t)rows)", "% (uint32_t)rows)"),
    "bucket-strict": ("if (b[j] <= x) k++;", "if (b[j] < x) k++;"),
    "hash-range-inclusive": ("id >= col->id_hi) return ROW_DROPPED;", "id > col->id_hi) return ROW_DROPPED;"),
    "mean-skips-default": ("n++;\n                if (r == ROW_DEFAULT) continue;      /* the zero row",
                           "if (r == ROW_DEFAULT) continue;      /* the zero row"),
    "mean-on-sum": ("y = (col->pool == O_MEAN) ? acc[d] / (double)n : acc[d];",
                    "y = acc[d] / (double)n;"),
    "grad-wrong-sample": ("G[s * sumD + off_c + d]", "G[s * sumD + d]"),
    "grad-no-mean-weight": ("w = (col->pool == O_MEAN) ? 1.0 / (double)n_of_bag[s] : 1.0;",
                            "w = 1.0;"),
    "sgd-sign": ("weight_store(col, r, d, w0 - lr * g[d]);", "weight_store(col, r, d, w0 + lr * g[d]);"),
    "adagrad-eps-inside": ("return e - lr * g / (sqrt(a2) + eps);", "return e - lr * g / sqrt(a2 + eps);"),
    "bf16-truncate": ("r = ldexp(rint(ldexp(m, 8)), e - 8);", "r = ldexp(floor(ldexp(m, 8)), e - 8);"),
    "init-shift": ("(double)(z >> 40), -24)", "(double)(z >> 41), -24)"),
    "trunc-last-off-by-one": ("return i >= len - col->seq_max;", "return i > len - col->seq_max;"),
    "trunc-first-inclusive": ("return i < col->seq_max;", "return i <= col->seq_max;"),
    "trunc-ends-swapped": ("if (col->seq_keep_last) return", "if (!col->seq_keep_last) return"),
    "mask-ignored": ("if (mask && mask[p] == 0) return 0;", "if (mask && mask[p] == 2) return 0;"),
    "weight-ignored-in-backward": ("if (pweights) w *= (double)pweights[list[j].pos];",
                                   "if (0) w *= (double)pweights[list[j].pos];"),
    "weight-bag-relative-index": ("(double)pweights[p] : 1.0;", "(double)pweights[p - offsets[b]] : 1.0;"),
    "default-row-not-read": ("} else if (col->default_row >= 0) {", "} else if (0) {"),
    "default-row-no-gradient": ("        if (col->default_row >= 0) {\n            for (int32_t s = 0; s < B; s++) {",
                                "        if (0) {\n            for (int32_t s = 0; s < B; s++) {"),
    "default-row-mean-weight": ("                    w = 1.0;\n                } else {",
                                "                    w = (col->pool == O_MEAN) ? 0.5 : 1.0;\n                } else {"),
    "weight-column-relative-index": ("w *= (double)pweights[list[j].pos];",
                                     "w *= (double)pweights[list[j].pos - a];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_pins(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mut = tmp_path / "oracle_mut.c"
    mut.write_text(src.replace(old, new))
    so = tmp_path / "liboracle_mut.so"
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-std=c11", "-shared", "-fPIC",
                           str(mut), "-o", str(so), "-lm"])
    env = dict(os.environ, ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
