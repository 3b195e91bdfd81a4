"""Sensitivity of the oracle pins: plant one plausible mistake at a time in a
copy of the oracle's C source (on the CPU), build it, and check that the pin
suite then fails.  The committed oracle source is never modified."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "lora_oracle.c")

MUTANTS = {
    "rslora_dropped": ("return alpha / sqrt((double)r);", "return alpha / (double)r;"),
    "plain_scale_off": ("    return alpha / (double)r;\n}", "    return alpha / (double)(r + 1);\n}"),
    "ties_away_from_zero": ("return (down & 1u) ? up : down;", "return up;"),
    "scale_not_applied": ("B_scaled[p][i] = B_in[p][i] * scale;", "B_scaled[p][i] = B_in[p][i];"),
    "B_transposed_in_pad": ("B_pad[p][o * R + j] = B_scaled[p][o * r + j];",
                            "B_pad[p][o * R + j] = B_scaled[p][j * out_dim[p] + o];"),
    "A_rows_not_padded": ("        arow += R;", "        arow += r;"),
    "sort_not_stable": ("if (kj <= key)", "if (kj < key)"),
    "base_sorted_first": ("int64_t key = slot[cur] == -1 ? (int64_t)L : slot[cur];",
                          "int64_t key = slot[cur];"),
    "no_truncation": ("        if (s == -1)\n            break;", "        if (s == -2)\n            break;"),
    "slice_offset_dropped": ("u[t * C + (int64_t)s * R + j]", "u[t * C + j]"),
    "A_transposed": ("acc += A[c * in_f + k] * x[t * in_f + k];", "acc += A[k * C + c] * x[t * in_f + k];"),
    "delta_sign": ("y_in[t * n_out + off + o] + acc;", "y_in[t * n_out + off + o] - acc;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutated = src.replace(old, new, 1)
    c = tmp_path / "mutant.c"
    so = tmp_path / "libmutant.so"
    c.write_text(mutated)
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", str(c), "-o",
                    str(so), "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
