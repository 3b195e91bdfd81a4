"""Sensitivity of the oracle pins: plant one plausible mistake at a time in a
copy of the oracle's C source or of its Python driver (on the CPU), build or
load the copy, and check that the pin suite then fails.  The committed oracle
source is never modified."""

import os
import shutil
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


# mistakes in the Python side of the oracle (oracle/oracle.py): the bf16
# decoder every bf16 reference value passes through
PY_MUTANTS = {
    "bf16_decode_shift": ("<< np.uint32(16)", "<< np.uint32(15)"),
    "bf16_decode_sign_lost": ("b = np.ascontiguousarray(bits, dtype=np.uint16)",
                              "b = np.ascontiguousarray(bits, dtype=np.uint16) & np.uint16(0x7FFF)"),
    "f32_stack_rounded": ('return bf16_to_f64(a) if dtype == "bf16" else np.asarray(a, dtype=np.float64)',
                          'return bf16_to_f64(a) if dtype == "bf16" else np.asarray(a, dtype=np.float16).astype(np.float64)'),
}


@pytest.mark.parametrize("name", ["unchanged"] + sorted(PY_MUTANTS))
def test_planted_python_mistake_is_caught(name, tmp_path):
    """"unchanged" is the control: the copied, unmutated package passes."""
    import oracle
    lib = oracle.library_path()
    if not os.path.exists(lib):
        oracle.build()
    old, new = PY_MUTANTS.get(name, ("def bf16_to_f64(", "def bf16_to_f64("))
    pkg = tmp_path / "oracle"
    shutil.copytree(os.path.join(ROOT, "oracle"), pkg, ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    src = (pkg / "oracle.py").read_text()
    assert src.count(old) == 1, f"mutation anchor for {name} not found"
    (pkg / "oracle.py").write_text(src.replace(old, new))
    # the mutated package first on the path, the repository after it (so the
    # test suite's conftest does not put the real package in front)
    code = ("import sys, pytest; sys.path[:0] = [%r, %r]; import oracle; "
            "print('ORACLE_FROM', oracle.__file__, flush=True); "
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', %r]))"
            % (str(tmp_path), ROOT, os.path.join(ROOT, "tests", "test_oracle_pins.py")))
    env = dict(os.environ, ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    assert f"ORACLE_FROM {pkg}" in r.stdout, r.stdout[-2000:]
    if name == "unchanged":
        assert r.returncode == 0, r.stdout[-2000:]
    else:
        assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
