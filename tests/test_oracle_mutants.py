"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that the pins
in test_oracle_pins.py reject every one of them.  The shipped oracle is never modified."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "causal_diagonal_excluded": ("if (is_causal && j > i)", "if (is_causal && j >= i)"),
    "causal_wrong_triangle": ("if (is_causal && j > i)", "if (is_causal && j < i)"),
    "mask_polarity_inverted": ("mask[b * ms[0] + h * ms[1] + i * ms[2] + j * ms[3]] == 0",
                               "mask[b * ms[0] + h * ms[1] + i * ms[2] + j * ms[3]] != 0"),
    "scale_dropped": ("s[j] = scale * dot;", "s[j] = dot;"),
    "k_index_dropped_d": ("load_elem(k, dtype, krow + d * ks[3])", "load_elem(k, dtype, krow)"),
    "q_row_and_col_swapped": ("load_elem(q, dtype, qrow + d * qs[3])",
                              "load_elem(q, dtype, qrow + d * qs[2])"),
    "v_indexed_by_query": ("j * vs[2] + d * vs[3]", "i * vs[2] + d * vs[3]"),
    "empty_row_not_zeroed": ("if (!any) {", "if (0) {"),
    "lse_drops_max": ("*lse_out = m + log(l);", "*lse_out = log(l);"),
    "softmax_not_normalised": ("for (int64_t j = 0; j < Lk; ++j) p[j] /= l;", ""),
    "max_not_subtracted_wrongly": ("exp(s[j] - m)", "exp(s[j] + m)"),
    "bf16_decode_shift": ("<< 16", "<< 15"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert old in src, f"mutation anchor for {name} no longer matches oracle.c"
    mutant_c = tmp_path / "oracle_mutant.c"
    mutant_c.write_text(src.replace(old, new, 1))
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", str(lib),
                    str(mutant_c), "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"pins accepted the mutant {name}:\n{r.stdout[-2000:]}"
