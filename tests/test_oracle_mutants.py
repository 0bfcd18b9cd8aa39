"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that the pins
reject every one of them: forward mistakes by test_oracle_pins.py, backward mistakes by
test_oracle_bwd_pins.py.  The shipped oracle is never modified."""
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
    "f16_exponent_bias": ("ldexp((double)(1024 + frac), ex - 25)", "ldexp((double)(1024 + frac), ex - 24)"),
    "f16_subnormal_scale": ("ldexp((double)frac, -24)", "ldexp((double)frac, -25)"),
    "f16_sign_dropped": ("return sign ? -mag : mag;", "return mag;"),
    "bias_subtracted": ("s[j] += bias[b * bs[0] + h * bs[1] + i * bs[2] + j * bs[3]];",
                        "s[j] -= bias[b * bs[0] + h * bs[1] + i * bs[2] + j * bs[3]];"),
    "bias_transposed": ("s[j] += bias[b * bs[0] + h * bs[1] + i * bs[2] + j * bs[3]];",
                        "s[j] += bias[b * bs[0] + h * bs[1] + j * bs[2] + i * bs[3]];"),
    "bias_scaled": ("s[j] += bias[b * bs[0] + h * bs[1] + i * bs[2] + j * bs[3]];",
                    "s[j] += scale * bias[b * bs[0] + h * bs[1] + i * bs[2] + j * bs[3]];"),
    "bias_minus_inf_kept": ("      if (s[j] == -INFINITY) continue;\n    }", "    }"),
}

# backward: (anchor, replacement) in oracle_sdpa_bwd
BWD_MUTANTS = {
    "bwd_rowsum_sign": ("P[i * Lk + j] * (dS[i * Lk + j] - rowsum)",
                        "P[i * Lk + j] * (dS[i * Lk + j] + rowsum)"),
    "bwd_rowsum_dropped": ("P[i * Lk + j] * (dS[i * Lk + j] - rowsum)",
                           "P[i * Lk + j] * dS[i * Lk + j]"),
    "bwd_rowsum_without_p": ("rowsum += P[i * Lk + j] * dot;", "rowsum += dot;"),
    "bwd_dk_scale_dropped": ("dk[(bh * Lk + j) * D + d] = scale * ak;",
                             "dk[(bh * Lk + j) * D + d] = ak;"),
    "bwd_dq_scale_dropped": ("dq[(bh * Lq + i) * D + d] = scale * a;",
                             "dq[(bh * Lq + i) * D + d] = a;"),
    "bwd_dk_from_dout": ("ak += dS[i * Lk + j] * load_elem(q, dtype, qb + i * qs[2] + d * qs[3]);",
                         "ak += dS[i * Lk + j] * load_elem(dout, dtype, ob + i * dos[2] + d * dos[3]);"),
    "bwd_dv_uses_ds": ("av += P[i * Lk + j] *", "av += dS[i * Lk + j] *"),
    "bwd_dp_uses_k": ("load_elem(v, dtype, vb + j * vs[2] + d * vs[3]);",
                      "load_elem(k, dtype, kb + j * ks[2] + d * ks[3]);"),
    "bwd_dq_uses_v": ("a += dS[i * Lk + j] * load_elem(k, dtype, kb + j * ks[2] + d * ks[3]);",
                      "a += dS[i * Lk + j] * load_elem(v, dtype, vb + j * vs[2] + d * vs[3]);"),
    "bwd_p_unnormalised": ("pr[j] = any ? pr[j] / l : 0.0;", "pr[j] = any ? pr[j] : 0.0;"),
    "bwd_empty_row_not_zeroed": ("pr[j] = any ? pr[j] / l : 0.0;", "pr[j] = pr[j] / l;"),
    "bwd_dout_row_stride": ("ob + i * dos[2] + d * dos[3]) *", "ob + i * dos[3] + d * dos[3]) *"),
    "bwd_bias_subtracted": ("pr[j] += bias[b * bs[0] + h * bs[1] + i * bs[2] + j * bs[3]];",
                            "pr[j] -= bias[b * bs[0] + h * bs[1] + i * bs[2] + j * bs[3]];"),
    "bwd_bias_transposed": ("pr[j] += bias[b * bs[0] + h * bs[1] + i * bs[2] + j * bs[3]];",
                            "pr[j] += bias[b * bs[0] + h * bs[1] + j * bs[2] + i * bs[3]];"),
    "bwd_bias_scaled": ("pr[j] += bias[b * bs[0] + h * bs[1] + i * bs[2] + j * bs[3]];",
                        "pr[j] += scale * bias[b * bs[0] + h * bs[1] + i * bs[2] + j * bs[3]];"),
    "bwd_bias_minus_inf_kept": ("            if (pr[j] == -INFINITY) continue;\n", ""),
}


ALL = {**{n: (o, r, "test_oracle_pins.py") for n, (o, r) in MUTANTS.items()},
       **{n: (o, r, "test_oracle_bwd_pins.py") for n, (o, r) in BWD_MUTANTS.items()}}


@pytest.mark.parametrize("name", sorted(ALL))
def test_pins_reject_mutant(name, tmp_path):
    old, new, pins = ALL[name]
    src = open(SRC).read()
    assert old in src, f"mutation anchor for {name} no longer matches oracle.c"
    mutant_c = tmp_path / "oracle_mutant.c"
    mutant_c.write_text(src.replace(old, new, 1))
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", str(lib),
                    str(mutant_c), "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", pins)],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"pins accepted the mutant {name}:\n{r.stdout[-2000:]}"
