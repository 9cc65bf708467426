"""The oracle's pins must catch plausible mistakes.

Each mutant below is a copy of oracle.c with one planted mistake (a dropped
term, a flipped sign, a transposed or wrong index, a missing guard).  The copy
is compiled on the CPU and the oracle pin tests are run against it in a child
process; every mutant must make at least one pin fail.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PIN_TESTS = ["tests/test_oracle_lse.py", "tests/test_oracle_partials.py",
             "tests/test_oracle_chain.py", "tests/test_oracle_axis_softmax.py"]

MUTANTS = {
    "lse_drops_max": ("  return m + log(s);\n}", "  return log(s);\n}"),
    "lse_sign_flip": ("s += exp((double)p[i * stride] - m);", "s += exp(m - (double)p[i * stride]);"),
    "lse_no_inf_guard": ("  if (isinf(m)) return m;\n", "\n"),
    "axis0_transposed": ("lse_strided(x + j, R, inner)", "lse_strided(x + j * R, R, 1)"),
    "rows_sign_flip": ("yr[c] = (double)row[c] - L;", "yr[c] = (double)row[c] + L;"),
    "partials_short_chunk": ("(c0 + chunk < cols) ? c0 + chunk : cols",
                             "(c0 + chunk < cols) ? c0 + chunk - 1 : cols"),
    "partials_no_ninf_guard": ("      } else if (m == -INFINITY) {\n        s = 0.0;",
                               "      } else if (0) {\n        s = 0.0;"),
    "merge_unguarded": ("S += sr[i] * ((mr[i] == M) ? 1.0 : exp(mr[i] - M));",
                        "S += sr[i] * exp(mr[i] - M);"),
    "merge_sign_flip": ("S += sr[i] * ((mr[i] == M) ? 1.0 : exp(mr[i] - M));",
                        "S += sr[i] * ((mr[i] == M) ? 1.0 : exp(M - mr[i]));"),
    "hardswish_no_gate": ("  return t * u / 6.0;", "  return u / 6.0;"),
    "hardswish_no_clamp": ("  if (u > 6.0) u = 6.0;\n", "\n"),
    "conv_kernel_transposed": ("w[((o * Cin + c) * K + i) * K + j]", "w[((o * Cin + c) * K + j) * K + i]"),
    "conv_no_bias": ("double acc = b ? (double)b[o] : 0.0;", "double acc = 0.0;"),
    "gn_unbiased_var": ("const double var = sq / (double)cnt;", "const double var = sq / (double)(cnt - 1);"),
    "gn_mean_wrong_count": ("const double mu = sum / (double)cnt;", "const double mu = sum / (double)P;"),
    "gn_interleaved_groups": ("const int64_t g = c / Cg;", "const int64_t g = c % G;"),
    "gn_no_eps": ("rstd_g[g] = 1.0 / sqrt(var + eps);", "rstd_g[g] = 1.0 / sqrt(var);"),
    "gn_affine_swapped": ("* rstd_g[g] * ga + be;", "* rstd_g[g] * be + ga;"),
    "chain_no_residual": ("const double v4 = v0 + oracle_hardswish(tanh(v1));",
                          "const double v4 = oracle_hardswish(tanh(v1));"),
    "chain_no_tanh": ("oracle_hardswish(tanh(v1))", "oracle_hardswish(v1)"),
    "chain_lse_drops_max": ("          r = m + log(s);", "          r = log(s);"),
    "softmax_sign_flip": ("yr[c] = exp((double)row[c] - L);", "yr[c] = exp(L - (double)row[c]);"),
    "softmax_unnormalised": ("yr[c] = exp((double)row[c] - L);", "yr[c] = exp((double)row[c]);"),
    "axis_outer_stride": ("lse_strided(x + o * R * inner + j, R, inner)",
                          "lse_strided(x + o * inner + j, R, inner)"),
    "axis_wrong_stride": ("lse_strided(x + o * R * inner + j, R, inner)",
                          "lse_strided(x + o * R * inner + j, R, 1)"),
    "lsm_axis_wrong_out": ("y[(o * R + r) * inner + j] = (double)base[r * inner] - L;",
                           "y[(o * R + r) * inner + j] = (double)base[r] - L;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    from oracle.oracle import compile_source
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/present"
    mutated = tmp_path / "oracle_mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = compile_source(str(mutated), str(tmp_path / "liboracle_mutant.so"))
    env = dict(os.environ, LSE_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *PIN_TESTS], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
