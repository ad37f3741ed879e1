"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of oracle/plx_oracle.c (on the CPU), builds
it, and runs tests/test_oracle_pins.py against it; at least one pin must fail.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "plx_oracle.c")

MUTANTS = {
    "correction_sign": ("o[c] = vbar[c] - dot(sigma", "o[c] = vbar[c] + dot(sigma"),
    # Centring only one side of the weighted covariance is an identity, not a mistake
    # (the weighted deviations sum to zero), so the planted mistake removes both.
    "not_centred": ("double wv = p[j] * (vj[c] - vbar[c]);\n            double* srow = sigma + (size_t)c * dqk;\n            for (int e = 0; e < dqk; ++e) srow[e] += wv * (kj[e] - kbar[e]);",
                    "double wv = p[j] * vj[c];\n            double* srow = sigma + (size_t)c * dqk;\n            for (int e = 0; e < dqk; ++e) srow[e] += wv * kj[e];"),
    "bessel_factor": ("for (int c = 0; c < dv; ++c) o[c] = vbar[c] - dot(sigma + (size_t)c * dqk, rho, dqk);",
                      "for (int c = 0; c < dv; ++c) o[c] = vbar[c] - (n > 1 ? n / (n - 1.0) : 1.0) * dot(sigma + (size_t)c * dqk, rho, dqk);"),
    "sigma_transposed": ("srow[e] += wv * (kj[e] - kbar[e]);",
                         "sigma[(size_t)e * dv + c] += wv * (kj[e] - kbar[e]);"),
    "t_scaled": ("t[j] = dot(rho, K + (size_t)j * dqk, dqk);",
                 "t[j] = scale * dot(rho, K + (size_t)j * dqk, dqk);"),
    "diagonal_key_dropped": ("Vb, i + 1, dqk, dv,", "Vb, i > 0 ? i : 1, dqk, dv,"),
    "beta_not_rescaled": ("st->beta *= alpha;", ";"),
    "p2_without_p1": ("double P2 = P1 * S2[j];", "double P2 = S2[j];"),
    "combine_sign": ("o[c] = (1.0 + tbar) * (st->O1[c] / st->l)",
                     "o[c] = (1.0 - tbar) * (st->O1[c] / st->l)"),
    "merge_no_rescale": ("dst->beta = fd * dst->beta + fs * src->beta;",
                         "dst->beta = dst->beta + src->beta;"),
    "sweighted_sign": ("double s = p[j] * (1.0 - (t[j] - tbar));",
                       "double s = p[j] * (1.0 + (t[j] - tbar));"),
    "seqlens_not_clamped": ("if (n > L_max) n = L_max;", "if (n > L_max) n = L_max - 1;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mut_c = tmp_path / "mut.c"
    mut_c.write_text(src.replace(old, new))
    so = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
                           str(mut_c), "-o", str(so), "-lm"])
    env = dict(os.environ, PLX_ORACLE_LIB=str(so), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"no pin caught mutant {name}:\n{r.stdout[-2000:]}"
    assert "failed" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]
