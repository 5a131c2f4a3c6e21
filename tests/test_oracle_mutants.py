"""The pins are strong enough: each plausible mistake planted in a copy of
the oracle's C source (on the CPU, in a temporary build) makes the pin suite
fail.  The real oracle is untouched."""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "adam_oracle.c")

MUTANTS = {
    "eps_inside_root": ("(sqrt(v_hat) + j->eps)", "sqrt(v_hat + j->eps)"),
    "no_bias_correction_m": ("double m_hat = m / j->bc1;", "double m_hat = m;"),
    "no_bias_correction_v": ("double v_hat = v / j->bc2;", "double v_hat = v;"),
    "wrong_sign": ("double delta = -j->lr", "double delta = j->lr"),
    "swapped_beta_terms": ("double m = b1 * (double)j->m[i] + one_minus_b1 * g;",
                           "double m = one_minus_b1 * (double)j->m[i] + b1 * g;"),
    "v_uses_g_not_g2": ("one_minus_b2 * (g * g)", "one_minus_b2 * fabs(g)"),
    "bias_uses_t_minus_1": ("pow(beta1, (double)t)", "pow(beta1, (double)(t - 1) + 0.5)"),
    "bf16_truncates": ("u += 0x7FFFu + lsb;", "u += 0u * lsb;"),
    "bf16_ties_away": ("u += 0x7FFFu + lsb;", "u += 0x8000u + 0u * lsb;"),
    "recast_old_master": ("double w = (double)j->master[i] + delta;\n        j->m[i] = (float)m;\n        j->v[i] = (float)v;\n        j->master[i] = (float)w;\n        if (j->w) j->w[i] = lso_oracle_bf16_rne(j->master[i]);",
                          "double w = (double)j->master[i] + delta;\n        j->m[i] = (float)m;\n        j->v[i] = (float)v;\n        if (j->w) j->w[i] = lso_oracle_bf16_rne(j->master[i]);\n        j->master[i] = (float)w;"),
    "sgd_sign": ("float delta = -prod;", "float delta = prod;"),
    "accumulate_drops": ("w[i] = w[i] + delta[i];", "w[i] = delta[i];"),
    "g32_read_as_bf16": ("double g = j->g32 ? (double)j->g32[i] : bf16_widen(j->g[i]);",
                         "double g = j->g32 ? bf16_widen((uint16_t)(bits_from_f32(j->g32[i]) >> 16))"
                         " : bf16_widen(j->g[i]);"),
    "sgd_g32_read_as_bf16": ("float gi = g32 ? g32[i] : f32_from_bits((uint32_t)g[i] << 16);",
                             "float gi = g32 ? f32_from_bits(bits_from_f32(g32[i]) & 0xFFFF0000u)"
                             " : f32_from_bits((uint32_t)g[i] << 16);"),
    "sq_norm_drops_last": ("for (uint64_t i = 0; i < n; ++i) {\n        double g = g32 ?",
                           "for (uint64_t i = 0; i + 1 < n; ++i) {\n        double g = g32 ?"),
    "sq_norm_abs": ("s += g * g;", "s += fabs(g);"),
    "sq_norm_bf16_path_reads_low_half": ("double g = g32 ? (double)g32[i] : bf16_widen(g16[i]);",
                                         "double g = g32 ? (double)g32[i] : (double)g16[i];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "m.c")
        so = os.path.join(d, "libm.so")
        open(c, "w").write(src.replace(old, new))
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-shared",
                               "-fPIC", "-pthread", c, "-o", so, "-lm"])
        env = dict(os.environ, LSO_ORACLE_LIB=so)
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
        assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
