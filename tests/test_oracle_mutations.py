"""The oracle's pins must catch plausible slips.

Each case plants one mistake in a temporary copy of the oracle's C source,
builds it, and runs the pin tests against that copy: every planted mistake
has to make at least one pin fail.  Everything runs on the CPU.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kda_oracle.c")

MUTANTS = {
    "no_decay": ("S[i * dv + j] *= a[i];", "S[i * dv + j] *= 1.0;"),
    "correction_sign": ("S[i * dv + j] += b * kh[i] * (vt[j] - u[j]);",
                        "S[i * dv + j] += b * kh[i] * (vt[j] + u[j]);"),
    "beta_on_value_only": ("S[i * dv + j] += b * kh[i] * (vt[j] - u[j]);",
                           "S[i * dv + j] += kh[i] * (b * vt[j] - u[j]);"),
    "conv_taps_reversed": ("acc += wconv[ch * W + j] * hist[j * nch + ch];",
                           "acc += wconv[ch * W + (W - 2 - j)] * "
                           "hist[j * nch + ch];"),
    "norm_sum_not_mean": ("ms /= (double)dv;", "ms /= 1.0;"),
    "no_key_l2_norm": ("rk = 1.0 / sqrt(sk + cfg->l2_eps);", "rk = 1.0;"),
    "q_scale_dropped": ("rq = cfg->q_scale / sqrt(sq + cfg->l2_eps);",
                        "rq = 1.0 / sqrt(sq + cfg->l2_eps);"),
    "q_scale_before_norm": ("rq = cfg->q_scale / sqrt(sq + cfg->l2_eps);",
                            "rq = cfg->q_scale / sqrt(cfg->q_scale * "
                            "cfg->q_scale * sq + cfg->l2_eps);"),
    "bf16_truncates": ("return ldexp(nearbyint(ldexp(f, 8)), e - 8);",
                       "return ldexp(trunc(ldexp(f, 8)), e - 8);"),
    "chunk_w_without_decay": ("exp(G[i * dk + c]) * KH[i * dk + c];",
                              "KH[i * dk + c];"),
    "chunk_final_state_sign": (
        "acc += exp(gl - G[i * dk + c]) * KH[i * dk + c] *",
        "acc -= exp(gl - G[i * dk + c]) * KH[i * dk + c] *"),
    "commit_wrong_record": (
        "memcpy(S, records + (long)(m - 1) * dk * dv",
        "memcpy(S, records + (long)(m < n ? m : m - 1) * dk * dv"),
    "gate_sign": ("double sig = 1.0 / (1.0 + exp(-x));",
                  "double sig = 1.0 / (1.0 + exp(x));"),
    "logit_decay_sign": ("exp(-softplus(alpha[i]))", "exp(-softplus(-alpha[i]))"),
    "logit_write_sign": ("1.0 / (1.0 + exp(-beta[i]))", "1.0 / (1.0 + exp(beta[i]))"),
    "softplus_positive_branch": ("x > 0.0 ? x + log1p(exp(-x))", "x > 0.0 ? log1p(exp(-x))"),
    "readout_before_write": (
        "        /* 6. read-out after the write */",
        "        for (i = 0; i < dk; ++i) for (j = 0; j < dv; ++j)"
        " S[i * dv + j] -= b * kh[i] * (vt[j] - u[j]);\n"
        "        /* 6. read-out after the write */"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    before, after = MUTANTS[name]
    src = open(SRC).read()
    assert before in src, f"mutation site of {name} not found"
    mutant = tmp_path / "mutant.c"
    mutant.write_text(src.replace(before, after, 1))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared",
                    "-ffp-contract=off", "-o", str(lib), str(mutant), "-lm"],
                   check=True)
    env = dict(os.environ, KDA_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x",
                        "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode != 0, f"planted mistake {name} passed every pin"
