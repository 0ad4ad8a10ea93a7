"""Plant plausible mistakes in a copy of the oracle and check the pins fail.

Each mutation is a one-line textual change to ``oracle/oracle.c`` compiled
into a temporary library on the CPU; the pin suite is then run against that
library in a subprocess and must fail. The committed oracle is not touched.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTATIONS = {
    "eps_outside_root": ("r = 1.0 / sqrt(var + eps);", "r = 1.0 / (sqrt(var) + eps);"),
    "unbiased_variance": ("double var = q / (double)K;",
                          "double var = q / (double)(K > 1 ? K - 1 : 1);"),
    "dropped_beta": ("a[k] = a[k] * g + b;", "a[k] = a[k] * g + 0.0 * b;"),
    "ignored_gamma": ("double g = gamma ? dec(gamma[k], dtype) : 1.0;", "double g = 1.0;"),
    "mean_sign": ("a[k] = (a[k] - mu) * r;", "a[k] = (a[k] + mu) * r;"),
    "rms_without_eps": ("r = 1.0 / sqrt(ms + eps);", "r = 1.0 / sqrt(ms);"),
    "transposed_weight": ("z += ar[k] * dec(wr[k], dtype);",
                          "z += ar[k] * dec(W[(k * N + cols[j]) % (N * K)], dtype);"),
    "bias_after_act": ("y_out[t] = apply_act(z, act);",
                       "y_out[t] = apply_act(z - (bias ? dec(bias[cols[j]], dtype) : 0.0), act)"
                       " + (bias ? dec(bias[cols[j]], dtype) : 0.0);"),
    "silu_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "ffn_h_not_activated": ("h[f] = apply_act(z, act);", "h[f] = z;"),
    "gated_up_not_biased": ("u += dec(b1[F + f], dtype);", "u += 0.0 * dec(b1[F + f], dtype);"),
    "gated_act_of_product": ("h[f] *= u;", "h[f] = apply_act(z * u, act);"),
    "relu_leaky": ("return z < 0.0 ? 0.0 : z;", "return z < 0.0 ? 0.01 * z : z;"),
    "gelu_erf_unscaled": ("return 0.5 * z * (1.0 + erf(z / sqrt(2.0)));",
                          "return 0.5 * z * (1.0 + erf(z));"),
    "f16_exponent_bias": ("v = ldexp(1.0 + (double)f / 1024.0, e - 15);",
                          "v = ldexp(1.0 + (double)f / 1024.0, e - 16);"),
    "bf16_fraction": ("v = ldexp(1.0 + (double)f / 128.0, e - 127);",
                      "v = ldexp(1.0 + (double)f / 256.0, e - 127);"),
}

# Mistakes in the inference-mode folding, caught by its own pins.
FOLD_MUTATIONS = {
    "fold_c1_sign": ("y_out[t] = apply_act(r * (acc - mu * c1[cols[j]]) + c2[cols[j]], act);",
                     "y_out[t] = apply_act(r * (acc + mu * c1[cols[j]]) + c2[cols[j]], act);"),
    "fold_c2_without_bias": ("c2[n] = s2 + (bias ? dec(bias[n], dtype) : 0.0);", "c2[n] = s2;"),
    "fold_gamma_dropped": ("double wf = w * gk;", "double wf = w;"),
    "fold_c1_of_unfolded_w": ("s1 += wf;", "s1 += w;"),
}
# Mistakes in the post-GEMM normalization, caught by its own pins.
POSTNORM_MUTATIONS = {
    "postnorm_uncentred_variance": ("q += (z[n] - mu) * (z[n] - mu);", "q += z[n] * z[n];"),
    "postnorm_rms_of_abs": ("q += z[n] * z[n];", "q += fabs(z[n]);"),
    "postnorm_no_bias": ("z[n] = acc + (bias ? dec(bias[n], dtype) : 0.0);", "z[n] = acc;"),
    "postnorm_gamma_ignored": ("y_out[i * n_cols + j] = (z[n] - mu) * r * g + b;",
                               "y_out[i * n_cols + j] = (z[n] - mu) * r + b;"),
}
PIN_FILE = {name: "test_oracle_pins.py" for name in MUTATIONS}
PIN_FILE.update({name: "test_oracle_fold.py" for name in FOLD_MUTATIONS})
PIN_FILE.update({name: "test_oracle_postnorm.py" for name in POSTNORM_MUTATIONS})
MUTATIONS.update(FOLD_MUTATIONS)
MUTATIONS.update(POSTNORM_MUTATIONS)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC, encoding="utf-8").read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(src.replace(old, new), encoding="utf-8")
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-o",
                    str(lib), str(mutated), "-lm"], check=True)
    env = dict(os.environ, NORM_GEMM_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", PIN_FILE[name])],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode != 0, f"pins did not catch mutation {name}:\n{res.stdout[-2000:]}"
