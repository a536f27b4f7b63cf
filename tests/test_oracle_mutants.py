"""The oracle's pins are discriminative: each plausible mistake planted in a copy
of the C oracle (a dropped term, a wrong sign, index or operand) makes at least
one pin in test_oracle_pins.py fail.  CPU only; the mistakes live in temporary
copies of the oracle, never in the product path."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kda_oracle.c")

# (name, original text, planted mistake)
MUTANTS = [
    ("softplus_sign", "return -softplus(x);", "return softplus(x);"),
    ("safe_gate_arg", "return lb * sigmoid(x);", "return lb * sigmoid(-x);"),
    ("conv_tap_order", "acc += c->conv_w[(int64_t)ch * W + j]", "acc += c->conv_w[(int64_t)ch * W + (W - 1 - j)]"),
    ("silu_dropped", "if (c->act == KDA_ORACLE_ACT_SILU) acc = acc * sigmoid(acc);", ""),
    ("q_norm_uses_k", "const double rq = 1.0 / sqrt(sq + c->eps)", "const double rq = 1.0 / sqrt(sk + c->eps)"),
    ("beta_sign", "sigmoid(c->beta_logit[row * H + h])", "sigmoid(-c->beta_logit[row * H + h])"),
    ("conv_carry_off_by_one", "const int64_t t = len - (W - 1) + r;", "const int64_t t = len - W + r;"),
    ("decay_wrong_axis", "S[i * dv + j] *= a[i];", "S[i * dv + j] *= a[j % dk];"),
    ("update_sign", "u[j] = b * (vt[j] - ktS[j]);", "u[j] = b * (vt[j] + ktS[j]);"),
    ("beta_dropped", "u[j] = b * (vt[j] - ktS[j]);", "u[j] = (vt[j] - ktS[j]);"),
    ("projection_uses_q", "ktS[j] += kt[i] * S[i * dv + j];", "ktS[j] += qt[i] * S[i * dv + j];"),
    ("readout_uses_k", "ot[j] += qt[i] * S[i * dv + j];", "ot[j] += kt[i] * S[i * dv + j];"),
    ("readout_before_update", "    /* o = S^T q */", "    for (int i = 0; i < dk; ++i) for (int j = 0; j < dv; ++j) "
     "S[i * dv + j] -= kt[i] * u[j];\n    /* o = S^T q */"),
    ("chunk_solve_sign", "x -= A[r * C + i] * U[i * dv + j];", "x += A[r * C + i] * U[i * dv + j];"),
    ("chunk_state_decay_dropped", "double acc = exp(G[(L - 1) * dk + d]) * S[d * dv + j];",
     "double acc = S[d * dv + j];"),
    ("chunk_cumsum_dropped", "run += c->g[((c0 + r) * H + h) * dk + d];", "run = c->g[((c0 + r) * H + h) * dk + d];"),
    ("chunk_P_strict", "P[r * C + i] = (i <= r) ? sp : 0.0;", "P[r * C + i] = (i < r) ? sp : 0.0;"),
    ("log_decay_is_g", "memcpy(c->log_a + (row * H + h) * dk, a,", "memcpy(c->log_a + (row * H + h) * dk, gt,"),
    ("log_update_is_v", "memcpy(c->log_u + (row * H + h) * dv, u,", "memcpy(c->log_u + (row * H + h) * dv, vt,"),
    ("rms_sum_not_mean", "sqrt(ss / dv + eps)", "sqrt(ss + eps)"),
    ("out_gate_sign", "sigmoid(z[r * dv + j])", "sigmoid(-z[r * dv + j])"),
]


def _run_mutant(tmpdir, name, orig, repl):
    src = open(SRC).read()
    assert src.count(orig) >= 1, f"mutant {name}: original text not found"
    mut = src.replace(orig, repl, 1)
    c_path = os.path.join(tmpdir, f"{name}.c")
    so_path = os.path.join(tmpdir, f"lib{name}.so")
    with open(c_path, "w") as f:
        f.write(mut)
    subprocess.run(["gcc", "-O1", "-std=c99", "-D_POSIX_C_SOURCE=200809L", "-fPIC", "-shared", "-o", so_path,
                    c_path, "-lm", "-lpthread"], check=True)
    env = dict(os.environ, KDA_ORACLE_LIB=so_path)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")], env=env, cwd=ROOT,
                       capture_output=True, text=True, timeout=600)
    return name, r.returncode


def test_every_planted_mistake_fails_a_pin(tmp_path):
    with ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(lambda m: _run_mutant(str(tmp_path), *m), MUTANTS))
    survivors = [n for n, rc in results if rc == 0]
    assert not survivors, f"mutants not caught by any pin: {survivors}"
    assert all(rc == 1 for _, rc in results), results  # failures, not crashes or collection errors
