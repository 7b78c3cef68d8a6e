"""Planted mistakes in the oracle must be caught by its pins.

Each case copies ``oracle/rgdr_oracle.c`` to a temporary folder, replaces one fragment
with a plausible mistake (a dropped term, a wrong sign or index, a wrong operand, an
off-by-one commit, a wrong rounding tie rule), builds that copy with gcc, and runs every
pin against it. At least one pin has to fail. All of this happens on the CPU; the
oracle itself is never modified.
"""
import os
import subprocess

import pytest

import oracle
import pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "rgdr_oracle.c")

MUTANTS = {
    "decay_drops_gk": ("* eg * egk;", "* eg;"),
    "decay_drops_g": ("* eg * egk;", "* egk;"),
    "decay_gk_wrong_index": ("double egk = exp(gkt[i]);", "double egk = exp(gkt[0]);"),
    "delta_wrong_sign": ("u[j] = (vt[j] - kv[j]) * beta[t];", "u[j] = (kv[j] - vt[j]) * beta[t];"),
    "delta_drops_beta": ("u[j] = (vt[j] - kv[j]) * beta[t];", "u[j] = (vt[j] - kv[j]);"),
    "read_uses_query": ("acc += S[(size_t)i * Dv + j] * kt[i];",
                        "acc += S[(size_t)i * Dv + j] * qt[i];"),
    "update_uses_query": ("+ kt[i] * u[j];", "+ qt[i] * u[j];"),
    "output_drops_scale": ("(qt[i] * scale);", "(qt[i]);"),
    "output_uses_key": ("(qt[i] * scale);", "(kt[i] * scale);"),
    "commit_off_by_one": ("if (t + 1 == n)", "if (t == n)"),
    "snapshot_head_major": ("memcpy(snap + (size_t)t * snap_stride,", "memcpy(snap + (size_t)t * nS,"),
    "snapshot_at_commit_only": ("if (snap)\n", "if (snap && t + 1 == n)\n"),
    "padding_not_zeroed": ("out[(size_t)t * Dv + j] = 0.0;", "(void)out;"),
    "gqa_modulo_map": ("int hq = (int)(((long long)h * a->Hq) / a->Hv);", "int hq = h % a->Hq;"),
    "length_not_clamped_low": ("int L = clampi(a->lens[b], 0, T);",
                               "int L = a->lens[b] > T ? T : a->lens[b]; if (L < 0) L = T;"),
    "bf16_tie_to_odd": ("fmod(fl, 2.0) != 0.0", "fmod(fl, 2.0) == 0.0"),
    "bf16_truncates": ("if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0))", "if (0)"),
    "bf16_subnormal_scale": ("x = ldexp((double)m, -133);", "x = ldexp((double)m, -134);"),
    "softplus_wrong_branch": ("return x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x));",
                              "return x > 0.0 ? log1p(exp(-x)) : log1p(exp(x));"),
    "sigmoid_wrong_sign": ("beta[e] = 1.0 / (1.0 + exp(-rd(b, ab_ty, e)));",
                           "beta[e] = 1.0 / (1.0 + exp(rd(b, ab_ty, e)));"),
    "gate_bias_dropped": ("double x = rd(a, ab_ty, e) + (double)dt_bias[h];",
                          "double x = rd(a, ab_ty, e);"),
    "gate_bias_wrong_axis": ("double x = rd(a, ab_ty, e) + (double)dt_bias[h];",
                             "double x = rd(a, ab_ty, e) + (double)dt_bias[r % H];"),
    "f16_exponent_bias": ("x = ldexp((double)(1024 + m), e - 25);",
                          "x = ldexp((double)(1024 + m), e - 24);"),
    "normalize_missing_sqrt": ("double nrm = sqrt(ss);", "double nrm = ss;"),
    "normalize_skips_key": ("l2_normalize(k + (size_t)t * Dk, Dk);", "(void)k;"),
    "normalize_short_vector": ("l2_normalize(q + (size_t)t * Dk, Dk);",
                               "l2_normalize(q + (size_t)t * Dk, Dk - 1);"),
    "normalize_abs_sum": ("ss += x[i] * x[i];", "ss += fabs(x[i]);"),
}


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"fragment for {name} not found"
    mutated = src.replace(old, new, 1)
    c_path = tmp_path / f"{name}.c"
    so_path = tmp_path / f"lib{name}.so"
    c_path.write_text(mutated)
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
                    "-w", "-o", str(so_path), str(c_path), "-lm"], check=True)
    return str(so_path)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(tmp_path, name):
    old, new = MUTANTS[name]
    m = oracle.Oracle(_build_mutant(tmp_path, name, old, new))
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(m)
        except (AssertionError, RuntimeError, ValueError, OverflowError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught mutant {name}"
