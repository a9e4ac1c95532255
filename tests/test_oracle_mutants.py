"""The oracle's pins must catch plausible mistakes.

Each case plants one slip in a private copy of the oracle's C source (never in
the tree), rebuilds it in a temporary directory and runs the pin suite against
that copy in a subprocess; the suite has to fail.  This shows the pins are
strong enough that a wrong oracle would not pass them.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "decay_after_add": ("row[n] = decay * row[n] + xs * bt[n];",
                        "row[n] = decay * (row[n] + xs * bt[n]);"),
    "wrong_group_of_head": ("const int g = h / hpg;", "const int g = h % G;"),
    "dropped_skip": ("double yp = acc + (D ? D[h] * xp : 0.0);", "double yp = acc;"),
    "readout_before_update": (
        "for (int n = 0; n < N; ++n) row[n] = decay * row[n] + xs * bt[n];\n"
        "        double acc = 0.0;\n"
        "        for (int n = 0; n < N; ++n) acc += row[n] * ct[n];",
        "double acc = 0.0;\n"
        "        for (int n = 0; n < N; ++n) acc += row[n] * ct[n];\n"
        "        for (int n = 0; n < N; ++n) row[n] = decay * row[n] + xs * bt[n];"),
    "sign_of_A": ("exp(delta * A[h])", "exp(-delta * A[h])"),
    "sign_of_bias": ("+ (dt_bias ? dt_bias[h] : 0.0)", "- (dt_bias ? dt_bias[h] : 0.0)"),
    "B_read_from_C": ("const double* bt = Bm +", "const double* bt = Cm +"),
    "gate_without_z": ("yp = yp * zz / (1.0 + exp(-zz));", "yp = yp / (1.0 + exp(-zz));"),
    "initial_state_transposed": (
        "memcpy(S, h0 + ((size_t)i * H + h) * (size_t)P * N,\n             sizeof(double) * (size_t)P * N);",
        "for (int q = 0; q < P * N; ++q) S[q] = h0[((size_t)i * H + h) * (size_t)P * N + (q % P) * N + q / P];"),
    "clamp_upper_ignored": ("if (delta > dt_max) delta = dt_max;", ""),
    "chunk_end_off_by_one": ("(t - t0) % chunk == chunk - 1", "(t - t0) % chunk == 0"),
    "input_dt_ignored": ("const double xs = input_dt ? delta * xp : xp;", "const double xs = xp;"),
    "input_dt_scales_skip": ("double yp = acc + (D ? D[h] * xp : 0.0);",
                             "double yp = acc + (D ? D[h] * xs : 0.0);"),
}

# slips in the backward (ssd_ref_bwd), caught by tests/test_oracle_bwd_pins.py
BWD_MUTANTS = {
    "bwd_dx_without_skip": ("dxt[p] = f * acc + (D ? D[h] * dy : 0.0);", "dxt[p] = f * acc;"),
    "bwd_input_dt_dx_unscaled": ("dxt[p] = f * acc + (D ? D[h] * dy : 0.0);",
                                 "dxt[p] = acc + (D ? D[h] * dy : 0.0);"),
    "bwd_input_dt_dB_unscaled": ("dbt[n] += grow[n] * (f * xt[p]);", "dbt[n] += grow[n] * xt[p];"),
    "bwd_input_dt_no_step_term": ("(da * A[h] + (input_dt ? din : 0.0)) * gd",
                                  "(da * A[h]) * gd"),
    "bwd_input_dt_recompute_unscaled": (
        "Sn[(size_t)p * N + n] = decay * Sp[(size_t)p * N + n] + (f * xt[p]) * bt[n];",
        "Sn[(size_t)p * N + n] = decay * Sp[(size_t)p * N + n] + xt[p] * bt[n];"),
    "bwd_silu_derivative_sign": ("(sg * (1.0 + zz * (1.0 - sg)))", "(sg * (1.0 - zz * (1.0 - sg)))"),
    "bwd_dB_before_adjoint_update": (
        "grow[n] += dy * ct[n];\n                acc += grow[n] * bt[n];\n                dbt[n] += grow[n] * (f * xt[p]);",
        "dbt[n] += grow[n] * (f * xt[p]);\n                grow[n] += dy * ct[n];\n                acc += grow[n] * bt[n];"),
    "bwd_dC_from_previous_state": ("dct[n] += srow[n] * dy;", "dct[n] += Sp[(size_t)p * N + n] * dy;"),
    "bwd_da_from_current_state": ("da += grow[n] * Sp[(size_t)p * N + n];", "da += grow[n] * srow[n];"),
    "bwd_da_not_decayed": ("da *= decay;", ""),
    "bwd_adjoint_not_decayed": ("for (size_t q = 0; q < PN; ++q) Gs[q] *= decay;", ""),
    "bwd_softplus_derivative": ("double g = dt_softplus ? 1.0 / (1.0 + exp(-u)) : 1.0;",
                                "double g = dt_softplus ? 1.0 / (1.0 + exp(u)) : 1.0;"),
    "bwd_clamp_passes_gradient": ("if (d < dt_min) { d = dt_min; g = 0.0; }", "if (d < dt_min) { d = dt_min; }"),
    "bwd_dA_times_A": ("sA += da * delta;", "sA += da * A[h];"),
    "bwd_bias_not_summed": ("sBias += du;", "sBias = du;"),
    "bwd_gate_uses_y_after_gate": ("dy = dy * zz * sg;", "dy = dy * zz;"),
}


# slips in the complex-A scan (ssd_ref_complex.c), caught by tests/test_oracle_complex_pins.py
COMPLEX_MUTANTS = {
    "complex_C_conjugated": ("cx_mul(ct[2 * n], ct[2 * n + 1], sk[0], sk[1], &pr, &pi);",
                             "cx_mul(ct[2 * n], -ct[2 * n + 1], sk[0], sk[1], &pr, &pi);"),
    "complex_rotation_sign": ("ai = mag * sin(delta * Ai);", "ai = -mag * sin(delta * Ai);"),
    "complex_no_softplus": ("const double delta = cx_softplus(dt[t * H + h]);",
                            "const double delta = dt[t * H + h];"),
    "complex_product_sign": ("*r = ar * br - ai * bi;", "*r = ar * br + ai * bi;"),
    "complex_decay_after_add": ("sk[0] = dr + ur;\n          sk[1] = di + ui;",
                                "sk[0] = ar * (sk[0] + ur) - ai * (sk[1] + ui);\n"
                                "          sk[1] = ar * (sk[1] + ui) + ai * (sk[0] + ur);"),
    "complex_initial_state_untransposed": (
        "const double* src = h0 + ((((size_t)i * H + h) * D + d) * N + n) * 2;",
        "const double* src = h0 + ((((size_t)i * H + h) * N + n) * D + d) * 2;"),
}

# slips in the stored-state forward (oracle/__init__.py), caught by
# tests/test_oracle_state_dtype_pins.py
STATE_MUTANTS = {
    "stored_chunk_states_not_rounded": (
        "Hin, final = state_passing(rnd(S), cs, meta, initial_states)",
        "Hin, final = state_passing(S, cs, meta, initial_states)"),
    "stored_carry_in_not_rounded": ("initial_states=rnd(Hin),", "initial_states=Hin,"),
    "final_state_rounded": ("return FwdResult(y.reshape(x.shape), final, None)",
                            "return FwdResult(y.reshape(x.shape), rnd(final), None)"),
    "bf16_truncated": ("r = ((u + np.uint64(0x7FFF) + keep)", "r = ((u)"),
    "bf16_ties_away": ("r = ((u + np.uint64(0x7FFF) + keep)", "r = ((u + np.uint64(0x8000))"),
}

CASES = [(n, MUTANTS[n], "tests/test_oracle_pins.py", "ssd_ref.c") for n in sorted(MUTANTS)] + \
        [(n, BWD_MUTANTS[n], "tests/test_oracle_bwd_pins.py", "ssd_ref.c")
         for n in sorted(BWD_MUTANTS)] + \
        [(n, COMPLEX_MUTANTS[n], "tests/test_oracle_complex_pins.py", "ssd_ref_complex.c")
         for n in sorted(COMPLEX_MUTANTS)] + \
        [(n, STATE_MUTANTS[n], "tests/test_oracle_state_dtype_pins.py", "__init__.py")
         for n in sorted(STATE_MUTANTS)]


@pytest.mark.slow
@pytest.mark.parametrize("name,mutation,pins,target", CASES, ids=[c[0] for c in CASES])
def test_pins_reject_mutant(name, mutation, pins, target, tmp_path):
    src = open(os.path.join(ROOT, "oracle", target)).read()
    before, after = mutation
    assert before in src, f"mutation site for {name} no longer in the oracle"
    work = tmp_path / "tree"
    shutil.copytree(os.path.join(ROOT, "oracle"), work / "oracle",
                    ignore=shutil.ignore_patterns("*.so", "__pycache__", "*.tmp"))
    shutil.copytree(os.path.join(ROOT, "tests"), work / "tests",
                    ignore=shutil.ignore_patterns("__pycache__"))
    (work / "oracle" / target).write_text(src.replace(before, after))
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                    "-std=c99", str(work / "oracle" / "ssd_ref.c"),
                    str(work / "oracle" / "ssd_ref_complex.c"), "-o",
                    str(work / "oracle" / "libssd_ref.so"), "-lm"], check=True)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        pins], cwd=work, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode != 0, f"pins did not catch mutant {name}:\n{r.stdout[-2000:]}"
    assert "failed" in r.stdout
