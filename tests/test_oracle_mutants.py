"""The oracle's pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of ``oracle/oracle.c`` (on the CPU,
in a temporary directory), builds that copy, and runs the pin tests of
``test_oracle_pins.py`` against it.  At least one pin must fail for every
mutant; the unmodified copy must pass them all.
"""
import importlib.util
import os
import shutil
import subprocess
import sys

import pytest

import test_oracle_pins as pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, original text, mutated text): each a plausible slip.
MUTANTS = [
    ("gae_no_done_mask", "a = done ? delta : delta + gamma * lam * a;",
     "a = delta + gamma * lam * a;"),
    ("gae_sign_of_value", "- vt;\n            int done = flag_at(term, n, t, T) || flag_at(trunc, n, t, T);\n            a =",
     "+ vt;\n            int done = flag_at(term, n, t, T) || flag_at(trunc, n, t, T);\n            a ="),
    ("truncation_wins", "    if (flag_at(term, n, t, T))\n        return 0.0;\n    if (flag_at(trunc, n, t, T))\n        return AT(tv, n, t, T);",
     "    if (flag_at(trunc, n, t, T))\n        return AT(tv, n, t, T);\n    if (flag_at(term, n, t, T))\n        return 0.0;"),
    ("truncation_ignores_bootstrap", "        return AT(tv, n, t, T);\n    return AT(v, n, t + 1, T + 1);",
     "        return AT(v, n, t + 1, T + 1);\n    return AT(v, n, t + 1, T + 1);"),
    ("returns_bootstrap_dropped", "double g = bootstrap != NULL ? bootstrap[n] : 0.0;",
     "double g = 0.0;"),
    ("td_lambda_mix_swapped", "((1.0 - lam) * AT(v, n, t + 1, T + 1) + lam * g)",
     "(lam * AT(v, n, t + 1, T + 1) + (1.0 - lam) * g)"),
    ("vtrace_trace_index_shifted", "double c = lam * fmin(c_bar, ratio);",
     "double c = lam * fmin(c_bar, t + 1 < T ? exp(AT(log_rho, n, t + 1, T)) : ratio);"),
    ("vtrace_lambda_on_rho", "double rho = fmin(rho_bar, ratio);",
     "double rho = lam * fmin(rho_bar, ratio);"),
    ("vtrace_pg_uses_values", "double nvs = term_t ? 0.0 : (done ? AT(tv, n, t, T) : v_next);",
     "double nvs = term_t ? 0.0 : (done ? AT(tv, n, t, T) : AT(v, n, t + 1, T + 1));"),
    ("retrace_trace_index_unshifted",
     "double c_next = lam * fmin(c_bar, exp(AT(log_rho, n, t + 1, T)));",
     "double c_next = lam * fmin(c_bar, exp(AT(log_rho, n, t, T)));"),
    ("retrace_keeps_eq_after_termination",
     "(term_t ? 0.0 : gamma * AT(eq, n, t, T))", "(gamma * AT(eq, n, t, T))"),
    ("retrace_trace_not_cut_at_truncation", "if (!done && t < T - 1) {",
     "if (!term_t && t < T - 1) {"),
    ("forward_reset_on_same_step",
     "            double zt = AT(x, n, t, T) + (prev_done ? 0.0 : gamma * lam * prev);\n"
     "            AT(z, n, t, T) = zt;\n            prev = zt;\n"
     "            prev_done = flag_at(term, n, t, T) || flag_at(trunc, n, t, T);",
     "            prev_done = flag_at(term, n, t, T) || flag_at(trunc, n, t, T);\n"
     "            double zt = AT(x, n, t, T) + (prev_done ? 0.0 : gamma * lam * prev);\n"
     "            AT(z, n, t, T) = zt;\n            prev = zt;"),
    ("forward_trace_ignores_lambda", "(prev_done ? 0.0 : gamma * lam * prev)",
     "(prev_done ? 0.0 : gamma * prev)"),
    ("cumsum_drops_carry_in", "double prev = s_init != NULL ? s_init[n] : 0.0;",
     "double prev = 0.0;"),
    ("cumsum_reset_ignores_truncation",
     "            double st = AT(x, n, t, T) + (prev_done ? 0.0 : prev);\n"
     "            AT(s, n, t, T) = st;\n            prev = st;\n"
     "            prev_done = flag_at(term, n, t, T) || flag_at(trunc, n, t, T);",
     "            double st = AT(x, n, t, T) + (prev_done ? 0.0 : prev);\n"
     "            AT(s, n, t, T) = st;\n            prev = st;\n"
     "            prev_done = flag_at(term, n, t, T);"),
    # window carries and the generic affine scan
    ("gae_carry_in_dropped",
     "double a = carry_in != NULL ? carry_in[n] : 0.0;\n        double a0 = 0.0, da = 1.0;\n"
     "        for (int64_t t = T - 1;",
     "double a = 0.0;\n        double a0 = 0.0, da = 1.0;\n        for (int64_t t = T - 1;"),
    ("gae_map_derivative_ignores_done", "da = done ? 0.0 : gamma * lam * da;",
     "da = gamma * lam * da;"),
    ("td_lambda_carry_out_keeps_value", "put_carry(carry_out, map_out, n, g - v0, g0 - v0, dg);",
     "put_carry(carry_out, map_out, n, g, g0 - v0, dg);"),
    ("vtrace_pg_ignores_carry", "double nvs = term_t ? 0.0 : (done ? AT(tv, n, t, T) : v_next);",
     "double nvs = term_t ? 0.0 : (done ? AT(tv, n, t, T) : v_next0);"),
    ("vtrace_map_trace_unclipped", "dvs_t = gamma * c * dv_next;", "dvs_t = gamma * lam * dv_next;"),
    ("retrace_carry_out_without_trace", "c0 * (qret_next - q0), c0 * (qret_next0 - q0),",
     "(qret_next - q0), c0 * (qret_next0 - q0),"),
    ("retrace_carry_undiscounted", "target += gamma * carry;", "target += carry;"),
    ("returns_map_keeps_truncated_carry",
     "succ = succ0 = AT(tv, n, t, T);\n                dsucc = 0.0;",
     "succ = succ0 = AT(tv, n, t, T);\n                dsucc = dg;"),
    ("eligibility_carry_out_unmasked",
     "        if (prev_done)\n            put_carry(carry_out, map_out, n, 0.0, 0.0, 0.0);\n"
     "        else\n            put_carry", "        put_carry"),
    ("cumsum_carry_out_unmasked", "double keep = prev_done ? 0.0 : 1.0;", "double keep = 1.0;"),
    ("affine_reset_ignored", "double b = flag_at(reset, n, t, T) ? 0.0 : AT(beta, n, t, T);",
     "double b = AT(beta, n, t, T);"),
    ("affine_direction_swapped", "int64_t t = reverse ? T - 1 - i : i;",
     "int64_t t = reverse ? i : T - 1 - i;"),
    ("affine_map_from_carry", "a0 = AT(alpha, n, t, T) + b * a0;", "a0 = AT(alpha, n, t, T) + b * a;"),
    # Retrace and V-trace from policy tables
    ("probs_expectation_from_current_state", "size_t next = here + (size_t)A;",
     "size_t next = here;"),
    ("probs_q_taken_from_next_state", "q_taken[n * T + t] = q[here + (size_t)actions[n * T + t]];",
     "q_taken[n * T + t] = q[next + (size_t)actions[n * T + t]];"),
    ("probs_ratio_inverted", "log_rho[n * T + t] = lp - lm;", "log_rho[n * T + t] = lm - lp;"),
    ("probs_log_prob_used_as_prob", "e += exp(log_pi[next + (size_t)b]) * q[next + (size_t)b];",
     "e += log_pi[next + (size_t)b] * q[next + (size_t)b];"),
    ("probs_truncation_uses_table",
     "if (flag_at(trunc, n, t, T) && !flag_at(term, n, t, T)) {\n                eq[n * T + t]",
     "if (0) {\n                eq[n * T + t]"),
    ("probs_behaviour_from_next_step",
     ": log_mu[((size_t)n * (size_t)T + (size_t)t) * (size_t)A + (size_t)a];",
     ": log_mu[((size_t)n * (size_t)T + (size_t)(t + 1 < T ? t + 1 : t)) * (size_t)A + (size_t)a];"),
    ("probs_taken_behaviour_shifted", "double lm = mu_taken ? log_mu[n * T + t]",
     "double lm = mu_taken ? log_mu[n * T + (t + 1 < T ? t + 1 : t)]"),
    ("vtrace_probs_table_stride",
     "derive_probs(N, T, A, 0, actions, log_pi, log_mu, mu_taken, log_rho) == 0",
     "derive_probs(N, T, A, 1, actions, log_pi, log_mu, mu_taken, log_rho) == 0"),
]

PIN_CASES = [
    (pins.test_returns_constant_reward_closed_form, dict(gamma=0.99)),
    (pins.test_returns_one_hot_and_bootstrap_closed_form, {}),
    (pins.test_returns_no_dones_matches_discounted_sum, {}),
    (pins.test_termination_zeroes_successor_truncation_bootstraps, {}),
    (pins.test_gae_special_cases, {}),
    (pins.test_td_lambda_equals_gae_plus_values, {}),
    (pins.test_vtrace_reductions, {}),
    (pins.test_retrace_reductions, {}),
    (pins.test_oracle_matches_forward_views, dict(seed=21, T=12)),
    (pins.test_trace_index_vtrace_from_t_retrace_from_t_plus_1, {}),
    (pins.test_exhaustive_boundaries_against_forward_views, dict(T=3)),
    (pins.test_no_leak_across_episode_boundary, dict(kind="term")),
    (pins.test_no_leak_across_episode_boundary, dict(kind="trunc")),
    (pins.test_window_bootstrap_counted_once_and_ignored_after_done, {}),
    (pins.test_affine_operator_scan_equals_gae_recurrence_exactly, {}),
    (pins.test_forward_recurrences_without_boundaries_are_library_cumsums, {}),
    (pins.test_forward_boundary_restarts_next_step, {}),
    (pins.test_forward_oracle_matches_forward_sums, dict(seed=82, T=13)),
    (pins.test_forward_exhaustive_boundaries, {}),
    (pins.test_forward_no_leak_bitwise, {}),
] + [(pins.test_window_split_reproduces_one_long_window, dict(kind=k, seed=91))
     for k in pins.CARRY_KINDS] + [
    (pins.test_carry_map_is_the_affine_map_of_the_carry, dict(kind=k)) for k in pins.CARRY_KINDS
] + [(pins.test_carry_map_closed_forms, dict(kind=k)) for k in pins.CARRY_KINDS] + [
    (pins.test_carry_closed_forms_one_step, {}),
    (pins.test_affine_scan_constant_beta_is_a_first_order_iir_filter, dict(reverse=True)),
    (pins.test_affine_scan_constant_beta_is_a_first_order_iir_filter, dict(reverse=False)),
    (pins.test_affine_scan_unit_beta_is_cumsum, {}),
    (pins.test_affine_scan_matches_sum_form, dict(reverse=True, seed=100, T=6)),
    (pins.test_affine_scan_matches_sum_form, dict(reverse=False, seed=100, T=6)),
    (pins.test_affine_scan_exact_in_rationals, {}),
    (pins.test_retrace_probs_is_retrace_of_the_table_quantities, dict(seed=113, A=18)),
    (pins.test_vtrace_probs_is_vtrace_of_the_table_ratio, dict(seed=115, A=6)),
    (pins.test_retrace_probs_single_action_and_greedy_target, {}),
    (pins.test_probs_action_relabeling_is_invariant, {}),
    (pins.test_probs_tables_are_read_only_where_the_definition_reads_them, {}),
    (pins.test_probs_taken_behaviour_entries_equal_the_table_form, {}),
]


def _load_variant(tmp_path, name, src_text):
    pkg = tmp_path / ("oracle_" + name)
    shutil.copytree(os.path.join(ROOT, "oracle"), pkg,
                    ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    (pkg / "oracle.c").write_text(src_text)
    subprocess.run([sys.executable, str(pkg / "build.py")], check=True,
                   stdout=subprocess.DEVNULL)
    spec = importlib.util.spec_from_file_location("oracle_" + name, pkg / "__init__.py",
                                                  submodule_search_locations=[str(pkg)])
    mod = importlib.util.module_from_spec(spec)
    sys.modules[spec.name] = mod
    spec.loader.exec_module(mod)
    return mod


def _failing_pins(monkeypatch, mod):
    monkeypatch.setattr(pins, "oracle", mod)
    failed = []
    for fn, kw in PIN_CASES:
        try:
            fn(**kw)
        except (AssertionError, ValueError):
            failed.append(fn.__name__)
    return failed


def _source():
    with open(os.path.join(ROOT, "oracle", "oracle.c")) as f:
        return f.read()


def test_unmodified_copy_passes_every_pin(tmp_path, monkeypatch):
    mod = _load_variant(tmp_path, "clean", _source())
    assert _failing_pins(monkeypatch, mod) == []


@pytest.mark.parametrize("name,orig,mut", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, monkeypatch, name, orig, mut):
    src = _source()
    assert src.count(orig) == 1, "mutation site for %s not found exactly once" % name
    mod = _load_variant(tmp_path, name, src.replace(orig, mut))
    failed = _failing_pins(monkeypatch, mod)
    assert failed, "no pin caught mutant %s" % name
