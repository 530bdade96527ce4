"""Each plausible slip planted in a copy of the oracle (on the CPU) must fail at
least one pin.  This shows the pins constrain every part of the step: the
order gate -> read -> correct -> query, the sign and weight of the correction,
the row/column role of the gate, the signed gates, the per-token prologue
(practical gates from logits, unit-norm keys and queries) and its backward."""
import pytest

import oracle
import test_oracle_bwd as bwdpins
import test_oracle_pins as pins
import test_oracle_prologue_bwd as ppins

ORIG_GATE = "S[(long)i * dv + j] *= a[i];"
ORIG_READ = "s[j] += S[(long)i * dv + j] * kk[i];"
ORIG_CORR = "S[(long)i * dv + j] += b * kk[i] * (vv[j] - s[j]);"

MUTANTS = {
    # query the state before the update
    "readout_before_update": [("  /* gate: Hbar = Diag(alpha) H */",
                               "  if (out) { for (int j = 0; j < dv; ++j) { out[j] = 0.0; "
                               "for (int i = 0; i < dk; ++i) out[j] += S[(long)i * dv + j] * qq[i]; } }\n"
                               "  /* gate: Hbar = Diag(alpha) H */"),
                              ("  if (out) {\n    for (int j = 0; j < dv; ++j) out[j] = 0.0;",
                               "  if (0) {\n    for (int j = 0; j < dv; ++j) out[j] = 0.0;")],
    # apply the gate after the correction instead of before it
    "gate_after_correction": [(ORIG_GATE, "(void)0;"),
                              ("  /* query the updated state: o = H^T q */",
                               "  for (int i = 0; i < dk; ++i) for (int j = 0; j < dv; ++j) "
                               "S[(long)i * dv + j] *= a[i];\n  /* query the updated state: o = H^T q */")],
    "correction_sign_flipped": [(ORIG_CORR, "S[(long)i * dv + j] -= b * kk[i] * (vv[j] - s[j]);")],
    "beta_dropped": [(ORIG_CORR, "S[(long)i * dv + j] += kk[i] * (vv[j] - s[j]);")],
    "beta_squared": [(ORIG_CORR, "S[(long)i * dv + j] += b * b * kk[i] * (vv[j] - s[j]);")],
    "gate_on_columns": [(ORIG_GATE, "S[(long)i * dv + j] *= a[j % dk];")],
    "gate_sign_dropped": [(ORIG_GATE, "S[(long)i * dv + j] *= fabs(a[i]);")],
    "read_before_gate": [(ORIG_GATE, "(void)0;"),
                         ("  /* correct: H = Hbar + beta k (v - s)^T */",
                          "  for (int i = 0; i < dk; ++i) for (int j = 0; j < dv; ++j) "
                          "S[(long)i * dv + j] *= a[i];\n  /* correct: H = Hbar + beta k (v - s)^T */")],
    "prediction_with_query": [(ORIG_READ, "s[j] += S[(long)i * dv + j] * qq[i];")],
    "value_not_subtracted": [(ORIG_CORR, "S[(long)i * dv + j] += b * kk[i] * vv[j];")],
    "query_reads_gated_state": [("      for (int j = 0; j < dv; ++j) out[j] += S[(long)i * dv + j] * qq[i];",
                                 "      for (int j = 0; j < dv; ++j) out[j] += (S[(long)i * dv + j] - b * kk[i] * "
                                 "(vv[j] - s[j])) * qq[i];")],
    # prologue (practical gates, unit-norm keys and queries)
    "gate_eps_wrong": [("  const double eps = exp(-5.0);", "  const double eps = exp(-4.0);")],
    "gate_tanh_without_half": [("  const double r = tanh(0.5 * a);", "  const double r = tanh(a);")],
    "gate_sign_negative_at_zero": [("  const double s = r >= 0.0 ? 1.0 : -1.0;", "  const double s = r > 0.0 ? 1.0 : -1.0;")],
    "gate_sign_dropped_in_prologue": [("  return s * (eps + (1.0 - eps) * fabs(r));", "  return (eps + (1.0 - eps) * fabs(r));")],
    "beta_not_doubled": [("static double practical_beta(double b) { return 2.0 / (1.0 + exp(-b)); }",
                          "static double practical_beta(double b) { return 1.0 / (1.0 + exp(-b)); }")],
    "beta_logit_sign": [("static double practical_beta(double b) { return 2.0 / (1.0 + exp(-b)); }",
                         "static double practical_beta(double b) { return 2.0 / (1.0 + exp(b)); }")],
    "norm_without_sqrt": [("      const double inv = 1.0 / sqrt(ss + 1e-6);", "      const double inv = 1.0 / (ss + 1e-6);")],
    "norm_flags_swapped": [("  unit_rows(k, dtype, ntok, dk, flags & PRO_NORM_K, kk);",
                            "  unit_rows(k, dtype, ntok, dk, flags & PRO_NORM_Q, kk);")],
    # DeltaProduct_2
    "dp2_gate_dropped": [("    for (long long e = 0; e < (long long)dk * dv; ++e) S[e] *= a;\n  }\n  for (int j = 0; j < 2; ++j) {",
                          "    (void)a;\n  }\n  for (int j = 0; j < 2; ++j) {")],
    "dp2_substep_keys_swapped": [("    for (int i = 0; i < dk; ++i) kk[i] = widen(k, (tok * 2 + j) * dk + i, dtype);",
                                  "    for (int i = 0; i < dk; ++i) kk[i] = widen(k, (tok * 2 + 1 - j) * dk + i, dtype);")],
    "dp2_one_beta": [("    householder_write(S, kk, vv, widen(beta, tok * 2 + j, dtype), w, dk, dv);",
                      "    householder_write(S, kk, vv, widen(beta, tok * 2, dtype), w, dk, dv);")],
    # backward
    "bwd_gate_not_carried": [("            G[(long)i * dv + j] = a[i] * dhb;", "            G[(long)i * dv + j] = dhb;")],
    "bwd_dq_from_previous_state": [("          for (int j = 0; j < dv; ++j) acc += Ht[(long)i * dv + j] * gd[j];",
                                    "          for (int j = 0; j < dv; ++j) acc += Hp[(long)i * dv + j] * gd[j];")],
    "bwd_ds_sign": [("          ds[j] = -b * du[j];", "          ds[j] = b * du[j];")],
    "bwd_dalpha_on_gated_state": [("            ga += dhb * Hp[(long)i * dv + j];", "            ga += dhb * Hb[(long)i * dv + j];")],
    # prologue backward (gate slope with the sign held constant, beta slope, normalisation)
    "pbwd_slope_without_one_minus_r2": [("r > 0.0 ? 0.5 * (1.0 - r * r) : r < 0.0 ? -0.5 * (1.0 - r * r) : 0.0",
                                         "r > 0.0 ? 0.5 : r < 0.0 ? -0.5 : 0.0")],
    "pbwd_sign_not_held": [("  return s * (1.0 - eps) * dabs;", "  return (1.0 - eps) * dabs;")],
    "pbwd_slope_at_kink": [("r > 0.0 ? 0.5 * (1.0 - r * r) : r < 0.0 ? -0.5 * (1.0 - r * r) : 0.0",
                            "r > 0.0 ? 0.5 * (1.0 - r * r) : r < 0.0 ? -0.5 * (1.0 - r * r) : 0.5")],
    "pbwd_beta_slope_halved": [("  return 2.0 * sg * (1.0 - sg);", "  return sg * (1.0 - sg);")],
    "pbwd_norm_radial_term_dropped": [("n * dy[t * dk + i] - n * n * n * widen(x, t * dk + i, dtype) * xdy",
                                       "n * dy[t * dk + i]")],
    "pbwd_norm_radial_power": [("n * dy[t * dk + i] - n * n * n * widen(x, t * dk + i, dtype) * xdy",
                                "n * dy[t * dk + i] - n * widen(x, t * dk + i, dtype) * xdy")],
    # DeltaProduct_2 backward (the adjoint of the token step)
    "dp2bwd_dk2_without_state_term": [
        ("          for (int j = 0; j < dv; ++j) acc += b2 * G[(long)i * dv + j] * e2[j] - Hm[(long)i * dv + j] * de2[j];",
         "          for (int j = 0; j < dv; ++j) acc += b2 * G[(long)i * dv + j] * e2[j];")],
    "dp2bwd_dk1_with_first_write_state": [
        ("          for (int j = 0; j < dv; ++j) acc += b1 * G[(long)i * dv + j] * e1[j] - Hb[(long)i * dv + j] * de1[j];",
         "          for (int j = 0; j < dv; ++j) acc += b1 * G[(long)i * dv + j] * e1[j] - Hm[(long)i * dv + j] * de1[j];")],
    "dp2bwd_dhm_sign": [("          for (int j = 0; j < dv; ++j) G[(long)i * dv + j] -= k2[i] * de2[j];   /* now dHm */",
                         "          for (int j = 0; j < dv; ++j) G[(long)i * dv + j] += k2[i] * de2[j];   /* now dHm */")],
    "dp2bwd_gate_not_carried": [("          G[e] *= a;\n        }\n        if (alpha) dalpha[tok] = ga;",
                                 "        }\n        if (alpha) dalpha[tok] = ga;")],
    "dp2bwd_dalpha_on_gated_state": [("          ga += G[e] * Hp[e];", "          ga += G[e] * Hb[e];")],
    "dp2_value_not_corrected": [("    for (int j = 0; j < dv; ++j) S[(long)i * dv + j] += b * kk[i] * (vv[j] - w[j]);",
                                 "    for (int j = 0; j < dv; ++j) S[(long)i * dv + j] += b * kk[i] * vv[j];")],
}

PIN_CALLS = [
    lambda o: pins.test_worked_trace_decay(o),
    lambda o: pins.test_worked_trace_of_one(o),
    lambda o: pins.test_worked_trace_write(o),
    lambda o: pins.test_two_reflections_make_rotation(o),
    lambda o: pins.test_one_step_modular_counter(o, 3),
    lambda o: pins.test_eq2_planar_transition(o, -0.7, 0.3),
    lambda o: pins.test_eq3_diagonal_as_axis_householders(o),
    lambda o: pins.test_transitions_non_expansive_and_spectrum(o),
    lambda o: pins.test_brute_force_tiny(o, 1),
    lambda o: pins.test_brute_force_tiny(o, 2),
    lambda o: pins.test_exact_retrieval_at_beta_one(o),
    lambda o: pins.test_pure_decay_at_beta_zero(o),
    lambda o: pins.test_gauge_sign_absorption(o),
    lambda o: pins.test_practical_gate_endpoints_and_zero(o),
    lambda o: pins.test_practical_gate_matches_sigmoid_form(o),
    lambda o: pins.test_practical_gate_sign_symmetry_and_range(o),
    lambda o: pins.test_practical_beta(o),
    lambda o: pins.test_unit_norm_keys_and_queries(o),
    lambda o: pins.test_fused_forward_is_the_recurrence_on_prepared_inputs(o),
    lambda o: pins.test_deltaproduct2_tracks_permutations_with_transposition_keys(o),
    lambda o: pins.test_deltaproduct2_transition_is_the_gated_householder_product(o),
    lambda o: pins.test_deltaproduct2_with_one_inactive_substep_is_the_delta_rule(o, 0),
    lambda o: pins.test_deltaproduct2_with_one_inactive_substep_is_the_delta_rule(o, 1),
    lambda o: pins.test_deltaproduct2_decode_continues_the_forward(o),
    lambda o: bwdpins.test_backward_matches_finite_differences(o, "uniform"),
    lambda o: bwdpins.test_backward_of_pure_decay_is_closed_form(o),
    lambda o: ppins.test_prologue_backward_matches_finite_differences(o, 7),
    lambda o: ppins.test_gate_slope_closed_form_and_zero_subgradient(o),
    lambda o: ppins.test_normalisation_backward_is_tangent(o),
    lambda o: ppins.test_fused_backward_matches_finite_differences(o, False),
    lambda o: ppins.test_deltaproduct2_backward_matches_finite_differences(o, True),
    lambda o: ppins.test_deltaproduct2_backward_matches_finite_differences(o, False),
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = oracle.source()
    for old, new in MUTANTS[name]:
        assert old in src, (name, old)
        src = src.replace(old, new, 1)
    mutant = oracle.build_variant(src, str(tmp_path / f"libmut_{name}.so"))
    caught = 0
    for call in PIN_CALLS:
        try:
            call(mutant)
        except AssertionError:
            caught += 1
    assert caught > 0, f"mutant {name} passed every pin"


def test_unmutated_copy_passes(tmp_path):
    """Control: the same harness on an unmodified copy passes every pin."""
    clean = oracle.build_variant(oracle.source(), str(tmp_path / "libclean.so"))
    for call in PIN_CALLS:
        call(clean)
