"""Planted mistakes in the oracle must fail its pins.

Each mutant is a copy of ``oracle/tri_oracle.c`` with one plausible mistake
(a flipped conjugate or sign, interleaved band pairing, a dropped term, a
wrong weight, a wrong tie-break or fire rule, ...), compiled with gcc into a
temporary directory.  The pins of ``test_oracle_pins.py`` run against it and
at least one must fail.  CPU only; the real oracle is never modified.
"""
import os

import pytest

import oracle
import test_oracle_calib as calib_pins
import test_oracle_curve as curve_pins
import test_oracle_gqa as gqa_pins
import test_oracle_pins as pins
import test_oracle_shared as shared_pins

MUTANTS = {
    "conjugate on the query": ("q * conj(k[f])", "conj(q) * k[f]"),
    "interleaved band pairing": ("K[f] + I * K[f + d / 2]", "K[2 * f] + I * K[2 * f + 1]"),
    "inverse RoPE rotates forward": ("cexp(-I * omega[f] * (double)p)", "cexp(I * omega[f] * (double)p)"),
    "offsets look backwards": ("p_now + offsets[o] - pos[i]", "p_now - offsets[o] - pos[i]"),
    "distance ignores key position": ("p_now + offsets[o] - pos[i]", "p_now + offsets[o]"),
    "norm term dropped": ("score[i] = t + nm", "score[i] = t"),
    "trig term dropped": ("score[i] = t + nm", "score[i] = nm"),
    "norm weighted by R instead of 1-R": ("(1.0 - q_mrl[f]) * q_mean_norm[f] * cabs(k[f])",
                                          "q_mrl[f] * q_mean_norm[f] * cabs(k[f])"),
    "norm not weighted by mean query norm": ("(1.0 - q_mrl[f]) * q_mean_norm[f] * cabs(k[f])",
                                             "(1.0 - q_mrl[f]) * cabs(k[f])"),
    "sum over offsets instead of mean": ("trig_sum / (double)n_off", "trig_sum"),
    "omega with d in place of d/2 pairing": ("-2.0 * (double)f / (double)d", "-1.0 * (double)f / (double)d"),
    "ties go to the later position": ("if (a->p != b->p) return a->p < b->p ? -1 : 1;",
                                      "if (a->p != b->p) return a->p < b->p ? 1 : -1;"),
    "ties by slot instead of position": ("if (a->p != b->p) return a->p < b->p ? -1 : 1;", ""),
    "NaN ranks highest": ("const ranked* b = (const ranked*)b_;\n    int an = isnan(a->s), bn = isnan(b->s);\n    if (an != bn) return an ? 1 : -1;",
                          "const ranked* b = (const ranked*)b_;\n    int an = isnan(a->s), bn = isnan(b->s);\n    if (an != bn) return an ? -1 : 1;"),
    "keeps the lowest scores": ("if (an != bn) return an ? 1 : -1;\n    if (!an) {\n        if (a->s > b->s) return -1;\n        if (a->s < b->s) return 1;\n    }\n    if (a->p != b->p)",
                                "if (an != bn) return an ? 1 : -1;\n    if (!an) {\n        if (a->s > b->s) return 1;\n        if (a->s < b->s) return -1;\n    }\n    if (a->p != b->p)"),
    "fire rule off by one": ("if ((int64_t)n <= (int64_t)budget + (int64_t)window) return 0;",
                             "if ((int64_t)n < (int64_t)budget + (int64_t)window) return 0;"),
    "kept list left in rank order": ("qsort(kept, (size_t)budget, sizeof(int32_t), by_int32);", ""),
    "gather copies the wrong row": ("s + (size_t)kept[r] * (size_t)row_bytes", "s + (size_t)r * (size_t)row_bytes"),
    "GQA sample instead of population deviation": ("sqrt(sq / (double)count)",
                                                   "sqrt(sq / (double)(count > 1 ? count - 1 : 1))"),
    "GQA min instead of max over the group": ("z > score[i]", "z < score[i]"),
    "GQA rows not centred": ("(s[i] - mean) / sd", "s[i] / sd"),
    "GQA every query head uses the first table": (
        "qc_re + (size_t)g * half, qc_im + (size_t)g * half,\n                              q_mean_norm + (size_t)g * half, q_mrl + (size_t)g * half",
        "qc_re, qc_im,\n                              q_mean_norm, q_mrl"),
    "GQA constant row gives NaN": ("z = flat ? 0.0 : (s[i] - mean) / sd", "z = (s[i] - mean) / sd"),
    "calibration R not divided by the mean norm": ("mrl[f] = m > 0.0 ? cabs(centre) / m : 0.0;",
                                                   "mrl[f] = cabs(centre);"),
    "calibration interleaved band pairing": (
        "Q[(size_t)t * d + f] + I * Q[(size_t)t * d + f + half]",
        "Q[(size_t)t * d + 2 * f] + I * Q[(size_t)t * d + 2 * f + 1]"),
    "calibration sum instead of mean": ("const double complex centre = sum / (double)n;",
                                        "const double complex centre = sum;"),
    "calibration norm of the mean instead of the mean norm": (
        "const double m = norm_sum / (double)n;", "const double m = cabs(sum) / (double)n;"),
    "curve conjugates the query instead of the key": (
        "s += creal(q * conj(k) * cexp(I * omega[f] * (double)deltas[j]));",
        "s += creal(conj(q) * k * cexp(I * omega[f] * (double)deltas[j]));"),
    "curve ignores the distance": ("s += creal(q * conj(k) * cexp(I * omega[f] * (double)deltas[j]));",
                                   "s += creal(q * conj(k));"),
    "linear offsets truncated": ("(double)max_distance * (double)k / (double)count + 0.5)",
                                 "(double)max_distance * (double)k / (double)count)"),
    "geometric offsets by four": ("for (int64_t x = 1; x <= max_distance; x *= 2) {",
                                  "for (int64_t x = 1; x <= max_distance; x *= 4) {"),
    "shared budget ranks NaN highest": ("if (an != bn) return an ? 1 : -1;   /* NaN below every number */",
                                        "if (an != bn) return an ? -1 : 1;"),
    "shared budget ties to the later position": ("if (a->p != b->p) return (a->p < b->p) ? -1 : 1;",
                                                 "if (a->p != b->p) return (a->p < b->p) ? 1 : -1;"),
    "shared budget ignores the floor": ("r[m].reserved = j < floor_;", "r[m].reserved = 0;"),
    "shared budget ties to the higher head": ("if (a->head != b->head) return a->head < b->head ? -1 : 1;",
                                              "if (a->head != b->head) return a->head < b->head ? 1 : -1;"),
    "shared budget reserves the worst keys": ("r[m].reserved = j < floor_;", "r[m].reserved = j >= n[h] - floor_;"),
    "shared budget fire rule without the window": (
        "if (all <= (int64_t)total + (int64_t)n_head * window) return 0;",
        "if (all <= (int64_t)total) return 0;"),
    "shared budget kept lists unsorted": (
        "qsort(kept + (size_t)h * total, (size_t)count[h], sizeof(int32_t), by_int32);", ";"),
    "non-finite keys keep their literal score": ("        if (!finite_row) {\n", "        if (0) {\n"),
    "bound drops |A_f|": ("cabs(qc_re[f] + I * qc_im[f]) * cabs(a)", "cabs(qc_re[f] + I * qc_im[f])"),
    "bound drops the norm weight": ("                + (1.0 - q_mrl[f]) * q_mean_norm[f];", "                ;"),
    "bound doubled": ("        bound[i] = m;", "        bound[i] = 2.0 * m;"),
    "bound takes the mean norm as the trig coefficient": (
        "cabs(qc_re[f] + I * qc_im[f]) * cabs(a)", "q_mean_norm[f] * cabs(a)"),
    "GQA statistics include non-finite scores": (
        "if (isfinite(s[i])) { sum += s[i]; ++count; if (fabs(s[i]) > big) big = fabs(s[i]); }",
        "{ sum += s[i]; ++count; if (fabs(s[i]) > big) big = fabs(s[i]); }"),
}


def _pin_calls():
    calls = [
        (pins.test_omega_matches_standard_rope, {}),
        (pins.test_unrotate_inverts_a_dense_rotation, {"d": 64}),
        (pins.test_unrotate_composes_and_preserves_band_norms, {}),
        (pins.test_trig_equals_bruteforce_rope_dot_products, {"d": 8, "n": 40, "theta": 10.0}),
        (pins.test_trig_equals_bruteforce_rope_dot_products, {"d": 64, "n": 64, "theta": 1e4}),
        (pins.test_single_offset_is_the_rope_attention_logit, {}),
        (pins.test_key_equal_to_centre_at_zero_distance_gives_squared_norm, {}),
        (pins.test_zero_query_centre_gives_zero_trig, {}),
        (pins.test_polar_per_band_form, {}),
        (pins.test_trig_swapping_query_and_key_roles_is_detected, {}),
        (pins.test_norm_term_special_cases_and_direct_sum, {}),
        (pins.test_norm_term_is_position_invariant, {}),
        (pins.test_score_is_sum_and_bounded, {}),
        (pins.test_folded_form_agrees, {}),
        (pins.test_bound_adds_over_bands, {}),
        (pins.test_nonfinite_keys_score_nan_and_are_evicted, {}),
        (pins.test_select_matches_numpy_lexsort, {}),
        (pins.test_select_invariants_and_fire_rule, {}),
        (pins.test_gather_matches_numpy_take_and_identity, {}),
    ]
    for i in range(len(pins._bound_golden()["examples"])):
        calls.append((pins.test_golden_bound_examples, {"i": i}))
    for seed in range(6):
        calls.append((pins.test_bound_is_the_largest_score_over_key_phases, {"seed": seed}))
    for ex in pins._golden()["score_examples"]:
        calls.append((pins.test_golden_score_examples, {"ex": ex}))
    for i in range(len(pins._golden()["select_examples"])):
        calls.append((pins.test_golden_select_examples, {"i": i}))
    for seed in range(12):
        calls.append((pins.test_select_equals_bruteforce_subset_search, {"seed": seed}))
    for i in range(len(gqa_pins._golden()["examples"])):
        calls.append((gqa_pins.test_gqa_golden_examples, {"i": i}))
    calls += [
        (curve_pins.test_curve_is_the_rope_logit_of_the_centres, {}),
        (curve_pins.test_curve_at_zero_distance_is_the_dot_product_and_hand_example, {}),
        (curve_pins.test_score_trig_term_of_a_key_at_the_centre_averages_the_curve, {}),
        (curve_pins.test_offset_sets, {}),
    ]
    for i in range(len(shared_pins._golden()["examples"])):
        calls.append((shared_pins.test_shared_golden_examples, {"i": i}))
    calls += [(shared_pins.test_floor_equal_to_budget_is_the_per_head_top_b, {}),
              (shared_pins.test_one_head_is_the_plain_top_b, {})]
    for seed in range(10):
        calls.append((shared_pins.test_shared_selection_properties, {"seed": seed}))
    for i in range(len(calib_pins._golden()["examples"])):
        calls.append((calib_pins.test_calib_golden_examples, {"i": i}))
    calls += [
        (calib_pins.test_calib_equal_and_opposite_samples, {}),
        (calib_pins.test_calib_recovers_a_known_concentration, {}),
        (calib_pins.test_calib_scale_and_rotation, {}),
    ]
    calls += [
        (gqa_pins.test_gqa_z_rows_have_zero_mean_and_unit_population_variance, {}),
        (gqa_pins.test_gqa_score_is_free_of_each_query_heads_scale, {}),
        (gqa_pins.test_gqa_single_query_head_keeps_the_plain_top_b, {}),
        (gqa_pins.test_gqa_equal_scores_give_zero, {}),
        (gqa_pins.test_gqa_nonfinite_key_is_left_out_of_the_statistics, {}),
        (gqa_pins.test_gqa_max_over_the_group_of_separately_normalized_heads, {}),
    ]
    return calls


def test_pins_pass_on_the_real_oracle():
    lib = oracle.load()
    for fn, kw in _pin_calls():
        fn(lib, **kw)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_pin(name, tmp_path):
    old, new = MUTANTS[name]
    with open(oracle.SOURCE) as f:
        src = f.read()
    assert src.count(old) == 1, "mutation site not found: %r" % old
    mutant_c = os.path.join(tmp_path, "mutant.c")
    with open(mutant_c, "w") as f:
        f.write(src.replace(old, new))
    lib = oracle.Oracle(oracle.compile_c(mutant_c, os.path.join(tmp_path, "libmutant.so")))
    failed = []
    for fn, kw in _pin_calls():
        try:
            fn(lib, **kw)
        except (AssertionError, ValueError, IndexError, TypeError):
            failed.append(fn.__name__)
    assert failed, "mutant '%s' passed every pin" % name
