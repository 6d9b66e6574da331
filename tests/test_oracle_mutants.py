"""Planted mistakes in a patched copy of the oracle (CPU only) must each be
caught by at least one pin: evidence that the pins constrain the oracle."""
import os
import subprocess

import pytest

import tests.test_oracle_pins as P
import tests.test_oracle_pins_match as M
import tests.test_oracle_pins_chain as C
import tests.test_oracle_pins_filtered as F
import tests.test_oracle_pins_exact as E
from oracle import build as B
from oracle import oracle as O

# (name, exact source text, planted replacement, pins that must catch it)
MUTANTS = [
    ("argmax ties keep the higher index", "if (x > best) {", "if (x >= best) {",
     [P.test_argmax_planted_first_maximum_config1, P.test_argmax_matches_numpy_first_occurrence]),
    ("top-k ties ordered by descending id", "return a < b;", "return a > b;",
     [P.test_topk_matches_lexsort]),
    ("logsumexp drops the factored maximum", "return M + std::log(s);", "return std::log(s);",
     [P.test_lse_closed_forms]),
    ("logsumexp ignores the temperature", "s += std::exp(static_cast<double>(R.at(r, i)) / T - M);",
     "s += std::exp(static_cast<double>(R.at(r, i)) - M);", [P.test_lse_matches_scipy]),
    ("top-p cut on the tempered distribution",
     "Z0 += (e[j] = std::exp(static_cast<double>(R.at(r, cand[j])) - z0));",
     "Z0 += (e[j] = std::exp((static_cast<double>(R.at(r, cand[j])) - z0) / T));",
     [P.test_sample_filter_order_worked_example]),
    ("accept test with p and q transposed", "if (!(lhs <= pt)) {", "if (!(static_cast<double>(u_acc[b * G + i]) * pt <= qt)) {",
     [P.test_mrs_is_lossless_and_hits_the_ceiling, E.mrs_exact_pin]),
    ("residual with the wrong sign", "std::max(p_of(L, x) - q_of(L, x), 0.0)", "std::max(q_of(L, x) - p_of(L, x), 0.0)",
     [P.test_mrs_is_lossless_and_hits_the_ceiling, E.mrs_exact_pin]),
    ("residual draw with the accept test's uniform", "      u = u_res[b * G + L];\n", "      u = u_acc[b * G + L];\n",
     [E.mrs_exact_pin]),
    ("residual taken from p when q exceeds it nowhere", "      if (W <= 0.0)\n", "      if (W <= 1.0)\n",
     [E.mrs_exact_pin]),
    ("coupling sum with max instead of min", "s += std::min(p_of(i, x), q_of(i, x));", "s += std::max(p_of(i, x), q_of(i, x));",
     [P.test_spec_invariants_config4_like]),
    ("bonus draw from the wrong target row", "w[x] = p_of(G, x);", "w[x] = p_of(G - 1, x);",
     [P.test_bonus_draw_comes_from_the_last_target_row]),
    ("excluded ids masked before the finite check",
     "const float x = R.at(r, i);\n      if (is_bad(x)) bad = true;\n      const float v = is_excluded[i] ? neg_inf : x;",
     "const float v = is_excluded[i] ? neg_inf : R.at(r, i);\n      if (is_bad(v)) bad = true;",
     [P.test_argmax_excluding_special_cases]),
    ("excluded set ignored", "const float v = is_excluded[i] ? neg_inf : x;", "const float v = x;",
     [P.test_argmax_excluding_matches_numpy_on_masked_rows, P.test_argmax_excluding_brute_force_subsets]),
    ("draw from the last crossing instead of the first", "if (target < c) {", "if (target < c && j + 1 == w.size()) {",
     [P.test_sample_u_grid_frequencies_and_support]),
    ("sampler-match accepts on a mismatch", "if (i == G || x != draft_tokens[b * G + i]) {",
     "if (i == G || x == draft_tokens[b * G + i]) {",
     [M.test_sampler_match_accepts_at_sum_pq_and_is_lossless, M.test_sampler_match_draws_follow_the_cumulative_sum,
      E.sm_exact_pin]),
    ("sampler-match draws from the draft distribution", "for (int64_t x = 0; x < V; ++x) w[x] = p_of(i, x);",
     "for (int64_t x = 0; x < V; ++x) w[x] = i < G ? q_of(i, x) : p_of(i, x);",
     [M.test_sampler_match_accepts_at_sum_pq_and_is_lossless, E.sm_exact_pin]),
    ("sampler-match emits the drafted token at the mismatch", "      tk[i] = x;\n",
     "      tk[i] = i < G ? draft_tokens[b * G + i] : x;\n",
     [M.test_sampler_match_chi_square_and_power, M.test_sampler_match_draws_follow_the_cumulative_sum]),
    ("sampler-match bonus from the last verify row", "for (int64_t x = 0; x < V; ++x) w[x] = p_of(i, x);",
     "for (int64_t x = 0; x < V; ++x) w[x] = p_of(std::min<int64_t>(i, G - 1), x);",
     [M.test_sampler_match_bonus_comes_from_the_last_target_row]),
    ("sum p q with min", "s += p_of(i, x) * q_of(i, x);", "s += std::min(p_of(i, x), q_of(i, x));",
     [M.test_sumprod_closed_forms]),
    ("typical order reversed", "return score(a) < score(b);", "return score(a) > score(b);",
     [C.test_worked_example]),
    ("top-n-sigma with the sample standard deviation", "std::sqrt(var / n)", "std::sqrt(var / (n - 1.0))",
     [C.test_top_n_sigma_matches_numpy_std]),
    ("top-p kept in typical order", "      std::sort(cand.begin(), cand.end(), by_value);\n", "",
     [C.test_worked_example, C.test_typical_and_top_p_cuts_satisfy_their_definitions]),
    ("min-p in tempered units", "const double thr = cmax + std::log(static_cast<double>(min_p));",
     "const double thr = cmax + T * std::log(static_cast<double>(min_p));",
     [C.test_worked_example, C.test_min_p_matches_a_numpy_mask]),
    ("filtered p not renormalised over the kept ids", "d.lse = M + std::log(s);", "d.lse = lse_row(R, r, V, T);",
     [F.test_filtered_coupling_sums_match_numpy]),
    ("draft rows left unfiltered", "dq[i] = row_dist(Dr, drow0 + i, V, T, top_k, top_p, min_p, &m);",
     "dq[i] = row_dist(Dr, drow0 + i, V, T, 0, 1.0f, 0.0f, &m);", [F.test_filtered_coupling_sums_match_numpy]),
    ("filtered top-p on the tempered distribution",
     "    for (uint32_t x : cand) Z += std::exp(z(x) - zmax);\n    double cum = 0.0;\n"
     "    for (size_t j = 0; j < cand.size(); ++j) {\n      const double prev = cum;\n"
     "      cum += std::exp(z(cand[j]) - zmax) / Z;",
     "    for (uint32_t x : cand) Z += std::exp((z(x) - zmax) / T);\n    double cum = 0.0;\n"
     "    for (size_t j = 0; j < cand.size(); ++j) {\n      const double prev = cum;\n"
     "      cum += std::exp((z(cand[j]) - zmax) / T) / Z;",
     [E.test_filtered_rules_worked_example]),
    ("filtered min-p in tempered units", "const double thr = zmax + std::log(static_cast<double>(min_p));",
     "const double thr = zmax + T * std::log(static_cast<double>(min_p));", [E.test_filtered_rules_worked_example]),
    ("filtered nucleus cut on the tempered distribution", "cum += std::exp(z(cand[j]) - zmax) / Z;",
     "cum += std::exp((z(cand[j]) - zmax) / T) / Z;", [F.test_filtered_coupling_sums_match_numpy]),
]


@pytest.mark.parametrize("name,find,repl,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, find, repl, pins):
    src = open(B.SRC).read()
    assert src.count(find) == 1, f"mutation anchor not unique: {find}"
    mut = tmp_path / "mutant.cpp"
    mut.write_text(src.replace(find, repl))
    so = tmp_path / "libmutant.so"
    subprocess.run(["g++", "-std=c++17", "-O1", "-fPIC", "-shared", "-pthread", str(mut), "-o", str(so)], check=True)
    saved = O._lib
    O._lib = O.load(str(so))
    try:
        caught = 0
        for pin in pins:
            try:
                pin(O)
            except AssertionError:
                caught += 1
        assert caught >= 1, f"no pin caught the planted mistake: {name}"
    finally:
        O._lib = saved
