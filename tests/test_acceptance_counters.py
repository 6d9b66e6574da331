"""The speculative run counters (CPU only), against the summary line the page
prints ("speculative-acceptance.md", "Reading the rule off a run"): 153 rounds
of 4 drafts, 612 proposed, 195 positions tested, 46 accepted, so
per_position_acceptance 46/195 = .2359, acceptance_rate 46/612 = .0752 and
mean_accepted_len 46/153 = .3007."""
import numpy as np

from vocab_row_reductions_amd.acceptance import acceptance_counters, summary_line


def page_run():
    # a set of rounds with those totals: with n rounds that accept all 4
    # drafts, 195 = (46 - 4n) + (153 - n) + 4n, so n = 4; the other 149 rounds
    # accept 30 drafts, one each in 30 of them
    L = np.array([4] * 4 + [1] * 30 + [0] * 119)
    np.random.default_rng(1).shuffle(L)
    return L


def test_counters_reproduce_the_page_run():
    c = acceptance_counters(page_run(), 4)
    assert (c["rounds"], c["proposed"], c["positions_tested"], c["accepted"]) == (153, 612, 195, 46)
    assert round(c["per_position_acceptance"], 4) == 0.2359
    assert round(c["acceptance_rate"], 4) == 0.0752
    assert round(c["mean_accepted_len"], 4) == 0.3007
    line = summary_line(c)
    assert ("rule=stochastic rounds=153 proposed=612 positions_tested=195 accepted=46 "
            "per_position_acceptance=0.2359 acceptance_rate=0.0752 mean_accepted_len=0.3007") in line


def test_rates_differ_by_the_truncated_positions():
    # acceptance_rate is depressed by exactly the positions the chains never tested
    L = page_run()
    c = acceptance_counters(L, 4)
    assert np.isclose(c["acceptance_rate"] * c["proposed"], c["per_position_acceptance"] * c["positions_tested"])
    untested = c["proposed"] - c["positions_tested"]
    assert untested == int(np.sum(4 - np.minimum(L + 1, 4)))


def test_closed_forms_average_over_the_tested_positions():
    L = np.array([0, 2, 3, -1])       # the last round failed closed: left out
    smin = np.array([[.5, 9, 9], [.6, .7, .8], [.1, .2, .3], [9, 9, 9]])
    sprod = smin / 2
    c = acceptance_counters(L, 3, smin, sprod, rule="sampler-match")
    assert c["rounds"] == 3 and c["positions_tested"] == 1 + 3 + 3
    assert np.isclose(c["closed_form_sum_min"], (.5 + .6 + .7 + .8 + .1 + .2 + .3) / 7)
    assert np.isclose(c["closed_form_sum_prod"], c["closed_form_sum_min"] / 2)
    assert "rule=sampler-match" in summary_line(c)
