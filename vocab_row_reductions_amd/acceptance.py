"""Run counters of speculative acceptance, read off a call's outputs on the host.

"speculative-acceptance.md", "Reading the rule off a run" prints one summary
line per speculative run, and "The two acceptance rates are not
interchangeable" defines its three ratios:
  per_position_acceptance = accepted / positions_tested (what the closed forms
                            predict),
  acceptance_rate         = accepted / proposed (moves with block length),
  mean_accepted_len       = accepted / rounds (tokens gained per target pass).
A chain stops at its first rejection, so a round of gamma drafts that accepted
L of them tested min(L + 1, gamma) positions.  "Verifying the gain before
trusting a throughput number" averages sum min(p, q) and sum p*q over the
positions the run actually tested.

These are summaries after the fact; nothing here takes part in the selection.
"""
from __future__ import annotations

import numpy as np


def acceptance_counters(lengths, gamma: int, summin=None, sumprod=None, rule: str = "stochastic") -> dict:
    """lengths: accepted drafts per round ([rounds] ints, -1 for a fail-closed
    round, which is left out); summin, sumprod: [rounds, gamma] closed forms of
    the same rounds, or None."""
    L = np.asarray(lengths, dtype=np.int64).reshape(-1)
    ok = L >= 0
    Lk = L[ok]
    rounds = int(Lk.size)
    proposed = rounds * int(gamma)
    tested_per = np.minimum(Lk + 1, gamma)
    tested = int(tested_per.sum())
    accepted = int(Lk.sum())
    nan = float("nan")
    out = dict(rule=rule, rounds=rounds, proposed=proposed, positions_tested=tested, accepted=accepted,
               per_position_acceptance=accepted / tested if tested else nan,
               acceptance_rate=accepted / proposed if proposed else nan,
               mean_accepted_len=accepted / rounds if rounds else nan)
    mask = np.arange(gamma)[None, :] < tested_per[:, None]
    for name, v in (("closed_form_sum_min", summin), ("closed_form_sum_prod", sumprod)):
        if v is not None:
            a = np.asarray(v, dtype=np.float64).reshape(L.size, gamma)[ok]
            out[name] = float(a[mask].mean()) if tested else nan
    return out


def summary_line(c: dict) -> str:
    """The counters as one line, in the order the page prints them."""
    s = (f"[Speculative acceptance] rule={c['rule']} rounds={c['rounds']} proposed={c['proposed']} "
         f"positions_tested={c['positions_tested']} accepted={c['accepted']} "
         f"per_position_acceptance={c['per_position_acceptance']:.4f} acceptance_rate={c['acceptance_rate']:.4f} "
         f"mean_accepted_len={c['mean_accepted_len']:.4f}")
    if "closed_form_sum_min" in c or "closed_form_sum_prod" in c:
        s += " diagnostic:"
        for k in ("closed_form_sum_min", "closed_form_sum_prod"):
            if k in c:
                s += f" {k}={c[k]:.4f}"
    return s
