"""Pins of the oracle's ordered sampler chain ("Chapter 21", section 21.7;
"speculative-acceptance.md", "The rules"): top-n-sigma, top-k, typical-p,
top-p and min-p on the untempered distribution, the temperature last.

The chain is checked against a hand-worked example (tests/golden/
sampler_chain.json: kept candidates and their draw order), against numpy for
the threshold filters (np.std for sigma, a plain mask for min-p) through
uniform-grid draw frequencies, against the chain's defining inequalities for
typical-p and top-p on larger rows, and against the plain sampler when the
new filters are off.
"""
import json
import os

import numpy as np
import pytest

import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def grid_draws(oracle, row, T, N, **kw):
    """Tokens the chain draws over an N-point midpoint grid of u."""
    x = np.repeat(np.asarray(row, np.float32)[None], N, 0)
    u = ((np.arange(N) + 0.5) / N).astype(np.float32)
    tok, _, _ = oracle.sample_chain(x, T, u, **kw)
    return tok


def expected_grid(row, kept, T, N):
    """Tokens an inverse-CDF draw over `kept` (in that order) gives on the same grid."""
    z = np.asarray(row, np.float64)
    w = np.exp((z[kept] - z.max()) / T)
    c = np.cumsum(w)
    u = (np.arange(N) + 0.5) / N
    j = np.searchsorted(c, u * c[-1], side="right")
    return np.asarray(kept)[np.minimum(j, len(kept) - 1)]


def test_worked_example(oracle):
    g = gold("sampler_chain.json")
    row = np.log(np.array(g["p"], np.float64)).astype(np.float32)
    for case in g["cases"]:
        for T in (1.0, 0.7):
            got = grid_draws(oracle, row, T, 2000, **case["params"])
            want = expected_grid(row, case["kept"], T, 2000)
            assert np.array_equal(got, want), case["why"]


def test_min_p_matches_a_numpy_mask(oracle):
    rng = np.random.default_rng(W.BASE_SEED + 90)
    for min_p in (0.05, 0.3, 0.9):
        row = rng.normal(0, 1.5, 40).astype(np.float32)
        z = row.astype(np.float64)
        kept = np.nonzero(np.exp(z - z.max()) >= min_p)[0]        # p >= min_p * max p, id order
        got = grid_draws(oracle, row, 0.8, 3000, min_p=min_p)
        assert np.array_equal(got, expected_grid(row, kept, 0.8, 3000))


def test_top_n_sigma_matches_numpy_std(oracle):
    rng = np.random.default_rng(W.BASE_SEED + 91)
    for n in (0.5, 1.0, 2.5):
        row = rng.normal(0, 2.0, 50).astype(np.float32)
        row[7] = -np.inf                                          # masks take no part in sigma
        z = row.astype(np.float64)
        fin = z[np.isfinite(z)]
        kept = np.nonzero(z >= z.max() - n * np.std(fin))[0]     # population std, id order
        got = grid_draws(oracle, row, 1.0, 3000, top_n_sigma=n)
        assert np.array_equal(got, expected_grid(row, kept, 1.0, 3000))


def test_typical_and_top_p_cuts_satisfy_their_definitions(oracle):
    """On larger rows every drawn token lies in the set the definitions give:
    typical-p keeps the lowest-scoring tokens whose mass first reaches
    typical_p; top-p then keeps the most likely of those whose renormalised
    mass first reaches top_p."""
    rng = np.random.default_rng(W.BASE_SEED + 92)
    row = (2.0 * rng.gumbel(size=300)).astype(np.float32)
    z = row.astype(np.float64)
    p = np.exp(z - z.max())
    p /= p.sum()
    H = -(p * np.log(p)).sum()
    order = np.argsort(np.abs(-np.log(p) - H), kind="stable")
    n_typ = int(np.searchsorted(np.cumsum(p[order]), 0.6) + 1)
    typ = order[:n_typ]
    tok = grid_draws(oracle, row, 1.0, 4000, typical_p=0.6)
    assert set(np.unique(tok)) <= set(typ)
    assert len(np.unique(tok)) >= min(len(typ), 5)
    # then top-p over the typical set, re-sorted by value
    by_val = typ[np.lexsort((typ, -z[typ]))]
    q = p[by_val] / p[by_val].sum()
    nuc = by_val[:int(np.searchsorted(np.cumsum(q), 0.5) + 1)]
    tok = grid_draws(oracle, row, 1.0, 4000, typical_p=0.6, top_p=0.5)
    assert np.array_equal(tok, expected_grid(row, nuc, 1.0, 4000))


def test_reduces_to_the_plain_sampler(oracle):
    x, u = W.sampling_rows(rows=16, vocab=3000, seed=93)
    for top_k, top_p in ((20, 0.95), (50, 1.0), (0, 1.0), (7, 0.5)):
        a = oracle.sample(x, 0.7, top_k, top_p, u)
        b = oracle.sample_chain(x, 0.7, u, top_k=top_k, top_p=top_p)
        assert np.array_equal(a[0], b[0])
        assert np.allclose(a[1], b[1], rtol=0, atol=1e-12)


def test_greedy_limits(oracle):
    x, u = W.sampling_rows(rows=8, vocab=500, seed=94)
    am = oracle.argmax(x)[0]
    for kw in (dict(min_p=0.1), dict(typical_p=0.5, top_n_sigma=1.0), dict(top_p=0.3)):
        t0, lp0, _ = oracle.sample_chain(x, 0.0, u, **kw)
        assert np.array_equal(t0, am) and np.all(lp0 == 0.0)
        t1, _, _ = oracle.sample_chain(x, 0.9, u, top_k=1, **kw)
        assert np.array_equal(t1, am)


def test_fail_closed_rows(oracle):
    x, u = W.sampling_rows(rows=3, vocab=200, seed=95)
    x = x.copy()
    x[1, 4] = np.nan
    tok, lp, _ = oracle.sample_chain(x, 0.7, u, min_p=0.1, top_n_sigma=1.0)
    assert tok[1] == 0xFFFFFFFF and np.isnan(lp[1]) and tok[0] != 0xFFFFFFFF
