"""Pins of the oracle's sampler-match rule and its sum p*q diagnostic
("speculative-acceptance.md", "The rules": sampler-match; "The acceptance
ceiling"; "Verifying the gain before trusting a throughput number").

Each pin checks the oracle against something other than itself: the rule's
closed-form acceptance probability sum_x p(x) q(x) integrated over uniform
grids, losslessness (every emitted token is a draw from p), closed forms of
sum p*q, a library softmax, the draw definition against numpy's cumsum +
searchsorted, a chi-square test of the emitted stream, and the greedy limit.
"""
import json
import os

import numpy as np
import pytest
from scipy.special import softmax

import workloads as W

SENT = 0xFFFFFFFF
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _softmax64(z, T=1.0):
    z = np.asarray(z, np.float64) / T
    e = np.exp(z - z.max())
    return e / e.sum()


def _match_grid(oracle, zt, zd, T, N):
    """Integrate the oracle's sampler-match rule over a uniform grid: drafted
    token t weighted by q(t), the position-0 uniform on an N-point midpoint
    grid.  gamma = 1.  Returns (P(accept), P(first emitted = x))."""
    V = len(zt)
    q = _softmax64(zd, T)
    u0 = ((np.arange(N) + 0.5) / N).astype(np.float32)
    um = np.stack([u0, np.full(N, 0.5, np.float32)], 1)
    target = np.repeat(np.array([zt], np.float32), 2 * N, 0)
    draft = np.repeat(np.array([zd], np.float32), N, 0)
    acc, emit = 0.0, np.zeros(V)
    for t in range(V):
        out = oracle.spec_match(target, draft, np.full(N, t, np.uint32), um, N, 1, T)
        acc += q[t] * (out["len_sm"] == 1).mean()
        emit += q[t] * np.bincount(out["tok_sm"][:, 0], minlength=V) / N
    return acc, emit


def test_sampler_match_accepts_at_sum_pq_and_is_lossless(oracle):
    zt = [0.2, 1.1, -0.5, 0.7, 0.0]
    zd = [1.0, -0.3, 0.4, 0.9, -1.2]
    for T in (1.0, 0.7):
        p, q = _softmax64(zt, T), _softmax64(zd, T)
        acc, emit = _match_grid(oracle, zt, zd, T, N=400)
        assert abs(acc - (p * q).sum()) < 2.0 / 400       # P(accept) = sum p q
        assert np.all(np.abs(emit - p) < 2.0 / 400)        # the emitted token is a draw from p
        assert acc < np.minimum(p, q).sum()                # below the coupling ceiling


def test_sumprod_closed_forms(oracle):
    V = 7
    u = np.zeros(V, np.float32)
    zt = np.array([0.3, -1.0, 2.0, 0.5, 0.0, 1.5, -0.4], np.float32)
    tok = np.zeros(1, np.uint32)
    um = np.full((1, 2), 0.5, np.float32)
    # uniform p and q: 1/V
    out = oracle.spec_match(np.stack([u, u]), u[None], tok, um, 1, 1, 1.0)
    assert abs(out["sumprod"][0, 0] - 1.0 / V) < 1e-14
    # identical rows: sum p^2
    p = _softmax64(zt)
    out = oracle.spec_match(np.stack([zt, zt]), zt[None], tok, um, 1, 1, 1.0)
    assert abs(out["sumprod"][0, 0] - (p ** 2).sum()) < 1e-14
    # one-hot q on d (prompt lookup): sum p q = sum min(p, q) = p(d)
    d = 4
    zd = np.full(V, -np.inf, np.float32)
    zd[d] = 0.0
    out = oracle.spec_match(np.stack([zt, zt]), zd[None], np.array([d], np.uint32), um, 1, 1, 1.0)
    mrs = oracle.spec_accept(np.stack([zt, zt]), zd[None], np.array([d], np.uint32), np.full(1, .5, np.float32),
                             np.full(1, .5, np.float32), np.full(1, .5, np.float32), 1, 1, 1.0)
    assert abs(out["sumprod"][0, 0] - p[d]) < 1e-14
    assert abs(out["sumprod"][0, 0] - mrs["summin"][0, 0]) < 1e-14


def test_sumprod_matches_library_softmax_and_stays_below_sum_min(oracle):
    d = W.speculative_batch(batch=3, gamma=4, vocab=3000, seed=31)
    um = W.uniforms(3 * 5, seed=31).reshape(3, 5)
    out = oracle.spec_match(d["target"], d["draft"], d["tokens"], um, 3, 4, 0.8)
    mrs = oracle.spec_accept(d["target"], d["draft"], d["tokens"], d["u_acc"], d["u_res"], d["u_bon"], 3, 4, 0.8)
    tg = d["target"].reshape(3, 5, -1).astype(np.float64)
    dr = d["draft"].reshape(3, 4, -1).astype(np.float64)
    for b in range(3):
        for i in range(4):
            T = float(np.float32(0.8))  # the oracle takes the temperature as float32
            ref = float(np.dot(softmax(tg[b, i] / T), softmax(dr[b, i] / T)))
            assert abs(out["sumprod"][b, i] - ref) < 1e-12
            assert out["sumprod"][b, i] <= mrs["summin"][b, i]


def test_sampler_match_draws_follow_the_cumulative_sum(oracle):
    """Every tested position's draw is numpy's inverse CDF of p_i in id order
    (the first x with u * sum(p) < cumsum(p)[x]); the chain stops at the first
    mismatch and emits that draw."""
    B, G, V, T = 6, 4, 600, 1.0
    d = W.speculative_batch(batch=B, gamma=G, vocab=V, seed=32)
    # drafts equal to the target's own draws at the first positions, so chains run long
    um = W.uniforms(B * (G + 1), seed=32).reshape(B, G + 1)
    tg = d["target"].reshape(B, G + 1, V)
    tok = d["tokens"].reshape(B, G).copy()
    for b in range(B):
        for i in range(G):
            if (b + i) % 3 != 2:
                p = _softmax64(tg[b, i], T)
                c = np.cumsum(p)
                tok[b, i] = np.searchsorted(c, np.float64(um[b, i]) * c[-1], side="right")
    out = oracle.spec_match(d["target"], d["draft"], tok.reshape(-1), um, B, G, T)
    for b in range(B):
        L = out["len_sm"][b]
        assert 0 <= L <= G
        for i in range(L + 1):
            p = _softmax64(tg[b, i], T)
            c = np.cumsum(p)
            x = np.searchsorted(c, np.float64(um[b, i]) * c[-1], side="right")
            if i < L:
                assert x == tok[b, i] and out["tok_sm"][b, i] == tok[b, i]
            else:
                assert out["tok_sm"][b, i] == x
                assert L == G or x != tok[b, i]
        assert np.all(out["tok_sm"][b, L + 1:] == SENT)
    assert np.any(out["len_sm"] >= 2)


def _chi2(counts, probs):
    n = counts.sum()
    e = probs * n
    return float(((counts - e) ** 2 / e).sum())


def test_sampler_match_chi_square_and_power(oracle):
    g = gold("chi_square.json")
    V = g["dof"] + 1
    n = g["draws"]
    p = np.array([0.4, 0.3, 0.1, 0.1, 0.05, 0.05])
    q = p[::-1].copy()
    zt, zd = np.log(p).astype(np.float32), np.log(q).astype(np.float32)
    pf, qf = _softmax64(zt), _softmax64(zd)
    rng = np.random.default_rng(W.BASE_SEED + 78)
    t = rng.choice(V, size=n, p=qf).astype(np.uint32)
    um = rng.random((n, 2), dtype=np.float32)
    out = oracle.spec_match(np.repeat(zt[None], 2 * n, 0), np.repeat(zd[None], n, 0), t, um, n, 1, 1.0)
    assert _chi2(np.bincount(out["tok_sm"][:, 0], minlength=V), pf) < g["threshold"]
    # power: rules that keep the drafted token, or emit argmax p, on a mismatch
    kept = t
    assert _chi2(np.bincount(kept, minlength=V), pf) > g["threshold"]
    greedy_fix = np.where(out["len_sm"] == 1, t, int(np.argmax(pf)))
    assert _chi2(np.bincount(greedy_fix, minlength=V), pf) > g["threshold"]
    # the measured acceptance sits at sum p q, not at sum min(p, q)
    acc = (out["len_sm"] == 1).mean()
    se = np.sqrt(acc * (1 - acc) / n)
    assert abs(acc - (pf * qf).sum()) < 4 * se
    assert abs(acc - np.minimum(pf, qf).sum()) > 4 * se


def test_sampler_match_temperature_zero_is_argmax_rule(oracle):
    d = W.speculative_batch(batch=5, gamma=3, vocab=300, seed=33)
    um = W.uniforms(5 * 4, seed=33).reshape(5, 4)
    out = oracle.spec_match(d["target"], d["draft"], d["tokens"], um, 5, 3, 0.0)
    aa = oracle.spec_accept(d["target"], d["draft"], d["tokens"], d["u_acc"], d["u_res"], d["u_bon"], 5, 3, 0.0)
    assert np.array_equal(out["len_sm"], aa["len_aa"])
    assert np.array_equal(out["tok_sm"], aa["tok_aa"])
    assert np.array_equal(out["sumprod"], aa["summin"])


def test_sampler_match_fail_closed(oracle):
    d = W.speculative_batch(batch=3, gamma=2, vocab=100, seed=34)
    tgt = d["target"].copy()
    tgt[1 * 3 + 2, 5] = np.inf               # bonus row of sequence 1
    tok = d["tokens"].copy()
    tok[2 * 2] = 1000                        # out-of-range draft in sequence 2
    um = W.uniforms(9, seed=34).reshape(3, 3)
    out = oracle.spec_match(tgt, d["draft"], tok, um, 3, 2, 1.0)
    assert out["len_sm"][0] >= 0 and out["len_sm"][1] == -1 and out["len_sm"][2] == -1
    assert np.all(out["tok_sm"][1:] == SENT) and np.all(np.isnan(out["sumprod"][1:]))


def test_sampler_match_bonus_comes_from_the_last_target_row(oracle):
    # One verify position whose only token has all the mass (the draft always
    # matches), so every chain reaches the bonus row, drawn over a u grid.
    zb = np.array([1.5, -1.0, 0.3, 0.0], np.float32)
    z0 = np.array([-np.inf, 0.0, -np.inf, -np.inf], np.float32)
    N = 4000
    ub = ((np.arange(N) + 0.5) / N).astype(np.float32)
    um = np.stack([np.full(N, 0.5, np.float32), ub], 1)
    target = np.tile(np.stack([z0, zb]), (N, 1))
    out = oracle.spec_match(target, np.repeat(zb[None], N, 0), np.full(N, 1, np.uint32), um, N, 1, 0.8)
    assert np.all(out["len_sm"] == 1) and np.all(out["tok_sm"][:, 0] == 1)
    freq = np.bincount(out["tok_sm"][:, 1], minlength=4) / N
    assert np.all(np.abs(freq - _softmax64(zb, 0.8)) <= 2.0 / N)
