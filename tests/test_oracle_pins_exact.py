"""Exact-rational pins of the oracle's speculative acceptance (CPU only).

Modified rejection sampling ("speculative-acceptance.md", "Modified rejection
sampling") and sampler-match ("The rules", "The acceptance ceiling") are
checked on vocabularies of 2 to 6 tokens against their exact structure:

* p and q are computed here, independently of the oracle, to 200 bits with
  mpmath from the float32 logits and held as Fractions.
* Every decision boundary the rule implies -- u = p(t)/q(t) for the accept
  test, the cumulative sums of normalize(relu(p - q)) for the residual draw
  and of p for the bonus and fresh draws (id order) -- is probed with the
  float32 uniforms on either side of it, 1e-12 away or more.  The oracle must
  take the decision the exact rule takes on each side.
* With the boundaries in place, the oracle's decision regions have exact
  rational measure.  Summed and weighted by q(t), they give P(accept) =
  sum min(p, q) (MRS) or sum p*q (sampler-match) and P(emit = x) = p(x),
  as exact Fractions: min(q, p) + relu(p - q) = p, pointwise.  The oracle's
  own float64 sums must equal those Fractions to 1e-13.

A hand-worked example of the filtered rules (tests/golden/filtered_rules.json:
top-k, then top-p and min-p on the untempered row, then the temperature) pins
the filtered p and q the same way.
"""
import json
import os
from fractions import Fraction

import mpmath as mp
import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
MARGIN = Fraction(1, 10 ** 12)
mp.mp.prec = 200


def frac(x) -> Fraction:
    m, e = mp.mpf(x).man_exp
    return Fraction(m) * Fraction(2) ** e


def exact_softmax(z, T):
    """softmax(z / T) of float32 logits z (T a float32), to 200 bits, as Fractions;
    -inf logits get 0."""
    t = mp.mpf(float(np.float32(T)))
    zs = [mp.mpf(float(v)) / t if np.isfinite(v) else None for v in np.asarray(z, np.float32)]
    m = max(v for v in zs if v is not None)
    e = [frac(mp.exp(v - m)) if v is not None else Fraction(0) for v in zs]
    s = sum(e)
    return [v / s for v in e]  # normalised exactly: the Fractions sum to 1


def below(b: Fraction):
    """The largest float32 u with u <= b - MARGIN (None if there is none in [0, 1))."""
    if b - MARGIN < 0:
        return None
    x = np.float32(float(b))
    while Fraction(float(x)) > b - MARGIN:
        x = np.nextafter(x, np.float32(-1))
    return x if x >= 0 else None


def above(b: Fraction):
    """The smallest float32 u with u >= b + MARGIN and u < 1 (None if there is none)."""
    x = np.float32(float(b))
    while Fraction(float(x)) < b + MARGIN:
        x = np.nextafter(x, np.float32(2))
    return x if x < 1 else None


def cdf(w):
    """Cumulative sums of w / sum(w) in id order (Fractions)."""
    W = sum(w)
    out, c = [], Fraction(0)
    for x in w:
        c += x
        out.append(c / W)
    return out


def draw_probes(w):
    """(u, expected token) pairs just inside both ends of every interval of the
    id-order inverse CDF of weights w: the first x with u * W < w_0 + ... + w_x."""
    probes = []
    lo = Fraction(0)
    for x, hi in enumerate(cdf(w)):
        if w[x] > 0 and hi - lo > 4 * MARGIN:
            for u in (above(lo) if lo > 0 else np.float32(0), below(hi)):
                if u is not None and Fraction(float(u)) >= lo and Fraction(float(u)) < hi:
                    probes.append((u, x))
        lo = hi
    return probes


def row_pairs():
    """Seeded float32 target, bonus and draft rows of 2 to 6 tokens."""
    rng = np.random.default_rng(20261203)
    cases = []
    for V in (2, 3, 4, 5, 6):
        for _ in range(3):
            zt = (rng.standard_normal(V) * 1.5).astype(np.float32)
            zb = (rng.standard_normal(V) * 1.5).astype(np.float32)
            zd = (zt + rng.standard_normal(V)).astype(np.float32)
            cases.append((zt, zb, zd))
    return cases


def run_mrs(oracle, zt, zb, zd, T, probes, **filters):
    """Run the oracle once over one sequence per probe (gamma = 1).
    probes: list of (t, u_acc, u_res, u_bon)."""
    B, V = len(probes), len(zt)
    target = np.empty((2 * B, V), np.float32)
    target[0::2] = zt
    target[1::2] = zb
    draft = np.repeat(np.asarray(zd, np.float32)[None], B, 0)
    t = np.array([p[0] for p in probes], np.uint32)
    ua = np.array([p[1] for p in probes], np.float32)
    ur = np.array([p[2] for p in probes], np.float32)
    ub = np.array([p[3] for p in probes], np.float32)
    return oracle.spec_accept(target, draft, t, ua, ur, ub, B, 1, T, **filters)


def run_sm(oracle, zt, zb, zd, T, probes, **filters):
    """probes: list of (t, u_match, u_bonus)."""
    B, V = len(probes), len(zt)
    target = np.empty((2 * B, V), np.float32)
    target[0::2] = zt
    target[1::2] = zb
    draft = np.repeat(np.asarray(zd, np.float32)[None], B, 0)
    t = np.array([p[0] for p in probes], np.uint32)
    um = np.array([[p[1], p[2]] for p in probes], np.float32)
    return oracle.spec_match(target, draft, t, um, B, 1, T, **filters)


def check_mrs(oracle, zt, zb, zd, T, p, pb, q, **filters):
    """Probe every boundary of modified rejection sampling with exact p, q (bonus
    row pb), then check the exact measures.  Returns the number of probes."""
    V = len(p)
    r = [max(p[x] - q[x], Fraction(0)) for x in range(V)]
    R = sum(r)
    resid = r if R > 0 else p
    res_probes = draw_probes(resid)
    bon_probes = draw_probes(pb)
    probes, expect = [], []
    for t in range(V):
        if q[t] == 0:
            continue
        b = p[t] / q[t]
        acc_u = [(np.float32(0), True)]
        if b < 1:
            for u, ok in ((below(b), True), (above(b), False)):
                if u is not None:
                    acc_u.append((u, ok))
        else:
            acc_u.append((np.float32(np.nextafter(np.float32(1), np.float32(0))), True))
        for u, ok in acc_u:
            if ok:
                for ub, x in bon_probes:
                    probes.append((t, u, np.float32(0.5), ub))
                    expect.append((1, t, x))
            else:
                for ur, x in res_probes:
                    probes.append((t, u, ur, np.float32(0.5)))
                    expect.append((0, x, None))
    out = run_mrs(oracle, zt, zb, zd, T, probes, **filters)
    for j, (L, first, second) in enumerate(expect):
        got = (int(out["len_mrs"][j]), int(out["tok_mrs"][j, 0]))
        assert got == (L, first), (probes[j], got, (L, first))
        if second is not None:
            assert int(out["tok_mrs"][j, 1]) == second, (probes[j], out["tok_mrs"][j])
    # exact measures of the decision regions the probes fixed
    acc = sum((q[t] * min(Fraction(1), p[t] / q[t]) for t in range(V) if q[t] > 0), Fraction(0))
    summin = sum((min(p[x], q[x]) for x in range(V)), Fraction(0))
    assert acc == summin
    rej = 1 - acc
    for x in range(V):
        emit = (q[x] * min(Fraction(1), p[x] / q[x]) if q[x] > 0 else 0) + rej * resid[x] / sum(resid)
        assert emit == p[x], (x, emit, p[x])
    assert np.allclose(out["summin"][:, 0], float(summin), rtol=0, atol=1e-13)
    return len(probes)


def check_sm(oracle, zt, zb, zd, T, p, pb, q, **filters):
    V = len(p)
    fresh = draw_probes(p)
    bon = draw_probes(pb)
    probes, expect = [], []
    for t in range(V):
        for u, x in fresh:
            if x == t:
                for ub, xb in bon:
                    probes.append((t, u, ub))
                    expect.append((1, t, xb))
            else:
                probes.append((t, u, np.float32(0.5)))
                expect.append((0, x, None))
    out = run_sm(oracle, zt, zb, zd, T, probes, **filters)
    for j, (L, first, second) in enumerate(expect):
        got = (int(out["len_sm"][j]), int(out["tok_sm"][j, 0]))
        assert got == (L, first), (probes[j], got, (L, first))
        if second is not None:
            assert int(out["tok_sm"][j, 1]) == second
    # the fresh draw lands on t with exact probability p(t): accept = sum q p
    sumprod = sum((p[x] * q[x] for x in range(V)), Fraction(0))
    assert sum((q[t] * p[t] for t in range(V)), Fraction(0)) == sumprod
    assert np.allclose(out["sumprod"][:, 0], float(sumprod), rtol=0, atol=1e-13)
    return len(probes)


def mrs_exact(oracle, T):
    n = 0
    for zt, zb, zd in row_pairs():
        p, pb, q = exact_softmax(zt, T), exact_softmax(zb, T), exact_softmax(zd, T)
        n += check_mrs(oracle, zt, zb, zd, T, p, pb, q)
    assert n > 500


def sm_exact(oracle, T):
    n = 0
    for zt, zb, zd in row_pairs():
        p, pb, q = exact_softmax(zt, T), exact_softmax(zb, T), exact_softmax(zd, T)
        n += check_sm(oracle, zt, zb, zd, T, p, pb, q)
    assert n > 300


@pytest.mark.parametrize("T", [1.0, 0.6])
def test_mrs_boundaries_and_exact_acceptance(oracle, T):
    mrs_exact(oracle, T)


@pytest.mark.parametrize("T", [1.0, 0.6])
def test_sampler_match_boundaries_and_exact_acceptance(oracle, T):
    sm_exact(oracle, T)


def mrs_exact_pin(oracle):
    """Both temperatures (for the planted-mistake checks)."""
    for T in (1.0, 0.6):
        mrs_exact(oracle, T)


def sm_exact_pin(oracle):
    for T in (1.0, 0.6):
        sm_exact(oracle, T)


def test_mrs_second_position_only_after_the_first_accepts(oracle):
    # gamma = 2: position 1 is tested only when position 0 accepted; u_acc = 0
    # always accepts, a u above p/q at position 0 always rejects there
    zt = np.array([0.5, -0.2, 1.0], np.float32)
    zd = np.array([1.2, -0.5, 0.1], np.float32)
    p, q = exact_softmax(zt, 1.0), exact_softmax(zd, 1.0)
    t0 = 0                       # q(0) > p(0): rejectable
    b = p[t0] / q[t0]
    assert b < 1
    target = np.tile(zt, (6, 1))
    draft = np.tile(zd, (4, 1))
    toks = np.array([t0, 2, t0, 2], np.uint32)
    ua = np.array([0, 0, above(b), 0], np.float32)
    out = oracle.spec_accept(target, draft, toks, ua, np.full(4, .5, np.float32), np.full(2, .5, np.float32),
                             2, 2, 1.0)
    assert list(out["len_mrs"]) == [2, 0]
    assert list(out["tok_mrs"][0, :2]) == [t0, 2]


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_filtered_rules_worked_example(oracle):
    g = gold("filtered_rules.json")
    T, filt = g["temperature"], dict(top_k=g["top_k"], top_p=g["top_p"], min_p=g["min_p"])
    zt = np.log(np.array(g["target_weights"], np.float64)).astype(np.float32)
    zd = np.log(np.array(g["draft_weights"], np.float64)).astype(np.float32)
    p = [Fraction(s) for s in g["p"]]
    q = [Fraction(s) for s in g["q"]]
    assert sum(p) == 1 and sum(q) == 1
    assert [x for x in range(5) if p[x] > 0] == g["kept_target"]
    assert [x for x in range(5) if q[x] > 0] == g["kept_draft"]
    assert sum(min(a, b) for a, b in zip(p, q)) == Fraction(g["summin"])
    assert sum(a * b for a, b in zip(p, q)) == Fraction(g["sumprod"])
    # the oracle's sums on the float32 logits (ln of the weights, rounded)
    B = 2
    target = np.tile(zt, (2 * B, 1))
    draft = np.tile(zd, (B, 1))
    toks = np.array([1, 3], np.uint32)
    half = np.full(B, .5, np.float32)
    out = oracle.spec_accept(target, draft, toks, half, half, half, B, 1, T, **filt)
    assert np.allclose(out["summin"], float(Fraction(g["summin"])), rtol=0, atol=1e-6)
    sm = oracle.spec_match(target, draft, toks, np.full((B, 2), .5, np.float32), B, 1, T, **filt)
    assert np.allclose(sm["sumprod"], float(Fraction(g["sumprod"])), rtol=0, atol=1e-6)
    # the decision boundaries of the worked example, probed either side
    assert Fraction(g["mrs"]["accept_below"]["1"]) == p[1] / q[1]
    assert [Fraction(s) for s in g["mrs"]["residual"]] == [max(a - b, 0) / Fraction(17, 21) for a, b in zip(p, q)]
    assert [Fraction(s) for s in g["bonus_cdf"]] == [c for c, w in zip(cdf(p), p) if w > 0]
    # probes 1e-6 from each boundary: the float32 logits move them by ~1e-7
    eps = 1e-6
    cases = [  # (t, u_acc, u_res, u_bon) -> (len, first token, second token)
        ((1, 5 / 21 - eps, .5, .1), (1, 1, 0)),
        ((1, 5 / 21 - eps, .5, 16 / 21 + eps), (1, 1, 1)),
        ((1, 5 / 21 - eps, .5, 20 / 21 + eps), (1, 1, 2)),
        ((1, 5 / 21 + eps, 16 / 17 - eps, .5), (0, 0, None)),
        ((1, 5 / 21 + eps, 16 / 17 + eps, .5), (0, 2, None)),
        ((3, eps, .3, .5), (0, 0, None)),
        ((3, .9, .99, .5), (0, 2, None)),
    ]
    Bc = len(cases)
    out = oracle.spec_accept(np.tile(zt, (2 * Bc, 1)), np.tile(zd, (Bc, 1)),
                             np.array([c[0][0] for c in cases], np.uint32),
                             np.array([c[0][1] for c in cases], np.float32),
                             np.array([c[0][2] for c in cases], np.float32),
                             np.array([c[0][3] for c in cases], np.float32), Bc, 1, T, **filt)
    for j, (_, (L, a, b)) in enumerate(cases):
        assert out["len_mrs"][j] == L and out["tok_mrs"][j, 0] == a, (cases[j], out["tok_mrs"][j])
        if b is not None:
            assert out["tok_mrs"][j, 1] == b
    sm_cases = [((1, 16 / 21 - eps, .5), (0, 0)), ((1, 16 / 21 + eps, .3), (1, 1)),
                ((1, 20 / 21 + eps, .5), (0, 2)), ((3, .97, .5), (0, 2)), ((3, .5, .5), (0, 0))]
    Bs = len(sm_cases)
    sm = oracle.spec_match(np.tile(zt, (2 * Bs, 1)), np.tile(zd, (Bs, 1)),
                           np.array([c[0][0] for c in sm_cases], np.uint32),
                           np.array([[c[0][1], c[0][2]] for c in sm_cases], np.float32), Bs, 1, T, **filt)
    for j, (_, (L, a)) in enumerate(sm_cases):
        assert sm["len_sm"][j] == L and sm["tok_sm"][j, 0] == a, (sm_cases[j], sm["tok_sm"][j])
