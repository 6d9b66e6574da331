"""Pins of the oracle's filtered speculative acceptance ("speculative-acceptance.md",
"The rules": p is the target distribution after top-k / top-p / min-p filtering
on the untempered distribution and the final temperature; q the distribution
the drafter drew from, here under the same sampler settings).

The filtered distributions are rebuilt here with numpy (lexsort, cumsum,
masks, softmax over the kept ids) and the oracle is checked against them:
acceptance probabilities and emitted distributions by integration over uniform
grids (modified rejection sampling accepts at sum min(p, q), sampler-match at
sum p q; both emit p), the page's regression guard that no emitted token lies
outside a top_k = 2 target's support, the coupling sums, and the top_k = 1
limit that reduces modified rejection sampling to the argmax rule.
"""
import numpy as np
import pytest

import workloads as W

SENT = 0xFFFFFFFF


def filtered(z, T, top_k=0, top_p=1.0, min_p=0.0):
    """The effective distribution of one row, from the definitions."""
    z = np.asarray(z, np.float64)
    V = len(z)
    cand = np.arange(V)
    if top_k or top_p < 1:
        cand = np.lexsort((np.arange(V), -z))          # value desc, id asc
        if top_k:
            cand = cand[:top_k]
        if top_p < 1:
            p0 = np.exp(z[cand] - z[cand].max())
            p0 /= p0.sum()
            cand = cand[:int(np.searchsorted(np.cumsum(p0), top_p)) + 1]
    if min_p > 0:
        cand = cand[z[cand] >= z[cand].max() + np.log(min_p)]
    p = np.zeros(V)
    e = np.exp((z[cand] - z[cand].max()) / T)
    p[cand] = e / e.sum()
    return p


FILTERS = [dict(top_k=3), dict(top_p=0.7), dict(min_p=0.3), dict(top_k=4, top_p=0.9, min_p=0.1)]
ZT = [0.2, 1.1, -0.5, 0.7, 0.4]
ZD = [1.0, -0.3, 0.4, 0.9, 0.6]


def _grid(oracle, rule, zt, zd, T, N, kw):
    """Integrate one rule over uniform grids with gamma = 1: the drafted token t
    weighted by the filtered q(t).  Returns (P(accept), P(first emitted = x))."""
    V = len(zt)
    q = filtered(zd, T, **kw)
    g = ((np.arange(N) + 0.5) / N).astype(np.float32)
    acc, emit = 0.0, np.zeros(V)
    for t in np.nonzero(q)[0]:
        if rule == "mrs":
            ua, ur = np.meshgrid(g, g, indexing="ij")
            B = ua.size
            target = np.repeat(np.array([zt], np.float32), 2 * B, 0)
            draft = np.repeat(np.array([zd], np.float32), B, 0)
            out = oracle.spec_accept(target, draft, np.full(B, t, np.uint32), ua.ravel(), ur.ravel(),
                                     np.full(B, 0.5, np.float32), B, 1, T, **kw)
            ok, first = out["len_mrs"] == 1, out["tok_mrs"][:, 0]
        else:
            B = N
            um = np.stack([g, np.full(N, 0.5, np.float32)], 1)
            target = np.repeat(np.array([zt], np.float32), 2 * B, 0)
            draft = np.repeat(np.array([zd], np.float32), B, 0)
            out = oracle.spec_match(target, draft, np.full(B, t, np.uint32), um, B, 1, T, **kw)
            ok, first = out["len_sm"] == 1, out["tok_sm"][:, 0]
        acc += q[t] * ok.mean()
        emit += q[t] * np.bincount(first, minlength=V) / B
    return acc, emit


@pytest.mark.parametrize("kw", FILTERS)
@pytest.mark.parametrize("T", [1.0, float(np.float32(0.7))])
def test_filtered_mrs_is_lossless_and_hits_the_ceiling(oracle, kw, T):
    p, q = filtered(ZT, T, **kw), filtered(ZD, T, **kw)
    acc, emit = _grid(oracle, "mrs", ZT, ZD, T, 120, kw)
    assert abs(acc - np.minimum(p, q).sum()) < 2.0 / 120
    assert np.all(np.abs(emit - p) < 3.0 / 120)


@pytest.mark.parametrize("kw", FILTERS)
def test_filtered_sampler_match_accepts_at_sum_pq(oracle, kw):
    T = float(np.float32(0.8))
    p, q = filtered(ZT, T, **kw), filtered(ZD, T, **kw)
    acc, emit = _grid(oracle, "sm", ZT, ZD, T, 4000, kw)
    assert abs(acc - (p * q).sum()) < 2.0 / 4000 * 5
    assert np.all(np.abs(emit - p) < 3.0 / 4000 * 5)


def test_filtered_support_is_never_violated(oracle):
    """No emitted token outside the target's filtered support, over both rules,
    a top_k = 2 target and a nucleus, drafts from the filtered q (zero tolerance)."""
    rng = np.random.default_rng(W.BASE_SEED + 600)
    B, G, V = 400, 3, 50
    tgt = (1.5 * rng.normal(size=(B * (G + 1), V))).astype(np.float32)
    dft = (tgt.reshape(B, G + 1, V)[:, :G] + rng.normal(0, 1.0, (B, G, V))).reshape(B * G, V).astype(np.float32)
    for kw in (dict(top_k=2), dict(top_p=0.5), dict(top_k=5, min_p=0.2)):
        T = 1.0
        toks = np.array([rng.choice(V, p=filtered(dft[r], T, **kw)) for r in range(B * G)], np.uint32)
        u = rng.random((4, B * G), dtype=np.float32)
        mrs = oracle.spec_accept(tgt, dft, toks, u[0], u[1], u[2, :B], B, G, T, **kw)
        sm = oracle.spec_match(tgt, dft, toks, rng.random((B, G + 1), dtype=np.float32), B, G, T, **kw)
        for out, L in ((mrs["tok_mrs"], mrs["len_mrs"]), (sm["tok_sm"], sm["len_sm"])):
            for b in range(B):
                for i in range(L[b] + 1):
                    assert filtered(tgt[b * (G + 1) + i], T, **kw)[out[b, i]] > 0, (kw, b, i)


def test_filtered_coupling_sums_match_numpy(oracle):
    d = W.speculative_batch(batch=3, gamma=3, vocab=3000, seed=601)
    T = float(np.float32(0.9))                          # the oracle takes the temperature as float32
    for kw in (dict(top_k=50), dict(top_p=0.9), dict(min_p=0.05), dict(top_k=200, top_p=0.95, min_p=0.01)):
        mrs = oracle.spec_accept(d["target"], d["draft"], d["tokens"], d["u_acc"], d["u_res"], d["u_bon"], 3, 3,
                                 T, **kw)
        sm = oracle.spec_match(d["target"], d["draft"], d["tokens"], np.full((3, 4), 0.5, np.float32), 3, 3, T,
                               **kw)
        for b in range(3):
            for i in range(3):
                p = filtered(d["target"][b * 4 + i], T, **kw)
                q = filtered(d["draft"][b * 3 + i], T, **kw)
                assert abs(mrs["summin"][b, i] - np.minimum(p, q).sum()) < 1e-12
                assert abs(sm["sumprod"][b, i] - (p * q).sum()) < 1e-12


def test_top_k_one_reduces_mrs_to_the_argmax_rule(oracle):
    """With top_k = 1 the drafter can only propose its argmax, q and p are one-hot,
    so accept iff the draft is the target's argmax, and the residual emits it."""
    d = W.speculative_batch(batch=8, gamma=4, vocab=2000, seed=602)
    toks = np.argmax(d["draft"], axis=1).astype(np.uint32)
    toks[::3] = np.argmax(d["target"].reshape(8, 5, -1)[:, :4].reshape(32, -1), axis=1)[::3]  # some agree
    out = oracle.spec_accept(d["target"], d["draft"], toks, d["u_acc"], d["u_res"], d["u_bon"], 8, 4, 1.0,
                             top_k=1)
    assert np.array_equal(out["len_mrs"], out["len_aa"])
    assert np.array_equal(out["tok_mrs"], out["tok_aa"])


def test_filters_off_reduce_to_the_unfiltered_rules(oracle):
    d = W.speculative_batch(batch=4, gamma=3, vocab=1000, seed=603)
    a = oracle.spec_accept(d["target"], d["draft"], d["tokens"], d["u_acc"], d["u_res"], d["u_bon"], 4, 3, 0.8)
    b = oracle.spec_accept(d["target"], d["draft"], d["tokens"], d["u_acc"], d["u_res"], d["u_bon"], 4, 3, 0.8,
                           top_k=0, top_p=1.0, min_p=0.0)
    for k in ("len_mrs", "tok_mrs", "len_aa", "tok_aa", "summin"):
        assert np.array_equal(a[k], b[k])
    assert np.all(np.isinf(b["filter_margin"]))
