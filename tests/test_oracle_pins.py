"""Pins of the CPU oracle to facts fixed by the pages and by mathematics.

Nothing here compares the oracle with itself: each check uses a closed form,
a documented library routine, brute force over tiny inputs, a page's printed
value (tests/golden/), or a theorem about the method (for acceptance, the
losslessness identity min(q, p) + relu(p - q) = p and the coupling ceiling).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp

import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")
SENT = 0xFFFFFFFF


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ geometry
def test_chunk_geometry_matches_figure_21_1(oracle):
    for c in gold("geometry.json")["cases"]:
        count, tail = oracle.chunk_geometry(c["n"], c["chunk"])
        assert count == c["chunks"] and tail == c["tail"]
        assert (count - 1) * c["chunk"] == c["full_elements"]
    # same arithmetic on the 248,320-column verify rows
    assert oracle.chunk_geometry(248320, 1024) == (243, 512)


# ------------------------------------------------------------------ argmax
def test_argmax_planted_first_maximum_config1(oracle):
    row, planted = W.greedy_single_row()
    idx, val = oracle.argmax(row)
    assert len(planted) == 3
    chunks = {p // 1024 for p in planted}
    assert len(chunks) == 3 and max(planted) >= 201728          # one copy in the 320-element tail
    assert idx[0] == min(planted)                                # lowest index holding the maximum
    assert val[0] == row[0].max()


def test_argmax_matches_numpy_first_occurrence(oracle):
    rng = np.random.default_rng(7)
    for V in (1, 2, 7, 63, 1024, 1025, 4097):
        x = (np.round(rng.normal(0, 1, (5, V)) * 4) / 4).astype(np.float32)  # coarse grid: many ties
        idx, _ = oracle.argmax(x)
        assert np.array_equal(idx, np.argmax(x, axis=1).astype(np.uint32))


def test_argmax_brute_force_binary_rows(oracle):
    rows = np.array(list(itertools.product([0.0, 1.0], repeat=8)), dtype=np.float32)
    idx, _ = oracle.argmax(rows)
    for r, i in zip(rows.tolist(), idx):
        assert i == r.index(max(r))


def test_argmax_fail_closed_and_masks(oracle):
    inf = np.inf
    x = np.array([[1, np.nan, 2, 0],
                  [1, inf, 2, 0],
                  [-inf, -inf, -inf, -inf],
                  [-inf, -3, -inf, -3],
                  [-0.0, 0.0, -1, -2],
                  [0.0, -0.0, -1, -2]], dtype=np.float32)
    idx, _ = oracle.argmax(x)
    assert list(idx) == [SENT, SENT, SENT, 1, 0, 0]


# ---- greedy serving variant ("Chapter 21", section 21.4): excluded ids are
# -inf inside the reduction only; any NaN / +inf in the row fails it closed.
def test_argmax_excluding_matches_numpy_on_masked_rows(oracle):
    rng = np.random.default_rng(11)
    for V in (1, 5, 64, 1025, 4097):
        x = (np.round(rng.normal(0, 1, (6, V)) * 4) / 4).astype(np.float32)  # coarse grid: many ties
        for n_ex in sorted({0, 1, min(V, 3), min(V, 40)}):
            ex = rng.choice(V, size=n_ex, replace=False).astype(np.uint32)
            idx, st = oracle.argmax_excluding(x, ex)
            masked = x.copy()
            masked[:, ex] = -np.inf
            for r in range(x.shape[0]):
                if np.all(np.isneginf(masked[r])):
                    assert st[r] == 2 and idx[r] == SENT
                else:
                    assert st[r] == 0 and idx[r] == np.argmax(masked[r])  # numpy: first occurrence
    # excluding every position that holds the maximum moves the answer to the next value
    x = np.array([[3, 9, 1, 9, 9, 7, 7]], np.float32)
    idx, st = oracle.argmax_excluding(x, [1, 3, 4])
    assert (idx[0], st[0]) == (5, 0)


def test_argmax_excluding_special_cases(oracle):
    inf = np.inf
    x = np.array([[1, 5, 3, 5, 2],
                  [1, np.nan, 3, 2, 0],     # NaN at an excluded id still fails closed
                  [1, inf, 3, 2, 0],        # so does +inf
                  [-inf, 4, -inf, -inf, -inf],
                  [2, 2, 2, 2, 2]], np.float32)
    idx, st = oracle.argmax_excluding(x, [1])
    assert list(st) == [0, 1, 1, 2, 0]
    assert list(idx) == [3, SENT, SENT, SENT, 0]
    # every id excluded: no candidate; ids past the vocabulary exclude nothing; duplicates are fine
    idx, st = oracle.argmax_excluding(x[:1], [0, 1, 2, 3, 4])
    assert (idx[0], st[0]) == (SENT, 2)
    idx, st = oracle.argmax_excluding(x[:1], [5, 99, 1 << 31, 1, 1])
    assert (idx[0], st[0]) == (3, 0)
    # an empty set is the plain argmax (the plain argmax is pinned above)
    y = np.random.default_rng(3).normal(0, 1, (4, 333)).astype(np.float32)
    assert np.array_equal(oracle.argmax_excluding(y, [])[0], oracle.argmax(y)[0])


def test_argmax_excluding_brute_force_subsets(oracle):
    # every subset of the ids of small rows with ties, against a direct reading
    rows = np.array([[0, 1, 1, 0, 1], [2, 2, 2, 2, 2], [-1, 3, -2, 3, 0]], np.float32)
    for r in rows:
        for mask in range(32):
            ex = [i for i in range(5) if mask >> i & 1]
            idx, st = oracle.argmax_excluding(r[None, :], ex)
            kept = [i for i in range(5) if i not in ex]
            if not kept:
                assert (idx[0], st[0]) == (SENT, 2)
            else:
                m = max(r[i] for i in kept)
                assert (idx[0], st[0]) == (min(i for i in kept if r[i] == m), 0)


def test_bf16_rows_widen_exactly(oracle):
    rng = np.random.default_rng(3)
    f = rng.normal(0, 4, (4, 777)).astype(np.float32)
    b = W.f32_to_bf16_bits(f)
    wide = W.bf16_bits_to_f32(b)
    i1, v1 = oracle.argmax(b)
    i2, v2 = oracle.argmax(wide)
    assert np.array_equal(i1, i2) and np.array_equal(v1, v2)
    assert np.array_equal(oracle.topk(b, 17)[1], oracle.topk(wide, 17)[1])
    # bfloat16 0x3F80 is 1.0 and 0xC000 is -2.0
    assert W.bf16_bits_to_f32(np.array([0x3F80, 0xC000], np.uint16)).tolist() == [1.0, -2.0]


# ------------------------------------------------------------------ top-k
def _lexsort_topk(row, k):
    ids = np.arange(row.size)
    order = np.lexsort((ids, -row.astype(np.float64)))[:k]
    return order


def test_topk_matches_lexsort(oracle):
    rng = np.random.default_rng(11)
    for V, k in [(1, 1), (7, 3), (7, 7), (100, 84), (1024, 64), (5000, 84), (5000, 1)]:
        x = (np.round(rng.normal(0, 2, (3, V)) * 8) / 8).astype(np.float32)
        vals, ids, am, _ = oracle.topk(x, k)
        for r in range(3):
            ref = _lexsort_topk(x[r], k)
            assert np.array_equal(ids[r], ref.astype(np.uint32))
            assert np.array_equal(vals[r].view(np.uint32), x[r, ref].view(np.uint32))
            assert am[r] == ids[r, 0]


def test_topk_brute_force_tiny(oracle):
    # every k-subset: the oracle's set is the unique one where no outside
    # element precedes an inside element in (value desc, id asc) order
    vals_grid = [-1.0, 0.0, 0.5]
    for row in itertools.product(vals_grid, repeat=5):
        x = np.array([row], dtype=np.float32)
        for k in (1, 2, 4, 5):
            _, ids, _, _ = oracle.topk(x, k)
            chosen = list(ids[0])
            precedes = lambda a, b: row[a] > row[b] or (row[a] == row[b] and a < b)
            outside = [i for i in range(5) if i not in chosen]
            assert all(precedes(c, o) for c in chosen for o in outside)
            assert all(precedes(chosen[j], chosen[j + 1]) for j in range(k - 1))


def test_topk_invariants_verify_rows(oracle):
    x = W.verify_topk_rows(rows=3, vocab=20000, seed=5)
    k = 84
    vals, ids, am, _ = oracle.topk(x, k)
    for r in range(3):
        v, i = vals[r], ids[r].astype(np.int64)
        assert am[r] == i[0]
        assert np.all(v[:-1] >= v[1:])
        eq = v[:-1] == v[1:]
        assert np.all(i[:-1][eq] < i[1:][eq])
        mask = np.ones(x.shape[1], bool)
        mask[i] = False
        last_tied = i[v == v[-1]].max()
        out = np.nonzero(mask)[0]
        assert np.all((x[r, out] < v[-1]) | ((x[r, out] == v[-1]) & (out > last_tied)))
        # the five +8 spikes sit in the top 84 (sanity, not a pin)
        assert (x[r, i] > 6).sum() >= 5


def test_topk_signed_zero_ties_and_masks(oracle):
    x = np.array([[-0.0, 0.0, -np.inf, 0.0, -np.inf]], dtype=np.float32)
    vals, ids, am, ls = oracle.topk(x, 5)
    assert list(ids[0]) == [0, 1, 3, 2, 4]
    assert vals[0].view(np.uint32)[0] == 0x80000000      # the row's own -0.0 bits
    y = np.full((1, 6), -np.inf, np.float32)
    vals, ids, am, ls = oracle.topk(y, 3)
    assert list(ids[0]) == [0, 1, 2] and am[0] == SENT and ls[0] == -np.inf
    z = np.array([[1.0, np.nan, 3.0]], np.float32)
    vals, ids, am, ls = oracle.topk(z, 2)
    assert ids[0, 0] == SENT and am[0] == SENT and np.isnan(ls[0])


# ------------------------------------------------------------------ logsumexp
def test_lse_closed_forms(oracle):
    for V, c in [(1, 0.0), (7, 2.5), (202048, -3.0), (1000, 80.0)]:
        x = np.full((1, V), c, np.float32)
        assert abs(oracle.lse(x)[0] - (c + math.log(V))) < 1e-12 * max(1, abs(c) + math.log(V))
    x = np.full((1, 9), -np.inf, np.float32)
    x[0, 4] = 1.25
    assert oracle.lse(x)[0] == 1.25
    assert oracle.lse(np.full((1, 3), -np.inf, np.float32))[0] == -np.inf


def test_lse_matches_scipy(oracle):
    rng = np.random.default_rng(2)
    x = rng.normal(0, 3, (4, 3001)).astype(np.float32)
    x[1, ::7] = -np.inf
    for T in (1.0, 0.7, 2.0):
        ref = logsumexp(x.astype(np.float64) / T, axis=1)
        assert np.allclose(oracle.lse(x, T), ref, rtol=0, atol=1e-12)


# ------------------------------------------------------------------ sampling
def test_sample_greedy_limits(oracle):
    x, u = W.sampling_rows(rows=8, vocab=3000, seed=9)
    am, _ = oracle.argmax(x)
    for T, k in ((0.0, 20), (0.7, 1)):
        tok, logp, _ = oracle.sample(x, T, k, 0.95, u)
        assert np.array_equal(tok, am) and np.all(logp == 0)


def test_sample_full_row_matches_numpy_categorical(oracle):
    # top_k = 0, top_p = 1: a plain categorical of softmax(z/T) in id order
    rng = np.random.default_rng(4)
    x = rng.normal(0, 2, (1, 50)).astype(np.float32)
    T = 0.7
    z = x[0].astype(np.float64) / T
    p = np.exp(z - z.max())
    cdf = np.cumsum(p) / p.sum()
    us = (np.arange(2000, dtype=np.float64) + 0.5) / 2000
    xs = np.repeat(x, len(us), axis=0)
    tok, logp, m = oracle.sample(xs, T, 0, 1.0, us.astype(np.float32))
    ref = np.searchsorted(cdf, us.astype(np.float32).astype(np.float64), side="right")
    ok = m[:, 0] > 1e-9
    assert np.array_equal(tok[ok], ref[ok].astype(np.uint32))
    assert np.allclose(logp, np.log(p[tok] / p.sum()), atol=1e-12)
    # top_k = V: same categorical taken in (value desc, id asc) order
    order = np.lexsort((np.arange(50), -x[0].astype(np.float64)))
    cdf2 = np.cumsum(p[order]) / p.sum()
    tok2, _, m2 = oracle.sample(xs, T, 50, 1.0, us.astype(np.float32))
    ref2 = order[np.searchsorted(cdf2, us.astype(np.float32).astype(np.float64), side="right")]
    ok2 = m2[:, 0] > 1e-9
    assert np.array_equal(tok2[ok2], ref2[ok2].astype(np.uint32))


def test_sample_filter_order_worked_example(oracle):
    # logits 2, 1, 0, -1, -inf with top_k = 3, top_p = 0.8, T = 0.5.
    # Untempered over the top 3: p0 = (1, e^-1, e^-2)/(1 + e^-1 + e^-2)
    #   = 0.665, 0.245, 0.090 -> the 0.8 nucleus keeps ids {0, 1}.
    # Tempered over the kept set: (1, e^-2)/(1 + e^-2) = 0.8808, 0.1192.
    # (Tempering first would keep id 0 alone, since 1/(1+e^-2+e^-4) = 0.867 >= 0.8.)
    x = np.array([[2.0, 1.0, 0.0, -1.0, -np.inf]], np.float32)
    p_keep0 = 1.0 / (1.0 + math.exp(-2.0))
    tok, logp, _ = oracle.sample(np.repeat(x, 2, 0), 0.5, 3, 0.8, np.array([0.5, 0.9], np.float32))
    assert list(tok) == [0, 1]
    assert abs(logp[0] - math.log(p_keep0)) < 1e-12
    assert abs(logp[1] - math.log(1.0 - p_keep0)) < 1e-12


def test_sample_u_grid_frequencies_and_support(oracle):
    # The draw over a uniform grid reproduces the kept distribution to 1/N,
    # and no token outside the top_k support is ever emitted.
    x = np.array([[0.3, 1.9, -0.4, 1.2, 0.8, -2.0]], np.float32)
    N = 20000
    us = ((np.arange(N) + 0.5) / N).astype(np.float32)
    for top_k, top_p, T in ((2, 1.0, 1.0), (4, 0.9, 0.7), (6, 1.0, 1.3)):
        tok, _, _ = oracle.sample(np.repeat(x, N, 0), T, top_k, top_p, us)
        order = np.lexsort((np.arange(6), -x[0].astype(np.float64)))[:top_k]
        assert set(np.unique(tok)) <= set(order.tolist())
        z = x[0, order].astype(np.float64)
        p0 = np.exp(z - z[0]) / np.exp(z - z[0]).sum()
        n = top_k if top_p >= 1 else int(np.argmax(np.cumsum(p0) >= top_p)) + 1
        w = np.exp((z[:n] - z[0]) / T)
        freq = np.array([(tok == order[j]).mean() for j in range(n)])
        assert np.all(np.abs(freq - w / w.sum()) <= 2.0 / N)


# ------------------------------------------------------------------ speculative acceptance
def _softmax64(z, T=1.0):
    z = np.asarray(z, np.float64) / T
    e = np.exp(z - z.max())
    return e / e.sum()


def _mrs_grid(oracle, zt, zd, T, N):
    """Integrate the oracle's modified rejection sampling over uniform grids:
    drafted token t weighted by q(t); u_acc and u_res on N-point midpoint grids.
    gamma = 1, so the first emitted token is t (accepted) or the residual draw.
    Returns (P(accept), P(first emitted = x))."""
    V = len(zt)
    q = _softmax64(zd, T)
    g = ((np.arange(N) + 0.5) / N).astype(np.float32)
    ua, ur = np.meshgrid(g, g, indexing="ij")
    ua, ur = ua.ravel(), ur.ravel()
    B = ua.size
    tgt_row = np.array(zt, np.float32)
    target = np.empty((B * 2, V), np.float32)
    target[0::2] = tgt_row
    target[1::2] = tgt_row       # bonus row
    draft = np.repeat(np.array([zd], np.float32), B, 0)
    acc = 0.0
    emit = np.zeros(V)
    for t in range(V):
        out = oracle.spec_accept(target, draft, np.full(B, t, np.uint32), ua, ur,
                                 np.full(B, 0.5, np.float32), B, 1, T)
        accepted = out["len_mrs"] == 1
        acc += q[t] * accepted.mean()
        first = out["tok_mrs"][:, 0]
        emit += q[t] * np.bincount(first, minlength=V) / B
    return acc, emit


def test_mrs_is_lossless_and_hits_the_ceiling(oracle):
    zt = [0.2, 1.1, -0.5, 0.7]
    zd = [1.0, -0.3, 0.4, 0.9]
    for T in (1.0, 0.6):
        p, q = _softmax64(zt, T), _softmax64(zd, T)
        acc, emit = _mrs_grid(oracle, zt, zd, T, N=160)
        assert abs(acc - np.minimum(p, q).sum()) < 2.0 / 160       # P(accept) = sum min(p, q)
        assert np.all(np.abs(emit - p) < 3.0 / 160)                 # emitted ~ p exactly


def test_ceiling_example_argmax_rule_vs_mrs(oracle):
    g = gold("acceptance_ceiling.json")
    p = np.array([g["p_a"], 0.25, 0.25, 0.2])
    q = np.array([g["q_a"], 0.02, 0.02, 0.01])
    zt, zd = np.log(p), np.log(q)
    pf, qf = _softmax64(np.float32(zt)), _softmax64(np.float32(zd))
    acc, _ = _mrs_grid(oracle, list(np.float32(zt)), list(np.float32(zd)), 1.0, N=200)
    ceiling = np.minimum(pf, qf).sum()
    assert abs(acc - ceiling) < 2.0 / 200
    assert abs(ceiling - 0.35) < 1e-6 and ceiling >= g["ceiling_about"]
    # argmax-against-argmax accepts exactly when the draft is argmax p = id 0: probability q(a)
    B = 4
    target = np.repeat(np.float32(zt)[None], 2 * B, 0)
    draft = np.repeat(np.float32(zd)[None], B, 0)
    out = oracle.spec_accept(target, draft, np.arange(B, dtype=np.uint32), np.full(B, .5, np.float32),
                             np.full(B, .5, np.float32), np.full(B, .5, np.float32), B, 1, 1.0)
    assert list(out["len_aa"]) == [1, 0, 0, 0]
    assert abs((qf * (out["len_aa"] == 1)).sum() - g["argmax_rule_acceptance"]) < 1e-6


def test_spec_invariants_config4_like(oracle):
    d = W.speculative_batch(batch=3, gamma=4, vocab=4000, seed=12)
    out = oracle.spec_accept(d["target"], d["draft"], d["tokens"], d["u_acc"], d["u_res"], d["u_bon"],
                             d["batch"], d["gamma"], d["temperature"])
    tg = d["target"].reshape(3, 5, -1)
    dr = d["draft"].reshape(3, 4, -1)
    for b in range(3):
        L = out["len_mrs"][b]
        assert 0 <= L <= 4
        assert np.array_equal(out["tok_mrs"][b, :L], d["tokens"].reshape(3, 4)[b, :L])
        assert np.all(out["tok_mrs"][b, L + 1:] == SENT)
        for i in range(4):
            p, q = _softmax64(tg[b, i]), _softmax64(dr[b, i])
            sm = out["summin"][b, i]
            assert abs(sm - (1 - 0.5 * np.abs(p - q).sum())) < 1e-12   # 1 - TV(p, q)
            assert sm >= (p * q).sum() and 0 <= sm <= 1
        Laa = out["len_aa"][b]
        amax = [int(np.argmax(tg[b, i])) for i in range(5)]
        assert out["tok_aa"][b, Laa] == amax[Laa]


def test_spec_identical_rows_accept_everything(oracle):
    d = W.speculative_batch(batch=4, gamma=3, vocab=500, seed=13)
    tgt = d["target"].reshape(4, 4, -1)
    draft = np.ascontiguousarray(tgt[:, :3]).reshape(12, -1)
    out = oracle.spec_accept(d["target"], draft, d["tokens"], d["u_acc"], d["u_res"], d["u_bon"], 4, 3, 1.0)
    assert np.all(out["len_mrs"] == 3)
    assert np.allclose(out["summin"], 1.0, atol=1e-12)


def test_spec_one_hot_draft(oracle):
    # Prompt-lookup style q: one-hot on d.  sum min(p, q) = sum p q = p(d).
    zt = np.array([0.5, 1.5, -1.0, 0.0, 2.0], np.float32)
    d = 3
    zd = np.full(5, -np.inf, np.float32)
    zd[d] = 0.0
    p = _softmax64(zt)
    us = np.array([0.01, 0.2, 0.5, 0.99], np.float32)
    B = len(us)
    out = oracle.spec_accept(np.repeat(zt[None], 2 * B, 0), np.repeat(zd[None], B, 0), np.full(B, d, np.uint32),
                             us, np.full(B, 0.3, np.float32), np.full(B, 0.3, np.float32), B, 1, 1.0)
    assert np.allclose(out["summin"][:, 0], p[d], atol=1e-12)
    assert list(out["len_mrs"]) == [int(u <= p[d]) for u in us.astype(np.float64)]
    # on rejection the residual is p restricted to x != d
    rej = out["len_mrs"] == 0
    assert np.all(out["tok_mrs"][rej, 0] != d)


def test_spec_temperature_zero_is_argmax_rule(oracle):
    d = W.speculative_batch(batch=5, gamma=3, vocab=300, seed=14)
    out = oracle.spec_accept(d["target"], d["draft"], d["tokens"], d["u_acc"], d["u_res"], d["u_bon"], 5, 3, 0.0)
    assert np.array_equal(out["len_mrs"], out["len_aa"])
    assert np.array_equal(out["tok_mrs"], out["tok_aa"])


def test_spec_fail_closed(oracle):
    d = W.speculative_batch(batch=3, gamma=2, vocab=100, seed=15)
    tgt = d["target"].copy()
    tgt[1 * 3 + 2, 17] = np.nan            # bonus row of sequence 1
    tok = d["tokens"].copy()
    tok[2 * 2 + 1] = 100                   # out-of-range draft in sequence 2
    out = oracle.spec_accept(tgt, d["draft"], tok, d["u_acc"], d["u_res"], d["u_bon"], 3, 2, 1.0)
    assert out["len_mrs"][0] >= 0 and out["len_mrs"][1] == -1 and out["len_mrs"][2] == -1
    assert np.all(out["tok_mrs"][1] == SENT)


def _chi2(counts, probs):
    n = counts.sum()
    e = probs * n
    return float(((counts - e) ** 2 / e).sum())


def test_chi_square_stream_and_power(oracle):
    g = gold("chi_square.json")
    V = g["dof"] + 1
    n = g["draws"]
    p = np.array([0.4, 0.3, 0.1, 0.1, 0.05, 0.05])
    q = p[::-1].copy()
    zt, zd = np.log(p).astype(np.float32), np.log(q).astype(np.float32)
    pf, qf = _softmax64(zt), _softmax64(zd)
    rng = np.random.default_rng(W.BASE_SEED + 77)
    t = rng.choice(V, size=n, p=qf).astype(np.uint32)
    ua, ur, ub = (rng.random(n, dtype=np.float32) for _ in range(3))
    out = oracle.spec_accept(np.repeat(zt[None], 2 * n, 0), np.repeat(zd[None], n, 0), t, ua, ur, ub, n, 1, 1.0)
    first = out["tok_mrs"][:, 0]
    stat = _chi2(np.bincount(first, minlength=V), pf)
    assert stat < g["threshold"]
    # power: argmax-against-argmax emits argmax p whenever it rejects
    stat_aa = _chi2(np.bincount(out["tok_aa"][:, 0], minlength=V), pf)
    assert stat_aa > g["threshold"]
    # power: a planted wrong rule that resamples from p instead of the residual
    accepted = out["len_mrs"] == 1
    cdf = np.cumsum(pf)
    resampled = np.searchsorted(cdf, ur.astype(np.float64), side="right")
    wrong = np.where(accepted, t, resampled)
    assert _chi2(np.bincount(wrong, minlength=V), pf) > g["threshold"]


def test_bonus_draw_comes_from_the_last_target_row(oracle):
    # Draft == verify row 0, so position 0 is always accepted and the bonus
    # token is drawn from p of the separate bonus row over a u_bon grid.
    z0 = np.array([0.1, 0.9, -0.2, 0.4], np.float32)
    zb = np.array([1.5, -1.0, 0.3, 0.0], np.float32)
    N = 4000
    ub = ((np.arange(N) + 0.5) / N).astype(np.float32)
    target = np.tile(np.stack([z0, zb]), (N, 1))
    draft = np.repeat(z0[None], N, 0)
    out = oracle.spec_accept(target, draft, np.full(N, 1, np.uint32), np.full(N, .999, np.float32),
                             np.full(N, .5, np.float32), ub, N, 1, 0.8)
    assert np.all(out["len_mrs"] == 1)
    freq = np.bincount(out["tok_mrs"][:, 1], minlength=4) / N
    assert np.all(np.abs(freq - _softmax64(zb, 0.8)) <= 2.0 / N)
