"""GPU parity of vsel_spec_accept with the oracle.

Bit-exact accepted lengths and emitted tokens for both rules, except after an
accept test whose oracle float64 margin |u*q(t) - p(t)| is below 1e-7 (later
outputs of that sequence are not compared) and for a draw whose margin to a
CDF boundary is below 1e-9 of the total.  Coupling sums (sum min(p, q) and the
sum p*q of the same pass) within 1e-6 absolute plus 1e-5 relative.
"""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu
ACC_MARGIN, DRAW_MARGIN = 1e-7, 1e-9


@pytest.fixture(scope="module")
def g():
    import tests.gpu_helpers as G
    import vocab_row_reductions_amd as vsel
    G.vsel = vsel
    return G


def run(g, d, target=None, draft=None, tokens=None, T=None):
    target = d["target"] if target is None else target
    draft = d["draft"] if draft is None else draft
    tokens = d["tokens"] if tokens is None else tokens
    T = d["temperature"] if T is None else T
    out = g.vsel.vsel_spec_accept(g.dev(target), g.dev(draft), g.dev(tokens), g.dev(d["u_acc"]), g.dev(d["u_res"]),
                                  g.dev(d["u_bon"]), d["batch"], d["gamma"], T)
    return {k: (g.u32(v) if k.startswith("tok") else v.cpu().numpy()) for k, v in out.items()}


def compare(g, oracle, d, target=None, draft=None, tokens=None, T=None):
    target = d["target"] if target is None else target
    draft = d["draft"] if draft is None else draft
    tokens = d["tokens"] if tokens is None else tokens
    T = d["temperature"] if T is None else T
    B, G = d["batch"], d["gamma"]
    got = run(g, d, target, draft, tokens, T)
    ref = oracle.spec_accept(target, draft, tokens, d["u_acc"], d["u_res"], d["u_bon"], B, G, T)
    # argmax-against-argmax involves no floating point: bit-exact everywhere
    assert np.array_equal(got["len_aa"], ref["len_aa"])
    assert np.array_equal(got["tok_aa"], ref["tok_aa"])
    ok = np.isfinite(ref["summin"])
    assert np.all(np.abs(got["summin"][ok] - ref["summin"][ok]) <= 1e-6 + 1e-5 * np.abs(ref["summin"][ok]))
    assert np.array_equal(np.isnan(got["summin"]), ~ok)
    # sum p*q from the same pass: the oracle's sampler-match sums of the same p and q
    rsp = oracle.spec_match(target, draft, tokens, np.full((B, G + 1), 0.5, np.float32), B, G, T)["sumprod"]
    ok = np.isfinite(rsp)
    assert np.all(np.abs(got["sumprod"][ok] - rsp[ok]) <= 1e-6 + 1e-5 * np.abs(rsp[ok]))
    assert np.array_equal(np.isnan(got["sumprod"]), ~ok)
    assert np.all(got["sumprod"][ok] <= got["summin"][ok] + 1e-6)
    exempt = 0
    for b in range(B):
        am = ref["acc_margin"][b]
        close = np.nonzero(am < ACC_MARGIN)[0]
        if len(close):                      # compare only what precedes the first near-tie
            i = close[0]
            exempt += 1
            assert np.array_equal(got["tok_mrs"][b, :i], ref["tok_mrs"][b, :i])
            continue
        assert got["len_mrs"][b] == ref["len_mrs"][b], f"sequence {b}: accepted length"
        L = ref["len_mrs"][b]
        if L < 0:
            assert np.all(got["tok_mrs"][b] == g.SENT)
            continue
        assert np.array_equal(got["tok_mrs"][b, :L], ref["tok_mrs"][b, :L])
        if ref["draw_margin"][b] >= DRAW_MARGIN:
            assert got["tok_mrs"][b, L] == ref["tok_mrs"][b, L], f"sequence {b}: drawn token"
        else:
            exempt += 1
        assert np.all(got["tok_mrs"][b, L + 1:] == g.SENT)
    return got, ref, exempt


def test_config4_speculative_batch(g, oracle):
    d = W.speculative_batch()
    got, ref, exempt = compare(g, oracle, d)
    assert exempt <= 2
    # the draw happened in every sequence that rejected, and the mean
    # per-position acceptance sits near the mean coupling sum (statistical)
    L = ref["len_mrs"]
    tested = np.minimum(L + 1, d["gamma"]).sum()
    assert 0.5 < L.sum() / tested <= 1.0


@pytest.mark.parametrize("V", [2, 7, 1000, 70001])
def test_shapes(g, oracle, V):
    d = W.speculative_batch(batch=6, gamma=4, vocab=V, seed=V, noise=1.5)
    compare(g, oracle, d)
    compare(g, oracle, d, T=0.6)


def test_identical_rows_accept_everything(g, oracle):
    d = W.speculative_batch(batch=5, gamma=3, vocab=20000, seed=41)
    tgt = d["target"].reshape(5, 4, -1)
    draft = np.ascontiguousarray(tgt[:, :3]).reshape(15, -1)
    got, ref, _ = compare(g, oracle, d, draft=draft)
    assert np.all(got["len_mrs"] == 3)
    assert np.allclose(got["summin"], 1.0, atol=1e-6)


def test_temperature_zero_is_the_argmax_rule(g, oracle):
    d = W.speculative_batch(batch=8, gamma=3, vocab=5000, seed=42)
    got, ref, _ = compare(g, oracle, d, T=0.0)
    assert np.array_equal(got["len_mrs"], got["len_aa"])
    assert np.array_equal(got["tok_mrs"], got["tok_aa"])


def test_fail_closed_sequences(g, oracle):
    d = W.speculative_batch(batch=4, gamma=2, vocab=3000, seed=43)
    tgt = d["target"].copy()
    tgt[1 * 3 + 2, 17] = np.nan          # bonus row of sequence 1
    tok = d["tokens"].copy()
    tok[2 * 2 + 1] = 3000                # out-of-range draft of sequence 2
    got, ref, _ = compare(g, oracle, d, target=tgt, tokens=tok)
    assert list(got["len_mrs"][1:3]) == [-1, -1] and got["len_mrs"][0] >= 0


def test_chi_square_of_the_emitted_stream(g, oracle):
    # 12,000 emitted first tokens on a 6-token vocabulary against p: the
    # regression guard of speculative-acceptance.md, run on the GPU path.
    import json
    import os
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "chi_square.json")))
    n, V = gold["draws"], gold["dof"] + 1
    p = np.array([0.4, 0.3, 0.1, 0.1, 0.05, 0.05])
    zt, zd = np.log(p).astype(np.float32), np.log(p[::-1].copy()).astype(np.float32)
    pf = np.exp(zt.astype(np.float64) - zt.max()); pf /= pf.sum()
    qf = np.exp(zd.astype(np.float64) - zd.max()); qf /= qf.sum()
    rng = np.random.default_rng(W.BASE_SEED + 99)
    t = rng.choice(V, size=n, p=qf).astype(np.uint32)
    d = dict(u_acc=rng.random(n, dtype=np.float32), u_res=rng.random(n, dtype=np.float32),
             u_bon=rng.random(n, dtype=np.float32), batch=n, gamma=1)
    got = run(g, d, np.repeat(zt[None], 2 * n, 0), np.repeat(zd[None], n, 0), t, 1.0)
    counts = np.bincount(got["tok_mrs"][:, 0], minlength=V)
    stat = float(((counts - n * pf) ** 2 / (n * pf)).sum())
    assert stat < gold["threshold"]
    counts_aa = np.bincount(got["tok_aa"][:, 0], minlength=V)
    assert float(((counts_aa - n * pf) ** 2 / (n * pf)).sum()) > gold["threshold"]


def test_boundary_uniforms_take_the_exact_draw(g, oracle):
    """The draws run with float32 terms first and stand only far from a CDF
    boundary.  u placed 3e-6 (relative to the mass) above and below boundaries
    of the residual normalize(max(p - q, 0)) and of the bonus row's p cannot be
    decided by float32 terms: the float64 passes must take them, and the
    tokens must still be the oracle's."""
    from scipy.special import logsumexp
    B, G, V = 12, 1, 50000
    d = W.speculative_batch(batch=B, gamma=G, vocab=V, seed=45)
    tg, dr = d["target"].astype(np.float64), d["draft"].astype(np.float64)
    tok = np.zeros(B, np.uint32)
    ua, ur, ub = np.zeros(B, np.float32), np.full(B, 0.5, np.float32), np.full(B, 0.5, np.float32)
    for b in range(B):
        p = np.exp(tg[2 * b] - logsumexp(tg[2 * b]))
        q = np.exp(dr[b] - logsumexp(dr[b]))
        side = 3e-6 if b % 2 == 0 else -3e-6
        if b < 8:   # rejected at position 0: the residual draw
            cand = np.nonzero(p < 0.5 * q)[0]
            t = int(cand[np.argmax(q[cand])])
            tok[b], ua[b] = t, np.float32(0.999)
            r = np.maximum(p - q, 0.0)
            c = np.cumsum(r) / r.sum()
        else:       # accepted (u = 0): the bonus draw from target row 1
            t = int(np.argmax(q))
            tok[b] = t
            pb = np.exp(tg[2 * b + 1] - logsumexp(tg[2 * b + 1]))
            c = np.cumsum(pb)
        # a boundary below one of the heavier tokens, with mass on both sides
        heavy = [x for x in np.argsort(-np.diff(np.concatenate([[0.0], c])))[:16] if 0.05 < c[x - 1] < 0.95]
        x = int(heavy[b % len(heavy)])
        u = np.float32(c[x - 1] + side)
        if b < 8:
            ur[b] = u
        else:
            ub[b] = u
    dd = dict(d, tokens=tok, u_acc=ua, u_res=ur, u_bon=ub)
    got, ref, exempt = compare(g, oracle, dd)
    assert exempt == 0
    assert list(ref["len_mrs"]) == [0] * 8 + [1] * 4


@pytest.mark.parametrize("T", [0.6, 1.7])
def test_large_logit_offsets(g, oracle, T):
    """Rows offset by +3000: every float32 exponent is taken relative to the
    row maximum, so the coupling sums and the draws keep their precision."""
    d = W.speculative_batch(batch=8, gamma=4, vocab=30000, seed=46, temperature=T)
    tgt = (d["target"] + np.float32(3000.0)).astype(np.float32)
    dft = (d["draft"] + np.float32(3000.0)).astype(np.float32)
    got, ref, exempt = compare(g, oracle, d, target=tgt, draft=dft, T=T)
    assert exempt <= 1
