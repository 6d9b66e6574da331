"""GPU parity of the filtered speculative rules (vsel_spec_accept_filtered,
vsel_spec_match_filtered: p and q after top-k / top-p / min-p on the
untempered rows, then the temperature) with the oracle.

Tolerances as the unfiltered tests: bit-exact lengths and tokens, except after
an accept test closer than 1e-7 to its boundary, at a draw closer than 1e-9 of
the mass to a CDF boundary, and for a sequence whose filtered sets have a row
whose top-p cut or min-p threshold lies within 1e-9 of a decision (the
oracle's filter margin: then the whole sequence is skipped, since its p or q
may legitimately differ).  Coupling sums within 1e-6 absolute plus 1e-5
relative.  Drafted tokens are drawn from the filtered q, computed here with
numpy from the definitions.
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests.test_oracle_pins_filtered import filtered

pytestmark = pytest.mark.gpu
ACC_MARGIN, DRAW_MARGIN, FILTER_MARGIN = 1e-7, 1e-9, 1e-9


@pytest.fixture(scope="module")
def g():
    import tests.gpu_helpers as G
    import vocab_row_reductions_amd as vsel
    G.vsel = vsel
    return G


def filtered_drafts(d, T, kw, seed):
    """Drafted tokens drawn from each draft row's filtered q (numpy, float64)."""
    rng = np.random.default_rng(W.BASE_SEED + seed)
    toks = [rng.choice(d["draft"].shape[1], p=filtered(row, T, **kw)) for row in d["draft"]]
    return np.asarray(toks, np.uint32)


def np_out(g, out):
    return {k: (g.u32(v) if k.startswith("tok") else v.cpu().numpy()) for k, v in out.items()}


def compare_mrs(g, oracle, d, toks, T, kw):
    B, G = d["batch"], d["gamma"]
    got = np_out(g, g.vsel.vsel_spec_accept_filtered(
        g.dev(d["target"]), g.dev(d["draft"]), g.dev(toks), g.dev(d["u_acc"]), g.dev(d["u_res"]), g.dev(d["u_bon"]),
        B, G, T, **kw))
    ref = oracle.spec_accept(d["target"], d["draft"], toks, d["u_acc"], d["u_res"], d["u_bon"], B, G, T, **kw)
    # sum p*q of the same pass against the oracle's sampler-match sums of the same filtered p and q
    rsp = oracle.spec_match(d["target"], d["draft"], toks, np.full((B, G + 1), 0.5, np.float32), B, G, T,
                            **kw)["sumprod"]
    assert np.array_equal(got["len_aa"], ref["len_aa"]) and np.array_equal(got["tok_aa"], ref["tok_aa"])
    skipped = 0
    for b in range(B):
        if ref["filter_margin"][b] < FILTER_MARGIN:
            skipped += 1
            continue
        ok = np.isfinite(ref["summin"][b])
        assert np.all(np.abs(got["summin"][b][ok] - ref["summin"][b][ok]) <= 1e-6 + 1e-5 * ref["summin"][b][ok])
        assert np.all(np.abs(got["sumprod"][b][ok] - rsp[b][ok]) <= 1e-6 + 1e-5 * rsp[b][ok])
        close = np.nonzero(ref["acc_margin"][b] < ACC_MARGIN)[0]
        if len(close):
            assert np.array_equal(got["tok_mrs"][b, :close[0]], ref["tok_mrs"][b, :close[0]])
            skipped += 1
            continue
        L = ref["len_mrs"][b]
        assert got["len_mrs"][b] == L, f"sequence {b}: accepted length ({kw})"
        if L < 0:
            assert np.all(got["tok_mrs"][b] == g.SENT)
            continue
        assert np.array_equal(got["tok_mrs"][b, :L], ref["tok_mrs"][b, :L])
        if ref["draw_margin"][b] >= DRAW_MARGIN:
            assert got["tok_mrs"][b, L] == ref["tok_mrs"][b, L], f"sequence {b}: drawn token ({kw})"
        else:
            skipped += 1
    return got, ref, skipped


def compare_sm(g, oracle, d, toks, um, T, kw):
    B, G = d["batch"], d["gamma"]
    got = np_out(g, g.vsel.vsel_spec_match_filtered(g.dev(d["target"]), g.dev(d["draft"]), g.dev(toks),
                                                     g.dev(um.reshape(-1)), B, G, T, **kw))
    ref = oracle.spec_match(d["target"], d["draft"], toks, um, B, G, T, **kw)
    skipped = 0
    for b in range(B):
        if ref["filter_margin"][b] < FILTER_MARGIN:
            skipped += 1
            continue
        ok = np.isfinite(ref["sumprod"][b])
        assert np.all(np.abs(got["sumprod"][b][ok] - ref["sumprod"][b][ok]) <= 1e-6 + 1e-5 * ref["sumprod"][b][ok])
        close = np.nonzero(ref["match_margin"][b] < DRAW_MARGIN)[0]
        if len(close):
            assert np.array_equal(got["tok_sm"][b, :close[0]], ref["tok_sm"][b, :close[0]])
            skipped += 1
            continue
        assert got["len_sm"][b] == ref["len_sm"][b], f"sequence {b}: accepted length ({kw})"
        assert np.array_equal(got["tok_sm"][b], ref["tok_sm"][b]), f"sequence {b}: tokens ({kw})"
    return got, ref, skipped


FILTERS = [dict(top_k=50, top_p=0.95),          # candidates of the per-wave top-k kernel
           dict(top_k=500, top_p=0.9, min_p=0.01),  # the workgroup top-k kernel
           dict(top_p=0.9),                     # the whole-row nucleus
           dict(min_p=0.05),                    # the whole-row threshold
           dict(top_k=20)]


@pytest.mark.parametrize("kw", FILTERS, ids=lambda k: ",".join(f"{a}={b}" for a, b in k.items()))
def test_speculative_batch(g, oracle, kw):
    d = W.speculative_batch()
    T = float(np.float32(d["temperature"]))
    toks = filtered_drafts(d, T, kw, 610)
    _, ref, skipped = compare_mrs(g, oracle, d, toks, T, kw)
    assert skipped <= 2
    um = W.uniforms(d["batch"] * (d["gamma"] + 1), seed=611).reshape(d["batch"], -1)
    _, _, skipped = compare_sm(g, oracle, d, toks, um, T, kw)
    assert skipped <= 2


@pytest.mark.parametrize("V", [7, 1000, 70001])
@pytest.mark.parametrize("ci", range(len(FILTERS)))
def test_shapes(g, oracle, V, ci):
    kw = dict(FILTERS[ci])
    d = W.speculative_batch(batch=5, gamma=3, vocab=V, seed=620 + V)
    T = float(np.float32(0.7))
    toks = filtered_drafts(d, T, kw, 621 + V)
    compare_mrs(g, oracle, d, toks, T, kw)
    um = W.uniforms(5 * 4, seed=622 + V).reshape(5, 4)
    compare_sm(g, oracle, d, toks, um, T, kw)


def test_filters_off_and_greedy_equal_the_unfiltered_rules(g):
    d = W.speculative_batch(batch=6, gamma=4, vocab=30000, seed=630)
    args = [g.dev(d[k]) for k in ("target", "draft", "tokens", "u_acc", "u_res", "u_bon")]
    um = g.dev(W.uniforms(6 * 5, seed=631))
    for T, kw in ((1.0, {}), (0.0, dict(top_k=7, top_p=0.5, min_p=0.1))):
        a = g.vsel.vsel_spec_accept(*args, 6, 4, T)
        b = g.vsel.vsel_spec_accept_filtered(*args, 6, 4, T, **kw)
        for k in a:
            assert torch.equal(a[k], b[k]), (T, k)
        a = g.vsel.vsel_spec_match(args[0], args[1], args[2], um, 6, 4, T)
        b = g.vsel.vsel_spec_match_filtered(args[0], args[1], args[2], um, 6, 4, T, **kw)
        for k in a:
            assert torch.equal(a[k], b[k]), (T, k)


def test_support_of_a_top_k_2_target_is_never_violated(g):
    """The page's regression guard, on the GPU: no emitted token outside the
    target's two largest logits, over many sequences and both rules."""
    rng = np.random.default_rng(W.BASE_SEED + 640)
    B, G, V = 512, 2, 3000
    tgt = (1.5 * rng.normal(size=(B * (G + 1), V))).astype(np.float32)
    dft = (tgt.reshape(B, G + 1, V)[:, :G] + rng.normal(0, 1.0, (B, G, V))).reshape(B * G, V).astype(np.float32)
    kw = dict(top_k=2)
    toks = np.array([rng.choice(V, p=filtered(r, 1.0, **kw)) for r in dft], np.uint32)
    u = rng.random((3, B * G), dtype=np.float32)
    top2 = np.argsort(-tgt, axis=1, kind="stable")[:, :2]
    mrs = np_out(g, g.vsel.vsel_spec_accept_filtered(g.dev(tgt), g.dev(dft), g.dev(toks), g.dev(u[0]), g.dev(u[1]),
                                                     g.dev(u[2, :B]), B, G, 1.0, **kw))
    sm = np_out(g, g.vsel.vsel_spec_match_filtered(g.dev(tgt), g.dev(dft), g.dev(toks),
                                                   g.dev(rng.random(B * (G + 1), dtype=np.float32)), B, G, 1.0, **kw))
    for tok, L in ((mrs["tok_mrs"], mrs["len_mrs"]), (sm["tok_sm"], sm["len_sm"])):
        for b in range(B):
            for i in range(L[b] + 1):
                assert tok[b, i] in top2[b * (G + 1) + i], (b, i)


def test_fail_closed(g, oracle):
    d = W.speculative_batch(batch=3, gamma=2, vocab=900, seed=650)
    d = dict(d)
    d["target"] = d["target"].copy()
    d["target"][1 * 3 + 2, 5] = np.nan           # bonus row of sequence 1
    toks = d["tokens"].copy()
    toks[2 * 2] = 900                            # out-of-range draft in sequence 2
    kw = dict(top_k=30, top_p=0.9)
    got, _, _ = compare_mrs(g, oracle, d, toks, 1.0, kw)
    assert list(got["len_mrs"][1:]) == [-1, -1]
    um = W.uniforms(3 * 3, seed=651).reshape(3, 3)
    got, _, _ = compare_sm(g, oracle, d, toks, um, 1.0, dict(top_p=0.8))
    assert list(got["len_sm"][1:]) == [-1, -1]


@pytest.mark.parametrize("kw", [dict(top_p=0.9), dict(top_p=0.5, min_p=0.02)],
                         ids=lambda k: ",".join(f"{a}={b}" for a, b in k.items()))
@pytest.mark.parametrize("T", [1.0, 0.7])
def test_wholerow_nucleus_windows(g, oracle, kw, T):
    """The whole-row nucleus of the filtered rules over rows from flat to
    peaked (each sequence's rows scaled by its own factor, 0.05 to 8), so
    that the cut windows of the floor-mode window pass differ widely in size:
    a handful of candidates in the peaked rows, thousands in the flat ones."""
    B, G, V = 6, 3, 50000
    d = W.speculative_batch(batch=B, gamma=G, vocab=V, seed=640)
    scale = np.array([0.05, 0.3, 1.0, 2.0, 4.0, 8.0], np.float32)
    tgt = (d["target"].reshape(B, G + 1, V) * scale[:, None, None]).reshape(B * (G + 1), V)
    dft = (d["draft"].reshape(B, G, V) * scale[:, None, None]).reshape(B * G, V)
    d = dict(d, target=np.ascontiguousarray(tgt, np.float32), draft=np.ascontiguousarray(dft, np.float32))
    T = float(np.float32(T))
    toks = filtered_drafts(d, T, kw, 641)
    _, _, skipped = compare_mrs(g, oracle, d, toks, T, kw)
    assert skipped <= 1
    um = W.uniforms(B * (G + 1), seed=642).reshape(B, G + 1)
    _, _, skipped = compare_sm(g, oracle, d, toks, um, T, kw)
    assert skipped <= 1
