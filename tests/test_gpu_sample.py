"""GPU parity of vsel_sample with the oracle.

Tokens bit-exact except where the oracle's float64 margin at a decision (the
draw boundary, or the top-p cut) is below 1e-9 -- there the last bits of the
two float64 evaluations may legitimately decide differently; such rows are
counted and must be rare.  Log-probabilities within 1e-5 absolute.
"""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu
MARGIN = 1e-9


@pytest.fixture(scope="module")
def g():
    import tests.gpu_helpers as G
    import vocab_row_reductions_amd as vsel
    G.vsel = vsel
    return G


def compare(g, oracle, x, T, top_k, top_p, u, ld=None, max_exempt_frac=0.02):
    xd = g.dev_rows(x, ld)
    tok, lp = g.vsel.vsel_sample(xd, T, top_k, top_p, g.dev(u), vocab=x.shape[1])
    otok, olp, om = oracle.sample(x, T, top_k, top_p, u)
    exempt = (om[:, 0] < MARGIN) | (om[:, 1] < MARGIN)
    assert exempt.mean() <= max_exempt_frac
    gt = g.u32(tok)
    assert np.array_equal(gt[~exempt], otok[~exempt]), "sampled tokens differ"
    same = (~exempt) & (otok != g.SENT)
    assert np.all(np.abs(lp.cpu().numpy()[same] - olp[same]) <= 1e-5)
    assert np.array_equal(np.isnan(lp.cpu().numpy()), np.isnan(olp))
    return gt, otok


def test_config3_sampling_rows(g, oracle):
    x, u = W.sampling_rows()
    gt, ot = compare(g, oracle, x, 0.7, 20, 0.95, u, max_exempt_frac=0.0)


def test_greedy_short_circuits_equal_argmax(g, oracle):
    x, u = W.sampling_rows(rows=16, vocab=50000, seed=31)
    xd = g.dev_rows(x)
    idx, _ = g.vsel.vsel_argmax(xd)
    for T, k in ((0.0, 20), (0.7, 1), (0.0, 0)):
        tok, lp = g.vsel.vsel_sample(xd, T, k, 1.0 if k == 0 else 0.9, g.dev(u))
        assert torch.equal(tok, idx)
        assert torch.all(lp == 0)


@pytest.mark.parametrize("V,top_k,top_p,T", [(1, 5, 0.5, 1.0), (7, 3, 0.8, 0.5), (1000, 50, 1.0, 1.3),
                                             (4097, 1024, 0.99, 0.9), (70001, 20, 0.95, 0.7),
                                             (70001, 300, 0.5, 2.0), (202048, 84, 0.9, 1.0)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_shapes_and_parameters(g, oracle, V, top_k, top_p, T, dtype):
    x, u = W.sampling_rows(rows=8, vocab=V, seed=V + top_k, masked_frac=0.01 if V > 100 else 0.0)
    if dtype == "bf16":
        x = W.f32_to_bf16_bits(x)
    compare(g, oracle, x, T, top_k, top_p, u, ld=V + 8 if dtype == "f32" else V + 3)


@pytest.mark.parametrize("V", [5, 3000, 202048])
def test_full_row_draw_in_id_order(g, oracle, V):
    x, u = W.sampling_rows(rows=12, vocab=V, seed=77 + V)
    compare(g, oracle, x, 0.8, 0, 1.0, u)
    compare(g, oracle, W.f32_to_bf16_bits(x), 1.1, 0, 1.0, u)


def test_support_never_violated(g, oracle):
    # top_k = 2: no token outside the two largest (speculative-acceptance.md, Regression guards)
    x = np.array([[0.3, 1.9, -0.4, 1.2, 0.8, -2.0]], np.float32)
    n = 4096
    u = ((np.arange(n) + 0.5) / n).astype(np.float32)
    xd = g.dev_rows(np.repeat(x, n, 0))
    tok, _ = g.vsel.vsel_sample(xd, 1.0, 2, 1.0, g.dev(u))
    assert set(np.unique(g.u32(tok)).tolist()) == {1, 3}


def test_fail_closed_rows(g, oracle):
    x, u = W.sampling_rows(rows=4, vocab=9000, seed=5)
    x[1, 10] = np.nan
    x[2, :] = -np.inf
    x[3, 5] = np.inf
    for k in (0, 1, 20):
        tok, lp = g.vsel.vsel_sample(g.dev_rows(x), 0.7, k, 1.0, g.dev(u))
        t = g.u32(tok)
        assert t[0] != g.SENT and np.all(t[1:] == g.SENT)
        assert np.all(np.isnan(lp.cpu().numpy()[1:]))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_whole_row_top_p(g, oracle, dtype):
    """top_k = 0 with top_p < 1: the nucleus over the whole row, in (value desc,
    id asc) order, as the ordered chain with top-p alone defines it."""
    x, u = W.sampling_rows(rows=64, seed=41)
    if dtype == "bf16":
        x = W.f32_to_bf16_bits(x)
    for T, top_p in ((0.7, 0.95), (1.2, 0.5)):
        tok, lp = g.vsel.vsel_sample(g.dev_rows(x), T, 0, top_p, g.dev(u), vocab=x.shape[1])
        otok, olp, om = oracle.sample_chain(x, T, u, top_p=top_p)
        exempt = np.any(om[:, :3] < MARGIN, axis=1)
        assert exempt.sum() <= 1
        gt = g.u32(tok)
        assert np.array_equal(gt[~exempt], otok[~exempt]), (T, top_p)
        assert np.all(np.abs(lp.cpu().numpy()[~exempt] - olp[~exempt]) <= 1e-5)
