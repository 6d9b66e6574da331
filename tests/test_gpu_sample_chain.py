"""GPU parity of vsel_sample_chain (the ordered sampler chain: top-n-sigma,
top-k, typical-p, top-p, min-p, then the temperature) with the oracle.

Tokens bit-exact except on rows where one of the oracle's float64 margins is
below 1e-9: the draw boundary, the typical-p or top-p cut, or the distance of
the top-n-sigma or min-p threshold to the nearest candidate value.  There the
last bits of two float64 evaluations (a different summation order for sigma,
another libm for exp and log) may legitimately decide differently; such rows
are counted and must be rare.  Log-probabilities within 1e-5 absolute.
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


def compare(g, oracle, x, T, u, ld=None, max_exempt_frac=0.02, exact_thresholds=False, **kw):
    """exact_thresholds: the rows' thresholds are exact on both sides (sigma 0,
    min_p 1), so an element lying on one is no reason to exempt the row.
    Every margin, the typicality-score gap beside the typical cut or the draw
    included, is the oracle's float64 margin of 1e-9."""
    xd = g.dev_rows(x, ld)
    tok, lp = g.vsel.vsel_sample_chain(xd, T, g.dev(u), vocab=x.shape[1], **kw)
    otok, olp, om = oracle.sample_chain(x, T, u, **kw)
    exempt = np.any((om[:, :3] if exact_thresholds else om[:, :5]) < MARGIN, axis=1) | (om[:, 5] < MARGIN)
    print(f"chain {kw} T={T} rows={len(otok)}: {int(exempt.sum())} exempt", flush=True)
    assert exempt.mean() <= max_exempt_frac, f"{exempt.sum()} rows within {MARGIN} of a decision"
    gt = g.u32(tok)
    bad = np.nonzero((gt != otok) & ~exempt)[0]
    assert len(bad) == 0, f"rows {bad[:8]}: gpu {gt[bad[:8]]} oracle {otok[bad[:8]]} ({kw})"
    same = (~exempt) & (otok != g.SENT)
    lpn = lp.cpu().numpy()
    assert np.all(np.abs(lpn[same] - olp[same]) <= 1e-5)
    assert np.array_equal(np.isnan(lpn), np.isnan(olp))
    return gt, otok


CHAINS = [
    dict(top_n_sigma=1.0, top_k=50, typical_p=0.9, top_p=0.95, min_p=0.05),
    dict(top_n_sigma=1.5),                                   # whole row, one threshold
    dict(min_p=0.1),
    dict(top_n_sigma=0.5, min_p=0.02),
    dict(top_k=100, typical_p=0.7),
    dict(top_k=128, typical_p=0.5, top_p=0.8, min_p=0.05, top_n_sigma=2.0),
    dict(top_k=500, top_n_sigma=1.0, min_p=0.01, top_p=0.9),  # k above the per-wave kernel's range
    dict(top_k=1024, min_p=0.2),
    dict(top_k=20, top_p=0.95),                              # the plain sampler's chain
    dict(top_k=300, typical_p=0.5),                          # typical-p on the workgroup kernel's candidates
    dict(top_k=1024, typical_p=0.8, top_p=0.9, min_p=0.01),
]


def test_config3_rows_full_chain(g, oracle):
    x, u = W.sampling_rows()
    compare(g, oracle, x, 0.7, u, max_exempt_frac=0.0, **CHAINS[0])


@pytest.mark.parametrize("ci", range(len(CHAINS)))
@pytest.mark.parametrize("V", [7, 1000, 70001, 202048])
def test_chains_over_shapes_f32(g, oracle, ci, V):
    kw = dict(CHAINS[ci])
    if kw.get("top_k", 0) > V:
        kw["top_k"] = V
    x, u = W.sampling_rows(rows=8, vocab=V, seed=300 + V + ci, masked_frac=0.01 if V > 100 else 0.0)
    compare(g, oracle, x, 0.9, u, ld=V + 8, **kw)


@pytest.mark.parametrize("ci", [0, 1, 3, 5, 6])
@pytest.mark.parametrize("ld_pad", [0, 3])
def test_chains_bf16(g, oracle, ci, ld_pad):
    """bf16 rows; an odd stride sends every top-k to the workgroup kernel."""
    V = 50021
    x, u = W.sampling_rows(rows=8, vocab=V, seed=400 + ci + ld_pad)
    xb = W.f32_to_bf16_bits(x)
    compare(g, oracle, xb, 1.2, u, ld=V + ld_pad, **CHAINS[ci])


def test_reduces_to_vsel_sample(g):
    x, u = W.sampling_rows(rows=16, vocab=30000, seed=401)
    xd, ud = g.dev_rows(x), g.dev(u)
    for top_k, top_p in ((20, 0.95), (0, 1.0), (300, 0.5), (128, 1.0)):
        a = g.vsel.vsel_sample(xd, 0.8, top_k, top_p, ud)
        b = g.vsel.vsel_sample_chain(xd, 0.8, ud, top_k=top_k, top_p=top_p)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_greedy_limits(g):
    x, u = W.sampling_rows(rows=16, vocab=9000, seed=402)
    xd, ud = g.dev_rows(x), g.dev(u)
    idx, _ = g.vsel.vsel_argmax(xd)
    for T, kw in ((0.0, dict(top_n_sigma=1.0, min_p=0.1)), (0.7, dict(top_k=1, typical_p=0.5)),
                  (0.0, dict(top_k=40, typical_p=0.3, top_p=0.2))):
        tok, lp = g.vsel.vsel_sample_chain(xd, T, ud, **kw)
        assert torch.equal(tok, idx) and torch.all(lp == 0)


def test_threshold_edge_rows(g, oracle):
    """Rows with one finite element (sigma 0), a large common offset (sigma
    from shifted sums), many ties at the maximum, and min_p = 1 (only the
    maximum's ties survive)."""
    V = 5000
    rng = np.random.default_rng(W.BASE_SEED + 403)
    x = rng.normal(0.0, 1.0, (6, V)).astype(np.float32)
    x[0, :] = -np.inf
    x[0, 1234] = 2.5                                   # sigma 0: only the maximum
    x[1] += np.float32(3000.0)                         # large offset
    x[2, ::7] = np.float32(6.0)                        # ties at the maximum
    x[3, :] = np.round(x[3] * 4) / 4                   # coarse grid: many equal values
    u = rng.random(6, dtype=np.float32)
    compare(g, oracle, x, 1.0, u, max_exempt_frac=0.0, exact_thresholds=True, top_n_sigma=1.0)
    compare(g, oracle, x, 1.0, u, max_exempt_frac=0.0, exact_thresholds=True, min_p=1.0)
    compare(g, oracle, x, 0.5, u, max_exempt_frac=0.0, exact_thresholds=True, top_k=64, top_n_sigma=0.3, min_p=0.5)
    tok, _ = g.vsel.vsel_sample_chain(g.dev_rows(x), 1.0, g.dev(u), min_p=1.0)
    assert g.u32(tok)[0] == 1234 and g.u32(tok)[2] % 7 == 0


def test_fail_closed(g, oracle):
    x, u = W.sampling_rows(rows=4, vocab=3000, seed=404)
    x = x.copy()
    x[1, 17] = np.nan
    x[2, 5] = np.inf
    for kw in (dict(top_n_sigma=1.0, min_p=0.1), dict(top_k=30, typical_p=0.8, top_n_sigma=1.0)):
        gt, _ = compare(g, oracle, x, 0.8, u, **kw)
        assert gt[1] == g.SENT and gt[2] == g.SENT and gt[0] != g.SENT


def test_support_of_each_filter(g):
    """Over a grid of uniforms, every drawn token lies in the filter's kept set
    (computed here with numpy), and every kept token is drawn."""
    z = np.array([2.0, 1.5, 1.4, 0.2, -0.5, -1.0, -3.0, -6.0], np.float32)
    n = 8192
    u = ((np.arange(n) + 0.5) / n).astype(np.float32)
    xd = g.dev_rows(np.repeat(z[None], n, 0))
    zz = z.astype(np.float64)
    cases = [(dict(min_p=0.3), np.nonzero(np.exp(zz - zz.max()) >= 0.3)[0]),
             (dict(top_n_sigma=1.0), np.nonzero(zz >= zz.max() - np.std(zz))[0]),
             (dict(top_k=6, top_n_sigma=0.8, min_p=0.1),
              np.nonzero((zz >= zz.max() - 0.8 * np.std(zz)) & (np.exp(zz - zz.max()) >= 0.1))[0])]
    for kw, kept in cases:
        tok, _ = g.vsel.vsel_sample_chain(xd, 1.0, g.dev(u), **kw)
        assert set(np.unique(g.u32(tok)).tolist()) == set(kept.tolist()), kw


# ---- top-p over whole rows (top_k = 0): the weighted selections in value order
ROW_NUCLEUS = [dict(top_p=0.9), dict(top_p=0.95, min_p=0.05), dict(top_p=0.5, top_n_sigma=1.0),
               dict(top_p=0.99, top_n_sigma=2.0, min_p=0.001), dict(top_p=0.3)]


def test_whole_row_top_p_sampling_rows(g, oracle):
    x, u = W.sampling_rows()
    compare(g, oracle, x, 0.7, u, max_exempt_frac=0.0, top_p=0.95)
    compare(g, oracle, x, 1.3, u, max_exempt_frac=0.0, top_p=0.9, top_n_sigma=1.5, min_p=0.01)


@pytest.mark.parametrize("ci", range(len(ROW_NUCLEUS)))
@pytest.mark.parametrize("V", [1, 7, 1000, 70001, 202048])
def test_whole_row_top_p_shapes(g, oracle, ci, V):
    x, u = W.sampling_rows(rows=8, vocab=V, seed=500 + V + ci, masked_frac=0.01 if V > 100 else 0.0)
    # one element: sigma is 0 on both sides, the threshold sits on the maximum exactly
    compare(g, oracle, x, 0.8, u, ld=V + 5, exact_thresholds=(V == 1), **ROW_NUCLEUS[ci])


@pytest.mark.parametrize("sd,top_p", [(0.3, 0.9), (1.0, 0.5), (0.05, 0.999), (3.0, 0.97)])
def test_whole_row_top_p_large_nuclei(g, oracle, sd, top_p):
    """Flat rows: the nucleus and the draw window hold far more candidates than
    one workgroup sorts, so the window is narrowed by key passes."""
    rng = np.random.default_rng(W.BASE_SEED + int(sd * 100) + int(top_p * 1000))
    x = rng.normal(0.0, sd, (6, W.V_DECODE)).astype(np.float32)
    u = rng.random(6, dtype=np.float32)
    compare(g, oracle, x, 1.0, u, top_p=top_p)
    compare(g, oracle, x, 0.5, u, top_p=top_p, min_p=0.5)


def test_whole_row_top_p_ties(g, oracle):
    """Equal values: the cut and the draw fall inside runs of ties, which only
    the ids order (key passes over the id bits)."""
    V = 7777
    rng = np.random.default_rng(W.BASE_SEED + 510)
    x = np.zeros((5, V), np.float32)
    x[1] = np.round(rng.normal(0, 1, V) * 2) / 2        # a few distinct values
    x[2, ::3] = 1.0                                     # two values
    x[3] = rng.normal(0, 1, V).astype(np.float32)
    x[3, 100:4200] = x[3].max()                         # 4,100 tied maxima
    x[4, :] = -np.inf
    x[4, 17] = 0.5                                      # one candidate
    u = rng.random(5, dtype=np.float32)
    for T, top_p in ((1.0, 0.9), (0.6, 0.37), (2.0, 0.999)):
        compare(g, oracle, x, T, u, max_exempt_frac=0.0, top_p=top_p)
    # the largest tie: the whole 202,048-element row equal
    xe = np.full((2, W.V_DECODE), 0.25, np.float32)
    compare(g, oracle, xe, 1.0, np.array([0.3, 0.8], np.float32), max_exempt_frac=0.0, top_p=0.9)


@pytest.mark.parametrize("ld_pad", [0, 3])
def test_whole_row_top_p_bf16(g, oracle, ld_pad):
    V = 50021
    x, u = W.sampling_rows(rows=8, vocab=V, seed=520 + ld_pad)
    compare(g, oracle, W.f32_to_bf16_bits(x), 1.1, u, ld=V + ld_pad, top_p=0.9, min_p=0.02)
    flat = np.random.default_rng(W.BASE_SEED + 521).normal(0, 0.5, (4, V)).astype(np.float32)
    compare(g, oracle, W.f32_to_bf16_bits(flat), 1.0, u[:4], ld=V + ld_pad, top_p=0.8)


def test_whole_row_top_p_fail_closed(g, oracle):
    x, u = W.sampling_rows(rows=4, vocab=3000, seed=530)
    x = x.copy()
    x[1, 17] = np.nan
    x[2, :] = -np.inf
    gt, _ = compare(g, oracle, x, 0.8, u, top_p=0.9, top_n_sigma=1.0)
    assert gt[1] == g.SENT and gt[2] == g.SENT and gt[0] != g.SENT


# ---- typical-p over whole rows (top_k = 0): the typical order is the distance
# to the p-weighted mean logit (float64, mantissa cut to 30 bits on the device)
TYP = [dict(typical_p=0.9), dict(typical_p=0.5, top_p=0.9), dict(typical_p=0.8, min_p=0.05),
       dict(typical_p=0.95, top_p=0.8, min_p=0.02, top_n_sigma=2.0), dict(typical_p=0.3)]


@pytest.mark.parametrize("ci", range(len(TYP)))
@pytest.mark.parametrize("V", [7, 1000, 70001, 202048])
def test_whole_row_typical_shapes(g, oracle, ci, V):
    x, u = W.sampling_rows(rows=8, vocab=V, seed=700 + V + ci, masked_frac=0.01 if V > 100 else 0.0)
    compare(g, oracle, x, 0.8, u, ld=V + 5, **TYP[ci])


def test_whole_row_typical_sampling_rows(g, oracle):
    x, u = W.sampling_rows()
    compare(g, oracle, x, 0.7, u, max_exempt_frac=0.0, typical_p=0.9)
    compare(g, oracle, x, 1.0, u, max_exempt_frac=0.0, typical_p=0.7, top_p=0.95, min_p=0.01)


def test_whole_row_typical_ties(g, oracle):
    """Equal values share a typicality score, so the cut and the draw fall inside
    runs of ties that only the ids order: windows far larger than LDS holds,
    narrowed by one workgroup's key passes."""
    V = 7777
    rng = np.random.default_rng(W.BASE_SEED + 720)
    x = np.zeros((5, V), np.float32)
    x[1] = np.round(rng.normal(0, 1, V) * 2) / 2        # a few distinct values
    x[2, ::3] = 1.0                                     # two values
    x[3] = rng.normal(0, 1, V).astype(np.float32)
    x[3, 100:4200] = x[3].max()                         # 4,100 tied maxima
    x[4, :] = -np.inf
    x[4, 17] = 0.5                                      # one candidate
    u = rng.random(5, dtype=np.float32)
    for T, kw in ((1.0, dict(typical_p=0.9)), (0.6, dict(typical_p=0.37, top_p=0.8)),
                  (2.0, dict(typical_p=0.999, min_p=0.1))):
        compare(g, oracle, x, T, u, max_exempt_frac=0.0, **kw)
    # the largest tie: the whole 202,048-element row equal
    xe = np.full((2, W.V_DECODE), 0.25, np.float32)
    compare(g, oracle, xe, 1.0, np.array([0.3, 0.8], np.float32), max_exempt_frac=0.0,
            typical_p=0.9)


@pytest.mark.parametrize("ld_pad", [0, 3])
def test_whole_row_typical_bf16_and_flat(g, oracle, ld_pad):
    """bf16 rows (runs of equal values: equal scores, ordered by id) and flat
    rows (typical sets far larger than one workgroup sorts)."""
    V = 50021
    x, u = W.sampling_rows(rows=8, vocab=V, seed=710 + ld_pad)
    compare(g, oracle, W.f32_to_bf16_bits(x), 1.1, u, ld=V + ld_pad,
            typical_p=0.9, top_p=0.95)
    flat = np.random.default_rng(W.BASE_SEED + 711).normal(0, 0.3, (4, V)).astype(np.float32)
    compare(g, oracle, flat, 1.0, u[:4], ld=V + ld_pad, typical_p=0.6)
