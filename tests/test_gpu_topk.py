"""GPU parity of vsel_topk (fused top-k + argmax + log-sum-exp) with the oracle.

Bit-exact: ids, values (the row's own bits) and argmax.  Log-sum-exp within
1e-5 absolute (p = exp(z - lse), so this is the 1e-5 relative probability
tolerance) plus the rounding of the float32 output, 2^-23 |lse|.  The
full-size bf16 batch is compared on every row, and checked through
properties as well.
"""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu
LSE_TOL = 1e-5


def lse_ok(got, ref):
    return np.abs(got - ref) <= LSE_TOL + np.abs(ref) * 2.0 ** -23


@pytest.fixture(scope="module")
def g():
    import tests.gpu_helpers as G
    import vocab_row_reductions_amd as vsel
    G.vsel = vsel
    return G


def compare(g, oracle, x, k, ld=None, rows=None):
    xd = g.dev_rows(x, ld)
    before = g.digest(xd)
    vals, ids, am, lse = g.vsel.vsel_topk(xd, k, vocab=x.shape[1])
    sel = slice(None) if rows is None else rows
    ov, oi, oam, olse = oracle.topk(x[sel], k)
    gi, gv = g.u32(ids)[sel], g.bits(vals)[sel]
    bad = oi[:, 0] == g.SENT
    assert np.array_equal(gi[bad, 0], oi[bad, 0])
    assert np.array_equal(gi[~bad], oi[~bad]), "top-k ids differ"
    assert np.array_equal(gv[~bad], ov[~bad].view(np.uint32)), "top-k values differ"
    assert np.array_equal(g.u32(am)[sel], oam), "argmax differs"
    gl = lse.cpu().numpy()[sel]
    fin = np.isfinite(olse)
    assert np.all(lse_ok(gl[fin], olse[fin]))
    assert np.array_equal(np.isnan(gl), np.isnan(olse)) and np.array_equal(np.isneginf(gl), np.isneginf(olse))
    assert g.digest(xd) == before
    return vals, ids, am, lse


def test_config2_verify_rows_49(g, oracle):
    x = W.verify_topk_rows(rows=49)
    vals, ids, _, _ = compare(g, oracle, x, 84)
    # the five +8 spikes of every row are among its candidates
    assert np.all((vals.cpu().numpy() > 6).sum(axis=1) >= 5)


def test_config2_verify_rows_3(g, oracle):
    compare(g, oracle, W.verify_topk_rows(rows=3), 84)


@pytest.mark.parametrize("k", [64, 84])
def test_config5_bf16_batch_full_size(g, oracle, k):
    bits, dup_rows = W.decode_batch_bf16()
    rows, ld = bits.shape
    V = W.V_DECODE
    xd = torch.from_numpy(bits.view(np.int16)).to(g.DEV).view(torch.bfloat16)
    vals, ids, am, lse = g.vsel.vsel_topk(xd, k, vocab=V)
    torch.cuda.synchronize()
    # every row against the oracle, in the launch configuration the benchmark
    # times (the duplicated maxima of 10% of the rows are bf16 ties at the top)
    ov, oi, oam, olse = oracle.topk(bits, k, vocab=V)
    gi, gv, ga = g.u32(ids), g.bits(vals), g.u32(am)
    for name, got, ref in (("ids", gi, oi), ("values", gv, ov.view(np.uint32)), ("argmax", ga, oam)):
        bad = np.nonzero(np.any((got != ref).reshape(rows, -1), axis=1))[0]
        assert len(bad) == 0, f"{name} differ on {len(bad)} rows, first {bad[:5]}"
    assert np.all(lse_ok(lse.cpu().numpy(), olse))
    # the rows with a copied maximum: a tie at the top, the lower id first
    assert len(dup_rows) > 0 and np.all(gv[dup_rows, 0] == gv[dup_rows, 1])
    assert np.all(gi[dup_rows, 0] < gi[dup_rows, 1])
    # properties on every row (float32 on the device, exact comparisons only)
    xf = xd[:, :V].float()
    v = vals
    assert torch.all(v[:, :-1] >= v[:, 1:])
    gathered = torch.gather(xf, 1, ids.long())
    assert torch.equal(gathered.view(torch.int32), v.view(torch.int32))
    kth = v[:, -1:]
    assert torch.all((xf > kth).sum(1) < k) and torch.all((xf >= kth).sum(1) >= k)
    assert torch.equal(am, ids[:, 0])
    rmax, _ = xf.max(1)
    assert torch.equal(v[:, 0], rmax)
    # the pad elements (bf16 NaN) were never read: no row latched
    assert not torch.any(ids[:, 0] == -1)


@pytest.mark.parametrize("V,k", [(1, 1), (7, 3), (7, 7), (63, 63), (1024, 64), (1025, 84), (4097, 1024),
                                 (5000, 1), (70001, 84), (70001, 256), (70001, 300), (202049, 1024)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_edge_shapes_and_k(g, oracle, V, k, dtype):
    rng = np.random.default_rng(V * 7 + k)
    x = (np.round(rng.normal(0, 2, (3, V)) * 8) / 8).astype(np.float32)
    if dtype == "bf16":
        x = W.f32_to_bf16_bits(x)
    for ld in (V, V + 1, V + 8):
        compare(g, oracle, x, k, ld=ld)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_adversarial_rows(g, oracle, dtype):
    V = 50000
    rng = np.random.default_rng(9)
    x = rng.normal(0, 1, (11, V)).astype(np.float32)
    x[0, :] = 1.5                                   # all equal: every element ties
    x[1, :] = np.arange(V, dtype=np.float32)        # ascending: the threshold keeps rising
    x[2, :] = -np.arange(V, dtype=np.float32)       # descending
    x[3, :] = -np.inf                               # all masked: ids 0..k-1, no argmax
    x[4, ::3] = -np.inf
    x[4, 1::3] = -np.inf                            # a third finite
    x[5, 777] = np.nan                              # fail closed
    x[6, 123] = np.inf                              # fail closed
    x[7, :] = 0.0
    x[7, ::2] = -0.0                                # signed zeros tie
    x[8, :] = np.round(x[8, :])                     # few distinct values
    x[9, 40000:] = 100.0                            # the winners all in the last segment
    x[10, :] = rng.normal(0, 1e30, V)               # huge magnitudes: the exp offset moves far
    if dtype == "bf16":
        x = W.f32_to_bf16_bits(x)
    for k in (1, 20, 84, 128, 129, 300, 1024):
        compare(g, oracle, x, k)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ascending_rows_with_a_ragged_end(g, oracle, dtype):
    """Ascending rows whose length is not a whole number of 16-byte groups:
    the candidate lists stay long to the end, and the last few elements (the
    largest) are added after the last flush."""
    for V in (50003, 202045, 4099):
        x = np.tile(np.arange(V, dtype=np.float32), (4, 1))
        x[1] = np.round(x[1] / 3)                   # runs of three equal values
        x[2] = x[2] * 1e-3 - 7.0
        x[3, -3:] = x[3, :3]                        # the smallest at the very end
        if dtype == "bf16":
            x = W.f32_to_bf16_bits(x)
        for k in (1, 20, 84, 128):
            compare(g, oracle, x, min(k, V), ld=(V + 7) // 8 * 8)   # 16-byte aligned rows: the per-wave kernel


def test_back_to_back_calls_reuse_workspace(g, oracle):
    for rep in range(12):
        rng = np.random.default_rng(500 + rep)
        rows = int(rng.integers(1, 64))
        V = int(rng.integers(3000, 150000))
        k = int(rng.choice([1, 20, 64, 84, 200]))
        x = (np.round(rng.normal(0, 3, (rows, V)) * 32) / 32).astype(np.float32)
        compare(g, oracle, x, min(k, V))


def compare_no_lse(g, oracle, x, k, ld=None):
    """vsel_topk without a log-sum-exp output: the plain fused kernel, whose
    segment-final partial tile is loaded in one round trip."""
    xd = g.dev_rows(x, ld)
    vals, ids, am, lse = g.vsel.vsel_topk(xd, k, vocab=x.shape[1], want_lse=False)
    assert lse is None
    ov, oi, oam, _ = oracle.topk(x, k)
    gi, gv = g.u32(ids), g.bits(vals)
    bad = oi[:, 0] == g.SENT
    assert np.array_equal(gi[bad, 0], oi[bad, 0])
    assert np.array_equal(gi[~bad], oi[~bad]), "top-k ids differ"
    assert np.array_equal(gv[~bad], ov[~bad].view(np.uint32)), "top-k values differ"
    assert np.array_equal(g.u32(am), oam), "argmax differs"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_partial_tiles_without_lse(g, oracle, dtype):
    """Rows whose segments end in partial tiles of every size, through the
    kernel without log-sum-exp: constant rows stage every group of that tile
    (the staging list overflows and the tile is read again, bounded by the
    row's end), ascending rows keep their largest elements in it, and few rows
    of 248,320 make the last segment a partial tile alone."""
    rng = np.random.default_rng(77)
    for V in (4099, 50003, 202045, 202048, 248320):
        x = rng.normal(0, 1, (6, V)).astype(np.float32)
        x[0, :] = 1.5
        x[1, :] = np.arange(V, dtype=np.float32)
        tail = min(5000, V // 2)
        x[2, -tail:] = 50.0 + np.arange(tail, dtype=np.float32)  # the winners in the partial tile
        x[3, :] = np.round(x[3, :])
        x[4, ::2] = -np.inf
        if dtype == "bf16":
            x = W.f32_to_bf16_bits(x)
        for k in (1, 20, 84, 128):
            compare_no_lse(g, oracle, x, min(k, V), ld=(V + 7) // 8 * 8)
    x = W.verify_topk_rows(rows=3)
    for k in (20, 84):
        compare_no_lse(g, oracle, x, k)
