"""GPU parity of vsel_argmax_excluding (the greedy serving variant) with the
oracle: bit-exact indices and status words on the same seeded rows and sets."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import tests.gpu_helpers as G
    import vocab_row_reductions_amd as vsel
    G.vsel = vsel
    return G


def run(g, xd, ex, V):
    exd = g.dev(np.asarray(ex, dtype=np.uint32).reshape(-1))
    idx, st = g.vsel.vsel_argmax_excluding(xd, exd, vocab=V)
    return g.u32(idx), g.u32(st)


def check(g, oracle, x, ex, ld=None, vocab=None):
    xd = g.dev_rows(x, ld)
    before = g.digest(xd)
    V = x.shape[1] if vocab is None else vocab
    idx, st = run(g, xd, ex, V)
    oi, os_ = oracle.argmax_excluding(x[:, :V], ex)
    assert np.array_equal(st, os_), (np.nonzero(st != os_)[0][:8], st[:8], os_[:8])
    assert np.array_equal(idx, oi), (np.nonzero(idx != oi)[0][:8], idx[:8], oi[:8])
    assert g.digest(xd) == before, "input rows were modified"
    return oi, os_


def test_config1_planted_maxima_excluded_in_turn(g, oracle):
    """The single greedy row with its planted copies of the maximum: excluding
    the lowest planted ids one after another moves the answer to another copy
    (the original occurrence is never excluded, so a copy always remains)."""
    row, planted = W.greedy_single_row()
    planted = sorted(planted)
    for n in range(len(planted) + 1):
        oi, os_ = check(g, oracle, row, planted[:n])
        assert os_[0] == 0
        assert oi[0] not in planted[:n] and row[0, oi[0]] == row.max()


@pytest.mark.parametrize("V", [1, 7, 63, 1023, 1025, 4097, 65537, 202049])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_edge_shapes(g, oracle, V, dtype):
    rng = np.random.default_rng(V + 17)
    x = (np.round(rng.normal(0, 2, (3, V)) * 4) / 4).astype(np.float32)   # coarse: many ties
    if dtype == "bf16":
        x = W.f32_to_bf16_bits(x)
    am = oracle.argmax(x)[0]
    tail = np.arange(max(0, V - 9), V, dtype=np.uint32)          # the ragged tail and its neighbours
    sets = [
        [],                                                      # empty set: the plain argmax
        am[:1],                                                  # row 0's argmax
        np.concatenate([am, tail]),                              # every row's argmax and the tail
        W.excluded_ids(V, 16, seed=V, out_of_range=3, duplicates=4),
        np.concatenate([am, W.excluded_ids(V, 256 - len(am), seed=V + 1)])[:256],   # the largest set
        np.array([V, V + 1, 0xFFFFFFFF], dtype=np.uint32),       # nothing in range
    ]
    for ld in (V, V + 3, V + 8):
        for ex in sets:
            check(g, oracle, x, np.asarray(ex, dtype=np.uint32), ld=ld)


def test_empty_set_matches_plain_argmax(g):
    rng = np.random.default_rng(3)
    x = (np.round(rng.normal(0, 2, (5, 70001)) * 8) / 8).astype(np.float32)
    xd = g.dev_rows(x)
    idx, st = run(g, xd, [], 70001)
    ref, _ = g.vsel.vsel_argmax(xd)
    assert np.array_equal(idx, g.u32(ref)) and not st.any()


def test_status_words(g, oracle):
    V = 9000
    rng = np.random.default_rng(11)
    x = rng.normal(0, 1, (9, V)).astype(np.float32)
    ex = np.array([5, 4321, 17, 8999, 100], dtype=np.uint32)
    x[0, 4321] = np.nan                 # NaN at an excluded id: still fails closed
    x[1, 17] = np.inf                   # +inf at an excluded id: still fails closed
    x[2, 6000] = np.nan                 # NaN elsewhere
    x[3, :] = -np.inf                   # nothing above -inf
    x[4, :] = -np.inf
    x[4, 8999] = 2.0                    # the only finite element is excluded: no candidate
    x[5, :] = -np.inf
    x[5, 8998] = -7.0                   # the element next to an excluded one survives
    x[6, 100] = 50.0                    # an excluded maximum
    x[7, 5] = -np.inf                   # -inf at an excluded id is fine
    x[8, :] = 1.0                       # all equal: first non-excluded index (0)
    oi, os_ = check(g, oracle, x, ex)
    assert list(os_) == [1, 1, 1, 2, 2, 0, 0, 0, 0]
    assert oi[5] == 8998 and oi[6] != 100 and oi[8] == 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_every_element_excluded(g, oracle, dtype):
    for V in (1, 5, 64, 200, 256):
        x = np.random.default_rng(V).normal(0, 1, (2, V)).astype(np.float32)
        if dtype == "bf16":
            x = W.f32_to_bf16_bits(x)
        ex = np.arange(V, dtype=np.uint32)[::-1].copy()
        oi, os_ = check(g, oracle, x, ex)
        assert (os_ == 2).all() and (oi == g.SENT).all()


def test_segmented_rows(g, oracle):
    """Few long rows split over several workgroups each, with the argmax and
    its tied copies excluded in different segments."""
    for rep in range(6):
        rng = np.random.default_rng(500 + rep)
        rows = int(rng.integers(1, 4))
        V = int(rng.integers(150000, 260000))
        x = (np.round(rng.normal(0, 3, (rows, V)) * 16) / 16).astype(np.float32)
        m = x.max(axis=1)
        cols = rng.integers(0, V, size=(rows, 4))
        for r in range(rows):
            x[r, cols[r]] = m[r]
        ex = np.concatenate([cols.reshape(-1), oracle.argmax(x)[0]]).astype(np.uint32)
        check(g, oracle, x, ex[: int(rng.integers(1, ex.size + 1))])


def test_decode_batch_bf16_full_size(g, oracle):
    """The 1024 x 202048 bf16 batch at its padded stride with a 16-id set that
    holds the argmax of 12 rows."""
    bits, _ = W.decode_batch_bf16()
    V = W.V_DECODE
    am = oracle.argmax(bits[:, :V], nthreads=8)[0]
    ex = np.concatenate([am[::90][:12], W.excluded_ids(V, 4, seed=99)]).astype(np.uint32)
    xd = torch.from_numpy(bits.view(np.int16)).to(g.DEV).view(torch.bfloat16)
    idx, st = run(g, xd, ex, V)
    oi, os_ = oracle.argmax_excluding(bits[:, :V], ex, nthreads=8)
    assert np.array_equal(st, os_) and np.array_equal(idx, oi)
    assert (idx[::90][:12] != am[::90][:12]).all()


def test_rejected_arguments(g):
    xd = g.dev_rows(np.zeros((2, 100), np.float32))
    with pytest.raises(g.vsel.VselError):
        g.vsel.vsel_argmax_excluding(xd, g.dev(np.zeros(257, np.uint32)))
