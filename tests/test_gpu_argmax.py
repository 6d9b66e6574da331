"""GPU parity of vsel_argmax with the oracle (bit-exact indices and values)."""
import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import tests.gpu_helpers as G
    import vocab_row_reductions_amd as vsel
    G.vsel = vsel
    return G


def check(g, oracle, x, ld=None, vocab=None):
    xd = g.dev_rows(x, ld)
    before = g.digest(xd)
    V = x.shape[1] if vocab is None else vocab
    idx, val = g.vsel.vsel_argmax(xd, vocab=V)
    oi, ov = oracle.argmax(x[:, :V])
    assert np.array_equal(g.u32(idx), oi)
    ok = oi != g.SENT
    assert np.array_equal(g.bits(val)[ok], ov.view(np.uint32)[ok])
    assert g.digest(xd) == before, "input rows were modified"


def test_config1_planted_first_maximum(g, oracle):
    row, planted = W.greedy_single_row()
    xd = g.dev_rows(row)
    idx, val = g.vsel.vsel_argmax(xd)
    assert g.u32(idx)[0] == min(planted) == oracle.argmax(row)[0][0]
    assert val.cpu().numpy()[0] == row.max()


@pytest.mark.parametrize("V", [1, 7, 63, 1023, 1024, 1025, 4097, 65537, 202049])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_edge_shapes(g, oracle, V, dtype):
    rng = np.random.default_rng(V)
    x = (np.round(rng.normal(0, 2, (3, V)) * 4) / 4).astype(np.float32)   # coarse: many ties
    if dtype == "bf16":
        x = W.f32_to_bf16_bits(x)
    for ld in (V, V + 3, V + 8):
        check(g, oracle, x, ld=ld)


def test_special_rows(g, oracle):
    V = 9000
    rng = np.random.default_rng(5)
    x = rng.normal(0, 1, (8, V)).astype(np.float32)
    x[0, 4321] = np.nan
    x[1, 17] = np.inf
    x[2, :] = -np.inf
    x[3, :] = -np.inf
    x[3, 8999] = -5.0
    x[4, :] = 0.0
    x[4, 100] = -0.0
    x[5, :] = -0.0
    x[6, ::2] = -np.inf
    x[7, :] = 3.0                     # all equal: first index
    check(g, oracle, x)


def test_many_rows_repeated_calls(g, oracle):
    # Many workgroups per row and back-to-back calls: the per-row tickets
    # must reset and partials must be visible across XCDs every time.
    for rep in range(20):
        rng = np.random.default_rng(1000 + rep)
        rows = int(rng.integers(1, 40))
        V = int(rng.integers(20000, 120000))
        x = (np.round(rng.normal(0, 3, (rows, V)) * 16) / 16).astype(np.float32)
        check(g, oracle, x)
