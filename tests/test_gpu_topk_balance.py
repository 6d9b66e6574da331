"""GPU parity of vsel_topk on large batches whose rows cost very different
amounts of candidate work (rising ramps keep raising the threshold, so their
workgroups stage and select far more candidates than those of noise rows).
The slow rows must give exactly the oracle's top-k, and every output (the
log-sum-exp included) must be the same bit for bit from call to call.
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


def uneven_batch(rows, vocab, dtype, seed):
    """Mostly N(0, 4^2) rows; every eighth row is a rising ramp with noise,
    which keeps raising the threshold, so its workgroup stages and selects far
    more candidates and finishes late."""
    rng = np.random.default_rng(seed)
    x = rng.normal(0.0, 4.0, (rows, vocab)).astype(np.float32)
    slow = np.arange(3, rows, 8)
    ramp = np.linspace(-60.0, 60.0, vocab, dtype=np.float32)
    x[slow] = ramp[None, :] + rng.normal(0.0, 0.25, (slow.size, vocab)).astype(np.float32)
    if dtype == "bf16":
        return W.f32_to_bf16_bits(x), slow
    return x, slow


def run(g, xd, k, V):
    vals, ids, am, lse = g.vsel.vsel_topk(xd, k, vocab=V)
    torch.cuda.synchronize()
    return [t.clone() for t in (vals, ids, am, lse)]


@pytest.mark.parametrize("dtype,rows,vocab,k", [("bf16", 512, 202048, 84), ("f32", 256, 131072, 64)])
def test_uneven_rows_match_the_oracle_and_repeat(g, oracle, dtype, rows, vocab, k):
    x, slow = uneven_batch(rows, vocab, dtype, seed=rows + k)
    xd = g.dev_rows(x)
    outs = [run(g, xd, k, vocab) for _ in range(3)]
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), "outputs differ between calls"
    vals, ids, am, lse = outs[0]
    rng = np.random.default_rng(7)
    sample = np.unique(np.concatenate([slow, rng.choice(rows, 24, replace=False)]))
    ov, oi, oam, olse = oracle.topk(x[sample], k, nthreads=8)
    assert np.array_equal(g.u32(ids)[sample], oi), "top-k ids differ"
    assert np.array_equal(g.bits(vals)[sample], ov.view(np.uint32)), "top-k values differ"
    assert np.array_equal(g.u32(am)[sample], oam), "argmax differs"
    assert np.all(lse_ok(lse.cpu().numpy()[sample], olse))


def test_decode_batch_repeats_bit_for_bit(g):
    bits, _ = W.decode_batch_bf16()
    xd = torch.from_numpy(bits.view(np.int16)).to(g.DEV).view(torch.bfloat16)
    outs = [run(g, xd, 84, W.V_DECODE) for _ in range(4)]
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), "outputs differ between calls"
