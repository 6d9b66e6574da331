"""The allocation-free top-k (vsel_topk_noalloc) against vsel_topk.

vsel_topk_noalloc runs the same kernels with their scratch in the library's
fixed device array.  Its outputs must equal vsel_topk's bit for bit (ids,
values, argmax and the log-sum-exp's float32 bits) on consecutive calls of
different shapes sharing that array: the large decode batch, then smaller
multi-segment verify rows (whose partial records live in the array), then
the large batch again, then a call at the row limit.  The verify rows are
also checked against the oracle.
"""
import ctypes as C

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


def same(g, x, k, vocab=None):
    print(f"noalloc: rows {x.shape[0]} ld {x.shape[1]} vocab {vocab} k {k} {x.dtype}", flush=True)
    a = g.vsel.vsel_topk(x, k, vocab=vocab)
    b = g.vsel.vsel_topk_noalloc(x, k, vocab=vocab)
    torch.cuda.synchronize()
    for name, p, q in zip(("vals", "ids", "argmax", "lse"), a, b):
        assert np.array_equal(g.bits(p), g.bits(q)), f"{name} differ from vsel_topk"
    return b


def test_noalloc_equals_topk_on_consecutive_calls(g, oracle):
    bits, _ = W.decode_batch_bf16()
    big = torch.from_numpy(bits.view(np.int16)).to(g.DEV).view(torch.bfloat16)
    same(g, big, 84, vocab=W.V_DECODE)
    # second call, smaller input: 3 verify rows of 248,320 float32, split into
    # segments whose records go through the scratch array
    x = W.verify_topk_rows(rows=3)
    vals, ids, am, lse = same(g, g.dev_rows(x), 84)
    ov, oi, oam, olse = oracle.topk(x, 84)
    assert np.array_equal(g.u32(ids), oi)
    assert np.array_equal(g.bits(vals), ov.view(np.uint32))
    assert np.array_equal(g.u32(am), oam)
    assert np.all(np.abs(lse.cpu().numpy() - olse) <= 1e-5 + np.abs(olse) * 2.0 ** -23)
    # the same shapes again (the kernels left the counters at zero), then k = 64
    same(g, g.dev_rows(x), 84)
    same(g, big, 64, vocab=W.V_DECODE)


def test_noalloc_at_the_row_limit(g):
    rows = g.vsel.NOALLOC_MAX_ROWS
    x = np.random.default_rng(7).standard_normal((rows, 1000)).astype(np.float32)
    same(g, g.dev_rows(x), 16)
    same(g, g.dev_rows(x[:5]), 16)


def test_noalloc_rejects_rows_beyond_the_limit(g):
    lib = g.vsel.lib
    fake = C.c_void_p(4096)  # never dereferenced: the row count is rejected first
    assert lib.vsel_topk_noalloc(fake, 0, g.vsel.NOALLOC_MAX_ROWS + 1, 100, 100, 5, fake, fake, None, None,
                                 None) == 1
