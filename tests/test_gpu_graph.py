"""Graph capture of the selection calls: every replay equals the eager result.

The kernels leave their workspace counters at zero and use no memset, so a
captured call can be replayed.  Each graph is replayed several times with
eager work and synchronisations in between, and every replay is checked."""
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


def replay_check(capture, outputs, eager_ref, eager_noise):
    graph = torch.cuda.CUDAGraph()
    capture()                       # warm the workspace cache outside the capture
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        capture()
    for rep in range(4):
        for t in outputs():
            t.fill_(-7)
        eager_noise()               # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, ref in zip(outputs(), eager_ref):
            assert torch.equal(got, ref), f"replay {rep} differs from the eager result"


def test_topk_and_argmax_graph(g):
    x = g.dev_rows(W.verify_topk_rows(rows=7, vocab=60001, seed=71))
    ref = [t.clone() for t in g.vsel.vsel_topk(x, 84)]
    out = dict(vals=torch.empty_like(ref[0]), ids=torch.empty_like(ref[1]), argmax=torch.empty_like(ref[2]),
               lse=torch.empty_like(ref[3]))
    y = g.dev_rows(W.verify_topk_rows(rows=3, vocab=9000, seed=72))
    replay_check(lambda: g.vsel.vsel_topk(x, 84, out=out), lambda: [out["vals"], out["ids"], out["argmax"], out["lse"]],
                 ref, lambda: g.vsel.vsel_argmax(y))


def test_sample_graph(g):
    xs, u = W.sampling_rows(rows=9, vocab=50000, seed=73)
    x, ud = g.dev_rows(xs), g.dev(u)
    for top_k in (20, 0):
        tok, lp = g.vsel.vsel_sample(x, 0.7, top_k, 0.95 if top_k else 1.0, ud)
        ref = [tok.clone(), lp.clone()]
        ot, ol = torch.empty_like(tok), torch.empty_like(lp)
        replay_check(lambda: g.vsel.vsel_sample(x, 0.7, top_k, 0.95 if top_k else 1.0, ud, out_token=ot, out_logprob=ol),
                     lambda: [ot, ol], ref, lambda: g.vsel.vsel_topk(x, 5))


def test_sample_chain_graph(g):
    xs, u = W.sampling_rows(rows=9, vocab=50000, seed=76)
    x, ud = g.dev_rows(xs), g.dev(u)
    for kw in (dict(top_n_sigma=1.0, top_k=40, typical_p=0.8, top_p=0.9, min_p=0.02), dict(top_n_sigma=0.7, min_p=0.01),
               dict(top_p=0.9, min_p=0.01), dict(typical_p=0.8, top_p=0.95)):
        tok, lp = g.vsel.vsel_sample_chain(x, 0.8, ud, **kw)
        ref = [tok.clone(), lp.clone()]
        ot, ol = torch.empty_like(tok), torch.empty_like(lp)
        replay_check(lambda: g.vsel.vsel_sample_chain(x, 0.8, ud, out_token=ot, out_logprob=ol, **kw),
                     lambda: [ot, ol], ref, lambda: g.vsel.vsel_topk(x, 5))


def test_spec_accept_graph(g):
    d = W.speculative_batch(batch=4, gamma=3, vocab=30000, seed=74)
    args = [g.dev(d[k]) for k in ("target", "draft", "tokens", "u_acc", "u_res", "u_bon")]
    ref = g.vsel.vsel_spec_accept(*args, 4, 3, 1.0)
    ref = {k: v.clone() for k, v in ref.items()}
    out = {k: torch.empty_like(v) for k, v in ref.items()}
    keys = list(ref)
    replay_check(lambda: g.vsel.vsel_spec_accept(*args, 4, 3, 1.0, out=out), lambda: [out[k] for k in keys],
                 [ref[k] for k in keys], lambda: g.vsel.vsel_argmax(args[0]))


def test_spec_match_graph(g):
    d = W.speculative_batch(batch=4, gamma=3, vocab=30000, seed=75)
    um = g.dev(W.uniforms(4 * 4, seed=75))
    args = [g.dev(d[k]) for k in ("target", "draft", "tokens")]
    ref = g.vsel.vsel_spec_match(*args, um, 4, 3, 1.0)
    ref = {k: v.clone() for k, v in ref.items()}
    out = {k: torch.empty_like(v) for k, v in ref.items()}
    keys = list(ref)
    replay_check(lambda: g.vsel.vsel_spec_match(*args, um, 4, 3, 1.0, out=out), lambda: [out[k] for k in keys],
                 [ref[k] for k in keys], lambda: g.vsel.vsel_argmax(args[0]))


def test_filtered_spec_graphs(g):
    d = W.speculative_batch(batch=4, gamma=3, vocab=30000, seed=77)
    args = [g.dev(d[k]) for k in ("target", "draft", "tokens", "u_acc", "u_res", "u_bon")]
    um = g.dev(W.uniforms(4 * 4, seed=77))
    for kw in (dict(top_k=40, top_p=0.9), dict(top_p=0.9, min_p=0.01), dict(min_p=0.05)):
        ref = {k: v.clone() for k, v in g.vsel.vsel_spec_accept_filtered(*args, 4, 3, 1.0, **kw).items()}
        out = {k: torch.empty_like(v) for k, v in ref.items()}
        keys = list(ref)
        replay_check(lambda: g.vsel.vsel_spec_accept_filtered(*args, 4, 3, 1.0, out=out, **kw),
                     lambda: [out[k] for k in keys], [ref[k] for k in keys], lambda: g.vsel.vsel_argmax(args[0]))
        ref = {k: v.clone() for k, v in g.vsel.vsel_spec_match_filtered(args[0], args[1], args[2], um, 4, 3, 1.0,
                                                                         **kw).items()}
        out = {k: torch.empty_like(v) for k, v in ref.items()}
        keys = list(ref)
        replay_check(lambda: g.vsel.vsel_spec_match_filtered(args[0], args[1], args[2], um, 4, 3, 1.0, out=out, **kw),
                     lambda: [out[k] for k in keys], [ref[k] for k in keys], lambda: g.vsel.vsel_argmax(args[0]))
