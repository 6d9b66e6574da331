"""Soak of the cross-workgroup merges against the oracle.

A reduction whose partial results are read before every workgroup has
written them gives wrong answers silently and only now and then ("Chapter 21
- Sampling, argmax, and grammar", section 21.5, on the two-phase reduction
and its stale partials).  Here a row's segments meet in the last workgroup to
arrive at a shared ticket.  Each path below runs thousands of calls that
split rows into many segments, on inputs whose oracle outputs are computed
once.  Every call writes its outputs to a slot of its own in a device buffer;
the slots are compared with the oracle in blocks, and the test stops at the
first mismatch, naming the call.  The comparison rules (and their float64
exemptions) are those of the parity tests.
"""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu
N_CALLS = 4000
BLOCK = 250


@pytest.fixture(scope="module")
def g():
    import tests.gpu_helpers as G
    import vocab_row_reductions_amd as vsel
    G.vsel = vsel
    return G


def soak(n, launch, check, name):
    """launch(i) issues call i into slot i; check(lo, hi) compares slots
    [lo, hi) and returns the first bad call or None."""
    done = 0
    while done < n:
        hi = min(n, done + BLOCK)
        for i in range(done, hi):
            launch(i)
        torch.cuda.synchronize()
        bad = check(done, hi)
        assert bad is None, f"{name}: call {bad} of {n} differs from the oracle"
        done = hi
    print(f"soak {name}: {n} calls equal to the oracle", flush=True)


def test_soak_single_row_argmax(g, oracle):
    """One 202,048-float row split into 99 segments: every call merges 99
    partials.  Four rows with their maximum planted in several segments."""
    rows = [W.greedy_single_row()[0][0]]
    for s in range(3):
        r, _ = W.greedy_single_row(seed=W.BASE_SEED + 900 + s)
        rows.append(r[0])
    xs = [g.dev_rows(r[None]) for r in rows]
    ref = np.array([oracle.argmax(r[None])[0][0] for r in rows], np.uint32)
    idx = torch.empty(N_CALLS, dtype=torch.int32, device=g.DEV)
    val = torch.empty(N_CALLS, dtype=torch.float32, device=g.DEV)

    def launch(i):
        g.vsel.vsel_argmax(xs[i % 4], out_idx=idx[i:i + 1], out_val=val[i:i + 1])

    def check(lo, hi):
        got = g.u32(idx[lo:hi])
        bad = np.nonzero(got != ref[np.arange(lo, hi) % 4])[0]
        return None if len(bad) == 0 else lo + int(bad[0])

    soak(N_CALLS, launch, check, "argmax 1 x 202,048 (99 segments)")


def test_soak_verify_topk(g, oracle):
    """Three 248,320-float verify rows at k = 84: 11 segments per row, each
    row's last workgroup merging 11 x 84 records."""
    xs, refs = [], []
    for s in range(2):
        x = W.verify_topk_rows(rows=3, seed=W.BASE_SEED + 910 + s)
        xs.append(g.dev_rows(x))
        refs.append(oracle.topk(x, 84))
    vals = torch.empty((N_CALLS, 3, 84), dtype=torch.float32, device=g.DEV)
    ids = torch.empty((N_CALLS, 3, 84), dtype=torch.int32, device=g.DEV)
    am = torch.empty((N_CALLS, 3), dtype=torch.int32, device=g.DEV)
    lse = torch.empty((N_CALLS, 3), dtype=torch.float32, device=g.DEV)

    def launch(i):
        g.vsel.vsel_topk(xs[i % 2], 84, out=dict(vals=vals[i], ids=ids[i], argmax=am[i], lse=lse[i]))

    def check(lo, hi):
        gi, gv, ga, gl = g.u32(ids[lo:hi]), g.bits(vals[lo:hi]), g.u32(am[lo:hi]), lse[lo:hi].cpu().numpy()
        for j in range(hi - lo):
            ov, oi, oam, olse = refs[(lo + j) % 2]
            if not (np.array_equal(gi[j], oi) and np.array_equal(gv[j], ov.view(np.uint32))
                    and np.array_equal(ga[j], oam)
                    and np.all(np.abs(gl[j] - olse) <= 1e-5 + np.abs(olse) * 2.0 ** -23)):
                return lo + j
        return None

    soak(N_CALLS, launch, check, "top-k 3 x 248,320, k = 84 (11 segments)")


def test_soak_topk_random_shapes(g, oracle):
    """Fifty seeded shapes (1-6 rows, 20,000-300,000 elements, k from 1 to 400,
    float32 and bfloat16, aligned and odd strides), eighty calls each."""
    rng = np.random.default_rng(W.BASE_SEED + 920)
    shapes = []
    for _ in range(50):
        rows = int(rng.integers(1, 7))
        V = int(rng.integers(20000, 300001))
        k = int(rng.choice([1, 7, 20, 64, 84, 128, 129, 400]))
        x = (np.round(rng.normal(0, 2, (rows, V)) * 16) / 16).astype(np.float32)
        if rng.random() < 0.5:
            x = W.f32_to_bf16_bits(x)
        ld = V + int(rng.choice([0, 3, 8]))
        shapes.append((g.dev_rows(x, ld), V, k, oracle.topk(x, k)))
    per = N_CALLS // len(shapes)
    outs = []
    for xd, V, k, _ in shapes:
        rows = xd.shape[0]
        outs.append((torch.empty((per, rows, k), dtype=torch.float32, device=g.DEV),
                     torch.empty((per, rows, k), dtype=torch.int32, device=g.DEV)))

    def launch(i):
        s, c = divmod(i, per)
        xd, V, k, _ = shapes[s]
        g.vsel.vsel_topk(xd, k, vocab=V, out=dict(vals=outs[s][0][c], ids=outs[s][1][c], argmax=None, lse=None))

    def check(lo, hi):
        for i in range(lo, hi):
            s, c = divmod(i, per)
            ov, oi, _, _ = shapes[s][3]
            if not (np.array_equal(g.u32(outs[s][1][c]), oi)
                    and np.array_equal(g.bits(outs[s][0][c]), ov.view(np.uint32))):
                return i
        return None

    soak(per * len(shapes), launch, check, "top-k, 50 random shapes")


def mrs_masks(ref, B, G):
    """Which MRS outputs the parity rules compare: not past an accept test whose
    float64 margin is below 1e-7, not a draw whose margin is below 1e-9."""
    len_mask = np.ones(B, bool)
    tok_mask = np.ones((B, G + 1), bool)
    for b in range(B):
        close = np.nonzero(ref["acc_margin"][b] < 1e-7)[0]
        if len(close):
            len_mask[b] = False
            tok_mask[b, close[0]:] = False
            continue
        L = ref["len_mrs"][b]
        if L >= 0 and ref["draw_margin"][b] < 1e-9:
            tok_mask[b, L] = False
    return len_mask, tok_mask


def test_soak_speculative_rules(g, oracle):
    """The 32 x 8 speculative batch (V = 202,048): modified rejection sampling
    and sampler-match, each call merging the position passes' segments and
    the draws' chunk masses."""
    d = W.speculative_batch()
    B, G, T = d["batch"], d["gamma"], d["temperature"]
    dv = {k: g.dev(d[k]) for k in ("target", "draft", "tokens", "u_acc", "u_res", "u_bon")}
    ref = oracle.spec_accept(d["target"], d["draft"], d["tokens"], d["u_acc"], d["u_res"], d["u_bon"], B, G, T)
    len_mask, tok_mask = mrs_masks(ref, B, G)
    um = W.uniforms(B * (G + 1), seed=W.BASE_SEED + 930).reshape(B, G + 1)
    umd = g.dev(um.reshape(-1))
    rsm = oracle.spec_match(d["target"], d["draft"], d["tokens"], um, B, G, T)
    sm_mask = np.ones(B, bool)
    for b in range(B):
        sm_mask[b] = not np.any(rsm["match_margin"][b] < 1e-9)
    n = N_CALLS // 2
    o = dict(len_mrs=torch.empty((n, B), dtype=torch.int32, device=g.DEV),
             tok_mrs=torch.empty((n, B, G + 1), dtype=torch.int32, device=g.DEV),
             len_aa=torch.empty((n, B), dtype=torch.int32, device=g.DEV),
             tok_aa=torch.empty((n, B, G + 1), dtype=torch.int32, device=g.DEV),
             summin=torch.empty((n, B, G), dtype=torch.float32, device=g.DEV))
    s = dict(len_sm=torch.empty((n, B), dtype=torch.int32, device=g.DEV),
             tok_sm=torch.empty((n, B, G + 1), dtype=torch.int32, device=g.DEV),
             sumprod=torch.empty((n, B, G), dtype=torch.float32, device=g.DEV))

    def launch(i):
        g.vsel.vsel_spec_accept(dv["target"], dv["draft"], dv["tokens"], dv["u_acc"], dv["u_res"], dv["u_bon"], B,
                                G, T, out={k: v[i] for k, v in o.items()})
        g.vsel.vsel_spec_match(dv["target"], dv["draft"], dv["tokens"], umd, B, G, T,
                               out={k: v[i] for k, v in s.items()})

    def near(a, b):
        ok = np.isfinite(b)
        return np.all(np.abs(a[..., ok] - b[ok]) <= 1e-6 + 1e-5 * np.abs(b[ok]))

    def check(lo, hi):
        lm, tm = o["len_mrs"][lo:hi].cpu().numpy(), g.u32(o["tok_mrs"][lo:hi])
        la, ta = o["len_aa"][lo:hi].cpu().numpy(), g.u32(o["tok_aa"][lo:hi])
        ls, ts = s["len_sm"][lo:hi].cpu().numpy(), g.u32(s["tok_sm"][lo:hi])
        smn, spr = o["summin"][lo:hi].cpu().numpy(), s["sumprod"][lo:hi].cpu().numpy()
        for j in range(hi - lo):
            good = (np.array_equal(la[j], ref["len_aa"]) and np.array_equal(ta[j], ref["tok_aa"])
                    and np.array_equal(lm[j][len_mask], ref["len_mrs"][len_mask])
                    and np.array_equal(tm[j][tok_mask], ref["tok_mrs"][tok_mask])
                    and np.array_equal(ls[j][sm_mask], rsm["len_sm"][sm_mask])
                    and np.array_equal(ts[j][sm_mask], rsm["tok_sm"][sm_mask])
                    and near(smn[j], ref["summin"]) and near(spr[j], rsm["sumprod"]))
            if not good:
                return lo + j
        return None

    soak(n, launch, check, "speculative 32 x 8 (both rules per call)")
