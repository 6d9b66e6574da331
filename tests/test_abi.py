"""Host-side checks of the C ABI (no kernel is launched): the library loads,
exports every entry point include/vsel.h declares, sizes workspaces and
rejects bad arguments synchronously."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vsel.h")


@pytest.fixture(scope="module")
def vsel():
    import vocab_row_reductions_amd as v
    return v


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vsel_[a-z_]+)\s*\(", text)))


def test_header_declares_the_operations():
    names = declared_functions()
    for op in ("vsel_argmax", "vsel_argmax_excluding", "vsel_topk", "vsel_topk_noalloc", "vsel_sample", "vsel_sample_chain",
               "vsel_spec_accept", "vsel_spec_match", "vsel_spec_accept_filtered", "vsel_spec_match_filtered",
               "vsel_workspace_bytes"):
        assert op in names


def test_library_exports_every_declared_symbol(vsel):
    lib = C.CDLL(vsel.library_path)
    for name in declared_functions():
        assert hasattr(lib, name), f"libvsel.so does not export {name}"


def test_version_and_status_strings(vsel):
    assert vsel.lib.vsel_version() >> 16 >= 1
    assert vsel.lib.vsel_status_string(0) == b"ok"
    assert b"invalid" in vsel.lib.vsel_status_string(1)


def test_workspace_sizes(vsel):
    wb = vsel.workspace_bytes
    for op, k in ((vsel.OP_ARGMAX, 0), (vsel.OP_TOPK, 84), (vsel.OP_SAMPLE, 20), (vsel.OP_SAMPLE, 0),
                  (vsel.OP_SPEC, 8), (vsel.OP_SAMPLE_CHAIN, 0), (vsel.OP_SAMPLE_CHAIN, 128)):
        n = wb(op, vsel.F32, 32, 202048, k)
        assert n > 0 and n % 256 == 0
    # the sampler is the chain with top-k and top-p only: one layout (the row
    # moments and, for top_k = 0, the whole-row nucleus after the candidates)
    for k in (0, 1, 50, 1024):
        assert wb(vsel.OP_SAMPLE_CHAIN, vsel.BF16, 64, 202048, k) == wb(vsel.OP_SAMPLE, vsel.BF16, 64, 202048, k)
    assert wb(vsel.OP_SAMPLE, vsel.F32, 64, 202048, 0) > wb(vsel.OP_SAMPLE, vsel.F32, 64, 202048, 20)
    assert wb(vsel.OP_SAMPLE_CHAIN, vsel.F32, 4, 100, 1025) == 0
    # the filtered rules hold the speculative workspace and the filter pass's after it
    assert wb(vsel.OP_SPEC_FILTERED, vsel.F32, 32, 202048, 8) > wb(vsel.OP_SPEC, vsel.F32, 32, 202048, 8) > 0
    assert wb(vsel.OP_SPEC_FILTERED, vsel.F32, 2, 100, 257) == 0
    assert wb(vsel.OP_TOPK, vsel.BF16, 1024, 202048, 84) > 0
    # rejected shapes size to 0
    assert wb(vsel.OP_TOPK, vsel.F32, 4, 100, 101) == 0          # k > vocab
    assert wb(vsel.OP_TOPK, vsel.F32, 4, 5000, 1025) == 0        # k > K_MAX
    assert wb(vsel.OP_ARGMAX, vsel.F32, 0, 100, 0) == 0          # no rows
    assert wb(vsel.OP_ARGMAX, 7, 4, 100, 0) == 0                 # unknown dtype
    assert wb(99, vsel.F32, 4, 100, 0) == 0                      # unknown op


def test_invalid_arguments_return_einval_before_launch(vsel):
    L = vsel.lib
    fake = C.c_void_p(4096)   # never dereferenced: every call below fails validation first
    ws = C.c_void_p(1 << 20)
    EINVAL, EWS = 1, 2
    assert L.vsel_argmax(None, 0, 4, 100, 100, fake, None, ws, 1 << 20, None) == EINVAL
    assert L.vsel_argmax(fake, 0, 0, 100, 100, fake, None, ws, 1 << 20, None) == EINVAL
    assert L.vsel_argmax(fake, 0, 4, 100, 99, fake, None, ws, 1 << 20, None) == EINVAL       # ld < vocab
    assert L.vsel_argmax(fake, 0, 4, 1 << 31, 1 << 31, fake, None, ws, 1 << 20, None) == EINVAL
    assert L.vsel_argmax(C.c_void_p(4097), 1, 4, 100, 100, fake, None, ws, 1 << 20, None) == EINVAL
    assert L.vsel_argmax(fake, 0, 4, 100, 100, fake, None, ws, 16, None) == EWS                # too small
    assert L.vsel_argmax(fake, 0, 4, 100, 100, fake, None, C.c_void_p((1 << 20) + 8), 1 << 20, None) == EWS
    def excl(n, ids=fake, status=fake, **kw):
        return L.vsel_argmax_excluding(fake, 0, kw.get("rows", 4), 100, 100, ids, n, fake, status, ws,
                                       kw.get("ws_bytes", 1 << 20), None)
    assert excl(-1) == EINVAL
    assert excl(257) == EINVAL                                  # above the set limit
    assert excl(3, ids=None) == EINVAL                          # ids missing
    assert excl(3, status=None) == EINVAL                       # status output missing
    assert excl(0, rows=0) == EINVAL
    assert excl(256, ws_bytes=16) == EWS
    assert L.vsel_topk(fake, 0, 4, 100, 100, 0, fake, fake, None, None, ws, 1 << 20, None) == EINVAL
    assert L.vsel_topk(fake, 0, 4, 100, 100, 101, fake, fake, None, None, ws, 1 << 20, None) == EINVAL
    assert L.vsel_topk(fake, 0, 4, 5000, 5000, 1025, fake, fake, None, None, ws, 1 << 20, None) == EINVAL
    assert L.vsel_topk(fake, 0, 4, 100, 100, 5, None, fake, None, None, ws, 1 << 20, None) == EINVAL
    # the allocation-free top-k: the row count is checked before any device call
    assert L.vsel_topk_noalloc(fake, 0, 0, 100, 100, 5, fake, fake, None, None, None) == EINVAL
    assert L.vsel_topk_noalloc(fake, 0, vsel.NOALLOC_MAX_ROWS + 1, 100, 100, 5, fake, fake, None, None,
                               None) == EINVAL
    bad_sample = [(-0.5, 20, 0.9), (0.7, -1, 0.9), (0.7, 20, 0.0), (0.7, 20, 1.5),
                  (0.7, 1025, 0.9), (float("nan"), 20, 0.9), (float("inf"), 20, 0.9)]
    for T, k, p in bad_sample:
        assert L.vsel_sample(fake, 0, 4, 100, 100, T, k, p, fake, fake, None, ws, 1 << 20, None) == EINVAL
    def chain(T=0.7, sig=0.0, k=20, typ=1.0, p=1.0, mp=0.0, u=fake, ws_bytes=1 << 20):
        return L.vsel_sample_chain(fake, 0, 4, 100, 100, T, sig, k, typ, p, mp, u, fake, None, ws, ws_bytes, None)
    bad_chain = [dict(sig=-1.0), dict(sig=float("inf")), dict(sig=float("nan")), dict(typ=0.0), dict(typ=1.5),
                 dict(mp=-0.1), dict(mp=1.01), dict(mp=float("nan")),
                 dict(k=-1), dict(k=1025), dict(p=0.0), dict(T=float("inf")),
                 dict(T=-0.1), dict(u=None)]
    for kw in bad_chain:
        assert chain(**kw) == EINVAL, kw
    assert chain(sig=1.0, ws_bytes=4096) == EWS
    args = dict(batch=2, gamma=3, vocab=100, T=1.0)
    def spec(**kw):
        a = {**args, **kw}
        return L.vsel_spec_accept(fake, a.get("ld_t", 100), fake, a.get("ld_d", 100), a["batch"], a["gamma"],
                                  a["vocab"], a["T"], fake, fake, fake, fake, fake, fake, None, None, None,
                                  None, ws, 1 << 20, None)
    assert spec(gamma=0) == EINVAL
    assert spec(gamma=257) == EINVAL
    assert spec(batch=0) == EINVAL
    assert spec(T=-1.0) == EINVAL
    assert spec(ld_t=99) == EINVAL
    assert spec(ld_d=50) == EINVAL
    def match(u=fake, ln=fake, tk=fake, **kw):
        a = {**args, **kw}
        return L.vsel_spec_match(fake, a.get("ld_t", 100), fake, a.get("ld_d", 100), a["batch"], a["gamma"],
                                 a["vocab"], a["T"], fake, u, ln, tk, None, ws, 1 << 20, None)
    assert match(u=None) == EINVAL                 # uniforms missing
    assert match(ln=None) == EINVAL                # length output missing
    assert match(tk=None) == EINVAL                # token output missing
    assert match(gamma=0) == EINVAL
    assert match(T=float("nan")) == EINVAL
    assert match(ld_t=99) == EINVAL
    def filt(fn, k=5, p=0.9, mp=0.0, ws_bytes=1 << 20):
        if fn == "accept":
            return L.vsel_spec_accept_filtered(fake, 100, fake, 100, 2, 3, 100, 1.0, k, p, mp, fake, fake, fake,
                                               fake, fake, fake, None, None, None, None, ws, ws_bytes, None)
        return L.vsel_spec_match_filtered(fake, 100, fake, 100, 2, 3, 100, 1.0, k, p, mp, fake, fake, fake, fake,
                                          None, ws, ws_bytes, None)
    for fn in ("accept", "match"):
        for kw in (dict(k=-1), dict(k=1025), dict(p=0.0), dict(p=1.5), dict(mp=-0.5), dict(mp=2.0),
                   dict(p=float("nan"))):
            assert filt(fn, **kw) == EINVAL, (fn, kw)
        assert filt(fn, ws_bytes=4096) == EWS
