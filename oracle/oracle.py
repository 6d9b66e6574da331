"""ctypes binding of the CPU oracle -- TEST INFRASTRUCTURE ONLY.

Arrays are numpy: float32 rows (dtype 0) or bfloat16 bit patterns stored as
uint16 (dtype 1), shape [rows, ld]; `vocab` (default ld) valid elements per row.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

_lib = None
SENTINEL = 0xFFFFFFFF


def load(path):
    """Load an oracle shared library and declare its signatures."""
    L = C.CDLL(path)
    i64, i32, vp, f32, f64 = C.c_int64, C.c_int32, C.c_void_p, C.c_float, C.c_double
    L.oracle_chunk_geometry.argtypes = [i64, i64, C.POINTER(i64), C.POINTER(i64)]
    L.oracle_argmax.argtypes = [vp, C.c_int, i64, i64, i64, vp, vp, C.c_int]
    L.oracle_lse.argtypes = [vp, C.c_int, i64, i64, i64, f64, vp, C.c_int]
    L.oracle_argmax_excluding.argtypes = [vp, C.c_int, i64, i64, i64, vp, i64, vp, vp, C.c_int]
    L.oracle_topk.argtypes = [vp, C.c_int, i64, i64, i64, i32, vp, vp, vp, vp, C.c_int]
    L.oracle_sample.argtypes = [vp, C.c_int, i64, i64, i64, f32, i32, f32, vp, vp, vp, vp, C.c_int]
    L.oracle_spec_accept.argtypes = [vp, i64, vp, i64, i64, i32, i64, f32, i32, f32, f32, vp, vp, vp, vp,
                                     vp, vp, vp, vp, vp, vp, vp, vp, C.c_int]
    L.oracle_sample_chain.argtypes = [vp, C.c_int, i64, i64, i64, f32, f32, i32, f32, f32, f32, vp, vp, vp, vp,
                                      C.c_int]
    L.oracle_spec_match.argtypes = [vp, i64, vp, i64, i64, i32, i64, f32, i32, f32, f32, vp, vp, vp, vp, vp, vp, vp,
                                    C.c_int]
    for f in (L.oracle_argmax, L.oracle_lse, L.oracle_topk, L.oracle_sample, L.oracle_spec_accept,
              L.oracle_argmax_excluding, L.oracle_spec_match, L.oracle_sample_chain):
        f.restype = C.c_int
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB) or os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC):
            _build.build()
        _lib = load(_build.LIB)
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _rows(x):
    x = np.ascontiguousarray(x)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    if x.dtype == np.float32:
        return x, 0
    if x.dtype == np.uint16:
        return x, 1
    raise TypeError("oracle rows must be float32 or uint16 (bfloat16 bits)")


def _check(rc):
    if rc != 0:
        raise ValueError("oracle rejected its arguments")


def chunk_geometry(n: int, chunk: int):
    c, t = C.c_int64(), C.c_int64()
    lib().oracle_chunk_geometry(n, chunk, C.byref(c), C.byref(t))
    return c.value, t.value


def argmax(x, vocab=None, nthreads=0):
    x, dt = _rows(x)
    R, ld = x.shape
    V = ld if vocab is None else vocab
    idx = np.empty(R, np.uint32)
    val = np.empty(R, np.float32)
    _check(lib().oracle_argmax(_p(x), dt, R, V, ld, _p(idx), _p(val), nthreads))
    return idx, val


def argmax_excluding(x, excluded, vocab=None, nthreads=0):
    """Greedy serving argmax with an excluded-id set: (idx, status) per row."""
    x, dt = _rows(x)
    R, ld = x.shape
    V = ld if vocab is None else vocab
    ex = np.ascontiguousarray(np.asarray(excluded, dtype=np.uint32).reshape(-1))
    idx = np.empty(R, np.uint32)
    status = np.empty(R, np.uint32)
    _check(lib().oracle_argmax_excluding(_p(x), dt, R, V, ld, _p(ex) if ex.size else None, ex.size, _p(idx),
                                         _p(status), nthreads))
    return idx, status


def lse(x, temperature=1.0, vocab=None, nthreads=0):
    x, dt = _rows(x)
    R, ld = x.shape
    V = ld if vocab is None else vocab
    out = np.empty(R, np.float64)
    _check(lib().oracle_lse(_p(x), dt, R, V, ld, float(temperature), _p(out), nthreads))
    return out


def topk(x, k, vocab=None, nthreads=0):
    x, dt = _rows(x)
    R, ld = x.shape
    V = ld if vocab is None else vocab
    vals = np.empty((R, k), np.float32)
    ids = np.empty((R, k), np.uint32)
    am = np.empty(R, np.uint32)
    ls = np.empty(R, np.float64)
    _check(lib().oracle_topk(_p(x), dt, R, V, ld, int(k), _p(vals), _p(ids), _p(am), _p(ls), nthreads))
    return vals, ids, am, ls


def sample(x, temperature, top_k, top_p, u, vocab=None, nthreads=0):
    x, dt = _rows(x)
    R, ld = x.shape
    V = ld if vocab is None else vocab
    u = np.ascontiguousarray(u, dtype=np.float32)
    assert u.shape == (R,)
    tok = np.empty(R, np.uint32)
    logp = np.empty(R, np.float64)
    margins = np.empty((R, 2), np.float64)
    _check(lib().oracle_sample(_p(x), dt, R, V, ld, float(temperature), int(top_k), float(top_p),
                               _p(u), _p(tok), _p(logp), _p(margins), nthreads))
    return tok, logp, margins


def sample_chain(x, temperature, u, top_n_sigma=0.0, top_k=0, typical_p=1.0, top_p=1.0, min_p=0.0, vocab=None,
                 nthreads=0):
    """The ordered sampler chain (top-n-sigma, top-k, typical-p, top-p, min-p,
    temperature) -> (tokens uint32[R], logp float64[R], margins float64[R, 6])."""
    x, dt = _rows(x)
    R, ld = x.shape
    V = ld if vocab is None else vocab
    u = np.ascontiguousarray(u, dtype=np.float32)
    assert u.shape == (R,)
    tok = np.empty(R, np.uint32)
    logp = np.empty(R, np.float64)
    margins = np.empty((R, 6), np.float64)
    _check(lib().oracle_sample_chain(_p(x), dt, R, V, ld, float(temperature), float(top_n_sigma), int(top_k),
                                     float(typical_p), float(top_p), float(min_p), _p(u), _p(tok), _p(logp),
                                     _p(margins), nthreads))
    return tok, logp, margins


def spec_accept(target, draft, tokens, u_acc, u_res, u_bon, batch, gamma, temperature,
                vocab=None, nthreads=0, top_k=0, top_p=1.0, min_p=0.0):
    target = np.ascontiguousarray(target, dtype=np.float32)
    draft = np.ascontiguousarray(draft, dtype=np.float32)
    assert target.shape[0] == batch * (gamma + 1) and draft.shape[0] == batch * gamma
    V = target.shape[1] if vocab is None else vocab
    tokens = np.ascontiguousarray(tokens, dtype=np.uint32).reshape(batch * gamma)
    u_acc = np.ascontiguousarray(u_acc, dtype=np.float32).reshape(batch * gamma)
    u_res = np.ascontiguousarray(u_res, dtype=np.float32).reshape(batch * gamma)
    u_bon = np.ascontiguousarray(u_bon, dtype=np.float32).reshape(batch)
    out = dict(
        len_mrs=np.empty(batch, np.int32), tok_mrs=np.empty((batch, gamma + 1), np.uint32),
        len_aa=np.empty(batch, np.int32), tok_aa=np.empty((batch, gamma + 1), np.uint32),
        summin=np.empty((batch, gamma), np.float64), acc_margin=np.empty((batch, gamma), np.float64),
        draw_margin=np.empty(batch, np.float64), filter_margin=np.empty(batch, np.float64))
    _check(lib().oracle_spec_accept(
        _p(target), target.shape[1], _p(draft), draft.shape[1], batch, gamma, V, float(temperature),
        int(top_k), float(top_p), float(min_p),
        _p(tokens), _p(u_acc), _p(u_res), _p(u_bon), _p(out["len_mrs"]), _p(out["tok_mrs"]),
        _p(out["len_aa"]), _p(out["tok_aa"]), _p(out["summin"]), _p(out["acc_margin"]),
        _p(out["draw_margin"]), _p(out["filter_margin"]), nthreads))
    return out


def spec_match(target, draft, tokens, u_match, batch, gamma, temperature, vocab=None, nthreads=0,
               top_k=0, top_p=1.0, min_p=0.0):
    """Sampler-match acceptance (fresh draw from p at each position, accept on
    equality, emit the draw) and the per-position sum_x p(x) q(x).
    u_match: float32 [batch, gamma+1].  Returns len_sm, tok_sm, sumprod and
    match_margin (the draw margin at each tested position, +inf elsewhere)."""
    target = np.ascontiguousarray(target, dtype=np.float32)
    draft = np.ascontiguousarray(draft, dtype=np.float32)
    assert target.shape[0] == batch * (gamma + 1) and draft.shape[0] == batch * gamma
    V = target.shape[1] if vocab is None else vocab
    tokens = np.ascontiguousarray(tokens, dtype=np.uint32).reshape(batch * gamma)
    u_match = np.ascontiguousarray(u_match, dtype=np.float32).reshape(batch * (gamma + 1))
    out = dict(len_sm=np.empty(batch, np.int32), tok_sm=np.empty((batch, gamma + 1), np.uint32),
               sumprod=np.empty((batch, gamma), np.float64),
               match_margin=np.empty((batch, gamma + 1), np.float64), filter_margin=np.empty(batch, np.float64))
    _check(lib().oracle_spec_match(
        _p(target), target.shape[1], _p(draft), draft.shape[1], batch, gamma, V, float(temperature),
        int(top_k), float(top_p), float(min_p),
        _p(tokens), _p(u_match), _p(out["len_sm"]), _p(out["tok_sm"]), _p(out["sumprod"]),
        _p(out["match_margin"]), _p(out["filter_margin"]), nthreads))
    return out
