"""vocab_row_reductions_amd -- vocab-row selection on MI355X (gfx950).

A thin ctypes binding of libvsel.so (include/vsel.h) with the same entry
point names.  PyTorch supplies device memory and the current HIP stream;
every step of the computation runs in the library's HIP kernels.  There is
no CPU fallback: importing the package fails if the library is missing.

uint32 outputs (ids, tokens) are returned as int32 tensors holding the same
bits, so VSEL_NONFINITE (0xFFFFFFFF) reads as -1.
"""
from __future__ import annotations

import ctypes as C
import os

import torch  # loads the HIP runtime that libvsel.so then shares

__all__ = ["vsel_argmax", "vsel_argmax_excluding", "vsel_topk", "vsel_topk_noalloc", "vsel_sample", "vsel_sample_chain", "vsel_spec_accept",
           "vsel_spec_match", "vsel_spec_accept_filtered", "vsel_spec_match_filtered",
           "workspace_bytes",
           "VselError", "NONFINITE", "K_MAX", "EXCLUDED_MAX", "library_path"]

HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(HERE, "libvsel.so")

NONFINITE = 0xFFFFFFFF
K_MAX = 1024
EXCLUDED_MAX = 256
NOALLOC_MAX_ROWS = 16384
NOALLOC_SCRATCH_BYTES = 8 << 20
F32, BF16 = 0, 1
OP_ARGMAX, OP_TOPK, OP_SAMPLE, OP_SPEC, OP_SAMPLE_CHAIN, OP_SPEC_FILTERED = 0, 1, 2, 3, 4, 5


class VselError(RuntimeError):
    pass


def _load():
    if not os.path.exists(library_path):
        raise ImportError(f"libvsel.so is not built ({library_path}); run __graft_entry__.build()")
    L = C.CDLL(library_path)
    i64, i32, vp, f32, sz = C.c_int64, C.c_int32, C.c_void_p, C.c_float, C.c_size_t
    L.vsel_version.restype = C.c_int
    L.vsel_status_string.restype = C.c_char_p
    L.vsel_status_string.argtypes = [C.c_int]
    L.vsel_workspace_bytes.restype = sz
    L.vsel_workspace_bytes.argtypes = [C.c_int, C.c_int, i64, i64, i32]
    L.vsel_argmax.argtypes = [vp, C.c_int, i64, i64, i64, vp, vp, vp, sz, vp]
    L.vsel_argmax_excluding.argtypes = [vp, C.c_int, i64, i64, i64, vp, i32, vp, vp, vp, sz, vp]
    L.vsel_topk.argtypes = [vp, C.c_int, i64, i64, i64, i32, vp, vp, vp, vp, vp, sz, vp]
    L.vsel_topk_noalloc.argtypes = [vp, C.c_int, i64, i64, i64, i32, vp, vp, vp, vp, vp]
    L.vsel_sample.argtypes = [vp, C.c_int, i64, i64, i64, f32, i32, f32, vp, vp, vp, vp, sz, vp]
    L.vsel_sample_chain.argtypes = [vp, C.c_int, i64, i64, i64, f32, f32, i32, f32, f32, f32, vp, vp, vp, vp, sz,
                                    vp]
    L.vsel_spec_accept.argtypes = [vp, i64, vp, i64, i64, i32, i64, f32, vp, vp, vp, vp, vp, vp, vp, vp,
                                   vp, vp, vp, sz, vp]
    L.vsel_spec_match.argtypes = [vp, i64, vp, i64, i64, i32, i64, f32, vp, vp, vp, vp, vp, vp, sz, vp]
    L.vsel_spec_accept_filtered.argtypes = [vp, i64, vp, i64, i64, i32, i64, f32, i32, f32, f32, vp, vp, vp, vp,
                                            vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.vsel_spec_match_filtered.argtypes = [vp, i64, vp, i64, i64, i32, i64, f32, i32, f32, f32, vp, vp, vp, vp,
                                           vp, vp, sz, vp]
    for f in (L.vsel_argmax, L.vsel_argmax_excluding, L.vsel_topk, L.vsel_topk_noalloc, L.vsel_sample, L.vsel_sample_chain,
              L.vsel_spec_accept, L.vsel_spec_match, L.vsel_spec_accept_filtered, L.vsel_spec_match_filtered):
        f.restype = C.c_int
    return L


lib = _load()
_ws_cache: dict = {}


def _check(rc: int, what: str, ws=None):
    if rc != 0:
        if rc == 3 and ws is not None:
            # a failed launch may leave the workspace's counters nonzero: the
            # next call of this signature gets a fresh zero-filled workspace
            for key in [key for key, t in _ws_cache.items() if t is ws]:
                del _ws_cache[key]
        raise VselError(f"{what}: {lib.vsel_status_string(rc).decode()} (status {rc})")


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("logit rows must be float32 or bfloat16")


def _rows(t: torch.Tensor, vocab):
    if not t.is_cuda:
        raise ValueError("logits must be a device tensor")
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("logits must be 2-D [rows, ld] with unit stride along the vocabulary")
    rows, cols = t.shape
    V = cols if vocab is None else int(vocab)
    if V > cols:
        raise ValueError("vocab exceeds the row length")
    return rows, V, t.stride(0)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(device) -> C.c_void_p:
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def workspace_bytes(op: int, dtype: int, rows: int, vocab: int, k: int) -> int:
    return int(lib.vsel_workspace_bytes(op, dtype, rows, vocab, k))


def _ws_key(op: int, dtype: int, rows: int, vocab: int, k: int, device):
    dev = torch.device(device)
    return (dev.index, torch.cuda.current_stream(dev).cuda_stream, op, dtype, rows, vocab, k)


def workspace(op: int, dtype: int, rows: int, vocab: int, k: int, device) -> torch.Tensor:
    """Zero-filled workspace for one call signature, cached per device, stream and
    signature (the kernels leave its counters at zero after every call; calls that
    share a workspace must be ordered on one stream).  A graph that captures a call
    keeps the capture stream's workspace; eager calls on another stream do not
    touch it."""
    key = _ws_key(op, dtype, rows, vocab, k, device)
    ws = _ws_cache.get(key)
    if ws is None:
        n = workspace_bytes(op, dtype, rows, vocab, k)
        if n == 0:
            raise VselError("arguments rejected when sizing the workspace")
        ws = torch.zeros(n, dtype=torch.uint8, device=torch.device(device))
        _ws_cache[key] = ws
    return ws


def vsel_argmax(logits: torch.Tensor, vocab=None, out_idx=None, out_val=None, want_val=True):
    """First-maximum argmax per row -> (idx int32[rows], val float32[rows] or None)."""
    rows, V, ld = _rows(logits, vocab)
    dt = _dtype(logits)
    dev = logits.device
    if out_idx is None:
        out_idx = torch.empty(rows, dtype=torch.int32, device=dev)
    if out_val is None and want_val:
        out_val = torch.empty(rows, dtype=torch.float32, device=dev)
    ws = workspace(OP_ARGMAX, dt, rows, V, 0, dev)
    _check(lib.vsel_argmax(_ptr(logits), dt, rows, V, ld, _ptr(out_idx), _ptr(out_val), _ptr(ws),
                           ws.numel(), _stream(dev)), "vsel_argmax", ws)
    return out_idx, out_val


def vsel_argmax_excluding(logits: torch.Tensor, excluded: torch.Tensor, vocab=None, out_idx=None,
                          out_status=None):
    """Greedy serving argmax with excluded ids -> (idx int32[rows], status int32[rows]).

    `excluded` is a 1-D int32/uint32-bit device tensor of at most EXCLUDED_MAX ids
    shared by every row; status 0 ok, 1 non-finite row, 2 no candidate."""
    rows, V, ld = _rows(logits, vocab)
    dt = _dtype(logits)
    dev = logits.device
    if excluded.dim() != 1 or excluded.dtype not in (torch.int32, torch.uint32) or not excluded.is_cuda:
        raise ValueError("excluded must be a 1-D int32 device tensor")
    if not excluded.is_contiguous():
        raise ValueError("excluded must be contiguous")
    n = excluded.numel()
    if out_idx is None:
        out_idx = torch.empty(rows, dtype=torch.int32, device=dev)
    if out_status is None:
        out_status = torch.empty(rows, dtype=torch.int32, device=dev)
    ws = workspace(OP_ARGMAX, dt, rows, V, 0, dev)
    _check(lib.vsel_argmax_excluding(_ptr(logits), dt, rows, V, ld, _ptr(excluded) if n else None, n,
                                     _ptr(out_idx), _ptr(out_status), _ptr(ws), ws.numel(), _stream(dev)),
           "vsel_argmax_excluding", ws)
    return out_idx, out_status


def vsel_topk(logits: torch.Tensor, k: int, vocab=None, want_argmax=True, want_lse=True, out=None):
    """Exact top-k per row -> (vals f32[rows,k], ids i32[rows,k], argmax i32[rows]|None, lse f32[rows]|None)."""
    rows, V, ld = _rows(logits, vocab)
    dt = _dtype(logits)
    dev = logits.device
    if out is None:
        out = dict(vals=torch.empty((rows, k), dtype=torch.float32, device=dev),
                   ids=torch.empty((rows, k), dtype=torch.int32, device=dev),
                   argmax=torch.empty(rows, dtype=torch.int32, device=dev) if want_argmax else None,
                   lse=torch.empty(rows, dtype=torch.float32, device=dev) if want_lse else None)
    ws = workspace(OP_TOPK, dt, rows, V, k, dev)
    _check(lib.vsel_topk(_ptr(logits), dt, rows, V, ld, int(k), _ptr(out["vals"]), _ptr(out["ids"]),
                         _ptr(out.get("argmax")), _ptr(out.get("lse")), _ptr(ws), ws.numel(), _stream(dev)),
           "vsel_topk", ws)
    return out["vals"], out["ids"], out.get("argmax"), out.get("lse")


def vsel_topk_noalloc(logits: torch.Tensor, k: int, vocab=None, want_argmax=True, want_lse=True, out=None):
    """vsel_topk whose scratch is the library's fixed device array (no workspace
    is allocated or passed) -> (vals, ids, argmax|None, lse|None)."""
    rows, V, ld = _rows(logits, vocab)
    dt = _dtype(logits)
    dev = logits.device
    if out is None:
        out = dict(vals=torch.empty((rows, k), dtype=torch.float32, device=dev),
                   ids=torch.empty((rows, k), dtype=torch.int32, device=dev),
                   argmax=torch.empty(rows, dtype=torch.int32, device=dev) if want_argmax else None,
                   lse=torch.empty(rows, dtype=torch.float32, device=dev) if want_lse else None)
    _check(lib.vsel_topk_noalloc(_ptr(logits), dt, rows, V, ld, int(k), _ptr(out["vals"]), _ptr(out["ids"]),
                                 _ptr(out.get("argmax")), _ptr(out.get("lse")), _stream(dev)), "vsel_topk_noalloc")
    return out["vals"], out["ids"], out.get("argmax"), out.get("lse")


def vsel_sample(logits: torch.Tensor, temperature: float, top_k: int, top_p: float, u: torch.Tensor,
                vocab=None, out_token=None, out_logprob=None):
    """Top-k then top-p temperature sampling with one uniform per row -> (token i32, logprob f32)."""
    rows, V, ld = _rows(logits, vocab)
    dt = _dtype(logits)
    dev = logits.device
    if u.dtype != torch.float32 or u.numel() != rows or not u.is_cuda:
        raise ValueError("u must be a float32 device tensor with one uniform per row")
    if out_token is None:
        out_token = torch.empty(rows, dtype=torch.int32, device=dev)
    if out_logprob is None:
        out_logprob = torch.empty(rows, dtype=torch.float32, device=dev)
    ws = workspace(OP_SAMPLE, dt, rows, V, int(top_k), dev)
    _check(lib.vsel_sample(_ptr(logits), dt, rows, V, ld, float(temperature), int(top_k), float(top_p),
                           _ptr(u.contiguous()), _ptr(out_token), _ptr(out_logprob), _ptr(ws), ws.numel(),
                           _stream(dev)), "vsel_sample", ws)
    return out_token, out_logprob


def vsel_sample_chain(logits: torch.Tensor, temperature: float, u: torch.Tensor, top_n_sigma=0.0, top_k=0,
                      typical_p=1.0, top_p=1.0, min_p=0.0, vocab=None, out_token=None, out_logprob=None):
    """The ordered sampler chain (top-n-sigma, top-k, typical-p, top-p, min-p,
    then the temperature) with one uniform per row -> (token i32, logprob f32)."""
    rows, V, ld = _rows(logits, vocab)
    dt = _dtype(logits)
    dev = logits.device
    if u.dtype != torch.float32 or u.numel() != rows or not u.is_cuda:
        raise ValueError("u must be a float32 device tensor with one uniform per row")
    if out_token is None:
        out_token = torch.empty(rows, dtype=torch.int32, device=dev)
    if out_logprob is None:
        out_logprob = torch.empty(rows, dtype=torch.float32, device=dev)
    ws = workspace(OP_SAMPLE_CHAIN, dt, rows, V, int(top_k), dev)
    _check(lib.vsel_sample_chain(_ptr(logits), dt, rows, V, ld, float(temperature), float(top_n_sigma), int(top_k),
                                 float(typical_p), float(top_p), float(min_p), _ptr(u.contiguous()), _ptr(out_token),
                                 _ptr(out_logprob), _ptr(ws), ws.numel(), _stream(dev)), "vsel_sample_chain", ws)
    return out_token, out_logprob


def vsel_spec_accept(target: torch.Tensor, draft: torch.Tensor, draft_tokens: torch.Tensor, u_accept: torch.Tensor,
                     u_resid: torch.Tensor, u_bonus: torch.Tensor, batch: int, gamma: int, temperature: float,
                     vocab=None, out=None):
    """Speculative acceptance for batch x gamma drafts -> dict of len_mrs, tok_mrs, len_aa, tok_aa, summin,
    sumprod (a caller's `out` may leave out any of the last four)."""
    if target.dtype != torch.float32 or draft.dtype != torch.float32:
        raise TypeError("speculative acceptance takes float32 rows")
    rt, Vt, ld_t = _rows(target, vocab)
    rd, Vd, ld_d = _rows(draft, vocab)
    if rt != batch * (gamma + 1) or rd != batch * gamma or Vt != Vd:
        raise ValueError("target must hold batch*(gamma+1) rows and draft batch*gamma rows")
    dev = target.device
    for t in (draft_tokens, u_accept, u_resid, u_bonus):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("token and uniform tensors must be contiguous device tensors")
    if draft_tokens.dtype not in (torch.int32,) or draft_tokens.numel() != batch * gamma:
        raise ValueError("draft_tokens must be int32[batch*gamma] (uint32 bits)")
    if out is None:
        out = dict(len_mrs=torch.empty(batch, dtype=torch.int32, device=dev),
                   tok_mrs=torch.empty((batch, gamma + 1), dtype=torch.int32, device=dev),
                   len_aa=torch.empty(batch, dtype=torch.int32, device=dev),
                   tok_aa=torch.empty((batch, gamma + 1), dtype=torch.int32, device=dev),
                   summin=torch.empty((batch, gamma), dtype=torch.float32, device=dev),
                   sumprod=torch.empty((batch, gamma), dtype=torch.float32, device=dev))
    ws = workspace(OP_SPEC, F32, batch, Vt, gamma, dev)
    _check(lib.vsel_spec_accept(_ptr(target), ld_t, _ptr(draft), ld_d, batch, gamma, Vt, float(temperature),
                                _ptr(draft_tokens), _ptr(u_accept), _ptr(u_resid), _ptr(u_bonus),
                                _ptr(out["len_mrs"]), _ptr(out["tok_mrs"]), _ptr(out.get("len_aa")),
                                _ptr(out.get("tok_aa")), _ptr(out.get("summin")), _ptr(out.get("sumprod")), _ptr(ws),
                                ws.numel(),
                                _stream(dev)), "vsel_spec_accept", ws)
    return out


def vsel_spec_match(target: torch.Tensor, draft: torch.Tensor, draft_tokens: torch.Tensor, u_match: torch.Tensor,
                    batch: int, gamma: int, temperature: float, vocab=None, out=None):
    """Sampler-match acceptance for batch x gamma drafts -> dict of len_sm, tok_sm, sumprod.

    u_match: float32[batch*(gamma+1)] (one uniform per position, then the bonus draw)."""
    if target.dtype != torch.float32 or draft.dtype != torch.float32:
        raise TypeError("speculative acceptance takes float32 rows")
    rt, Vt, ld_t = _rows(target, vocab)
    rd, Vd, ld_d = _rows(draft, vocab)
    if rt != batch * (gamma + 1) or rd != batch * gamma or Vt != Vd:
        raise ValueError("target must hold batch*(gamma+1) rows and draft batch*gamma rows")
    dev = target.device
    for t in (draft_tokens, u_match):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("token and uniform tensors must be contiguous device tensors")
    if draft_tokens.dtype not in (torch.int32,) or draft_tokens.numel() != batch * gamma:
        raise ValueError("draft_tokens must be int32[batch*gamma] (uint32 bits)")
    if u_match.dtype != torch.float32 or u_match.numel() != batch * (gamma + 1):
        raise ValueError("u_match must be float32[batch*(gamma+1)]")
    if out is None:
        out = dict(len_sm=torch.empty(batch, dtype=torch.int32, device=dev),
                   tok_sm=torch.empty((batch, gamma + 1), dtype=torch.int32, device=dev),
                   sumprod=torch.empty((batch, gamma), dtype=torch.float32, device=dev))
    ws = workspace(OP_SPEC, F32, batch, Vt, gamma, dev)
    _check(lib.vsel_spec_match(_ptr(target), ld_t, _ptr(draft), ld_d, batch, gamma, Vt, float(temperature),
                               _ptr(draft_tokens), _ptr(u_match), _ptr(out["len_sm"]), _ptr(out["tok_sm"]),
                               _ptr(out.get("sumprod")), _ptr(ws), ws.numel(), _stream(dev)), "vsel_spec_match", ws)
    return out


def vsel_spec_accept_filtered(target: torch.Tensor, draft: torch.Tensor, draft_tokens: torch.Tensor,
                              u_accept: torch.Tensor, u_resid: torch.Tensor, u_bonus: torch.Tensor, batch: int,
                              gamma: int, temperature: float, top_k=0, top_p=1.0, min_p=0.0, vocab=None, out=None):
    """vsel_spec_accept with p and q filtered by top-k, top-p and min-p before the temperature."""
    if target.dtype != torch.float32 or draft.dtype != torch.float32:
        raise TypeError("speculative acceptance takes float32 rows")
    rt, Vt, ld_t = _rows(target, vocab)
    rd, Vd, ld_d = _rows(draft, vocab)
    if rt != batch * (gamma + 1) or rd != batch * gamma or Vt != Vd:
        raise ValueError("target must hold batch*(gamma+1) rows and draft batch*gamma rows")
    dev = target.device
    for t in (draft_tokens, u_accept, u_resid, u_bonus):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("token and uniform tensors must be contiguous device tensors")
    if draft_tokens.dtype not in (torch.int32,) or draft_tokens.numel() != batch * gamma:
        raise ValueError("draft_tokens must be int32[batch*gamma] (uint32 bits)")
    if out is None:
        out = dict(len_mrs=torch.empty(batch, dtype=torch.int32, device=dev),
                   tok_mrs=torch.empty((batch, gamma + 1), dtype=torch.int32, device=dev),
                   len_aa=torch.empty(batch, dtype=torch.int32, device=dev),
                   tok_aa=torch.empty((batch, gamma + 1), dtype=torch.int32, device=dev),
                   summin=torch.empty((batch, gamma), dtype=torch.float32, device=dev),
                   sumprod=torch.empty((batch, gamma), dtype=torch.float32, device=dev))
    ws = workspace(OP_SPEC_FILTERED, F32, batch, Vt, gamma, dev)
    _check(lib.vsel_spec_accept_filtered(
        _ptr(target), ld_t, _ptr(draft), ld_d, batch, gamma, Vt, float(temperature), int(top_k), float(top_p),
        float(min_p), _ptr(draft_tokens), _ptr(u_accept), _ptr(u_resid), _ptr(u_bonus), _ptr(out["len_mrs"]),
        _ptr(out["tok_mrs"]), _ptr(out.get("len_aa")), _ptr(out.get("tok_aa")), _ptr(out.get("summin")),
        _ptr(out.get("sumprod")), _ptr(ws), ws.numel(), _stream(dev)), "vsel_spec_accept_filtered", ws)
    return out


def vsel_spec_match_filtered(target: torch.Tensor, draft: torch.Tensor, draft_tokens: torch.Tensor,
                             u_match: torch.Tensor, batch: int, gamma: int, temperature: float, top_k=0, top_p=1.0,
                             min_p=0.0, vocab=None, out=None):
    """vsel_spec_match with p and q filtered by top-k, top-p and min-p before the temperature."""
    if target.dtype != torch.float32 or draft.dtype != torch.float32:
        raise TypeError("speculative acceptance takes float32 rows")
    rt, Vt, ld_t = _rows(target, vocab)
    rd, Vd, ld_d = _rows(draft, vocab)
    if rt != batch * (gamma + 1) or rd != batch * gamma or Vt != Vd:
        raise ValueError("target must hold batch*(gamma+1) rows and draft batch*gamma rows")
    dev = target.device
    for t in (draft_tokens, u_match):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("token and uniform tensors must be contiguous device tensors")
    if draft_tokens.dtype not in (torch.int32,) or draft_tokens.numel() != batch * gamma:
        raise ValueError("draft_tokens must be int32[batch*gamma] (uint32 bits)")
    if u_match.dtype != torch.float32 or u_match.numel() != batch * (gamma + 1):
        raise ValueError("u_match must be float32[batch*(gamma+1)]")
    if out is None:
        out = dict(len_sm=torch.empty(batch, dtype=torch.int32, device=dev),
                   tok_sm=torch.empty((batch, gamma + 1), dtype=torch.int32, device=dev),
                   sumprod=torch.empty((batch, gamma), dtype=torch.float32, device=dev))
    ws = workspace(OP_SPEC_FILTERED, F32, batch, Vt, gamma, dev)
    _check(lib.vsel_spec_match_filtered(
        _ptr(target), ld_t, _ptr(draft), ld_d, batch, gamma, Vt, float(temperature), int(top_k), float(top_p),
        float(min_p), _ptr(draft_tokens), _ptr(u_match), _ptr(out["len_sm"]), _ptr(out["tok_sm"]),
        _ptr(out.get("sumprod")), _ptr(ws), ws.numel(), _stream(dev)), "vsel_spec_match_filtered", ws)
    return out
