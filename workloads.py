"""Seeded synthetic logit workloads for vocab-row selection.

Input construction only: this module draws random rows shaped like the
workloads the pages describe and holds none of the selection arithmetic
(no argmax rule, top-k order, softmax, sampling or acceptance test).  Both
the CPU oracle tests and the GPU path consume these arrays; expected values
always come from the oracle, never from here.

Shapes follow the pages: a 202,048-entry vocabulary for the single-row
greedy decode ("Chapter 21 - Sampling, argmax, and grammar", section 21.1
and Figure 21.1), 248k-column verify rows of 3 and 49 positions with k = 84
(llama.cpp PR #49, "Problem" and "Change"), and a speculative verify batch
("speculative-acceptance.md", "The rules").

Every generator is a pure function of its seed.  Uniforms come from a
separate PCG64 stream (seed + 1000) as float32 values in [0, 1).
"""
from __future__ import annotations

import numpy as np

BASE_SEED = 20261202

V_DECODE = 202_048          # vocabulary of the greedy decode chapter
V_VERIFY = 248_320          # vocabulary of the 248k verify rows
LD_PADDED = 202_112         # padded row stride of the large bf16 batch (64 pad elements)
BF16_NAN = 0x7FC0           # poison written into pad elements


def seed_of(config_no: int) -> int:
    return BASE_SEED + config_no


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16 (round to nearest, ties to even)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = 0x7FFF + ((u >> 16) & 1)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32 (for input construction)."""
    return (b.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- config 1
def greedy_single_row(vocab: int = V_DECODE, seed: int | None = None, chunk: int = 1024):
    """1 row of float32 logits ~ N(0, 3^2) rounded to multiples of 2^-8.

    The row maximum value M is copied to three further indices in three
    different `chunk`-element chunks: one low index placed before the first
    original occurrence of M (so the lowest planted index is the expected
    first maximum whenever the original is not at index 0), one in a middle
    chunk and one in the ragged tail chunk.
    Returns (row[1, vocab] float32, planted index list).
    """
    rng = np.random.default_rng(seed_of(1) if seed is None else seed)
    x = rng.normal(0.0, 3.0, size=vocab)
    x = (np.round(x * 256.0) / 256.0).astype(np.float32)
    m = x.max()
    first = int(np.flatnonzero(x == m)[0])
    n_chunks = -(-vocab // chunk)
    tail_start = (n_chunks - 1) * chunk
    planted = []
    if n_chunks >= 3 and first >= 1 and first // chunk < n_chunks - 2:
        lo = int(rng.integers(0, min(first, 61 * chunk)))
        lo_chunk = lo // chunk
        mid_chunk = int(rng.integers(lo_chunk + 1, n_chunks - 1))
        planted.append(lo)
        planted.append(mid_chunk * chunk + int(rng.integers(0, chunk)))
        planted.append(tail_start + int(rng.integers(0, vocab - tail_start)))
    else:
        planted = sorted(set(int(i) for i in rng.integers(0, vocab, size=3)))
    for i in planted:
        x[i] = m
    return x.reshape(1, vocab), planted


# ---------------------------------------------------------------- config 2
def verify_topk_rows(rows: int = 49, vocab: int = V_VERIFY, seed: int | None = None,
                     n_spikes: int = 5, spike: float = 8.0):
    """rows x vocab float32 logits ~ N(0, 2^2) with +8 added at 5 distinct ids per row."""
    rng = np.random.default_rng(seed_of(2) * 100 + rows if seed is None else seed)
    x = rng.normal(0.0, 2.0, size=(rows, vocab)).astype(np.float32)
    for r in range(rows):
        ids = rng.choice(vocab, size=min(n_spikes, vocab), replace=False)
        x[r, ids] += np.float32(spike)
    return x


# ---------------------------------------------------------------- config 3
def sampling_rows(rows: int = 64, vocab: int = V_DECODE, seed: int | None = None,
                  masked_frac: float = 0.01):
    """rows x vocab float32 logits ~ 2 * Gumbel(0, 1) with 1% of ids set to -inf.

    Returns (logits, u) where u holds one float32 uniform in [0, 1) per row.
    """
    s = seed_of(3) if seed is None else seed
    rng = np.random.default_rng(s)
    x = (2.0 * rng.gumbel(0.0, 1.0, size=(rows, vocab))).astype(np.float32)
    n_mask = int(round(masked_frac * vocab))
    for r in range(rows):
        if n_mask:
            x[r, rng.choice(vocab, size=n_mask, replace=False)] = -np.inf
    u = np.random.default_rng(s + 1000).random(rows, dtype=np.float32)
    return x, u


# ---------------------------------------------------------------- config 4
def speculative_batch(batch: int = 32, gamma: int = 8, vocab: int = V_DECODE,
                      temperature: float = 1.0, seed: int | None = None,
                      noise: float = 0.5):
    """Target rows [batch*(gamma+1), vocab] ~ N(0, 2^2); draft rows [batch*gamma, vocab]
    are the first gamma target rows of each sequence plus N(0, noise^2).

    Drafted tokens are drawn from the draft distribution at `temperature` by
    the Gumbel-max construction (argmax of logits/T plus independent Gumbel
    noise, in float64), i.e. the harness plays the drafter.  Uniforms for the
    accept test, the residual draw and the bonus draw come from the separate
    uniform stream.
    """
    s = seed_of(4) if seed is None else seed
    rng = np.random.default_rng(s)
    tgt = rng.normal(0.0, 2.0, size=(batch, gamma + 1, vocab)).astype(np.float32)
    dft = (tgt[:, :gamma, :] + rng.normal(0.0, noise, size=(batch, gamma, vocab))).astype(np.float32)
    g = rng.gumbel(0.0, 1.0, size=(batch, gamma, vocab))
    t = temperature if temperature > 0 else 1.0
    tokens = np.argmax(dft.astype(np.float64) / t + g, axis=2).astype(np.uint32)
    urng = np.random.default_rng(s + 1000)
    u_acc = urng.random((batch, gamma), dtype=np.float32)
    u_res = urng.random((batch, gamma), dtype=np.float32)
    u_bon = urng.random(batch, dtype=np.float32)
    return dict(target=tgt.reshape(batch * (gamma + 1), vocab),
                draft=dft.reshape(batch * gamma, vocab),
                tokens=tokens.reshape(batch * gamma),
                u_acc=u_acc.reshape(batch * gamma), u_res=u_res.reshape(batch * gamma),
                u_bon=u_bon, batch=batch, gamma=gamma, vocab=vocab,
                temperature=float(temperature))


# ---------------------------------------------------------------- config 5
def decode_batch_bf16(rows: int = 1024, vocab: int = V_DECODE, ld: int = LD_PADDED,
                      seed: int | None = None, tail_frac: float = 0.001,
                      tail_scale: float = 6.0, dup_frac: float = 0.10, block: int = 64):
    """rows x ld bfloat16 bit patterns (uint16): N(0, 4^2) logits, 0.1% of ids
    raised by Exp(1)*6, the row maximum copied to one other random index in 10%
    of rows, and bf16 NaN poison in the ld - vocab pad elements of every row.
    Returns (bits[rows, ld] uint16, list of rows with a copied maximum).
    """
    assert ld >= vocab
    rng = np.random.default_rng(seed_of(5) if seed is None else seed)
    out = np.full((rows, ld), BF16_NAN, dtype=np.uint16)
    dup_rows = []
    for r0 in range(0, rows, block):
        nb = min(block, rows - r0)
        x = rng.standard_normal(size=(nb, vocab), dtype=np.float32) * np.float32(4.0)
        hot = rng.random((nb, vocab), dtype=np.float32) < np.float32(tail_frac)
        x[hot] += rng.exponential(1.0, size=int(hot.sum())).astype(np.float32) * np.float32(tail_scale)
        out[r0:r0 + nb, :vocab] = f32_to_bf16_bits(x)
    dup = rng.random(rows) < dup_frac
    for r in np.nonzero(dup)[0]:
        vals = bf16_bits_to_f32(out[r, :vocab])
        m = vals.max()
        others = np.nonzero(vals != m)[0]
        if len(others) == 0:
            continue
        j = int(others[rng.integers(0, len(others))])
        out[r, j] = f32_to_bf16_bits(np.array([m], dtype=np.float32))[0]
        dup_rows.append(int(r))
    return out, dup_rows


def uniforms(n: int, seed: int) -> np.ndarray:
    """n float32 uniforms in [0, 1) from the uniform stream of `seed`."""
    return np.random.default_rng(seed + 1000).random(n, dtype=np.float32)


# ---------------------------------------------------------------- greedy serving
def excluded_ids(vocab: int, n: int, seed: int, out_of_range: int = 0, duplicates: int = 0) -> np.ndarray:
    """An end-of-generation id set as a serving request would hold it: n distinct
    ids drawn uniformly from [0, vocab), then `out_of_range` ids at or past
    vocab and `duplicates` repeats of ids already in the set, shuffled.
    Returns uint32[n + out_of_range + duplicates]."""
    rng = np.random.default_rng(seed)
    n = min(n, vocab)
    ids = rng.choice(vocab, size=n, replace=False).astype(np.uint32)
    extra = [vocab + rng.integers(0, 1000, size=out_of_range)] if out_of_range else []
    if duplicates and n:
        extra.append(ids[rng.integers(0, n, size=duplicates)])
    allids = np.concatenate([ids] + [np.asarray(e, dtype=np.uint32) for e in extra])
    rng.shuffle(allids)
    return allids.astype(np.uint32)
