"""Benchmark of the vocab-row selection path on one MI355X.

Step = one vsel_topk call (first-maximum argmax + exact top-84 (value, id) +
log-sum-exp, fused in one pass) over a batch of 1,024 bfloat16 logit rows of
202,048 entries at a padded stride of 202,112.  Inputs are resident in HBM
and rotate over three copies (1.24 GB, well past the 256 MB Infinity Cache),
so every step streams its rows from HBM.

Prints one JSON line (rank 0).  `roofline` prices the fused kernel against
the 8 TB/s HBM peak with its algorithmic bytes (valid input elements plus the
outputs); `cpu_baseline` times the CPU oracle on a bounded sample of the same
rows; `extra` holds the latency-bound configurations in microseconds per call.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "logit rows/sec + achieved HBM GB/s, fused argmax+top-k(k=84), V=202048, 1 GPU"

# HBM bytes per launch of the fused kernel from two rocprofv3 counter runs
# (FETCH_SIZE, WRITE_SIZE; scaled by the counters' reading for a plain copy of
# known size), valid for the kernel sources they were taken on.
TRAFFIC_BYTES = 414_951_184
TRAFFIC_SOURCES = ("vocab_row_reductions_amd/csrc/topk_wave.hip", "vocab_row_reductions_amd/csrc/device.hpp",
                   "vocab_row_reductions_amd/csrc/internal.hpp")
TRAFFIC_SHA256 = "4a19aa6b07f632779c5b8a3d1c580bce36736571e55b8bc3ed892956a3f878e7"


def sources_digest():
    """SHA-256 of the fused kernel's sources with comments and whitespace
    removed, so that only a change of code makes the counters stale."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def measured_traffic():
    """Bytes per launch from the counter runs, or None if the kernel changed since."""
    return TRAFFIC_BYTES if sources_digest() == TRAFFIC_SHA256 else None
HBM_PEAK_GBS = 8000.0
ROWS, V, LD, K = 1024, 202_048, 202_112, 84


def algorithmic_bytes(rows, vocab, elem, k):
    # valid input elements + top-k values and ids + argmax + log-sum-exp
    return rows * (vocab * elem + k * 8 + 4 + 4)


RAMP_S = 0.03  # calls before each extra measurement, so the clocks are up (they drop when idle)


def ramp_up(fn):
    import torch
    t, i = time.perf_counter(), 0
    while time.perf_counter() - t < RAMP_S:
        fn(i)
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def time_calls(fn, n, warmup, stream):
    import torch
    ramp_up(fn)
    for _ in range(warmup):
        fn(0)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(n):
        fn(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) * 1e3 / n  # microseconds per call


def time_graph(fn, n, stream):
    """Device microseconds per call: n calls captured in one graph, replayed."""
    import torch
    fn(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    ramp_up(lambda i: g.replay())
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    reps = 5
    ev0.record()
    for _ in range(reps):
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) * 1e3 / (reps * n)


def _only_rows(torch, W, dev):
    x, u = W.sampling_rows()
    return torch.from_numpy(x).to(dev), torch.from_numpy(u).to(dev)


def _only_spec(torch, W, dev):
    d = W.speculative_batch()
    g = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return g(d["target"]), g(d["draft"]), (g(d["tokens"].view(np.int32)), g(d["u_acc"]), g(d["u_res"]),
                                            g(d["u_bon"]), 32, 8, 1.0)


def _only_topp(torch, vsel, W, dev):
    x, u = _only_rows(torch, W, dev)
    return lambda i: vsel.vsel_sample_chain(x, 0.7, u, top_p=0.95)


def _only_typical(torch, vsel, W, dev):
    x, u = _only_rows(torch, W, dev)
    return lambda i: vsel.vsel_sample_chain(x, 0.7, u, typical_p=0.9)


def _only_threshold(torch, vsel, W, dev):
    x, u = _only_rows(torch, W, dev)
    return lambda i: vsel.vsel_sample_chain(x, 0.7, u, top_n_sigma=1.0, min_p=0.05)


def _only_sample(torch, vsel, W, dev):
    x, u = _only_rows(torch, W, dev)
    return lambda i: vsel.vsel_sample(x, 0.7, 20, 0.95, u)


def _only_chain(torch, vsel, W, dev):
    x, u = _only_rows(torch, W, dev)
    return lambda i: vsel.vsel_sample_chain(x, 0.7, u, top_n_sigma=1.0, top_k=50, typical_p=0.9, top_p=0.95,
                                            min_p=0.05)


def _only_spec_accept(torch, vsel, W, dev):
    tg, dr, args = _only_spec(torch, W, dev)
    return lambda i: vsel.vsel_spec_accept(tg, dr, *args)


def _only_spec_match(torch, vsel, W, dev):
    tg, dr, args = _only_spec(torch, W, dev)
    um = torch.from_numpy(W.uniforms(32 * 9, seed=W.BASE_SEED + 930)).to(dev)
    return lambda i: vsel.vsel_spec_match(tg, dr, args[0], um, 32, 8, 1.0)


def _only_spec_filtered(torch, vsel, W, dev):
    tg, dr, args = _only_spec(torch, W, dev)
    return lambda i: vsel.vsel_spec_accept_filtered(tg, dr, *args, top_p=0.9)


def _only_verify(torch, vsel, W, dev):
    x = torch.from_numpy(W.verify_topk_rows(rows=3)).to(dev)
    return lambda i: vsel.vsel_topk(x, 84)


# --only: one configuration, for profiling its kernels
ONLY = {"wholerow-topp": _only_topp, "wholerow-typical": _only_typical, "wholerow-threshold": _only_threshold,
        "sample": _only_sample,
        "chain": _only_chain, "spec-accept": _only_spec_accept, "spec-match": _only_spec_match,
        "spec-filtered-wholerow": _only_spec_filtered,
        "verify3": _only_verify}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--ramp-ms", type=float, default=100.0,
                    help="untimed calls for this long before the warm-up steps (the GPU clocks ramp under load)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=40)
    ap.add_argument("--only", choices=sorted(ONLY),
                    help="profiling: run --steps calls of one other configuration (after --warmup calls) and print "
                         "its time per call instead of the benchmark line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (the selection path has no multi-GPU leg); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import vocab_row_reductions_amd as vsel
    import workloads as W

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    if args.only:
        fn = ONLY[args.only](torch, vsel, W, dev)
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for i in range(args.steps):
            fn(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        print(json.dumps({"only": args.only, "steps": args.steps, "warmup": args.warmup,
                          "us_per_call": ev0.elapsed_time(ev1) * 1e3 / max(1, args.steps)}), flush=True)
        return
    print(f"bench: generating {ROWS} x {V} bf16 rows (ld {LD})", file=sys.stderr, flush=True)
    bits, _ = W.decode_batch_bf16(rows=ROWS, vocab=V, ld=LD)
    base = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
    bufs = [base] + [base.clone() for _ in range(2)]
    out = dict(vals=torch.empty((ROWS, K), dtype=torch.float32, device=dev),
               ids=torch.empty((ROWS, K), dtype=torch.int32, device=dev),
               argmax=torch.empty(ROWS, dtype=torch.int32, device=dev),
               lse=torch.empty(ROWS, dtype=torch.float32, device=dev))

    def step(i):
        vsel.vsel_topk(bufs[i % 3], K, vocab=V, out=out)

    # The GPU raises its clocks over the first tens of milliseconds of load (and
    # again after an idle second): without this ramp the first few hundred calls
    # run about 10% slower than the steady state a serving loop sees.
    ramp_calls, t_r = 0, time.perf_counter()
    while (time.perf_counter() - t_r) * 1e3 < args.ramp_ms:
        for _ in range(20):
            step(ramp_calls)
            ramp_calls += 1
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step(0)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    us_per_launch = ev0.elapsed_time(ev1) * 1e3 / args.steps
    ms_per_step = wall * 1e3 / args.steps
    rows_per_s = ROWS / (ms_per_step / 1e3)
    abytes = algorithmic_bytes(ROWS, V, 2, K)
    achieved = abytes / (us_per_launch * 1e-6) / 1e9

    result = {
        "metric": METRIC, "value": rows_per_s, "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "large-batch decode selection: 1024 rows x 202048 bf16 logits, ld 202112, "
                               "fused argmax + top-k k=84 + logsumexp, inputs rotated over 3 HBM copies",
                   "rows": ROWS, "vocab": V, "ld": LD, "k": K,
                   "clock_ramp": {"ms": args.ramp_ms, "calls": ramp_calls}},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "kernel": "topk_wave_kernel<bf16, lse>", "us_per_launch": us_per_launch,
                     "algorithmic_bytes_per_launch": abytes},
    }

    # the read-only streaming floor of this machine: the faster of a plain full-batch
    # reduction (torch.amax) and the library's argmax-only pass, over the same
    # rotated buffers; bytes = every element of the padded rows
    stream_bytes = ROWS * LD * 2
    fl_amax = time_calls(lambda i: torch.amax(bufs[i % 3]), 50, 5, stream)
    fl_arg = time_calls(lambda i: vsel.vsel_argmax(bufs[i % 3], vocab=V, want_val=False), 50, 5, stream)
    floor_gbs = max(stream_bytes / (fl_amax * 1e-6), ROWS * V * 2 / (fl_arg * 1e-6)) / 1e9
    result["roofline"]["stream_floor"] = {
        "gbs": floor_gbs, "frac_of_floor": achieved / floor_gbs,
        "torch_amax_us": fl_amax, "argmax_only_us": fl_arg,
        "what": "read-only streaming floor measured on this box: the faster of torch.amax over the padded batch "
                "and the library's argmax-only pass"}

    if not args.no_cpu_baseline:
        from oracle import oracle as O
        import statistics
        cores = len(os.sched_getaffinity(0))

        def rate(nthreads, rows, reps):
            t = time.perf_counter()
            for _ in range(reps):
                O.topk(bits[:rows], K, vocab=V, nthreads=nthreads)
            return rows * reps / (time.perf_counter() - t)

        O.topk(bits[:2], K, vocab=V, nthreads=cores)
        t_all = time.perf_counter()
        multi = statistics.median(rate(cores, ROWS, args.cpu_reps) for _ in range(3))
        single = statistics.median(rate(1, 64, 1) for _ in range(3))
        spent = time.perf_counter() - t_all
        model = ""
        try:
            with open("/proc/cpuinfo") as f:
                model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
        except OSError:
            pass
        result["cpu_baseline"] = {
            "value": multi, "unit": "rows/s", "cores": cores, "kind": "oracle",
            "sample": f"the whole {ROWS}-row batch {args.cpu_reps} times per run, median of 3 runs, same fused "
                      f"outputs (top-84, argmax, float64 logsumexp); single-thread: 64 rows, median of 3; "
                      f"{spent:.1f} s of CPU work in all",
            "value_1thread": single, "cpu_model": model}

    if not args.no_extra:
        result["extra"] = extras(torch, vsel, W, dev, stream, bufs, out)

    print(json.dumps(result), flush=True)


def extras(torch, vsel, W, dev, stream, bufs, out):
    """Microseconds per call for the other configurations (cold: inputs rotated
    over >= 1 GB of copies; warm: one buffer, as right after the LM head)."""
    from vocab_row_reductions_amd.acceptance import acceptance_counters, summary_line
    ex = {}
    ex["topk_k84_us"] = time_calls(lambda i: vsel.vsel_topk(bufs[i % 3], K, vocab=V, out=out), 50, 5, stream)
    out64 = dict(vals=torch.empty((ROWS, 64), dtype=torch.float32, device=dev),
                 ids=torch.empty((ROWS, 64), dtype=torch.int32, device=dev),
                 argmax=torch.empty(ROWS, dtype=torch.int32, device=dev),
                 lse=torch.empty(ROWS, dtype=torch.float32, device=dev))
    ex["topk_k64_us"] = time_calls(lambda i: vsel.vsel_topk(bufs[i % 3], 64, vocab=V, out=out64), 50, 5, stream)
    ex["topk_k64_gbs"] = algorithmic_bytes(ROWS, V, 2, 64) / (ex["topk_k64_us"] * 1e-6) / 1e9
    ex["argmax_only_bf16_1024rows_us"] = time_calls(lambda i: vsel.vsel_argmax(bufs[i % 3], vocab=V), 50, 5, stream)
    # greedy serving variant: a 16-id end-of-generation set, status word per row
    exd = torch.from_numpy(W.excluded_ids(V, 16, seed=7).view(np.int32)).to(dev)
    ex["argmax_excluding16_bf16_1024rows_us"] = time_calls(
        lambda i: vsel.vsel_argmax_excluding(bufs[i % 3], exd, vocab=V), 50, 5, stream)

    def cold_copies(x, total=1 << 30):
        n = max(1, -(-total // (x.numel() * x.element_size())))
        return [x] + [x.clone() for _ in range(n - 1)]

    # Latency-bound configurations: eager microseconds per call (includes the
    # Python binding and the launch) and device microseconds per call (graph
    # replay); cold = inputs rotated over >= 256 MB of copies, warm = one buffer.
    def lat(name, fn_warm, fn_cold, n=100):
        ex[name + "_eager_us"] = time_calls(fn_warm, n, 5, stream)
        ex[name + "_device_warm_us"] = time_graph(fn_warm, 20, stream)
        ex[name + "_device_cold_us"] = time_graph(fn_cold, 20, stream)

    # config 1: one row argmax
    row, _ = W.greedy_single_row()
    r1 = cold_copies(torch.from_numpy(row).to(dev), 1 << 28)
    o1 = torch.empty(1, dtype=torch.int32, device=dev)
    lat("argmax_1x202048", lambda i: vsel.vsel_argmax(r1[0], out_idx=o1, want_val=False),
        lambda i: vsel.vsel_argmax(r1[i % len(r1)], out_idx=o1, want_val=False))
    del r1
    # config 2: verify rows, k = 84
    for rows in (3, 49):
        x = W.verify_topk_rows(rows=rows)
        xs = cold_copies(torch.from_numpy(x).to(dev), 1 << 28)
        o2 = dict(vals=torch.empty((rows, 84), dtype=torch.float32, device=dev),
                  ids=torch.empty((rows, 84), dtype=torch.int32, device=dev),
                  argmax=torch.empty(rows, dtype=torch.int32, device=dev), lse=None)
        lat(f"topk_{rows}x248320_k84", lambda i: vsel.vsel_topk(xs[0], 84, out=o2),
            lambda i: vsel.vsel_topk(xs[i % len(xs)], 84, out=o2))
        del xs
    # config 3: sampling
    x, u = W.sampling_rows()
    xs = cold_copies(torch.from_numpy(x).to(dev), 1 << 28)
    ud = torch.from_numpy(u).to(dev)
    ot = torch.empty(64, dtype=torch.int32, device=dev)
    ol = torch.empty(64, dtype=torch.float32, device=dev)
    lat("sample_64x202048", lambda i: vsel.vsel_sample(xs[0], 0.7, 20, 0.95, ud, out_token=ot, out_logprob=ol),
        lambda i: vsel.vsel_sample(xs[i % len(xs)], 0.7, 20, 0.95, ud, out_token=ot, out_logprob=ol))
    # the ordered chain on the same rows: the moments pass, then top-k with
    # top-n-sigma, typical-p, top-p and min-p on the candidates; and the
    # whole-row draw with the two threshold filters
    chain = dict(top_n_sigma=1.0, top_k=50, typical_p=0.9, top_p=0.95, min_p=0.05)
    lat("sample_chain_64x202048", lambda i: vsel.vsel_sample_chain(xs[0], 0.7, ud, out_token=ot, out_logprob=ol,
                                                                   **chain),
        lambda i: vsel.vsel_sample_chain(xs[i % len(xs)], 0.7, ud, out_token=ot, out_logprob=ol, **chain))
    ex["sample_chain_rowdraw_64x202048_device_cold_us"] = time_graph(
        lambda i: vsel.vsel_sample_chain(xs[i % len(xs)], 0.7, ud, top_n_sigma=1.0, min_p=0.05, out_token=ot,
                                         out_logprob=ol), 20, stream)
    ex["sample_chain_typical09_wholerow_64x202048_device_cold_us"] = time_graph(
        lambda i: vsel.vsel_sample_chain(xs[i % len(xs)], 0.7, ud, typical_p=0.9, out_token=ot, out_logprob=ol), 10,
        stream)
    ex["sample_chain_topp095_wholerow_64x202048_device_cold_us"] = time_graph(
        lambda i: vsel.vsel_sample_chain(xs[i % len(xs)], 0.7, ud, top_p=0.95, out_token=ot, out_logprob=ol), 20,
        stream)
    del xs
    # config 4: speculative acceptance (target + draft rows: 440 MB, already past the Infinity Cache)
    d = W.speculative_batch()
    g = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    tg, dr = g(d["target"]), g(d["draft"])
    args = (g(d["tokens"].view(np.int32)), g(d["u_acc"]), g(d["u_res"]), g(d["u_bon"]), 32, 8, 1.0)
    so = vsel.vsel_spec_accept(tg, dr, *args)
    ex["spec_accept_32x8_eager_us"] = time_calls(lambda i: vsel.vsel_spec_accept(tg, dr, *args, out=so), 50, 5, stream)
    ex["spec_accept_32x8_device_us"] = time_graph(lambda i: vsel.vsel_spec_accept(tg, dr, *args, out=so), 10, stream)
    # the run counters and both closed forms of the same pass, over the tested positions
    cm = acceptance_counters(so["len_mrs"].cpu().numpy(), 8, so["summin"].cpu().numpy(), so["sumprod"].cpu().numpy())
    ex["spec_accept_32x8_counters"] = cm
    print(summary_line(cm), file=sys.stderr, flush=True)
    # the same batch under sampler-match (one uniform per position and the bonus)
    um = g(W.uniforms(32 * 9, seed=2026))
    margs = (args[0], um, 32, 8, 1.0)
    mo = vsel.vsel_spec_match(tg, dr, *margs)
    ex["spec_match_32x8_eager_us"] = time_calls(lambda i: vsel.vsel_spec_match(tg, dr, *margs, out=mo), 50, 5, stream)
    ex["spec_match_32x8_device_us"] = time_graph(lambda i: vsel.vsel_spec_match(tg, dr, *margs, out=mo), 10, stream)
    cs = acceptance_counters(mo["len_sm"].cpu().numpy(), 8, so["summin"].cpu().numpy(), mo["sumprod"].cpu().numpy(),
                             rule="sampler-match")
    ex["spec_match_32x8_counters"] = cs
    print(summary_line(cs), file=sys.stderr, flush=True)
    # both rules with filtered p and q (top-k 50 then top-p 0.95; top-p 0.9 over whole rows)
    for name, kw in (("k50_p095", dict(top_k=50, top_p=0.95)), ("wholerow_p09", dict(top_p=0.9))):
        fo = vsel.vsel_spec_accept_filtered(tg, dr, *args, **kw)
        ex[f"spec_accept_filtered_{name}_32x8_device_us"] = time_graph(
            lambda i: vsel.vsel_spec_accept_filtered(tg, dr, *args, out=fo, **kw), 10, stream)
        fm = vsel.vsel_spec_match_filtered(tg, dr, *margs, **kw)
        ex[f"spec_match_filtered_{name}_32x8_device_us"] = time_graph(
            lambda i: vsel.vsel_spec_match_filtered(tg, dr, *margs, out=fm, **kw), 10, stream)
    del tg, dr
    # fp32 variant of the headline batch (one buffer pair, 827 MB each)
    x32 = bufs[0][:, :V].float().contiguous()
    x32b = [x32, x32.clone()]
    o32 = dict(vals=torch.empty((ROWS, K), dtype=torch.float32, device=dev),
               ids=torch.empty((ROWS, K), dtype=torch.int32, device=dev),
               argmax=torch.empty(ROWS, dtype=torch.int32, device=dev),
               lse=torch.empty(ROWS, dtype=torch.float32, device=dev))
    us32 = time_calls(lambda i: vsel.vsel_topk(x32b[i % 2], K, out=o32), 30, 3, stream)
    ex["topk_fp32_1024x202048_k84_us"] = us32
    ex["topk_fp32_1024x202048_k84_gbs"] = algorithmic_bytes(ROWS, V, 4, K) / (us32 * 1e-6) / 1e9
    del x32b, x32
    # a plain device-to-device copy of the same batch (read + write), for context
    src = bufs[0]
    dst = torch.empty_like(src)
    cu = time_calls(lambda i: dst.copy_(bufs[i % 3]), 30, 3, stream)
    ex["torch_copy_bf16_batch_us"] = cu
    ex["torch_copy_bf16_batch_gbs"] = 2 * src.numel() * 2 / (cu * 1e-6) / 1e9
    # three decimals for times and rates; four significant digits for probabilities below 0.01
    return {k: (float(f"{v:.4g}") if isinstance(v, float) and abs(v) < 0.01 else round(v, 3) if isinstance(v, float) else v)
            for k, v in ex.items()}


if __name__ == "__main__":
    main()
