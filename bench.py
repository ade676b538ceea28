#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

A step is one pass of the whole path over one synthetic batch already resident
in HBM: assign (task map) + persistent split + combine.  A layer is split +
combine with the step's task map reused, as every layer of the model reuses
it.  Before every timed step or layer a 512 MiB buffer is streamed through so
neither L2 nor the 256 MB Infinity Cache still holds K/V from the previous one.
HIP events on the launch stream bracket each step (one pair, nothing between
the kernels), each layer (one pair), and -- through the library's timing hook --
each kernel's own start and end.  The default flush reads the buffer (a
reduction), so the caches hold clean lines and no write-back competes with the
timed kernels.

Prints ONE JSON line.  The headline workload is the long-context batch (8
requests of 64K-256K tokens, 64/8 heads, bf16: the largest single-GPU
configuration).  value = achieved HBM GB/s of a layer (algorithmic bytes /
mean layer time); ms_per_step is the whole step with assign.  The line also
carries the per-kernel times, the split kernel's roofline, a block with the
same figures for the other configurations (one GPU's TP8 share, the skewed
batch, the fp8 batch, the minimum-work-floor case), the static split-KV
comparison on the skewed batch, and the CPU oracle timed on the host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FLUSH_BYTES = 512 << 20
CALIB_BYTES = 256 << 20
SPLIT_SRC = os.path.join(ROOT, "load_balanced_split_assign_amd", "csrc", "lbsa_attention.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "split_kernel_traffic.json")


def alg_bytes(seqlens, Hq, Hkv, D, kv_dtype, q_len=1):
    """Bytes the method must move: live K/V (+ scales), Q (+ scale), bf16 out,
    page-table entries and lengths.  Partials are overhead, reported apart.
    With q_len query tokens per request, Q and out scale with q_len; K/V is
    read once for all of them."""
    e_kv, s_kv, e_q, s_q = (2, 0, 2, 0) if kv_dtype == "bf16" else (1, 8, 1, 4)
    B = len(seqlens)
    n_tiles = sum((L + 63) // 64 for L in seqlens)
    kv = sum(seqlens) * Hkv * (2 * D * e_kv + s_kv)
    q = B * q_len * Hq * (D * e_q + s_q)
    out = B * q_len * Hq * D * 2
    meta = 4 * n_tiles + 4 * B
    return {"kv": kv, "q": q, "out": out, "meta": meta, "layer": kv + q + out + meta, "split": kv + q + meta}


def summarize(xs):
    xs = sorted(xs)
    return {"mean": statistics.fmean(xs), "median": statistics.median(xs), "min": xs[0],
            "p90": xs[min(len(xs) - 1, int(math.ceil(0.9 * len(xs))) - 1)]}


def source_sha(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


class Path:
    """Preallocated buffers for one batch: assign() enqueues the assign kernel,
    layer() the split + combine of lbsa_decode (single-chunk segments written by
    the split kernel), split()/combine() the two halves as separate calls."""

    def __init__(self, batch, P, F=0):
        import torch

        from load_balanced_split_assign_amd import lbsa
        self.lbsa, self.b, self.P, self.F = lbsa, batch, P, F
        B, Hq, Hkv = batch["B"], batch["num_heads"], batch["num_kv_heads"]
        self.q_len = batch.get("q_len", 1)
        dev = batch["q"].device
        self.tm = torch.empty(lbsa.task_map_bytes(B, Hkv, P), dtype=torch.uint8, device=dev)
        self.ws = torch.empty(lbsa.workspace_bytes(B, Hq, Hkv, P, q_len=self.q_len), dtype=torch.uint8, device=dev)
        self.out = torch.empty(tuple(batch["q"].shape), dtype=torch.bfloat16, device=dev)

    def assign(self):
        b = self.b
        self.lbsa.plan(b["seqlens"], b["num_heads"], b["num_kv_heads"], b["max_pages"], self.P, self.F,
                       task_map=self.tm)

    def layer(self):
        b = self.b
        self.lbsa.decode(b["q"], b["k_cache"], b["v_cache"], b["page_table"], self.tm, self.P, b["softmax_scale"],
                         q_scale=b["q_scale"], k_scale=b["k_scale"], v_scale=b["v_scale"], workspace=self.ws,
                         out=self.out)

    def split(self):
        b = self.b
        self.lbsa.decode_split(b["q"], b["k_cache"], b["v_cache"], b["page_table"], self.tm, self.P,
                               b["softmax_scale"], q_scale=b["q_scale"], k_scale=b["k_scale"],
                               v_scale=b["v_scale"], workspace=self.ws)

    def combine(self):
        b = self.b
        self.lbsa.decode_combine(b["B"], b["num_heads"], b["num_kv_heads"], self.P, self.tm, self.ws,
                                 out=self.out, q_len=self.q_len)


def auto_P(batch, q_len=None):
    """lbsa_auto_workgroups for a batch built on this host (its lengths are known here)."""
    from load_balanced_split_assign_amd import lbsa
    sl = [int(x) for x in batch["seqlens"].cpu()]
    kv = batch.get("kv_dtype") or ("fp8" if batch.get("k_scale") is not None else "bf16")
    return lbsa.auto_workgroups(sl, batch["num_kv_heads"], kv, q_len or batch.get("q_len", 1) or 1)


def make_flush(mode):
    """Evicts K/V of the previous step from L2 and the Infinity Cache.  'read'
    streams a 512 MiB buffer through a reduction (the caches are left holding
    clean lines, so the next kernel pays no write-back); 'write' rewrites it;
    'none' leaves the caches warm."""
    import torch
    buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda:0")
    if mode == "read":
        return lambda i: buf.sum()
    if mode == "write":
        return lambda i: buf.fill_(float(i & 7))
    return lambda i: None


MIN_WARM_S = 0.25   # seconds of untimed steps before any timed pass


def _warm(run_once, warmup, flush):
    """At least `warmup` untimed runs and MIN_WARM_S of busy GPU (synchronised
    one by one): after an idle stretch (the CPU leg, a batch built on the host)
    the clocks take tens of ms of load to come back up, and a few short runs do
    not cover that."""
    import torch
    t_end = time.perf_counter() + MIN_WARM_S
    i = 0
    while i < warmup or time.perf_counter() < t_end:
        flush(i)
        run_once()
        torch.cuda.synchronize()
        i += 1


def _pairs(n):
    import torch
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]


def time_steps(path, steps, warmup, flush):
    """Per-step times (us) in three passes, the flush outside every event pair:
    `step` = assign + split + combine under one pair (as a decode step runs);
    `layer` = split + combine under one pair with the map built beforehand (as
    every layer runs); `*_kernel` = each kernel's own start-to-end stamps from the
    library's timing hook (no marker packets between the launches, so no added
    dispatch gaps: the durations rocprofv3 reports) -- the assign kernel's in a
    step, the split and combine kernels' in a layer."""
    import torch

    from load_balanced_split_assign_amd import lbsa
    stream = torch.cuda.current_stream()
    _warm(lambda: (path.assign(), path.layer()), warmup, flush)
    whole = _pairs(steps)
    for i in range(steps):
        flush(i)
        whole[i][0].record(stream)
        path.assign(); path.layer()
        whole[i][1].record(stream)
    lay = _pairs(steps)
    path.assign()
    for i in range(steps):
        flush(i)
        lay[i][0].record(stream)
        path.layer()
        lay[i][1].record(stream)
    aev = _pairs(steps)                             # the assign kernel, as in a step
    kev = [_pairs(2) for _ in range(steps)]         # split and combine, as in a layer (map reused)
    for e in [aev] + kev:
        for a, b in e:
            a.record(stream); b.record(stream)      # torch creates an event at its first record
    torch.cuda.synchronize()
    for i in range(steps):
        flush(i)
        lbsa.time_next_kernels([aev[i]])
        path.assign(); path.layer()
    path.assign()
    for i in range(steps):
        flush(i)
        lbsa.time_next_kernels(kev[i])              # the split and the combine of decode
        path.layer()
    torch.cuda.synchronize()
    us = lambda ps: [1000.0 * a.elapsed_time(b) for a, b in ps]  # noqa: E731
    return {"step": us(whole), "layer": us(lay), "assign_kernel": us(aev),
            "split_kernel": us([e[0] for e in kev]), "combine_kernel": us([e[1] for e in kev])}


def time_steps_graph(path, steps, warmup, flush):
    """Per-step times (us) of the assign + split + combine sequence captured in
    one HIP graph and replayed (the flush runs eagerly between replays)."""
    import torch
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        path.assign(); path.layer()
    stream = torch.cuda.current_stream()
    _warm(g.replay, warmup, flush)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        flush(i)
        ev[i][0].record(stream)
        g.replay()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return [1000.0 * a.elapsed_time(b) for a, b in ev]


def graph_bench(args):
    """The step (assign + split + combine) launched eagerly against the same
    three launches captured in one HIP graph and replayed, on tp8_share, the
    smallest Table 3 mix and skewed (medians, us)."""
    import torch

    from load_balanced_split_assign_amd import lbsa
    flush = make_flush(args.flush)
    rows = []
    for name in ("tp8_share", "t3_64x0.5K", "skewed"):
        b = gpu_batch(name)
        path = Path(b, auto_P(b))
        eager = summarize(time_steps(path, args.steps, args.warmup, flush)["step"])["median"]
        graph = summarize(time_steps_graph(path, args.steps, args.warmup, flush))["median"]
        rows.append({"workload": name, "eager_step_us": round(eager, 2), "graph_step_us": round(graph, 2)})
        del b, path
        torch.cuda.empty_cache()
    print(json.dumps({"graph_vs_eager": rows, "unit": "us", "flush": args.flush}), flush=True)


def time_static(batch, S, steps, warmup, flush, stamps=False):
    """Static split-KV (split + fixed-S combine) under one event pair per call;
    with stamps=True also each kernel's own start/end (summaries in us)."""
    import torch

    from load_balanced_split_assign_amd import lbsa
    B, Hq, Hkv = batch["B"], batch["num_heads"], batch["num_kv_heads"]
    ws = torch.empty(lbsa.static_workspace_bytes(B, Hq, Hkv, S), dtype=torch.uint8, device=batch["q"].device)
    out = torch.empty((B, Hq, 128), dtype=torch.bfloat16, device=batch["q"].device)

    def run():
        lbsa.decode_static(batch["q"], batch["k_cache"], batch["v_cache"], batch["page_table"], batch["seqlens"],
                           S, batch["softmax_scale"], q_scale=batch["q_scale"], k_scale=batch["k_scale"],
                           v_scale=batch["v_scale"], workspace=ws, out=out)
    stream = torch.cuda.current_stream()
    _warm(run, warmup, flush)
    ev = _pairs(steps)
    for i in range(steps):
        flush(i)
        ev[i][0].record(stream)
        run()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    res = summarize([1000.0 * a.elapsed_time(b) for a, b in ev])
    if stamps:
        kev = [_pairs(2) for _ in range(steps)]
        for e in kev:
            for a, b in e:
                a.record(stream); b.record(stream)
        torch.cuda.synchronize()
        for i in range(steps):
            flush(i)
            lbsa.time_next_kernels(kev[i])
            run()
        torch.cuda.synchronize()
        res["split_kernel"] = statistics.fmean(1000.0 * e[0][0].elapsed_time(e[0][1]) for e in kev)
        res["combine_kernel"] = statistics.fmean(1000.0 * e[1][0].elapsed_time(e[1][1]) for e in kev)
    torch.cuda.synchronize()
    return res


def time_layer(path, steps, warmup, flush, with_assign=False):
    """Event time (us) of split + combine (lbsa_decode; plus assign if asked) with
    one event pair around them, as a layer (or a step) runs in use."""
    import torch
    stream = torch.cuda.current_stream()

    def run():
        if with_assign:
            path.assign()
        path.layer()
    path.assign()            # the map the layers reuse
    _warm(run, warmup, flush)
    ev = _pairs(steps)
    for i in range(steps):
        flush(i)
        ev[i][0].record(stream)
        run()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return summarize([1000.0 * a.elapsed_time(b) for a, b in ev])


def static_sweep(batch, P, steps, warmup, flush, splits=(1, 2, 4, 8, 16, 32, 64)):
    """Static split-KV at the heuristic S = ceil(P / (B * Hkv)) and over a sweep of S."""
    heur = max(1, -(-P // (batch["B"] * batch["num_kv_heads"])))
    sweep = {S: time_static(batch, S, steps, warmup, flush)["mean"] for S in splits}
    heur_t = sweep.get(heur) or time_static(batch, heur, steps, warmup, flush)["mean"]
    best = min(sweep, key=sweep.get)
    return heur, heur_t, best, sweep


def table3(args):
    """The six KV-length mixes of the vLLM post's Table 3 (fp8 KV, 8 query heads /
    1 KV head): dynamic (map reused: split + combine; and with assign) against
    the static split-KV kernel at the heuristic S and at the best S of a sweep,
    each with its kernels' own start/end stamps."""
    import torch

    from load_balanced_split_assign_amd import lbsa
    from load_balanced_split_assign_amd import workload as wl
    flush = make_flush(args.flush)
    rows = []
    for name in wl.TABLE3:
        b = gpu_batch(name)
        w = wl.WORKLOADS[name]
        P = args.workgroups or auto_P(b)
        sl = [int(x) for x in b["seqlens"].cpu()]
        ab = alg_bytes(sl, b["num_heads"], b["num_kv_heads"], 128, w.kv_dtype)
        path = Path(b, P)
        t = {k: summarize(v)["mean"] for k, v in time_steps(path, args.steps, args.warmup, flush).items()}
        m = lbsa.read_task_map(path.tm, b["B"], b["num_kv_heads"], P)
        heur, heur_t, best, sweep = static_sweep(b, P, max(10, args.steps // 2), 3, flush)
        st = time_static(b, best, max(10, args.steps // 2), 3, flush, stamps=True)
        layer = t["layer"]
        rows.append({"mix": name[3:], "batch": b["B"], "live_tokens": sum(sl), "alg_bytes": ab["layer"],
                     "K": m["K"], "Ndesc": m["Ndesc"], "single_chunk_segments": int((m["seg_num_chunks"] == 1).sum()),
                     "dynamic_layer_us": round(layer, 2), "dynamic_step_us": round(t["step"], 2),
                     "dynamic_split_kernel_us": round(t["split_kernel"], 2),
                     "dynamic_combine_kernel_us": round(t["combine_kernel"], 2),
                     "assign_kernel_us": round(t["assign_kernel"], 2),
                     "layer_GBps": round(ab["layer"] / layer / 1e3, 1),
                     "static_heuristic_S": heur, "static_heuristic_us": round(heur_t, 2),
                     "static_best_S": best, "static_best_us": round(sweep[best], 2),
                     "static_best_split_kernel_us": round(st["split_kernel"], 2),
                     "static_best_combine_kernel_us": round(st["combine_kernel"], 2),
                     "static_sweep_us": {str(k): round(v, 2) for k, v in sweep.items()},
                     "speedup_vs_static_best": round(sweep[best] / layer, 3),
                     "speedup_vs_static_heuristic": round(heur_t / layer, 3)})
        del b, path
        torch.cuda.empty_cache()
    print(json.dumps({"table3": rows, "P": P, "unit": "us", "flush": args.flush}), flush=True)


def mtp_bench(args):
    """Multi-token decode (2 query tokens per request: verifying one draft token
    of a multi-token-prediction layer) against one-token decode on the same
    lengths: layer time (split + combine, map reused) for each."""
    import torch

    from load_balanced_split_assign_amd import lbsa
    from load_balanced_split_assign_amd import workload as wl
    flush = make_flush(args.flush)
    rows = []
    for name in ("tp8_share", "skewed", "fp8"):
        w = wl.WORKLOADS[name]
        row = {"workload": name, "kv_dtype": w.kv_dtype, "num_heads": w.num_heads, "num_kv_heads": w.num_kv_heads}
        for ql in (1, 2):
            b = wl.make_batch(name, tail="normal", device="cuda:0", q_len=ql)
            P = args.workgroups or w.num_workgroups or auto_P(b, ql)
            row[f"q{ql}_P"] = P
            sl = [int(x) for x in b["seqlens"].cpu()]
            ab = alg_bytes(sl, b["num_heads"], b["num_kv_heads"], 128, w.kv_dtype, q_len=ql)
            tl = time_layer(Path(b, P), args.steps, args.warmup, flush)
            t = tl["mean"]
            row[f"q{ql}_layer_us"] = round(t, 2)
            row[f"q{ql}_layer_median_us"] = round(tl["median"], 2)
            row[f"q{ql}_layer_p90_us"] = round(tl["p90"], 2)
            row[f"q{ql}_GBps"] = round(ab["layer"] / t / 1e3, 1)
            row["batch"] = b["B"]
            del b
            torch.cuda.empty_cache()
        row["q2_over_q1"] = round(row["q2_layer_us"] / row["q1_layer_us"], 3)
        rows.append(row)
    print(json.dumps({"multi_token_decode": rows, "unit": "us", "flush": args.flush}), flush=True)


# HPC-Ops latency (ms) on one H20 from the vLLM post's Table 4: context for the
# same shapes here, not a target measured on this machine
TABLE4_H20_MS = {"q512": 0.047, "q1ks2k": 0.406, "q2k": 0.530, "q4k": 2.002, "q8k": 7.883, "2q1ks4k": 1.835,
                 "8q1s1k": 0.019, "16q1s2k": 0.054, "32q1s1k": 0.057, "64q1s4k": 0.299}
MFMA_BF16_PEAK_TFLOPS = 2500.0


def causal_flops(B, QL, L, Hq, D=128):
    """2 matmuls x 2 flops per multiply-add over the (query, token) pairs the
    causal rule keeps: query i of a request sees L - QL + i + 1 tokens."""
    seen = sum(max(0, min(L, L - QL + i + 1)) for i in range(QL))
    return 4 * B * Hq * D * seen


def table4(args):
    """The attention shapes of the vLLM post's Table 4 at 64 query / 8 KV heads,
    bf16: prefill and extend through lbsa_prefill (TFLOP/s of the causal
    work), decode through the load-balanced path (assign + split + combine)."""
    import torch

    from load_balanced_split_assign_amd import lbsa
    from load_balanced_split_assign_amd import workload as wl
    flush = make_flush(args.flush)
    stream = torch.cuda.current_stream()
    rows = []
    for name, (kind, B, QL, L) in wl.TABLE4.items():
        if args.shapes and name not in args.shapes.split(","):
            continue
        b = wl.make_table4_batch(name, device="cuda:0")
        torch.cuda.synchronize()
        row = {"shape": name, "kind": kind, "batch": B, "q_len": QL, "kv_len": L,
               "pages_h20_ms": TABLE4_H20_MS[name]}
        if kind == "decode":
            P = args.workgroups or auto_P(b)
            path = Path(b, P)
            t = time_layer(path, args.steps, args.warmup, flush, with_assign=True)["mean"]
            ab = alg_bytes([L] * B, 64, 8, 128, "bf16")
            row.update({"us": round(t, 2), "GBps": round(ab["layer"] / t / 1e3, 1),
                        "pct_of_hbm_peak": round(100 * ab["layer"] / t / 1e3 / HBM_PEAK_GBS, 2)})
            del path
        else:
            out = torch.empty_like(b["q"])

            def run():
                lbsa.prefill(b["q"], b["k_cache"], b["v_cache"], b["page_table"], b["seqlens"],
                             b["softmax_scale"], out=out)
            for i in range(args.warmup):
                flush(i)
                run()
            torch.cuda.synchronize()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.steps)]
            for i in range(args.steps):
                flush(i)
                ev[i][0].record(stream)
                run()
                ev[i][1].record(stream)
            torch.cuda.synchronize()
            t = summarize([1000.0 * x.elapsed_time(y) for x, y in ev])["mean"]
            fl = causal_flops(B, QL, L, 64)
            row.update({"us": round(t, 2), "TFLOPs": round(fl / t / 1e6, 1),
                        "pct_of_mfma_peak": round(100 * fl / t / 1e6 / MFMA_BF16_PEAK_TFLOPS, 2)})
            del out
        row["speedup_vs_pages_h20"] = round(row["pages_h20_ms"] * 1000.0 / row["us"], 2)
        rows.append(row)
        del b
        torch.cuda.empty_cache()
    print(json.dumps({"table4": rows, "unit": "us", "flush": args.flush}), flush=True)


def _timed(run, steps, warmup, flush):
    """Mean event time (us) of run() with one event pair per call, the flush outside."""
    import torch
    stream = torch.cuda.current_stream()
    _warm(run, warmup, flush)
    ev = _pairs(steps)
    for i in range(steps):
        flush(i)
        ev[i][0].record(stream)
        run()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return summarize([1000.0 * a.elapsed_time(b) for a, b in ev])["mean"]


def _timed_alternating(runs, steps, warmup, flush):
    """Mean event time (us) of each closure in `runs` (name -> run), the
    closures taking turns within every round (flush before each call, outside
    its event pair), so that every one meets the same clock and cache history;
    `warmup` untimed rounds first."""
    import torch
    stream = torch.cuda.current_stream()
    names = list(runs)
    k = 0

    def round_once():
        for n in names:
            runs[n]()
    _warm(round_once, warmup, flush)
    ev = {n: _pairs(steps) for n in names}
    for i in range(steps):
        for n in names:
            flush(k)
            k += 1
            ev[n][i][0].record(stream)
            runs[n]()
            ev[n][i][1].record(stream)
    torch.cuda.synchronize()
    return {n: summarize([1000.0 * a.elapsed_time(b) for a, b in ev[n]])["mean"] for n in names}


def varlen_bench(args):
    """The --varlen mode: varlen_rows with the command line's steps, warm-up, flush and P."""
    rows = varlen_rows(args.steps, args.warmup, make_flush(args.flush), args.workgroups)
    print(json.dumps({"varlen": rows, "unit": "us", "flush": args.flush}), flush=True)


def varlen_rows(steps, warmup, flush, P_arg=0):
    """Prefill / extend and decode rows on one task map (query-block segments)
    against the grid path: lbsa_prefill for the requests with new tokens and the
    decode task map for the decode rows.  Workloads: the mixed batch (one 8K
    extend of an 8K context beside 63 decode rows, 64/8 heads) and a q8k prefill
    alone.  Per path: the step (with its plans) and the layer (plans reused),
    event pairs with the read flush before each; the map path's split kernel
    (which also merges the cut segments) also by its own stamps.  The paths
    take turns in every round after at least 10 warm-up rounds: the clocks
    still rise over the first tens of milliseconds of load, and timing one path
    after the other favours the second."""
    import torch

    from load_balanced_split_assign_amd import lbsa
    from load_balanced_split_assign_amd import workload as wl
    rows = []
    cases = {"mixed_extend": dict(wl.MIXED_EXTEND),
             "q8k_prefill": dict(wl.MIXED_EXTEND, extend_len=8192, extend_q=8192, decode_rows=0)}
    for name, cfg in cases.items():
        sl, ql = wl.mixed_extend_lengths(**cfg)
        b = wl.make_batch(seqlens=sl, qlens=ql, num_heads=64, num_kv_heads=8, kv_dtype="bf16", seed=cfg["seed"],
                          tail="normal", device="cuda:0")
        tq = int(sum(ql))
        B, mp = b["B"], b["max_pages"]
        P = P_arg or lbsa.varlen_auto_workgroups(ql, 8)
        tm = torch.empty(lbsa.varlen_task_map_bytes(B, 8, P, tq), dtype=torch.uint8, device="cuda:0")
        ws = torch.empty(lbsa.varlen_workspace_bytes(64, 8, P), dtype=torch.uint8, device="cuda:0")
        out = torch.empty_like(b["q"])

        def vplan():
            lbsa.plan_varlen(b["seqlens"], b["qlens"], 64, 8, mp, P, 0, total_q=tq, task_map=tm)

        def vattend():
            lbsa.attend_varlen(b["q"], b["k_cache"], b["v_cache"], b["page_table"], tm, P, b["softmax_scale"], B,
                               workspace=ws, out=out)
        vplan()
        stamps = []

        def vattend_stamped():
            e = _pairs(1)
            e[0][0].record()
            e[0][1].record()
            lbsa.time_next_kernels(e)
            vattend()
            stamps.append(e[0])
        m = lbsa.read_varlen_task_map(tm, B, 8, P, tq)

        # the grid path: lbsa_prefill for the request with new tokens, the decode map for the rest
        eq = ql[0]
        ext_q = b["q"][:eq].reshape(1, eq, 64, 128)
        ext_out = torch.empty_like(ext_q)
        ext_pt = b["page_table"][:1].contiguous()
        ext_sl = b["seqlens"][:1].contiguous()
        nd = B - 1
        if nd:
            dec = {"q": b["q"][eq:].contiguous(), "k_cache": b["k_cache"], "v_cache": b["v_cache"],
                   "k_scale": None, "v_scale": None, "q_scale": None, "page_table": b["page_table"][1:].contiguous(),
                   "seqlens": b["seqlens"][1:].contiguous(), "num_heads": 64, "num_kv_heads": 8, "B": nd,
                   "max_pages": mp, "softmax_scale": b["softmax_scale"], "q_len": 1}
            dpath = Path(dec, auto_P(dec))
            dpath.assign()

        def grid_layer():
            lbsa.prefill(ext_q, b["k_cache"], b["v_cache"], ext_pt, ext_sl, b["softmax_scale"], out=ext_out)
            if nd:
                dpath.layer()

        def grid_step():
            if nd:
                dpath.assign()
            grid_layer()
        runs = {"map_layer": vattend, "grid_layer": grid_layer, "map_step": lambda: (vplan(), vattend()),
                "grid_step": grid_step, "map_stamped": vattend_stamped}
        t = _timed_alternating(runs, steps, max(warmup, 10), flush)
        torch.cuda.synchronize()
        layer, step, g_layer, g_step = t["map_layer"], t["map_step"], t["grid_layer"], t["grid_step"]
        split_k = statistics.fmean(1000.0 * x.elapsed_time(y) for x, y in stamps[-steps:])
        flops = causal_flops(1, eq, sl[0], 64) + sum(4 * 64 * 128 * L for L in sl[1:])
        rows.append({"workload": name, "batch": B, "total_q": tq, "extend": {"L": sl[0], "q": eq},
                     "decode_rows": nd, "P": P, "T": m["T"], "K": m["K"], "Ndesc": m["Ndesc"],
                     "cut_segments": int((m["seg_num_chunks"] > 1).sum()), "flops": flops,
                     "map_layer_us": round(layer, 2), "map_step_us": round(step, 2),
                     "map_split_kernel_us": round(split_k, 2),
                     "grid_layer_us": round(g_layer, 2), "grid_step_us": round(g_step, 2),
                     "map_layer_TFLOPs": round(flops / layer / 1e6, 1),
                     "map_layer_pct_of_mfma_peak": round(100 * flops / layer / 1e6 / MFMA_BF16_PEAK_TFLOPS, 2),
                     "grid_layer_TFLOPs": round(flops / g_layer / 1e6, 1),
                     "speedup_map_vs_grid_layer": round(g_layer / layer, 3),
                     "speedup_map_vs_grid_step": round(g_step / step, 3)})
        del b, tm, ws, out
        if nd:
            del dpath, dec
        torch.cuda.empty_cache()
    return rows


ROUTER_M = (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096)


def router_bench(args):
    """Split-bf16 router GEMM on the SGLang post's K = 4096, N = 192 sweep over M
    tokens, against an fp32 GEMM of the same scores (torch / hipBLASLt, with and
    without the bf16 -> fp32 cast of X), each timed with its own event pair
    (flush before each launch); the max |error| of both against fp64 on the
    exact fp32 weights."""
    import numpy as np
    import torch

    from load_balanced_split_assign_amd import lbsa
    flush = make_flush(args.flush)
    stream = torch.cuda.current_stream()
    K, N = 4096, 192
    g = torch.Generator(device="cuda:0").manual_seed(120)
    w = torch.randn(N, K, generator=g, device="cuda:0") * 0.02
    wt = w.t().contiguous()
    hi, lo = lbsa.router_split_weights(w)

    def timed(fn):
        for i in range(args.warmup):
            flush(i)
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for i in range(args.steps):
            flush(i)
            ev[i][0].record(stream)
            fn()
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        return summarize([1000.0 * a.elapsed_time(b) for a, b in ev])["mean"]

    rows = []
    w64 = w.double()
    for M in ROUTER_M:
        x = torch.randn(M, K, generator=g, device="cuda:0").to(torch.bfloat16)
        xf = x.float()
        out = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
        need = lbsa.router_workspace_bytes(M, N, K)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda:0")
        t_ours = timed(lambda: lbsa.router_gemm(x, hi, lo, out=out, workspace=ws))
        t_f32 = timed(lambda: torch.mm(xf, wt))
        t_f32_cast = timed(lambda: torch.mm(x.float(), wt))
        exact = x.double() @ w64.t()
        lbsa.router_gemm(x, hi, lo, out=out, workspace=ws)
        err = float((out.double() - exact).abs().max())
        err_f32 = float((torch.mm(xf, wt).double() - exact).abs().max())
        flops = 2 * 2 * M * N * K
        nbytes = M * K * 2 + 2 * N * K * 2 + M * N * 4
        rows.append({"M": M, "us": round(t_ours, 2), "fp32_gemm_us": round(t_f32, 2),
                     "fp32_cast_gemm_us": round(t_f32_cast, 2), "speedup_vs_fp32": round(t_f32 / t_ours, 2),
                     "speedup_vs_fp32_cast": round(t_f32_cast / t_ours, 2),
                     "TFLOPs": round(flops / t_ours / 1e6, 2), "GBps": round(nbytes / t_ours / 1e3, 1),
                     "max_abs_err": err, "fp32_max_abs_err": err_f32})
        del x, xf, out, ws
    print(json.dumps({"router_gemm": rows, "K": K, "N": N, "unit": "us", "flush": args.flush}), flush=True)


def prologue_bytes(T, Hq, Hkv, fp8):
    """Bytes the prologue must move: the fused QKV rows in, positions and slots,
    the two norm weights, Q out (+ scale) and the K / V cache rows (+ scales)."""
    e = 1 if fp8 else 2
    s = 4 if fp8 else 0
    return (T * (Hq + 2 * Hkv) * 128 * 2 + T * 12 + 2 * 128 * 4
            + T * Hq * (128 * e + s) + 2 * T * Hkv * (128 * e + s))


def prologue_bench(args):
    """The fused prologue on the decode- and prefill-shaped inputs: mean event
    time and achieved GB/s per workload (cache flush before every launch)."""
    import torch

    from load_balanced_split_assign_amd import lbsa
    from load_balanced_split_assign_amd import workload as wl
    flush = make_flush(args.flush)
    stream = torch.cuda.current_stream()
    rows = []
    for name, kw in wl.PROLOGUE_WORKLOADS.items():
        g = {k: (v.to("cuda:0") if isinstance(v, torch.Tensor) else v)
             for k, v in wl.make_prologue_inputs(**kw).items()}
        fp8 = g["kv_dtype"] == "fp8"
        T, Hq, Hkv = g["tokens"], g["num_heads"], g["num_kv_heads"]
        q = torch.empty((T, Hq, 128), dtype=torch.float8_e4m3fn if fp8 else torch.bfloat16, device="cuda:0")
        qs = torch.empty((T, Hq), dtype=torch.float32, device="cuda:0") if fp8 else None

        def run():
            lbsa.prologue(g["qkv"], g["positions"], g["slot_mapping"], g["q_weight"], g["k_weight"], Hq, Hkv,
                          g["k_cache"], g["v_cache"], rope_theta=g["theta"], eps=g["eps"], k_scale=g["k_scale"],
                          v_scale=g["v_scale"], q_out=q, q_scale_out=qs)
        for i in range(args.warmup):
            flush(i)
            run()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for i in range(args.steps):
            flush(i)
            ev[i][0].record(stream)
            run()
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        t = summarize([1000.0 * a.elapsed_time(b) for a, b in ev])
        nbytes = prologue_bytes(T, Hq, Hkv, fp8)
        rows.append({"workload": name, "tokens": T, "num_heads": Hq, "num_kv_heads": Hkv,
                     "kv_dtype": g["kv_dtype"], "bytes": nbytes, "us_mean": round(t["mean"], 3),
                     "us_median": round(t["median"], 3), "GBps": round(nbytes / t["mean"] / 1e3, 1),
                     "pct_of_peak": round(100 * nbytes / t["mean"] / 1e3 / HBM_PEAK_GBS, 2)})
        del g, q, qs
        torch.cuda.empty_cache()
    # a plain device copy that moves as many bytes as the bf16 prefill (half
    # read, half written): the streaming rate these compare with in practice
    big = max(rows, key=lambda r: r["bytes"])
    src = torch.empty(big["bytes"] // 8, dtype=torch.int32, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for i in range(args.warmup):
        flush(i)
        dst.copy_(src)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        flush(i)
        ev[i][0].record(stream)
        dst.copy_(src)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    t = summarize([1000.0 * a.elapsed_time(b) for a, b in ev])
    nbytes = 2 * src.numel() * 4
    copy = {"bytes": nbytes, "us_mean": round(t["mean"], 3), "GBps": round(nbytes / t["mean"] / 1e3, 1),
            "pct_of_peak": round(100 * nbytes / t["mean"] / 1e3 / HBM_PEAK_GBS, 2)}
    print(json.dumps({"prologue": rows, "device_copy": copy, "unit": "us", "flush": args.flush}), flush=True)


def gpu_batch(name, tail="normal"):
    import torch

    from load_balanced_split_assign_amd import workload as wl
    b = wl.make_batch(name, tail=tail, device="cuda:0")
    torch.cuda.synchronize()
    return b


def cpu_baseline(batch, out, P, budget_s):
    """The CPU oracle (as it stands) timed on this host: assign + fp64 attention
    over a bounded sample of the workload's (request, query head) rows, on a
    host copy of the very batch the GPU ran.  The sampled rows and the task map
    are also checked against the GPU results (max abs error, bit-exact map)."""
    import numpy as np
    import torch

    from load_balanced_split_assign_amd import lbsa
    from oracle import oracle
    b = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in batch.items()}
    B, Hq, Hkv = b["B"], b["num_heads"], b["num_kv_heads"]
    sl = [int(x) for x in b["seqlens"]]
    threads = oracle.num_threads()
    # rows are taken in (request, head) order until the estimated work fits the budget,
    # using a rate measured on one row of the first request
    t0 = time.perf_counter()
    oracle.attention_rows(b, np.array([[0, 0]], np.int32))
    per_token_s = max(1e-9, (time.perf_counter() - t0) / max(1, sl[0]))
    rows, tokens = [], 0
    for r in range(B * Hq):
        req = r // Hq
        if rows and (tokens + sl[req]) * per_token_s / threads > budget_s:
            break
        rows.append((req, r % Hq))
        tokens += sl[req]
    rows = np.array(rows, np.int32)
    t0 = time.perf_counter()
    ref, _ = oracle.attention_rows(b, rows)
    t_attn = time.perf_counter() - t0
    t0 = time.perf_counter()
    om = oracle.assign(b["seqlens"], Hq, Hkv, P, 2, b["max_pages"])
    t_assign = time.perf_counter() - t0
    full = len(rows) == B * Hq
    # each row is charged its own Q and output plus 1/G of its segment's K/V bytes
    G = Hq // Hkv
    e_kv, s_kv, e_q, s_q = (2, 0, 2, 0) if b["kv_dtype"] == "bf16" else (1, 8, 1, 4)
    row_tokens = sum(sl[r] for r, _ in rows)
    sample_bytes = row_tokens * (2 * 128 * e_kv + s_kv) / G + len(rows) * (128 * e_q + s_q + 128 * 2)
    got = out.float().cpu().numpy()[rows[:, 0], rows[:, 1]].astype(np.float64)
    err = float(np.max(np.abs(got - ref))) if len(rows) else 0.0
    gm = lbsa.read_task_map(batch["_tm"], B, Hkv, P)
    same = all(np.array_equal(np.asarray(gm[k]), np.asarray(om[k]))
               for k in ("bin_desc_begin", "desc", "seg_first_desc", "seg_num_chunks"))
    same = same and all(int(gm[k]) == int(om[k]) for k in ("T", "K", "q", "r", "Ndesc"))
    return {"value": round(sample_bytes / (t_attn + t_assign) / 1e9, 4), "unit": "GB/s",
            "cores": threads, "kind": "oracle",
            "sample": (f"{'all' if full else len(rows)} of {B * Hq} (request, query head) rows"
                       f" ({row_tokens} token-rows), fp64 attention + assign"),
            "attn_s": round(t_attn, 3), "assign_us": round(1e6 * t_assign, 1),
            "check": {"rows": len(rows), "max_abs_err": err, "map_bitexact": bool(same)}}


def _pmc_rows(run_dir, counter):
    """(kernel name, value in KiB) per dispatch, in dispatch order, from the
    counter_collection CSV files of one rocprofv3 --pmc run."""
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    rows.sort()
    return [(k, v) for _, k, v in rows]


def _load_traffic():
    if not os.path.exists(TRAFFIC_FILE):
        return {}
    rec = json.load(open(TRAFFIC_FILE))
    return rec.get("workloads", {})


def write_traffic(fetch_dir, write_dir, workload, P):
    """HBM bytes per split launch on `workload` = FETCH_SIZE + WRITE_SIZE of the
    split kernel, each scaled by CALIB_BYTES / what the same counter reads for
    the calibration copy (the first device-to-device copy dispatch of a
    --calib-copy run).  The file keeps one entry per workload, each stamped with
    the kernel source it was taken on and the number of bins P of that run."""
    rec = {"source_sha256": source_sha(SPLIT_SRC), "kernel": "split_kernel", "workload": workload, "P": P,
           "calib_bytes": CALIB_BYTES}
    total = 0.0
    for key, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = _pmc_rows(d, counter)
        calib = next(v for k, v in rows if "copyBuffer" in k)
        split = [v for k, v in rows if "split_kernel" in k]
        factor = CALIB_BYTES / (calib * 1024.0)
        mean_kib = statistics.fmean(split)
        rec[key] = {"counter": counter, "calib_kib": calib, "factor": round(factor, 4),
                    "split_kib_mean": round(mean_kib, 2), "launches": len(split),
                    "bytes_per_launch": round(mean_kib * 1024.0 * factor)}
        total += mean_kib * 1024.0 * factor
    rec["bytes_per_launch"] = round(total)
    entries = _load_traffic()
    entries[workload] = rec
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump({"kernel": "split_kernel", "workloads": dict(sorted(entries.items()))}, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def traffic_from_profile(workload, P):
    """HBM bytes per split launch from committed PMC counters, if they were taken
    on the current kernel source, on this workload and with the same number of
    bins (else None)."""
    rec = _load_traffic().get(workload)
    if not rec or rec.get("source_sha256") != source_sha(SPLIT_SRC) or rec.get("P") != P:
        return None
    return rec.get("bytes_per_launch")


def measure_workload(name, steps, warmup, flush, workgroups=0):
    """Step, layer and per-kernel times of one workload; returns (record, batch, path)."""
    from load_balanced_split_assign_amd import lbsa
    from load_balanced_split_assign_amd import workload as wl
    w = wl.WORKLOADS[name]
    batch = gpu_batch(name)
    P = workgroups or w.num_workgroups or auto_P(batch)
    sl = [int(x) for x in batch["seqlens"].cpu()]
    ab = alg_bytes(sl, batch["num_heads"], batch["num_kv_heads"], 128, w.kv_dtype)
    path = Path(batch, P)
    t = time_steps(path, steps, warmup, flush)
    m = lbsa.read_task_map(path.tm, batch["B"], batch["num_kv_heads"], P)
    st = {k: summarize(v) for k, v in t.items()}
    gbs = lambda nbytes, us: nbytes / (us * 1e-6) / 1e9  # noqa: E731
    layer_us, step_us, split_us = st["layer"]["mean"], st["step"]["mean"], st["split_kernel"]["mean"]
    single = int((m["seg_num_chunks"] == 1).sum())
    rec = {"workload": name, "desc": w.note, "batch": batch["B"], "num_heads": batch["num_heads"],
           "num_kv_heads": batch["num_kv_heads"], "kv_dtype": w.kv_dtype, "seed": w.seed, "live_tokens": sum(sl),
           "P": P, "T": m["T"], "K": m["K"], "Ndesc": m["Ndesc"], "single_chunk_segments": single,
           "alg_bytes_layer": ab["layer"], "alg_bytes_split": ab["split"],
           "t_step_us": round(step_us, 3), "t_layer_us": round(layer_us, 3),
           "t_assign_kernel_us": round(st["assign_kernel"]["mean"], 3),
           "t_split_kernel_us": round(split_us, 3), "t_combine_kernel_us": round(st["combine_kernel"]["mean"], 3),
           "layer_GBps": round(gbs(ab["layer"], layer_us), 1),
           "pct_of_peak_layer": round(100.0 * gbs(ab["layer"], layer_us) / HBM_PEAK_GBS, 2),
           "step_GBps": round(gbs(ab["layer"], step_us), 1),
           "pct_of_peak_step": round(100.0 * gbs(ab["layer"], step_us) / HBM_PEAK_GBS, 2),
           "split_GBps": round(gbs(ab["split"], split_us), 1),
           "pct_of_peak_split": round(100.0 * gbs(ab["split"], split_us) / HBM_PEAK_GBS, 2),
           "partial_bytes": 2 * (m["Ndesc"] - single) * 8 * (128 + 1) * 4}
    return rec, st, batch, path, ab


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="long")
    ap.add_argument("--only", action="store_true",
                    help="time the headline workload alone (no other configs, static sweep or CPU baseline)")
    ap.add_argument("--workgroups", type=int, default=0, help="persistent workgroups (0 = CUs x occupancy)")
    ap.add_argument("--no-static", action="store_true", help="skip the static split-KV comparison")
    ap.add_argument("--no-varlen", action="store_true", help="skip the prefill-on-map block of the default line")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flush", choices=("read", "write", "none"), default="read",
                    help="cache eviction before each timed step")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one 256 MiB device copy first (reference for PMC byte counters)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work (bounded sample)")
    ap.add_argument("--table4", action="store_true",
                    help="instead of the headline line: Table 4 prefill / extend / decode shapes (64/8 heads)")
    ap.add_argument("--shapes", default="", help="with --table4: comma-separated subset of the shapes")
    ap.add_argument("--router", action="store_true",
                    help="instead of the headline line: split-bf16 router GEMM, K 4096, N 192, M sweep")
    ap.add_argument("--mtp", action="store_true",
                    help="instead of the headline line: 2-query-token decode vs 1-token decode")
    ap.add_argument("--prologue", action="store_true",
                    help="instead of the headline line: the fused QK-Norm/RoPE/KV-write prologue")
    ap.add_argument("--graph", action="store_true",
                    help="eager launches against one HIP graph of assign + split + combine (step times)")
    ap.add_argument("--varlen", action="store_true",
                    help="instead of the headline line: prefill / extend / decode rows on one task map vs the grid")
    ap.add_argument("--table3", action="store_true",
                    help="instead of the headline line: the six fp8 KV-length mixes, dynamic vs static")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU work: turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; each with "
                         "--calib-copy) into the split kernel's HBM bytes per launch")
    args = ap.parse_args()
    if args.traffic_from:
        if not args.workgroups:
            ap.error("--traffic-from needs --workgroups: the P of the profiled run")
        write_traffic(*args.traffic_from, args.workload, args.workgroups)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the path needs no collectives; "
              "KV-head or request sharding across GPUs runs independent copies of it.", file=sys.stderr)
        sys.exit(2)

    import torch

    from load_balanced_split_assign_amd import lbsa
    from load_balanced_split_assign_amd import workload as wl

    if args.calib_copy:   # a plain copy of known size: FETCH_SIZE / WRITE_SIZE reference
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.table3:
        table3(args)
        return
    if args.varlen:
        varlen_bench(args)
        return
    if args.prologue:
        prologue_bench(args)
        return
    if args.mtp:
        mtp_bench(args)
        return
    if args.table4:
        table4(args)
        return
    if args.router:
        router_bench(args)
        return
    if args.graph:
        graph_bench(args)
        return

    name = args.workload
    w = wl.WORKLOADS[name]
    flush = make_flush(args.flush)
    head, st, batch, path, ab = measure_workload(name, args.steps, args.warmup, flush, args.workgroups)
    P = head["P"]
    layer_us, step_us, split_us = st["layer"]["mean"], st["step"]["mean"], st["split_kernel"]["mean"]
    value = ab["layer"] / (layer_us * 1e-6) / 1e9
    split_gbs = ab["split"] / (split_us * 1e-6) / 1e9
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    dtype = "bf16" if w.kv_dtype == "bf16" else "fp8-e4m3 (fp8 MFMA QK^T, bf16 MFMA PV)"

    rec = {
        "metric": "decode-attn µs/step + achieved HBM GB/s (% of peak), mixed-length paged KV batch",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(step_us / 1000.0, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "config": {k: head[k] for k in ("workload", "desc", "batch", "num_heads", "num_kv_heads", "kv_dtype",
                                        "seed", "live_tokens", "P", "T", "K", "Ndesc")},
        "value_is": "layer GB/s = algorithmic bytes / t_layer (split + combine, the step's task map reused)",
        "us_per_step": round(step_us, 3), "us_per_layer": round(layer_us, 3),
        "pct_of_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "step_GBps": head["step_GBps"], "pct_of_peak_step": head["pct_of_peak_step"],
        "occupancy": {"workgroups": P, "compute_units": cus, "per_cu": round(P / cus, 3)},
        "times_us": {k: {kk: round(vv, 3) for kk, vv in v.items()} for k, v in st.items()},
        "alg_bytes": ab,
        "partial_bytes": head["partial_bytes"],
        "roofline": {"kernel": "split_kernel", "bound": "hbm", "achieved": round(split_gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(split_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profile(name, P), "alg_bytes_per_launch": ab["split"],
                     "avg_launch_us": round(split_us, 3), "workload": name,
                     "timing": "kernel start/end events (hipExtLaunchKernel), live in this run"},
    }
    if not args.no_cpu_baseline and not args.only:
        batch["_tm"] = path.tm                       # the map and output of the last timed layer
        rec["cpu_baseline"] = cpu_baseline(batch, path.out, P, args.cpu_budget)
    del batch, path
    torch.cuda.empty_cache()

    if not args.only:
        configs = []
        for other in ("tp8_share", "skewed", "fp8", "floor"):
            if other == name:
                continue
            r, _, b2, p2, _ = measure_workload(other, min(args.steps, 50), min(args.warmup, 5), flush)
            configs.append(r)
            del b2, p2
            torch.cuda.empty_cache()
        rec["configs"] = configs

    if not args.no_varlen and not args.only:
        # prefill / extend and decode rows on one task map against the grid path
        # (the --varlen mode's measurement, fewer rounds)
        rec["prefill_on_map"] = {"unit": "us", "rows": varlen_rows(min(args.steps, 20), 10, flush)}

    if not args.no_static and not args.only:
        sk = gpu_batch("skewed")
        Pk = lbsa.default_workgroups(0, "bf16")            # the heuristic S is defined on the resident count
        Pd = auto_P(sk)
        dyn = time_layer(Path(sk, Pd), 20, 3, flush)
        heur, heur_t, best_S, sweep = static_sweep(sk, Pk, 10, 2, flush)
        rec["static_baseline"] = {
            "workload": "skewed", "P": Pd, "P_resident": Pk, "dynamic_layer_us": round(dyn["mean"], 2),
            "static_heuristic_S": heur, "static_heuristic_us": round(heur_t, 2),
            "static_best_S": best_S, "static_best_us": round(sweep[best_S], 2),
            "static_sweep_us": {str(k): round(v, 2) for k, v in sweep.items()},
            "speedup_vs_static_heuristic": round(heur_t / dyn["mean"], 3),
            "speedup_vs_static_best": round(sweep[best_S] / dyn["mean"], 3)}
        del sk
        torch.cuda.empty_cache()

    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
