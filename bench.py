#!/usr/bin/env python3
"""Paged decode attention benchmark on one MI355X.

One step runs the decode path once over one batch:
  1. pa_paged_decode_f16 over the fp16 cache,
  2. pa_paged_decode_int8 over the INT8 cache.
The INT8 codes are written by pa_quantize_kv_int8 on every live physical
block (K and V) once before the timed steps; the quantize is timed on its own.
Each call is bracketed by its own HIP events on the stream it runs on.

Default workload: pool of 65,536 blocks x 16 tokens, 64 sequences with
context ~ U[512, 16384], 32 query heads / 8 KV heads, head_dim 128, groups of
4 sequences sharing their first 64 physical blocks; q/K/V ~ N(0,1), seeded.

Prints one JSON line. `value` is context (KV) tokens attended per second over
the step (both decodes: 2 x sum(ctx) per step). `roofline` is the dominant
decode's (algorithmic bytes over its mean event-timed call in the steps), and
`roofline.per_call` holds every call of the path -- the INT8 quantize, the
fp16, INT8 and FP8 (OCP E4M3) decodes, the FP8 quantize -- each as a series
of 200 event-timed launches after 20 warm-ups (p10/p50/p90/mean), with its
algorithmic bytes, GB/s, fraction of the 8 TB/s peak and the HBM bytes the
committed counter profile measured. `cpu_baseline` is the oracle on the same
step (median of 3 wall-clock runs on the host's threads) and carries the
parity of the GPU outputs against it.

After that, under `paths`: the next token's append (pa_append_kv_f16 /
pa_append_kv_int8), the eviction choice (pa_evict_select, 15 % of the
allocated blocks at 1,024, 16,384 and 65,536 blocks), the host block manager
(this batch's tables built with prefix-hash sharing) and the copy-on-write
block copy, each timed on its own. Under `configs`: the decode latencies of
the smaller configurations (tiny, the Qwen2-shaped layer at 1/4/8 sequences,
the Gaussian and the heavy-tailed INT8 batches; fp16, INT8 and FP8 caches;
per call, median/p10/p90 over 50 replays of a graph of 20 back-to-back
calls, each replay between its own event pair, and the median of 200 eager
calls, each between its own event pair; the last two configurations also
cold, each call of the graph on the next of several pool copies that
together exceed 1 GiB) with their quality against the fp32 computation on
the fp16 cache; under `hbm_probe`, the HBM rates the library's streaming
probes and torch's own copy and sum reach.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode attn tokens/sec + achieved HBM GB/s (% of peak), fp16 & INT8 KV"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E


def code_digest(path: str) -> str:
    """SHA-256 of a C/C++/HIP source with its comments and whitespace removed:
    the code the counters were taken with, unchanged by edits to comments."""
    import hashlib
    import re

    with open(path) as f:
        text = f.read()
    # string literals are kept whole (inline asm templates live in them);
    # comments and runs of whitespace become one space
    token = re.compile(r'("(?:\\.|[^"\\])*")|((?://[^\n]*|/\*.*?\*/|\s+)+)|([^"/\s]+|/)', re.S)
    code = "".join(m.group(1) or (" " if m.group(2) else m.group(3)) for m in token.finditer(text))
    return hashlib.sha256(code.strip().encode()).hexdigest()


def measured_traffic(call: str, workload: str):
    """HBM bytes per launch of `call` from the committed counter profile, or None
    when there is none for this workload or the kernel sources changed since
    (comments aside)."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get("calls", {}).get(call)
    if rec is None:
        return None
    for src, digest in rec["sources"].items():
        if code_digest(os.path.join(ROOT, src)) != digest:
            return None
    return rec["fetch_bytes"] + rec["write_bytes"]


CONFIGS = (
    ("tiny", lambda W: W.tiny()),
    ("qwen2_s1", lambda W: W.qwen2_layer(1)),
    ("qwen2_s4", lambda W: W.qwen2_layer(4)),
    ("qwen2_s8", lambda W: W.qwen2_layer(8)),
    ("int8_gaussian", lambda W: W.int8_gaussian()),
    ("int8_heavy_tailed", lambda W: W.int8_heavy_tailed()),
)
# pools of these two fit, or nearly fit, the 256 MB last-level cache: they are
# also timed cold, each launch on the next of several copies of the pools
COLD = ("int8_gaussian", "int8_heavy_tailed")
COLD_ROTATION_BYTES = 1 << 30
GRAPH_CALLS = 20  # decode calls per captured graph in the per-configuration latencies


def per_launch_us(torch, np, launch, n=200, warm=20):
    """p10/p50/p90 of n launches, each between its own pair of events on the
    current stream (the one the library launches on); launch(i) gets the
    launch index."""
    for i in range(warm):
        launch(i)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(ev):
        a.record()
        launch(i)
        b.record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    return [round(float(x), 2) for x in np.percentile(t, [10, 50, 90])]


SERIES_CALLS = 200  # event-timed launches per call of the path, after
SERIES_WARMUP = 20  # untimed warm-up launches


def launch_stats(torch, np, launch, n=SERIES_CALLS, warm=SERIES_WARMUP):
    """p10/p50/p90/mean (microseconds) of n launches after `warm` warm-up
    launches, each between its own event pair on the current stream (the one
    the library launches on)."""
    for i in range(warm):
        launch(i)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(ev):
        a.record()
        launch(i)
        b.record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    p10, p50, p90 = (round(float(x), 2) for x in np.percentile(t, [10, 50, 90]))
    return {"n": n, "p10_us": p10, "p50_us": p50, "p90_us": p90, "mean_us": round(float(t.mean()), 2)}


def config_table(pa, W, torch, np, dev, with_oracle):
    """Decode latency of every smaller configuration on the three caches, and
    (with_oracle) each output's distance to the oracle's fp32 computation on
    the fp16 cache (quality) and to the oracle's computation on the same codes
    (parity), with the oracle's own time."""
    if with_oracle:
        import oracle

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    table = {}
    for name, make in CONFIGS:
        w = make(W)
        q, tables, ctx = up(w.q), up(w.block_tables), up(w.context_lens)
        k16, v16 = up(w.k_pool), up(w.v_pool)
        ids = up(w.live_block_ids())
        k8, kf = (torch.zeros(k16.shape, dtype=t, device=dev) for t in (torch.int8, torch.uint8))
        v8, vf = torch.zeros_like(k8), torch.zeros_like(kf)
        ks, vs, kfs, vfs = (torch.zeros(k16.shape[:2], dtype=torch.float32, device=dev)
                            for _ in range(4))
        pa.pa_quantize_kv_int8(k16, v16, k8, v8, ks, vs, ids)
        pa.pa_quantize_kv_fp8(k16, v16, kf, vf, kfs, vfs, ids)
        S, sum_ctx = w.num_seqs, int(w.context_lens.sum())
        rec = {"num_seqs": S, "sum_ctx": sum_ctx, "q_heads": w.num_q_heads,
               "kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "pool_blocks": w.num_blocks}
        outs = {}
        for path, pools, fn, alg in (
            ("fp16", (k16, v16), pa.pa_paged_decode_f16, W.algorithmic_bytes(w, 2, False)),
            ("int8", (k8, v8, ks, vs), pa.pa_paged_decode_int8, W.algorithmic_bytes(w, 1, True)),
            ("fp8", (kf, vf, kfs, vfs), pa.pa_paged_decode_fp8, W.algorithmic_bytes(w, 1, True)),
        ):
            out = torch.empty(q.shape, dtype=torch.float32, device=dev)
            ws = pa.workspace_for(q, pools[0], tables, 0)
            copies = [pools]
            if name in COLD:
                per_copy = sum(x.numel() * x.element_size() for x in pools)
                copies += [tuple(x.clone() for x in pools)
                           for _ in range(COLD_ROTATION_BYTES // per_copy)]

            def launch(i, fn=fn, out=out, ws=ws, copies=copies, rotate=False):
                c = copies[i % len(copies)] if rotate else copies[0]
                fn(q, *c, tables, ctx, out, w.softmax_scale, 0, ws)

            # eager: host work of the call (binding, checks, launches) included
            # whenever the GPU waits for it
            eager = per_launch_us(torch, np, launch)
            # GRAPH_CALLS back-to-back calls captured into one graph and
            # replayed: per call, the device time of its kernels and the gaps
            # between them, without the host's launch cost. The warm graph
            # reuses the first pool copy; the cold one moves to the next copy
            # at every call.
            def graph_of(rotate):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for c in range(GRAPH_CALLS):
                        launch(c, rotate=rotate)
                return g

            def per_call(g):
                return [round(x / GRAPH_CALLS, 2)
                        for x in per_launch_us(torch, np, lambda i: g.replay(), n=50, warm=5)]

            warm_graph = graph_of(False)
            p10, p50, p90 = per_call(warm_graph)
            r = {"p10_us": p10, "p50_us": p50, "p90_us": p90, "eager_p50_us": eager[1],
                 "eager_p90_us": eager[2],
                 "decode_tokens_per_s": round(S / (p50 * 1e-6), 1),
                 "kv_tokens_per_s": round(sum_ctx / (p50 * 1e-6), 1), "alg_bytes": alg,
                 "gbs": round(alg / p50 / 1e3, 1), "frac_of_peak": round(alg / p50 / 1e3 / HBM_PEAK_GBS, 4)}
            launch(0)
            outs[path] = out.cpu().numpy()
            if len(copies) > 1:
                c10, c50, c90 = per_call(graph_of(True))
                r["cold"] = {"copies": len(copies), "p10_us": c10, "p50_us": c50, "p90_us": c90,
                             "gbs": round(alg / c50 / 1e3, 1),
                             "frac_of_peak": round(alg / c50 / 1e3 / HBM_PEAK_GBS, 4)}
            del copies, warm_graph
            rec[path] = r
        if with_oracle:
            live = w.live_block_ids()
            t0 = time.perf_counter()
            ref = oracle.decode_workload_f16(w)
            rec["oracle_fp16_ms"] = round((time.perf_counter() - t0) * 1e3, 2)
            rec["out_std"] = round(float(ref.std()), 6)
            codes = {"int8": oracle.quantize_kv_int8, "fp8": oracle.quantize_kv_fp8}
            same = {"fp16": ref}
            for path, quant in codes.items():
                kc, ksc = quant(w.k_pool, live)
                vc, vsc = quant(w.v_pool, live)
                dec = oracle.paged_decode_int8 if path == "int8" else oracle.paged_decode_fp8
                same[path] = dec(w.q, kc, vc, ksc, vsc, w.block_tables, w.context_lens,
                                 w.softmax_scale)
            for path, o in outs.items():
                err = o.astype(np.float64) - ref
                rec[path]["vs_fp32"] = {"rmse": float(np.sqrt(np.mean(err * err))),
                                        "max_abs": float(np.max(np.abs(err)))}
                rec[path]["parity_max_abs"] = float(np.max(np.abs(o - same[path])))
        table[name] = rec
        del k16, v16, k8, v8, kf, vf
        torch.cuda.empty_cache()
    return table


def hbm_probe(pa, torch, np, dev):
    """HBM rates for context: the library's streaming-read probe over 4 GiB
    (the practical read ceiling) and its read-and-write probe (4 GiB read, 2
    GiB written: the quantizer's mix), each the best of 1,024, 2,048 and
    4,096 workgroups, each the median of 10 calls; torch's sum of the same 4
    GiB (bytes read / time) and a 2 GiB device copy (bytes read + written /
    time); medians of 10."""
    res = {}
    x = torch.ones(1 << 30, dtype=torch.float32, device=dev)
    best = best_rw = 0.0
    half = torch.empty(1 << 29, dtype=torch.float32, device=dev)  # 2 GiB
    for groups in (1024, 2048, 4096):
        sink = torch.empty(groups, dtype=torch.int32, device=dev)
        us = per_launch_us(torch, np, lambda i: pa.pa_hbm_read_probe(x, sink), n=10, warm=3)[1]
        best = max(best, round((1 << 32) / us / 1e3, 1))
        us = per_launch_us(torch, np, lambda i: pa.pa_hbm_rw_probe(x, half, groups), n=10, warm=3)[1]
        best_rw = max(best_rw, round(3 * (1 << 31) / us / 1e3, 1))
    res["stream_read_gbs"] = best
    # the quantizer's mix: 4 GiB read, 2 GiB written (bytes read + written / time)
    res["stream_read2_write1_gbs"] = best_rw
    del half
    src = torch.ones(1 << 31, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for key, fn, nbytes in (("sum_read_gbs", lambda: x.sum(), 1 << 32),
                            ("copy_gbs", lambda: dst.copy_(src), 2 << 31)):
        us = per_launch_us(torch, np, lambda i: fn(), n=10, warm=3)[1]
        res[key] = round(nbytes / us / 1e3, 1)
    del x, src, dst
    torch.cuda.empty_cache()
    return res


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mixed_prefix",
                    choices=["mixed_prefix", "int8_gaussian", "int8_heavy_tailed", "qwen2_s8",
                             "tiny"])
    ap.add_argument("--partition-tokens", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle leg (CPU timing and output check)")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip timing the FP8 cache (quantize + decode) after the step")
    ap.add_argument("--no-blockmgr", action="store_true",
                    help="skip timing the block manager and the block copy after the step")
    ap.add_argument("--no-evict", action="store_true",
                    help="skip timing the eviction choice after the step")
    ap.add_argument("--no-append", action="store_true",
                    help="skip timing the next-token append calls after the step")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration decode latencies, quality table and "
                         "HBM probe after the step")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="first run one plain device-to-device copy of this many bytes "
                         "(a known-size reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): the decode path is "
              "built and measured on one GPU (one GPU's share of a sharded batch: by sequence "
              "or by KV head, with no exchange between GPUs)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import paged_kv_cache_228_amd as pa
    from paged_kv_cache_228_amd import workloads as W

    pa.lib()  # fail loudly before any work if the library is missing
    dev = torch.device("cuda:0")
    if args.copy_bytes > 0:
        src = torch.ones(args.copy_bytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    t_gen = time.time()
    w = {
        "mixed_prefix": W.mixed_prefix,
        "int8_gaussian": W.int8_gaussian,
        "int8_heavy_tailed": W.int8_heavy_tailed,
        "qwen2_s8": lambda: W.qwen2_layer(8),
        "tiny": W.tiny,
    }[args.workload]()
    print(f"[bench] generated {w.name} in {time.time() - t_gen:.1f}s", file=sys.stderr, flush=True)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    q, tables, ctx = up(w.q), up(w.block_tables), up(w.context_lens)
    k16, v16 = up(w.k_pool), up(w.v_pool)
    live = w.live_block_ids()
    ids = up(live)
    k8 = torch.zeros(k16.shape, dtype=torch.int8, device=dev)
    v8 = torch.zeros_like(k8)
    ks = torch.zeros(k16.shape[:2], dtype=torch.float32, device=dev)
    vs = torch.zeros_like(ks)
    out16 = torch.empty(q.shape, dtype=torch.float32, device=dev)
    out8 = torch.empty_like(out16)
    ws16 = pa.workspace_for(q, k16, tables, args.partition_tokens)
    ws8 = pa.workspace_for(q, k8, tables, args.partition_tokens)
    shares = {name: pa.pa_decode_shares(w.num_seqs, w.num_kv_heads, w.head_dim, w.max_blocks_per_seq,
                                        16, args.partition_tokens, kv_format=pa.KV_INT8 if i8 else pa.KV_F16)
              for name, i8 in (("fp16", False), ("int8", True))}
    torch.cuda.synchronize()

    # The bulk quantize of the live blocks runs once before the timed steps
    # (the INT8 decode reads the codes it writes); it is timed on its own below.
    pa.pa_quantize_kv_int8(k16, v16, k8, v8, ks, vs, ids)
    torch.cuda.synchronize()

    def step(ev):
        ev[0].record()
        pa.pa_paged_decode_f16(q, k16, v16, tables, ctx, out16, w.softmax_scale,
                               args.partition_tokens, ws16)
        ev[1].record()
        pa.pa_paged_decode_int8(q, k8, v8, ks, vs, tables, ctx, out8, w.softmax_scale,
                                args.partition_tokens, ws8)
        ev[2].record()

    warm = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(max(1, args.warmup))]
    for i in range(args.warmup):
        step(warm[i])
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(f"[bench] timed {args.steps} steps in {wall:.3f}s", file=sys.stderr, flush=True)
    in_step = {name: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs]))
               for i, name in enumerate(["fp16", "int8"])}

    # Every call of the path also as a series of SERIES_CALLS launches after
    # SERIES_WARMUP warm-up launches, each between its own event pair:
    # p10/p50/p90/mean per call. The quantize series runs first, so the INT8
    # decode series reads codes the quantize wrote, as in a serving step.
    kf = torch.zeros(k16.shape, dtype=torch.uint8, device=dev)
    vf = torch.zeros_like(kf)
    kfs, vfs = torch.zeros_like(ks), torch.zeros_like(ks)
    outf = torch.empty_like(out16)
    wsf = pa.workspace_for(q, kf, tables, args.partition_tokens)
    calls = {
        "quantize": lambda i: pa.pa_quantize_kv_int8(k16, v16, k8, v8, ks, vs, ids),
        "fp16": lambda i: pa.pa_paged_decode_f16(q, k16, v16, tables, ctx, out16, w.softmax_scale,
                                                 args.partition_tokens, ws16),
        "int8": lambda i: pa.pa_paged_decode_int8(q, k8, v8, ks, vs, tables, ctx, out8,
                                                  w.softmax_scale, args.partition_tokens, ws8),
        "quantize_fp8": lambda i: pa.pa_quantize_kv_fp8(k16, v16, kf, vf, kfs, vfs, ids),
        "fp8": lambda i: pa.pa_paged_decode_fp8(q, kf, vf, kfs, vfs, tables, ctx, outf,
                                                w.softmax_scale, args.partition_tokens, wsf),
    }
    if args.no_fp8:
        del calls["quantize_fp8"], calls["fp8"]
    series = {name: launch_stats(torch, np, fn, n=SERIES_CALLS, warm=SERIES_WARMUP)
              for name, fn in calls.items()}

    ms_step = wall * 1e3 / args.steps
    sum_ctx = int(w.context_lens.sum())
    S, d, hkv = w.num_seqs, w.head_dim, w.num_kv_heads
    n_live = int(live.size)
    quant_alg = n_live * hkv * 16 * d * 2 * (2 + 1) + n_live * hkv * 2 * 4 + n_live * 4
    alg = {
        "fp16": W.algorithmic_bytes(w, 2, False),
        "int8": W.algorithmic_bytes(w, 1, True),
        "fp8": W.algorithmic_bytes(w, 1, True),
        # read fp16 K+V, write 8-bit K+V and two scales per (block, head), read the id list
        "quantize": quant_alg,
        "quantize_fp8": quant_alg,
    }
    api = {"quantize": "pa_quantize_kv_int8", "fp16": "pa_paged_decode_f16",
           "int8": "pa_paged_decode_int8", "quantize_fp8": "pa_quantize_kv_fp8",
           "fp8": "pa_paged_decode_fp8"}
    per_call = {}
    for name, st in series.items():
        gbs = alg[name] / st["p50_us"] / 1e3
        rec = {"call": api[name], "alg_bytes": alg[name], **st, "gbs_p50": round(gbs, 1),
               "frac_p50": round(gbs / HBM_PEAK_GBS, 4)}
        if name in in_step:
            g = alg[name] / (in_step[name] * 1e-3) / 1e9
            rec["in_step_ms"] = round(in_step[name], 5)
            rec["gbs"] = round(g, 1)
            rec["frac"] = round(g / HBM_PEAK_GBS, 4)
            rec["decode_tokens_per_s"] = round(S / (in_step[name] * 1e-3), 1)
            rec["kv_tokens_per_s"] = round(sum_ctx / (in_step[name] * 1e-3), 1)
        traffic = measured_traffic(api[name], w.name)
        rec["traffic"] = traffic
        if traffic is not None:
            rec["traffic_over_alg"] = round(traffic / alg[name], 4)
        per_call[name] = rec
    # the dominant kernel of the step: the decode with the longer mean in-step time
    dom = max(in_step, key=lambda n: in_step[n])
    roofline = {"bound": "hbm", "achieved": per_call[dom]["gbs"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": per_call[dom]["frac"],
                "traffic": per_call[dom]["traffic"], "kernel": api[dom],
                "achieved_from": "algorithmic bytes / mean event-timed call (decode + merge "
                                 "kernels) over the timed steps",
                "traffic_unit": "HBM bytes per call (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                "calibrated on a plain copy; null once the sources changed)",
                "per_call": per_call}

    result = {
        "metric": METRIC,
        "value": round(2 * sum_ctx / (ms_step * 1e-3), 1),
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16+int8 KV, fp32 accumulate",
        "data": "synthetic",
        "config": {
            "workload": w.name, "num_seqs": S, "sum_ctx": sum_ctx,
            "ctx_min": int(w.context_lens.min()), "ctx_max": int(w.context_lens.max()),
            "num_q_heads": w.num_q_heads, "num_kv_heads": hkv, "head_dim": d,
            "block_size": 16, "pool_blocks": w.num_blocks, "live_blocks": n_live,
            "shares_per_kv_head": shares,
            "step": "fp16 decode + int8 decode (the int8 codes quantized before the steps)",
        },
        "roofline": roofline,
        "cpu_baseline": None,
    }
    paths = {}
    result["paths"] = paths

    if not args.no_cpu_baseline:
        import oracle

        # the outputs of the last series calls (every call rewrites them)
        calls["fp16"](0)
        calls["int8"](0)
        torch.cuda.synchronize()
        out16_h, out8_h = out16.cpu().numpy(), out8.cpu().numpy()
        kc_h, vc_h, ks_h, vs_h = (x.cpu().numpy() for x in (k8, v8, ks, vs))
        threads = oracle.max_threads()
        tq = time.perf_counter()
        okc, oks = oracle.quantize_kv_int8(w.k_pool, live)
        ovc, ovs = oracle.quantize_kv_int8(w.v_pool, live)
        tq = time.perf_counter() - tq
        runs = []
        for _ in range(3):  # the step on the host: both decodes over the whole batch
            t0 = time.perf_counter()
            ref16 = oracle.decode_workload_f16(w)
            t1 = time.perf_counter()
            ref8 = oracle.decode_workload_int8(w, okc, ovc, oks, ovs)
            t2 = time.perf_counter()
            runs.append((t2 - t0, t1 - t0, t2 - t1))
        cpu_s, c16, c8 = sorted(runs)[1]
        # the INT8 decode on one host thread, over the first two sequences
        one = np.arange(2, dtype=np.int32)
        oracle.set_threads(1)
        t4 = time.perf_counter()
        oracle.paged_decode_int8(w.q, okc, ovc, oks, ovs, w.block_tables, w.context_lens,
                                 w.softmax_scale, seq_ids=one)
        t5 = time.perf_counter()
        oracle.set_threads(threads)
        cpu_model = ""
        if os.path.exists("/proc/cpuinfo"):
            with open("/proc/cpuinfo") as f:
                cpu_model = next((ln.split(":", 1)[1].strip() for ln in f
                                  if ln.startswith("model name")), "")
        parity = {
            "codes_scales_bit_exact": bool(
                np.array_equal(kc_h[live], okc[live]) and np.array_equal(vc_h[live], ovc[live])
                and np.array_equal(ks_h[live].view(np.uint32), oks[live].view(np.uint32))
                and np.array_equal(vs_h[live].view(np.uint32), ovs[live].view(np.uint32))),
            "fp16_max_abs": float(np.max(np.abs(out16_h - ref16))),
            "int8_max_abs": float(np.max(np.abs(out8_h - ref8))),
            "tolerance": {"fp16": 2e-3, "int8": 1e-3},
        }
        result["cpu_baseline"] = {
            "value": round(2 * sum_ctx / cpu_s, 1), "unit": "KV tokens/s",
            "cores": threads, "kind": "oracle",
            "sample": (f"the step on the host (fp16 decode {c16:.2f}s + INT8 decode {c8:.2f}s "
                       f"of all {S} sequences, the median of 3 wall-clock runs); the oracle's "
                       f"quantize of the {n_live} live blocks took {tq:.2f}s once"),
            "cpu_model": cpu_model,
            "one_thread_int8_decode": {
                "value": round(int(w.context_lens[:2].sum()) / (t5 - t4), 1), "unit": "KV tokens/s",
                "sample": f"INT8 decode of the first 2 sequences ({int(w.context_lens[:2].sum())} "
                          f"context tokens, {t5 - t4:.2f}s)"},
            "parity": parity,
        }
    # The FP8 (OCP E4M3) cache's codes and decode (timed in the series above)
    # against the oracle.
    if not args.no_fp8 and not args.no_cpu_baseline:
        import oracle

        okf, okfs = oracle.quantize_kv_fp8(w.k_pool, live)
        ovf, ovfs = oracle.quantize_kv_fp8(w.v_pool, live)
        reff = oracle.paged_decode_fp8(w.q, okf, ovf, okfs, ovfs, w.block_tables,
                                       w.context_lens, w.softmax_scale)
        gkf, gvf = kf.cpu().numpy(), vf.cpu().numpy()
        gkfs, gvfs = kfs.cpu().numpy(), vfs.cpu().numpy()
        parity = result["cpu_baseline"]["parity"]
        parity["fp8_codes_scales_bit_exact"] = bool(
            np.array_equal(gkf[live], okf[live]) and np.array_equal(gvf[live], ovf[live])
            and np.array_equal(gkfs[live].view(np.uint32), okfs[live].view(np.uint32))
            and np.array_equal(gvfs[live].view(np.uint32), ovfs[live].view(np.uint32)))
        parity["fp8_max_abs"] = float(np.max(np.abs(outf.cpu().numpy() - reff)))

    # The append of the next token (timed on its own after the step, not part
    # of it): every sequence writes one K and one V row, fp16 and INT8.
    if not args.no_append:
        app = W.append_inputs(w, w.seed + 1, grow_frac=0.25)
        a_tab, a_pos = up(app.block_tables), up(app.positions)
        a_k, a_v = up(app.k_new), up(app.v_new)
        app_calls = {
            "append_f16": lambda: pa.pa_append_kv_f16(a_k, a_v, k16, v16, a_tab, a_pos),
            "append_int8": lambda: pa.pa_append_kv_int8(a_k, a_v, k8, v8, ks, vs, a_tab, a_pos),
        }
        n_app = int((app.positions >= 0).sum())
        row = hkv * d
        app_alg = {
            # new K/V rows read and written, one table entry and position per sequence
            "append_f16": n_app * row * 2 * 2 * 2 + S * 8,
            # + per (block, head) two scales read and written; the INT8 rows are written
            "append_int8": n_app * row * 2 * (2 + 1) + n_app * hkv * 2 * 8 + S * 8,
        }
        for name, fn in app_calls.items():
            for _ in range(5):
                fn()
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            torch.cuda.synchronize()
            e[0].record()
            for _ in range(200):
                fn()
            e[1].record()
            torch.cuda.synchronize()
            us = e[0].elapsed_time(e[1]) * 1e3 / 200
            paths[name] = {"us": round(us, 3), "alg_bytes": app_alg[name],
                           "gbs": round(app_alg[name] / us / 1e3, 1), "sequences": n_app,
                           "note": "launch-bound: a few hundred bytes per (sequence, KV head)"}
        if not args.no_cpu_baseline:
            import oracle

            ok, ov = oracle.append_kv_f16(w.k_pool, w.v_pool, app.k_new, app.v_new,
                                          app.block_tables, app.positions)
            touched = np.unique(app.block_tables[np.arange(S), np.maximum(app.positions, 0) // 16]
                                [app.positions >= 0])
            tix = up(touched.astype(np.int64))
            gk, gv = k16[tix].cpu().numpy(), v16[tix].cpu().numpy()
            o8 = oracle.append_kv_int8(okc, ovc, oks, ovs, app.k_new, app.v_new,
                                       app.block_tables, app.positions)
            g8 = [x[tix].cpu().numpy() for x in (k8, v8, ks, vs)]
            result["cpu_baseline"]["parity"]["append_bit_exact"] = bool(
                np.array_equal(gk.view(np.uint16), ok[touched].view(np.uint16))
                and np.array_equal(gv.view(np.uint16), ov[touched].view(np.uint16))
                and all(np.array_equal(g.view(np.uint8), r[touched].view(np.uint8))
                        for g, r in zip(g8, o8)))
    # The block manager (host) and the block copy of copy-on-write (timed on
    # their own): build this batch's block tables through the manager, the
    # 64 prefix blocks of each group of 4 sequences shared by prefix hash,
    # then release everything; copy 1,024 whole blocks (K and V) on the GPU.
    if not args.no_blockmgr:
        bm = pa.BlockManager(w.num_blocks)
        nblk = [(int(n) + 15) // 16 for n in w.context_lens]
        t0 = time.perf_counter()
        held = []
        for s_i, n in enumerate(nblk):
            grp = s_i // 4
            for j in range(n):
                held.append(bm.allocate((grp << 20) | j if j < 64 else None)[0])
        t1 = time.perf_counter()
        for b in held:
            bm.release(b)
        t2 = time.perf_counter()
        n_ops = 2 * len(held)
        rec = {"ops": n_ops, "blocks_used": len(set(held)),
               "blocks_match_batch": len(set(held)) == n_live,
               "alloc_release_us_per_op": round((t2 - t0) * 1e6 / n_ops, 3),
               "internal_fragmentation": round(pa.pa_internal_fragmentation(w.context_lens), 6),
               "note": "host C++ behind a Python binding; the per-op time is mostly the binding"}
        n_cp = 1024
        rng_cp = np.random.default_rng(5)
        src_cp = up(rng_cp.choice(w.num_blocks // 2, n_cp, replace=False).astype(np.int32))
        dst_cp = up((w.num_blocks // 2 + rng_cp.choice(w.num_blocks // 2, n_cp, replace=False)).astype(np.int32))
        k_cp, v_cp = torch.empty_like(k16), torch.empty_like(v16)

        def cp():
            pa.pa_copy_blocks(k16, k_cp, src_cp, dst_cp)
            pa.pa_copy_blocks(v16, v_cp, src_cp, dst_cp)

        for _ in range(3):
            cp()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        e[0].record()
        for _ in range(20):
            cp()
        e[1].record()
        torch.cuda.synchronize()
        us = e[0].elapsed_time(e[1]) * 1e3 / 20
        cp_bytes = 2 * n_cp * hkv * 16 * d * 2 * 2  # K and V blocks, read and written
        rec["copy_blocks"] = {"blocks": n_cp, "us": round(us, 2), "bytes": cp_bytes,
                              "gbs": round(cp_bytes / us / 1e3, 1)}
        del k_cp, v_cp
        paths["block_manager"] = rec

    # The eviction choice (timed on its own, not part of the step): 15 % of
    # the allocated blocks, at the README's pool sizes and on this batch's pool
    # with its reference counts; p50 of per-call event times like the README.
    if not args.no_evict:
        ev = {}
        for nb_ev in (1024, 16384, w.num_blocks):
            ref_h, last_h = W.eviction_inputs(nb_ev, 50 + nb_ev,
                                              refcount=w.refcount if nb_ev == w.num_blocks else None)
            k_ev = (int((ref_h > 0).sum()) * 15) // 100
            ref_d, last_d = up(ref_h), up(last_h)
            out_d = torch.empty(max(k_ev, 1), dtype=torch.int32, device=dev)
            for _ in range(10):
                pa.pa_evict_select(ref_d, last_d, 10_000, k_ev, out_d)
            times = []
            for _ in range(200):
                e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                e[0].record()
                pa.pa_evict_select(ref_d, last_d, 10_000, k_ev, out_d)
                e[1].record()
                e[1].synchronize()
                times.append(e[0].elapsed_time(e[1]) * 1e3)
            rec = {"blocks": nb_ev, "evict": k_ev, "p50_us": round(float(np.median(times)), 2),
                   "p90_us": round(float(np.percentile(times, 90)), 2)}
            if not args.no_cpu_baseline:
                import oracle.evict as OE

                got = out_d[:k_ev].cpu().numpy()
                rec["bit_exact"] = bool(np.array_equal(got, OE.evict_select(ref_h, last_h, 10_000, k_ev)))
            ev[str(nb_ev)] = rec
        paths["evict_select"] = ev

    if not args.no_configs:
        t_cfg = time.time()
        result["configs"] = config_table(pa, W, torch, np, dev, not args.no_cpu_baseline)
        result["hbm_probe"] = hbm_probe(pa, torch, np, dev)
        # the dominant decode against the read ceiling the device reaches
        ceiling = result["hbm_probe"]["stream_read_gbs"]
        result["roofline"]["measured_ceiling"] = {
            "gbs": ceiling, "probe": "stream_read_gbs",
            "frac": round(per_call[dom]["gbs"] / ceiling, 4)}
        print(f"[bench] configs and probe in {time.time() - t_cfg:.1f}s", file=sys.stderr, flush=True)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
