#!/usr/bin/env python3
"""Decode-step benchmark of libkpa on one MI355X.

One step = kpa_cache_append of the step's new token(s) (with the
Kronecker-separable RoPE on B^K) followed by the factor-space decode
(kpa_decode, or kpa_decode_multiq for the multi-query workload) over the whole
cached context of every sequence, on seeded synthetic inputs already resident
in HBM.  The default workload is 32 sequences x 32768 cached tokens,
h = 4x4, d_h = 8x16, R_K = R_V = 2, bfloat16 factors.

Prints ONE JSON line with the cached-tokens-attended rate, the roofline of
the split-KV decode kernel (algorithmic bytes or flops / that kernel's
average duration, bracketed with HIP events on its own stream by the
library's measurement hook), and the CPU oracle timed on a bounded sample.
After the timed steps a plain streaming read of the same cache bytes
(kpa_stream_xor, nontemporal 16-byte loads) is timed the same way; the
roofline carries its rate and the decode kernel's fraction of it, the
measured ceiling beside the published 8 TB/s.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Profile summaries (text, under profiles/) are written from rocprofv3 output
by the same file:

    python bench.py --summarize-trace STATS_DIR --bench-json FILE --cmd "..."
    python bench.py --summarize-pmc FETCH_DIR WRITE_DIR --copy-mib 256 --cmd "..." --cmd "..."

The traffic summary carries a hash of the kernel sources; the JSON line's
roofline.traffic is filled from it only while the sources still hash the same.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

HBM_PEAK_GBPS = 8000.0        # MI355X published HBM3E bandwidth
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X published dense bf16 matrix throughput
ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "factorized_kv_cache_kpa_amd", "csrc")
METRIC = "cached tokens attended/sec (decode) + achieved HBM GB/s as % of MI355X peak"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="kpa_32k")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU-oracle sample time")
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--factored-query", type=int, default=0, metavar="R_Q",
                    help="decode with a factored query of rank R_Q (kpa_decode_factored) instead of a dense one")
    ap.add_argument("--prewarm-s", type=float, default=0.3,
                    help="seconds of untimed steps before the warm-up steps, so that the clocks reach their "
                         "steady state (a compute-bound step runs ~15%% slower in the first ~50 ms)")
    ap.add_argument("--event-every", type=int, default=5,
                    help="time the decode kernel of every N-th timed step with HIP events")
    ap.add_argument("--unfused", action="store_true",
                    help="step as two calls (kpa_cache_append, then the decode) instead of kpa_append_decode")
    ap.add_argument("--call-events", action="store_true",
                    help="also bracket each whole decode call (kernel + merge) with events")
    ap.add_argument("--no-stream-read", action="store_true",
                    help="skip the streaming-read measurement of the cache bytes after the timed steps")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after timing, copy MIB MiB device-to-device 3 times (HBM counter calibration)")
    ap.add_argument("--summarize-trace", default=None, metavar="STATS_DIR")
    ap.add_argument("--bench-json", default=None, help="JSON line of the profiled run")
    ap.add_argument("--plain-json", default=None, help="JSON line of the same command run without the profiler")
    ap.add_argument("--summarize-pmc", nargs=2, default=None, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--copy-mib", type=int, default=256)
    ap.add_argument("--sweep", choices=["flashtpa", "headsplit", "project", "append"], default=None,
                    help="time the decode over FlashTPA's benchmark shapes instead of one workload")
    ap.add_argument("--sweep-out", default=None, help="write the sweep table (markdown) here")
    ap.add_argument("--summarize-util", default=None, metavar="PMC_DIR",
                    help="write profiles/decode_util_<workload>.md from one --pmc run of the activity counters")
    ap.add_argument("--cmd", action="append", default=[], help="command recorded in a summary")
    return ap.parse_args()


def main():
    args = parse()
    if args.summarize_trace:
        return summarize_trace(args)
    if args.summarize_pmc:
        return summarize_pmc(args)
    if args.summarize_util:
        return summarize_util(args)
    if args.sweep == "project":
        return sweep_project(args)
    if args.sweep == "headsplit":
        return sweep_headsplit(args)
    if args.sweep == "append":
        return sweep_append(args)
    if args.sweep:
        return sweep_flashtpa(args)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(the decode would shard by sequence, with no communication)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import factorized_kv_cache_kpa_amd as kpa
    from workloads import CONFIGS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    kpa.load()
    cfg = workload_config(args.workload)
    dev = "cuda"
    dims = kpa.make_dims(cfg.p1, cfg.p2, cfg.q1, cfg.q2, cfg.r_k, cfg.r_v, dtype=cfg.dtype,
                         rope_base=cfg.rope_base)
    n_q = cfg.n_q
    nb, ctx = cfg.batch, cfg.ctx
    n_new = n_q  # tokens appended per step: the decode queries' own tokens
    log(f"workload {cfg.name}: batch {nb} ctx {ctx} n_q {n_q} path {kpa.kpa_decode_path(dims, n_q)}")

    t0 = time.time()
    inp = make_inputs(cfg, seed=0)
    log(f"inputs generated ({time.time() - t0:.1f}s)")

    # --- setup: fill slots [0, ctx - n_new) once (untimed) ------------------------
    cache = kpa.alloc_cache(dims, nb, ctx, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    prefix = ctx - n_new
    chunk = 8192
    for s0 in range(0, prefix, chunk):
        s1 = min(prefix, s0 + chunk)
        sl = slice(s0, s1)
        kpa.kpa_cache_append(dims, cache, nb, ctx, inp.a_k[:, sl].contiguous().to(dev),
                             inp.b_k[:, sl].contiguous().to(dev), inp.a_v[:, sl].contiguous().to(dev),
                             inp.b_v[:, sl].contiguous().to(dev), inp.positions[:, sl].contiguous().to(dev),
                             torch.full((nb,), s0, dtype=torch.int32, device=dev), n_new=s1 - s0,
                             dev_status=status)
    torch.cuda.synchronize()
    log(f"cache filled: {cache.numel() / 1e6:.1f} MB")

    # --- the step's inputs, resident in HBM ---------------------------------------
    sl = slice(prefix, ctx)
    new_ak = inp.a_k[:, sl].contiguous().to(dev)
    new_bk = inp.b_k[:, sl].contiguous().to(dev)
    new_av = inp.a_v[:, sl].contiguous().to(dev)
    new_bv = inp.b_v[:, sl].contiguous().to(dev)
    new_pos = inp.positions[:, sl].contiguous().to(dev)
    slot0 = torch.full((nb,), prefix, dtype=torch.int32, device=dev)
    ctx_len = inp.ctx_len.to(dev)
    q = inp.q.to(dev).contiguous()
    q_pos = inp.q_pos.to(dev).contiguous()
    h, dh = cfg.h, cfg.d_h
    out = torch.empty((nb, n_q, h, dh), device=dev)
    lse = torch.empty((nb, n_q, h), device=dev)
    ws = kpa.alloc_workspace(dims, nb, ctx, n_q, args.num_splits, device=dev)

    if args.factored_query > 0:
        from workloads import make_query_factors
        a_q, b_q = (t.to(dev).contiguous() for t in make_query_factors(cfg, args.factored_query, seed=0))

    def decode():
        if args.factored_query > 0:
            kpa.kpa_decode_factored(dims, args.factored_query, cache, nb, ctx, ctx_len, ctx, n_q, 1, a_q, b_q,
                                    q_pos, out, lse, ws, args.num_splits)
        elif n_q == 1:
            kpa.kpa_decode(dims, cache, nb, ctx, ctx_len, ctx, q.view(nb, h, dh), q_pos.view(nb),
                           out.view(nb, h, dh), lse.view(nb, h), ws, args.num_splits)
        else:
            kpa.kpa_decode_multiq(dims, cache, nb, ctx, ctx_len, ctx, n_q, 1, q, q_pos, out, lse, ws,
                                  args.num_splits)

    fused = not args.unfused and args.factored_query == 0

    def step(ev=None):
        if fused:
            # one call: the matrix-core decode kernel writes the new tokens itself
            if ev is not None:
                ev[0].record()
            kpa.kpa_append_decode(dims, cache, nb, ctx, new_ak, new_bk, new_av, new_bv, new_pos, slot0, ctx_len,
                                  ctx, n_q, 1, q, q_pos, out, lse, ws, args.num_splits, n_new=n_new)
            if ev is not None:
                ev[1].record()
            return
        kpa.kpa_cache_append(dims, cache, nb, ctx, new_ak, new_bk, new_av, new_bv, new_pos, slot0,
                             n_new=n_new)
        if ev is not None:
            ev[0].record()
        decode()
        if ev is not None:
            ev[1].record()

    def timing_events(n):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for e0, e1 in ev:  # create the HIP events before the timed region
            e0.record()
            e1.record()
        return ev

    # Every event_every-th timed step's split-KV decode kernel is bracketed by
    # a pair of HIP events on its stream, stamped by the launch itself with
    # the kernel's own start and end (the whole-call pair only on request).
    # Not every step: even these events cost the stream time between
    # dispatches (~10 us a step on kpa_32k, measured).
    every = max(1, args.event_every)
    sampled = list(range(every - 1, args.steps, every)) or [args.steps - 1]
    kern_ev = dict(zip(sampled, timing_events(len(sampled))))
    call_ev = dict(zip(sampled, timing_events(len(sampled)))) if args.call_events else None

    # One step and its output check first: every host-side first use (torch's
    # own kernels included) happens here, not between the warm-up and the
    # timed steps.  An idle gap there (tens of ms) lets the clocks drop, and
    # the timed steps then ran in the recovery transient (measured: long_512k
    # 130 -> 160-190 us per dispatch for the next few ms).
    step()
    torch.cuda.synchronize()
    if not torch.isfinite(out).all():
        log("non-finite decode output")
        sys.exit(1)

    # untimed steps until the clocks settle, then the warm-up steps proper,
    # then the timed steps with no host work in between
    t_pre = time.perf_counter()
    n_pre = 0
    while time.perf_counter() - t_pre < args.prewarm_s:
        for _ in range(10):
            step()
        n_pre += 10
        torch.cuda.synchronize()
    if n_pre:
        log(f"pre-warm: {n_pre} steps in {time.perf_counter() - t_pre:.2f} s")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K steps.
    t_start = time.perf_counter()
    for k in range(args.steps):
        if k in kern_ev:
            kpa.kpa_time_next_decode_kernel(*kern_ev[k])
            step(call_ev[k] if call_ev else None)
        else:
            step()
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    if not torch.isfinite(out).all():
        log("non-finite decode output")
        sys.exit(1)
    log(f"warm-up {args.warmup} steps, then {args.steps} timed")
    ms_per_step = (t_end - t_start) * 1e3 / args.steps
    kern_ev = list(kern_ev.values())
    call_ev = list(call_ev.values()) if call_ev else None
    kern_ms = np.array([a.elapsed_time(b) for a, b in kern_ev])
    call_ms = np.array([a.elapsed_time(b) for a, b in call_ev]) if call_ev else None
    log(f"timed {args.steps} steps: {ms_per_step:.4f} ms/step, decode kernel {kern_ms.mean() * 1e3:.1f} us "
        f"over {len(kern_ms)} sampled steps "
        f"(median {np.median(kern_ms) * 1e3:.1f})"
        + (f", decode call {call_ms.mean() * 1e3:.1f} us" if call_ev else ""))

    # Measured ceiling: a plain streaming read (kpa_stream_xor) of the same
    # cache bytes, its launches timed like the decode kernel's (each stamps
    # its own start and end), three workgroups per CU.
    # (before the calibration copies, which a counter summary expects last)
    stream_gbps = None if args.no_stream_read else stream_read_gbps(cache, dev)

    if args.copy_calibration > 0:
        # a plain device-to-device copy of known size, after the timed region,
        # for scaling the HBM byte counters of a profiling pass
        n = args.copy_calibration << 18
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration: 3 copies of {args.copy_calibration} MiB")
        del src, dst

    tokens = int(inp.ctx_len.sum().item())  # cached tokens attended per step (per query)
    value = tokens / (ms_per_step / 1e3)
    # the fused kernel also reads the step's new factors and writes them (and
    # their positions) into the cache
    app_bytes = nb * n_new * (2 * cfg.bytes_per_token + 2 * 4) if fused else 0
    roofline = decode_roofline(cfg, tokens, q.numel() * 4 + out.numel() * 4 + lse.numel() * 4 + app_bytes,
                               float(kern_ms.mean()), float(call_ms.mean()) if call_ev else None,
                               kpa.kpa_decode_path(dims, n_q))
    # the roofline takes the average launch (what rocprofv3's average reports);
    # the median of the same samples, for comparison
    roofline["launch_us_median"] = round(float(np.median(kern_ms)) * 1e3, 2)
    if stream_gbps:
        roofline["stream_read_gbps"] = round(stream_gbps, 1)
        roofline["hbm_frac_of_stream_read"] = round(roofline["hbm_gbps"] / stream_gbps, 4)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, cfg, args.cpu_seconds, tokens)

    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "cached tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded normal factors; no dataset)",
        "config": {"workload": cfg.name, "batch": nb, "ctx": ctx, "n_q": n_q,
                   "split": [cfg.p1, cfg.p2, cfg.q1, cfg.q2], "ranks": [cfg.r_k, cfg.r_v],
                   "path": kpa.kpa_decode_path(dims, n_q), "step": ("append new token(s) + decode, one call (kpa_append_decode)" if fused
                            else "append new token(s) + decode, two calls"),
                   "query": f"factored, R_Q = {args.factored_query}" if args.factored_query > 0 else "dense",
                   "parallelism": "single GPU"},
        "achieved_hbm_gbps": roofline["hbm_gbps"], "hbm_pct_of_peak": round(100 * roofline["hbm_gbps"] / HBM_PEAK_GBPS, 2),
        "roofline": roofline, "cpu_baseline": cpu,
        "event_every": max(1, args.event_every), "prewarm_s": args.prewarm_s,
    }
    if n_q > 1:
        # (query, cached token) pairs the causal decode scores per second:
        # query n of a sequence with c cached tokens sees c - n_q + n + 1
        cl = inp.ctx_len.to(torch.int64)
        pairs = sum(int((cl - n_q + n + 1).clamp(min=0).minimum(cl).sum().item()) for n in range(n_q))
        res["query_token_pairs_per_s"] = round(pairs / (ms_per_step / 1e3), 1)
    line = json.dumps(res)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")


def stream_read_gbps(buf, dev, launches=20):
    """GB/s of kpa_stream_xor over the bytes of `buf` (mean over `launches`
    launches, each bracketed by its own start and end events)."""
    import numpy as np
    import torch

    import factorized_kv_cache_kpa_amd as kpa

    nbytes = buf.numel() * buf.element_size() // 16 * 16
    n_blocks = 3 * torch.cuda.get_device_properties(dev).multi_processor_count
    partial = torch.empty(n_blocks, dtype=torch.int32, device=dev)
    for _ in range(5):
        kpa.kpa_stream_xor(buf, partial, nbytes=nbytes)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
    for a, b in ev:
        a.record()
        b.record()
    torch.cuda.synchronize()
    for a, b in ev:
        kpa.kpa_time_next_decode_kernel(a, b)
        kpa.kpa_stream_xor(buf, partial, nbytes=nbytes)
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    log(f"streaming read of the cache ({nbytes / 1e6:.1f} MB, {n_blocks} workgroups): {ms * 1e3:.1f} us, "
        f"{nbytes / (ms * 1e-3) / 1e9:.1f} GB/s")
    return nbytes / (ms * 1e-3) / 1e9


def alg_flops_per_query_token(cfg):
    """Multiply-adds x 2 per (query, cached token) of the factor-space decode:
    both contractions of the scores and of the values, (R_K + R_V) h (q1 q2 + q1)."""
    return 2 * (cfg.r_k + cfg.r_v) * cfg.h * (cfg.q1 * cfg.q2 + cfg.q1)


def decode_roofline(cfg, tokens, io_bytes, kern_ms, call_ms, path):
    """Roofline of the split-KV decode kernel.  Algorithmic bytes per launch:
    every attended token's factors once plus the queries and outputs (no tile
    padding, no partial results); algorithmic flops: see
    alg_flops_per_query_token.  The bound is the one the algorithmic
    intensity selects against the MI355X ridge point."""
    alg_bytes = tokens * cfg.bytes_per_token + io_bytes
    alg_flops = tokens * cfg.n_q * alg_flops_per_query_token(cfg)
    hbm_gbps = alg_bytes / (kern_ms / 1e3) / 1e9
    tflops = alg_flops / (kern_ms / 1e3) / 1e12
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    mfma_bound = cfg.dtype == "bf16" and alg_flops / alg_bytes > ridge
    if mfma_bound:
        bound, achieved, peak, unit = "mfma", tflops, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
    else:
        bound, achieved, peak, unit = "hbm", hbm_gbps, HBM_PEAK_GBPS, "GB/s"
    r = {"bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 4), "traffic": None,
         "kernel": f"split-KV decode kernel ({path})", "launch_us": round(kern_ms * 1e3, 2),
         "alg_bytes_per_launch": alg_bytes, "alg_flops_per_launch": alg_flops,
         "hbm_gbps": round(hbm_gbps, 1), "tflops": round(tflops, 2)}
    if call_ms:
        r["call_us"] = round(call_ms * 1e3, 2)
        r["call_frac"] = round(achieved * kern_ms / call_ms / peak, 4)
    t = stored_traffic(cfg.name)
    if t is not None:
        r["traffic"] = t
        r["traffic_over_alg_bytes"] = round(t / alg_bytes, 4)
    return r


def workload_config(name):
    """A named workload: one of the configurations, or split_<h1>x<h2>, a head
    split the KPA page ablates (d1 = d2 = 8, R_K = R_V = 2) on 16 sequences of
    32768 cached tokens."""
    import re

    from workloads import CONFIGS, headsplit_config
    if name in CONFIGS:
        return CONFIGS[name]
    m = re.fullmatch(r"split_(\d+)x(\d+)", name)
    if m:
        return headsplit_config(int(m.group(1)), int(m.group(2)), 16, 32768).scaled(name=name)
    raise SystemExit(f"unknown workload {name!r}")


def kernel_sources_hash():
    import hashlib
    h = hashlib.sha256()
    for fn in sorted(os.listdir(CSRC)):
        if fn.endswith((".hip", ".hpp")):
            h.update(fn.encode())
            with open(os.path.join(CSRC, fn), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def traffic_summary_path(workload):
    return os.path.join(PROFILES, f"decode_traffic_{workload}.md")


def _summary_fields(path):
    fields = {}
    with open(path) as f:
        for line in f:
            line = line.strip().lstrip("-* ").strip()
            if ":" in line and line.split(":", 1)[0].replace("_", "").isalnum():
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    return fields


def stored_traffic(workload):
    """HBM bytes per decode launch from the committed counter summary, or None
    if there is none or the kernel sources changed since it was taken."""
    path = traffic_summary_path(workload)
    if not os.path.exists(path):
        return None
    f = _summary_fields(path)
    if f.get("kernel_sources_sha256") != kernel_sources_hash():
        log("traffic summary predates the current kernel sources: traffic = null")
        return None
    try:
        return int(f["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _read_csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _find(dirname, suffix):
    for root, _, files in os.walk(dirname):
        for fn in sorted(files):
            if fn.endswith(suffix):
                return os.path.join(root, fn)
    raise FileNotFoundError(f"no *{suffix} under {dirname}")


def _short_kernel(name):
    name = name.replace("kpa::(anonymous namespace)::", "").replace("kpa::mfma::", "").replace("(kpa::DecodeParams)", "")
    name = name.replace("kpa::(anonymous namespace)::", "")
    return name if len(name) < 110 else name[:107] + "..."


def summarize_trace(args):
    """profiles/decode_kernels_<workload>.md from a rocprofv3 --kernel-trace
    --stats run of this file and the JSON line that run printed."""
    with open(args.bench_json) as f:
        res = json.loads(f.read().strip().splitlines()[-1])
    wl = res["config"]["workload"]
    rows = _read_csv(_find(args.summarize_trace, "kernel_stats.csv"))
    lines = [f"# Kernel trace: {wl} decode step", "",
             "Command (from the repository root on the MI355X; the output directory is scratch):", ""]
    lines += [f"    {c}" for c in args.cmd] + [""]
    lines += ["rocprofv3 kernel statistics (all launches of the run, warm-up included):", "",
              "| kernel | calls | avg us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"| `{_short_kernel(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")
    rf = res["roofline"]
    dec = [r for r in rows if "decode_" in r["Name"] and "_kernel" in r["Name"]]
    lines += ["", "Same run, bench.py's own figures (HIP events on the launch stream, every "
                  f"{res.get('event_every', 1)}-th timed step):", "",
              f"- decode kernel average: {rf['launch_us']} us"]
    if "call_us" in rf:
        lines.append(f"- decode call (kernel + merge) average: {rf['call_us']} us")
    lines += [f"- ms per step: {res['ms_per_step']}",
              f"- roofline: {rf['achieved']} {rf['unit']} of {rf['peak']} ({100 * rf['frac']:.1f}%), bound {rf['bound']}"]
    avg = float(dec[0]["AverageNs"]) / 1e3 if dec else None
    # the last K decode dispatches are the timed steps; every event_every-th carried events
    k = int(res["steps"])
    every = int(res.get("event_every", 1))
    trace = [r for r in _read_csv(_find(args.summarize_trace, "kernel_trace.csv"))
             if "decode_" in r["Kernel_Name"] and "_kernel" in r["Kernel_Name"]]
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in trace]
    if len(durs) >= k:
        timed = durs[-k:]
        sampled = [timed[i] for i in range(every - 1, k, every)] or [timed[-1]]
        s_avg = sum(sampled) / len(sampled)
        lines.append(f"- rocprofv3, the {len(sampled)} dispatches the events timed: average {s_avg:.1f} us "
                     f"({100 * (rf['launch_us'] - s_avg) / s_avg:+.1f}% for the events)")
        lines.append(f"- rocprofv3, all {k} timed steps: decode kernel average {sum(timed) / k:.1f} us")
    if avg:
        lines.append(f"- rocprofv3 decode kernel average over every dispatch of the run: {avg:.1f} us")
    if "stream_read_gbps" in rf:
        lines.append(f"- streaming read of the same cache bytes (kpa_stream_xor, events): {rf['stream_read_gbps']} GB/s; "
                     f"the decode kernel moves {rf['hbm_frac_of_stream_read']:.3f} of that rate")
    srows = [r for r in rows if "stream_xor_kernel" in r["Name"]]
    if srows:
        lines.append(f"- rocprofv3 streaming-read kernel average: {float(srows[0]['AverageNs']) / 1e3:.1f} us "
                     f"over {srows[0]['Calls']} dispatches")
    if args.plain_json:
        with open(args.plain_json) as f:
            plain = json.loads(f.read().strip().splitlines()[-1])
        pr = plain["roofline"]
        lines += ["", "The same bench.py command without the profiler (same box, right before; the profiler "
                      "lengthens each dispatch as the events see it):", "",
                  f"- decode kernel average: {pr['launch_us']} us"
                  + (f" ({100 * (pr['launch_us'] - avg) / avg:+.1f}% against rocprofv3's average)" if avg else ""),
                  f"- ms per step: {plain['ms_per_step']}",
                  f"- roofline: {pr['achieved']} {pr['unit']} of {pr['peak']} ({100 * pr['frac']:.1f}%), bound {pr['bound']}"]
        if "stream_read_gbps" in pr:
            lines.append(f"- streaming read of the same cache bytes: {pr['stream_read_gbps']} GB/s; the decode kernel "
                         f"moves {pr['hbm_frac_of_stream_read']:.3f} of that rate")
    out = os.path.join(PROFILES, f"decode_kernels_{wl}.md")
    os.makedirs(PROFILES, exist_ok=True)
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)


def summarize_pmc(args):
    """profiles/decode_traffic_<workload>.md from two rocprofv3 --pmc runs of
    this file with --copy-calibration (FETCH_SIZE, then WRITE_SIZE).  The
    counters of the calibration copies (the last three dispatches of each run,
    MIB MiB read and written each) give the scale from counter KiB to bytes."""
    out = {}
    for counter, d in zip(("FETCH_SIZE", "WRITE_SIZE"), args.summarize_pmc):
        rows = [r for r in _read_csv(_find(d, "counter_collection.csv")) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        copies = rows[-3:]
        if len({r["Kernel_Name"] for r in copies}) != 1:
            raise SystemExit(f"{counter}: the last three dispatches are not one copy kernel")
        copy_kib = sum(float(r["Counter_Value"]) for r in copies) / 3
        dec = [r for r in rows if "decode_" in r["Kernel_Name"] and "_kernel" in r["Kernel_Name"]]
        if not dec:
            raise SystemExit(f"{counter}: no decode kernel dispatches")
        names = {r["Kernel_Name"] for r in dec}
        dec_kib = sum(float(r["Counter_Value"]) for r in dec) / len(dec)
        scale = args.copy_mib * 1024 / copy_kib
        out[counter] = dict(copy_kernel=copies[0]["Kernel_Name"], copy_kib=copy_kib, scale=scale,
                            dec_kib=dec_kib, n=len(dec), kernel=sorted(names))
    fetch = out["FETCH_SIZE"]["dec_kib"] * 1024 * out["FETCH_SIZE"]["scale"]
    write = out["WRITE_SIZE"]["dec_kib"] * 1024 * out["WRITE_SIZE"]["scale"]
    wl = None
    for c in args.cmd:
        if "--workload" in c:
            wl = c.split("--workload", 1)[1].split()[0]
    wl = wl or "kpa_32k"
    cfg = workload_config(wl)
    n_q = cfg.n_q
    alg = cfg.batch * cfg.ctx * cfg.bytes_per_token + cfg.batch * n_q * cfg.h * (2 * cfg.d_h + 1) * 4
    lines = [f"# HBM traffic of the split-KV decode kernel: {wl}", "",
             "Two counter passes of the same bench command (one counter each), from the repository root:", ""]
    lines += [f"    {c}" for c in args.cmd] + [""]
    lines += [f"Decode kernel: `{_short_kernel(k)}`" for k in out["FETCH_SIZE"]["kernel"]] + [""]
    lines += ["| counter | copy kernel KiB/dispatch | copy bytes | scale | decode KiB/dispatch (raw) | dispatches | decode bytes (scaled) |",
              "|---|---|---|---|---|---|---|"]
    for counter, v in out.items():
        lines.append(f"| {counter} | {v['copy_kib']:.1f} | {args.copy_mib} MiB | {v['scale']:.4f} | "
                     f"{v['dec_kib']:.1f} | {v['n']} | {v['dec_kib'] * 1024 * v['scale']:.0f} |")
    lines += ["", f"Calibration kernel: `{_short_kernel(out['FETCH_SIZE']['copy_kernel'])}`, "
                  f"{args.copy_mib} MiB read and {args.copy_mib} MiB written per dispatch.", "",
              f"- fetch_bytes_per_launch: {fetch:.0f}",
              f"- write_bytes_per_launch: {write:.0f}",
              f"- traffic_bytes_per_launch: {fetch + write:.0f}",
              f"- alg_bytes_per_launch: {alg}",
              f"- traffic_over_alg: {(fetch + write) / alg:.4f}",
              f"- kernel_sources_sha256: {kernel_sources_hash()}", ""]
    path = traffic_summary_path(wl)
    os.makedirs(PROFILES, exist_ok=True)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(path)


def sweep_project(args):
    """kpa_project_append (factor projection of hidden states into the cache,
    one GEMM on the matrix cores) for every bf16 configuration, d_model =
    h * d_h, at the decode step's token count and at 4096 and 32768 tokens.
    Weights and hidden states are seeded bf16 normals drawn on the GPU (parity
    is tested at these shapes in tests/test_gpu_project.py).  Kernel time from
    HIP events stamped by the launch (median of 10); the HBM roofline counts
    x, W, the factors written and the positions once; the matrix-core
    roofline counts 2 * tokens * d_model * F flop.  The CPU column is the
    float64 oracle projection (NumPy, x @ W^T plus the B^K rotation) timed on
    a sample of at most 256 tokens."""
    import numpy as np
    import torch

    import factorized_kv_cache_kpa_amd as kpa
    from workloads import CONFIGS

    kpa.load()
    dev = "cuda"
    g = torch.Generator(device=dev).manual_seed(0)
    rows = []
    for name in ("tpa_degenerate", "kpa_32k", "long_512k", "multiq_16"):
        cfg = CONFIGS[name]
        dims = kpa.make_dims(cfg.p1, cfg.p2, cfg.q1, cfg.q2, cfg.r_k, cfg.r_v, dtype=cfg.dtype,
                             rope_base=cfg.rope_base)
        d_model = cfg.h * cfg.d_h
        n_feat = (cfg.r_k + cfg.r_v) * (cfg.p1 * cfg.q1 + cfg.p2 * cfg.q2)
        w = (torch.randn((n_feat, d_model), generator=g, device=dev) / d_model ** 0.5).to(torch.bfloat16)
        for nb, n_new in ((cfg.batch, cfg.n_q), (1, 4096), (1, 32768)):
            m = nb * n_new
            cap = n_new
            x = torch.randn((nb, n_new, d_model), generator=g, device=dev).to(torch.bfloat16)
            pos = torch.arange(n_new, dtype=torch.int32, device=dev).repeat(nb, 1).contiguous()
            slot0 = torch.zeros(nb, dtype=torch.int32, device=dev)
            cache = kpa.alloc_cache(dims, nb, cap, device=dev)

            def call():
                kpa.kpa_project_append(dims, cache, nb, cap, x, w, pos, slot0, n_new=n_new)

            for _ in range(3):
                call()
            reps = 10
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
            for a, b in ev:
                a.record()
                b.record()
            torch.cuda.synchronize()
            for a, b in ev:
                kpa.kpa_time_next_decode_kernel(a, b)
                call()
            torch.cuda.synchronize()
            kern = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3
            nbytes = m * d_model * 2 + n_feat * d_model * 2 + m * n_feat * 2 + m * 4
            gbs = nbytes / (kern * 1e-6) / 1e9
            tfl = 2.0 * m * d_model * n_feat / (kern * 1e-6) / 1e12
            cpu_tps = cpu_baseline_project(cfg, x.reshape(m, d_model), w, pos.reshape(-1))
            rows.append((name, d_model, n_feat, m, kern, gbs, tfl, m / (kern * 1e-6), cpu_tps))
            log(f"{name} d_model={d_model} F={n_feat} tokens={m}: {kern:.1f} us, {gbs:.0f} GB/s, {tfl:.1f} TFLOP/s")
            del cache, x
            torch.cuda.empty_cache()
    lines = ["| config | d_model | F | tokens | kernel us | GB/s | of 8 TB/s | TFLOP/s | of 2.5 PFLOP/s | "
             "tokens/s | CPU oracle tokens/s |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for name, d_model, n_feat, m, kern, gbs, tfl, tps, cpu in rows:
        lines.append(f"| {name} | {d_model} | {n_feat} | {m} | {kern:.1f} | {gbs:.0f} | {100 * gbs / HBM_PEAK_GBPS:.1f}% "
                     f"| {tfl:.1f} | {100 * tfl / 2500.0:.2f}% | {tps:.3e} | {cpu:.3e} |")
    table = "\n".join(lines)
    print(table)
    if args.sweep_out:
        with open(args.sweep_out, "w") as f:
            f.write(table + "\n")


def sweep_append(args):
    """kpa_cache_append for every configuration: the decode step's new tokens
    (n_q per sequence) and a bulk fill of min(8192, ctx) tokens per sequence,
    for the configuration's batch.  Factors are the seeded inputs of the
    configuration (torch CPU generator), already on the GPU.  Time: stream
    events around each call, which is one kernel (median of 10 after 30 ms of
    untimed calls).  HBM bytes: the factors read and written once and the
    positions read and written.  The CPU column is the float64 oracle's
    append (the B^K rotation, NumPy) on a sample of at most 256 tokens."""
    import numpy as np
    import torch

    import factorized_kv_cache_kpa_amd as kpa
    from oracle import kpa_ref
    from workloads import CONFIGS, make_inputs

    kpa.load()
    dev = "cuda"
    rows = []
    for name in ("tiny_f32", "tpa_degenerate", "kpa_32k", "long_512k", "multiq_16"):
        cfg = CONFIGS[name]
        dims = kpa.make_dims(cfg.p1, cfg.p2, cfg.q1, cfg.q2, cfg.r_k, cfg.r_v, dtype=cfg.dtype,
                             rope_base=cfg.rope_base)
        nb = cfg.batch
        for n_new in (cfg.n_q, min(8192, cfg.ctx)):
            inp = make_inputs(cfg, seed=0, batch=nb, ctx=n_new)
            t = [x.contiguous().to(dev) for x in (inp.a_k, inp.b_k, inp.a_v, inp.b_v, inp.positions)]
            slot0 = torch.zeros(nb, dtype=torch.int32, device=dev)
            cache = kpa.alloc_cache(dims, nb, n_new, device=dev)

            def call():
                kpa.kpa_cache_append(dims, cache, nb, n_new, *t, slot0, n_new=n_new)

            t_w, n_w = time.perf_counter(), 0
            while n_w < 3 or time.perf_counter() - t_w < 0.03:
                call()
                n_w += 1
                if n_w % 20 == 0:
                    torch.cuda.synchronize()
            reps = 10
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
            torch.cuda.synchronize()
            for a, b in ev:
                a.record()
                call()
                b.record()
            torch.cuda.synchronize()
            us = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3
            m = nb * n_new
            nbytes = m * (2 * cfg.bytes_per_token + 8)
            gbs = nbytes / (us * 1e-6) / 1e9
            # CPU: the oracle's rotation of B^K (the copies are free) on a sample
            ms = min(m, 256)
            bk = inp.b_k.reshape(m, *inp.b_k.shape[2:])[:ms].to(torch.float64).numpy()
            ps = inp.positions.reshape(-1)[:ms].numpy()
            t0 = time.perf_counter()
            for i in range(ms):
                kpa_ref.append_rotate(bk[i], int(ps[i]), cfg.rope_base)
            cpu_tps = ms / (time.perf_counter() - t0)
            rows.append((name, nb, n_new, us, gbs, m / (us * 1e-6), cpu_tps))
            log(f"{name} {nb} x {n_new} tokens: {us:.1f} us, {gbs:.0f} GB/s")
            del cache, t
            torch.cuda.empty_cache()
    lines = ["| config | sequences | new tokens each | call us | GB/s | of 8 TB/s | tokens/s | CPU oracle tokens/s |",
             "|---|---|---|---|---|---|---|---|"]
    for name, nb, n_new, us, gbs, tps, cpu in rows:
        lines.append(f"| {name} | {nb} | {n_new} | {us:.1f} | {gbs:.0f} | {100 * gbs / HBM_PEAK_GBPS:.1f}% | "
                     f"{tps:.3e} | {cpu:.3e} |")
    table = "\n".join(lines)
    print(table)
    if args.sweep_out:
        with open(args.sweep_out, "w") as f:
            f.write(table + "\n")


def cpu_baseline_project(cfg, x, w, positions, max_tokens=256):
    """CPU baseline of the projection: the float64 oracle (NumPy x @ W^T, then
    the B^K rotation) on the first max_tokens tokens; tokens per second."""
    import numpy as np
    import torch

    from oracle import kpa_ref

    ms = min(x.shape[0], max_tokens)
    xs = x[:ms].to(torch.float64).cpu().numpy()
    wsd = w.to(torch.float64).cpu().numpy()
    ps = positions[:ms].cpu().numpy()
    t0 = time.perf_counter()
    kpa_ref.projected_cache_values(xs, wsd, ps, cfg.r_k, cfg.r_v, cfg.p1, cfg.q1, cfg.p2, cfg.q2, cfg.rope_base)
    return ms / (time.perf_counter() - t0)


def _time_decode_shape(kpa, cfg, g, dev, r_q=0):
    """Fill a cache of cfg's shape (factors drawn on the GPU with cfg's
    deviations, written by kpa_cache_append in chunks), then time the decode
    of one query per sequence at the last position: medians of 30 calls after
    at least 50 ms of untimed ones.  The query is dense (kpa_decode); with
    r_q > 0 the same cache is also decoded with a factored query of rank r_q
    (kpa_decode_factored; factors scaled so the expanded query has
    unit-variance elements).  Returns (kernel us, call us, kernel GB/s), or a
    pair of them (dense, factored) when r_q > 0."""
    import numpy as np
    import torch

    nb, ctx = cfg.batch, cfg.ctx
    dims = kpa.make_dims(cfg.p1, cfg.p2, cfg.q1, cfg.q2, cfg.r_k, cfg.r_v, dtype=cfg.dtype)
    cache = kpa.alloc_cache(dims, nb, ctx, device=dev)
    chunk = 8192
    for s0 in range(0, ctx, chunk):
        n = min(chunk, ctx - s0)

        def draw(r, p, q, sd):
            return (torch.randn((nb, n, r, p, q), generator=g, device=dev) * sd).to(torch.bfloat16)

        pos = torch.arange(s0, s0 + n, dtype=torch.int32, device=dev).repeat(nb, 1).contiguous()
        kpa.kpa_cache_append(dims, cache, nb, ctx, draw(cfg.r_k, cfg.p1, cfg.q1, cfg.sigma_a),
                             draw(cfg.r_k, cfg.p2, cfg.q2, cfg.sigma_b), draw(cfg.r_v, cfg.p1, cfg.q1, cfg.sigma_a),
                             draw(cfg.r_v, cfg.p2, cfg.q2, cfg.sigma_b), pos,
                             torch.full((nb,), s0, dtype=torch.int32, device=dev), n_new=n)
    h, dh = cfg.h, cfg.d_h
    q = torch.randn((nb, h, dh), generator=g, device=dev)
    q_pos = torch.full((nb,), ctx - 1, dtype=torch.int32, device=dev)
    ctx_len = torch.full((nb,), ctx, dtype=torch.int32, device=dev)
    out = torch.empty((nb, h, dh), device=dev)
    lse = torch.empty((nb, h), device=dev)
    ws = kpa.alloc_workspace(dims, nb, ctx, device=dev)

    def dense():
        kpa.kpa_decode(dims, cache, nb, ctx, ctx_len, ctx, q, q_pos, out, lse, ws)

    def timed(decode):
        # at least 50 ms of calls before timing (clocks settle; no idle gap after)
        t_w, n_w = time.perf_counter(), 0
        while n_w < 3 or time.perf_counter() - t_w < 0.05:
            decode()
            n_w += 1
            if n_w % 20 == 0:
                torch.cuda.synchronize()
        reps = 30
        kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in kev + cev:
            a.record()
            b.record()
        torch.cuda.synchronize()
        for k in range(reps):
            kpa.kpa_time_next_decode_kernel(*kev[k])
            cev[k][0].record()
            decode()
            cev[k][1].record()
        torch.cuda.synchronize()
        kern = float(np.median([a.elapsed_time(b) for a, b in kev])) * 1e3
        call = float(np.median([a.elapsed_time(b) for a, b in cev])) * 1e3
        return kern, call, (nb * ctx * cfg.bytes_per_token) / (kern * 1e-6) / 1e9

    res = timed(dense)
    if r_q > 0:
        s_f = (r_q ** 0.5) ** 0.5
        a_q = (torch.randn((nb, 1, r_q, cfg.p1, cfg.q1), generator=g, device=dev) * s_f).contiguous()
        b_q = (torch.randn((nb, 1, r_q, cfg.p2, cfg.q2), generator=g, device=dev) * s_f).contiguous()
        qp1, out1, lse1 = q_pos.view(nb, 1), out.view(nb, 1, h, dh), lse.view(nb, 1, h)

        def factored():
            kpa.kpa_decode_factored(dims, r_q, cache, nb, ctx, ctx_len, ctx, 1, 1, a_q, b_q, qp1, out1, lse1, ws)

        res = (res, timed(factored))
    del cache, ws
    torch.cuda.empty_cache()
    return res


def _write_table(args, lines):
    table = "\n".join(lines)
    print(table)
    if args.sweep_out:
        with open(args.sweep_out, "w") as f:
            f.write(table + "\n")


def sweep_flashtpa(args):
    """Decode over FlashTPA's benchmark grid as the TPA summary page states it
    (TPA split, d_h = 64, R_K = R_V = 1, a factored query of rank R_Q = 16;
    h = 16 / 32 / 48, i.e. d_model 1024 / 2048 / 3072; batch 1, 2, 4, 8, 16;
    2^12 .. 2^19 cached tokens per sequence), with the dense query beside it.
    Factors and queries are drawn on the GPU from a seeded generator (no
    oracle here: the same shapes are parity-tested at small sizes); the cache
    is filled by kpa_cache_append before timing.  One line per shape: kernel
    times of both query forms, the factored call's time (decode + merge),
    cached tokens/s and the factored kernel's HBM roofline fraction."""
    import torch

    import factorized_kv_cache_kpa_amd as kpa
    from workloads import FLASHTPA_BATCHES, FLASHTPA_HEADS, FLASHTPA_RQ, FLASHTPA_SEQS, flashtpa_config

    kpa.load()
    dev = "cuda"
    g = torch.Generator(device=dev).manual_seed(0)
    rows = []
    for h in FLASHTPA_HEADS:
        for nb in FLASHTPA_BATCHES:
            for ctx in FLASHTPA_SEQS:
                (kd, _, _), (kf, cf, gbs) = _time_decode_shape(kpa, flashtpa_config(h, nb, ctx), g, dev,
                                                              r_q=FLASHTPA_RQ)
                rows.append((h, nb, ctx, kd, kf, cf, nb * ctx / (cf * 1e-6), gbs))
                log(f"h={h} batch={nb} seq={ctx}: dense {kd:.1f} us, factored {kf:.1f} us (call {cf:.1f}), "
                    f"{gbs:.0f} GB/s")
    lines = [f"| h | batch | seq | dense-query kernel us | factored-query (R_Q = {FLASHTPA_RQ}) kernel us | "
             "factored call (kernel + merge) us | cached tokens/s (factored call) | factored kernel GB/s | "
             "of 8 TB/s |", "|---|---|---|---|---|---|---|---|---|"]
    for h, nb, ctx, kd, kf, cf, tps, gbs in rows:
        lines.append(f"| {h} | {nb} | {ctx} | {kd:.1f} | {kf:.1f} | {cf:.1f} | {tps:.3e} | {gbs:.0f} | "
                     f"{100 * gbs / HBM_PEAK_GBPS:.1f}% |")
    _write_table(args, lines)


def sweep_headsplit(args):
    """Decode over the head splits the KPA page ablates (h = p1 x p2, d1 = d2
    = 8, R_K = R_V = 2): 16 sequences of 32768 cached tokens each, one query
    per sequence, factors drawn on the GPU (each split is parity-tested at
    small sizes).  One line per split: the kernel path, kernel and whole-call
    time, cached tokens/s and the kernel's HBM roofline fraction."""
    import torch

    import factorized_kv_cache_kpa_amd as kpa
    from workloads import SWEEP_SHAPES, headsplit_config

    kpa.load()
    dev = "cuda"
    g = torch.Generator(device=dev).manual_seed(0)
    nb, ctx = 16, 32768
    lines = ["| split (h1 x h2) | h | bytes/token | path | decode kernel us | call (kernel + merge) us | cached tokens/s "
             "| kernel GB/s | of 8 TB/s |", "|---|---|---|---|---|---|---|---|---|"]
    for p1, p2 in SWEEP_SHAPES:
        cfg = headsplit_config(p1, p2, nb, ctx)
        dims = kpa.make_dims(cfg.p1, cfg.p2, cfg.q1, cfg.q2, cfg.r_k, cfg.r_v, dtype=cfg.dtype)
        path = kpa.kpa_decode_path(dims, 1)
        kern, call, gbs = _time_decode_shape(kpa, cfg, g, dev)
        log(f"split {p1}x{p2}: {path}, kernel {kern:.1f} us, call {call:.1f} us, {gbs:.0f} GB/s")
        lines.append(f"| {p1} x {p2} | {cfg.h} | {cfg.bytes_per_token} | {path} | {kern:.1f} | {call:.1f} | "
                     f"{nb * ctx / (call * 1e-6):.3e} | {gbs:.0f} | {100 * gbs / HBM_PEAK_GBPS:.1f}% |")
    _write_table(args, lines)


def summarize_util(args):
    """profiles/decode_util_<workload>.md: matrix-core and vector-ALU activity
    of the decode kernel from one rocprofv3 --pmc run.  GRBM_GUI_ACTIVE sums
    the busy cycles of the 8 XCDs; SQ_VALU_MFMA_BUSY_CYCLES sums the matrix
    pipe's busy cycles over all 1024 SIMDs (it equals the kernel's MFMA count
    times their issue cycles, 32 per 32x32x16 and 16 per 16x16x32 bf16);
    SQ_ACTIVE_INST_VALU counts vector instructions issued, each holding its
    SIMD for 4 cycles (64 lanes on 16)."""
    rows = _read_csv(_find(args.summarize_util, "counter_collection.csv"))
    dec = [r for r in rows if "decode_" in r["Kernel_Name"] and "_kernel" in r["Kernel_Name"]]
    # the run's first decode dispatch also carries the kernel's first use
    # (code object loading: ~10x the cycles of the others): left out
    ids = sorted({int(r["Dispatch_Id"]) for r in dec})
    dec = [r for r in dec if int(r["Dispatch_Id"]) != ids[0]] if len(ids) > 1 else dec
    if not dec:
        raise SystemExit("no decode kernel dispatches")
    n_disp = len({int(r["Dispatch_Id"]) for r in dec})
    vals = {}
    for r in dec:
        vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    avg = {k: sum(v) / len(v) for k, v in vals.items()}
    wl = None
    for c in args.cmd:
        if "--workload" in c:
            wl = c.split("--workload", 1)[1].split()[0]
    wl = wl or "kpa_32k"
    simds, xcds = 1024, 8
    cycles = avg["GRBM_GUI_ACTIVE"] / xcds
    mfma = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / simds / cycles
    valu = (avg["SQ_ACTIVE_INST_VALU"] * 4) / simds / cycles
    lines = [f"# Matrix-core and vector-ALU activity of the split-KV decode kernel: {wl}", "",
             "One counter pass of the bench command, from the repository root:", ""]
    lines += [f"    {c}" for c in args.cmd] + [""]
    lines += [f"Decode kernel: `{_short_kernel(dec[0]['Kernel_Name'])}`, {n_disp} dispatches (averages below; the "
              "run's first decode dispatch, which also loads the kernel, is left out)", "",
              "| counter | per dispatch |", "|---|---|"]
    for k in sorted(avg):
        lines.append(f"| {k} | {avg[k]:.0f} |")
    lines += ["", "Derived (GRBM_GUI_ACTIVE sums 8 XCDs; the SQ busy/issue counters sum 1024 SIMDs;"
                  " a vector instruction holds its SIMD 4 cycles):", "",
              f"- kernel cycles per XCD: {cycles:.0f}",
              f"- matrix-core pipe busy: {100 * mfma:.1f}% of SIMD cycles",
              f"- vector ALU issue busy: {100 * valu:.1f}% of SIMD cycles",
              f"- vector instructions per matrix instruction: "
              f"{(avg['SQ_INSTS_VALU'] - avg['SQ_INSTS_MFMA']) / max(avg['SQ_INSTS_MFMA'], 1):.1f}",
              f"- kernel_sources_sha256: {kernel_sources_hash()}", ""]
    path = os.path.join(PROFILES, f"decode_util_{wl}.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(path)


def cpu_model():
    """The host CPU's model name (the first "model name" line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(inp, cfg, target_s, tokens_total):
    """Time the float64 C oracle on a bounded sample of the same decode.

    The sample is a set of (sequence, query, head) rows; rows / h full decodes
    of one sequence's heads, each over that sequence's context.  Rate in the
    same unit: cached tokens attended per second (a token counts once per
    full set of h heads)."""
    import numpy as np

    from oracle import kpa_oracle

    kpa_oracle.build(force=False)
    threads = kpa_oracle.max_threads()
    h = cfg.h
    n_q = inp.q.shape[1]
    rows_total = inp.batch * n_q * h
    rng = np.random.default_rng(0)
    order = rng.permutation(rows_total)

    def run(k):
        idx = order[:k]
        items = np.stack([idx // (n_q * h), (idx // h) % n_q, idx % h], axis=1).astype(np.int32)
        t0 = time.perf_counter()
        kpa_oracle.decode(inp.a_k, inp.b_k, inp.a_v, inp.b_v, inp.positions, inp.ctx_len, inp.q, inp.q_pos,
                          items=items, n_threads=threads)
        return time.perf_counter() - t0, items

    k = min(rows_total, max(threads, 1))
    dt, _ = run(k)
    if dt < target_s and k < rows_total:
        k = int(min(rows_total, max(k, k * target_s / max(dt, 1e-3))))
        k = max(threads, (k // threads) * threads) if k < rows_total else rows_total
        dt, items = run(k)
    else:
        items = None
    ctx = inp.ctx_len.numpy()
    n_q_eff = n_q
    # tokens attended by the sampled rows, in whole-decode units
    idx = order[:k]
    b_idx = idx // (n_q * h)
    tok = float(ctx[b_idx].sum()) / h
    log(f"cpu oracle: {k} rows in {dt:.2f}s on {threads} threads")
    return {"value": round(tok / dt, 1), "unit": "cached tokens/s", "cores": threads, "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"{k} of {rows_total} (sequence, query, head) rows of the same workload "
                      f"(float64 C oracle, {n_q_eff} quer{'y' if n_q_eff == 1 else 'ies'} per sequence), "
                      f"{dt:.2f} s"}


if __name__ == "__main__":
    main()
