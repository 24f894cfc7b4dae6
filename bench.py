#!/usr/bin/env python3
"""Decode-step benchmark of libkpa on one MI355X.

One step = kpa_cache_append of the step's new token(s) (with the
Kronecker-separable RoPE on B^K) followed by the factor-space decode
(kpa_decode, or kpa_decode_multiq for the multi-query workload) over the whole
cached context of every sequence, on seeded synthetic inputs already resident
in HBM.  The default workload is 32 sequences x 32768 cached tokens,
h = 4x4, d_h = 8x16, R_K = R_V = 2, bfloat16 factors.

Prints ONE JSON line with the cached-tokens-attended rate, the roofline of
the decode kernel (algorithmic bytes / kernel time, timed with HIP events on
the launch stream), and the CPU oracle timed on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBPS = 8000.0  # MI355X published HBM3E bandwidth
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
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(the decode shards by sequence with no communication; see DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import factorized_kv_cache_kpa_amd as kpa
    from workloads import CONFIGS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    kpa.load()
    cfg = CONFIGS[args.workload]
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

    def decode():
        if n_q == 1:
            kpa.kpa_decode(dims, cache, nb, ctx, ctx_len, ctx, q.view(nb, h, dh), q_pos.view(nb),
                           out.view(nb, h, dh), lse.view(nb, h), ws, args.num_splits)
        else:
            kpa.kpa_decode_multiq(dims, cache, nb, ctx, ctx_len, ctx, n_q, 1, q, q_pos, out, lse, ws,
                                  args.num_splits)

    def step(ev=None):
        kpa.kpa_cache_append(dims, cache, nb, ctx, new_ak, new_bk, new_av, new_bv, new_pos, slot0,
                             n_new=n_new)
        if ev is not None:
            ev[0].record()
        decode()
        if ev is not None:
            ev[1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if not torch.isfinite(out).all():
        log("non-finite decode output")
        sys.exit(1)
    log(f"warmup done ({args.warmup} steps)")

    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    ms_per_step = (t_end - t_start) * 1e3 / args.steps
    decode_ms = float(np.mean([a.elapsed_time(b) for a, b in events]))
    log(f"timed {args.steps} steps: {ms_per_step:.4f} ms/step, decode {decode_ms * 1e3:.1f} us")

    tokens = int(inp.ctx_len.sum().item())  # cached tokens attended per step (per query)
    value = tokens / (ms_per_step / 1e3)
    # algorithmic bytes of one decode launch: every attended token's factors
    # once, plus the queries and outputs (no padding, no partial results)
    alg_bytes = tokens * cfg.bytes_per_token + q.numel() * 4 + out.numel() * 4 + lse.numel() * 4
    achieved = alg_bytes / (decode_ms / 1e3) / 1e9
    roofline = {"bound": "hbm", "kernel": "kpa_decode (split-KV decode + log-sum-exp merge)",
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                "alg_bytes_per_launch": alg_bytes, "launch_us": round(decode_ms * 1e3, 2)}

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
                   "path": kpa.kpa_decode_path(dims, n_q), "step": "append new token(s) + decode",
                   "parallelism": "single GPU"},
        "achieved_hbm_gbps": round(achieved, 1), "hbm_pct_of_peak": round(100 * achieved / HBM_PEAK_GBPS, 2),
        "roofline": roofline, "cpu_baseline": cpu,
    }
    line = json.dumps(res)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")


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
    return {"value": round(tok / dt, 1), "unit": "cached tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{k} of {rows_total} (sequence, query, head) rows of the same workload "
                      f"(float64 C oracle, {n_q_eff} quer{'y' if n_q_eff == 1 else 'ies'} per sequence), "
                      f"{dt:.2f} s"}


if __name__ == "__main__":
    main()
