#!/usr/bin/env python3
"""Benchmark of one SVG2 sparse-attention layer on one MI355X.

A step is one pass of the whole path over one layer's synthetic Q/K/V already
resident in HBM: cold k-means++ seeding and 5 Lloyd rounds on Q (400
clusters) and K (1000 clusters), permutation of Q, K, V, centroid scores with
top-p selection, variable-block attention, un-permutation.  Default workload:
the HunyuanVideo-720p-shaped layer (24 heads x 118,800 tokens x 128, bf16)
with top-p bisected to ~25% density.

Prints one JSON line.  `value` = effective attention TFLOP/s of the whole
step: 4 * head_dim * (computed query-key pairs) / step time.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-attn effective TFLOP/s + layer latency at 118k tokens; k-means iters/s"
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (256 CU x 2.4 GHz)
PEAK_F32_TFLOPS = 157.3


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="hunyuan720p")
    ap.add_argument("--top-p", type=float, default=None, help="fixed top-p (default: config / bisection)")
    ap.add_argument("--density", type=float, default=0.25, help="bisection target when top-p is tuned")
    ap.add_argument("--warm-iters", type=int, default=2)
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work in the CPU leg")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (counter calibration)")
    return ap.parse_args()


ATTN_SOURCE = os.path.join(ROOT, "sparse_attention_video_head_amd", "csrc", "attn.hip")
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "k_attn_bf16_hunyuan720p_counters.md")


def attn_traffic_per_launch():
    """HBM bytes per attention launch from the committed counter summary, if it
    was taken on the attention source as it is now (else None)."""
    import hashlib
    try:
        sha = hashlib.sha256(open(ATTN_SOURCE, "rb").read()).hexdigest()[:16]
        fields = {}
        for line in open(TRAFFIC_PROFILE):
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip()
        if fields.get("attn.hip sha256[:16]") != sha:
            return None
        return float(fields["calibrated HBM bytes per launch"])
    except (OSError, KeyError, ValueError):
        return None


def copy_calibration(mib: int):
    import torch
    n = mib * (1 << 20) // 2
    src = torch.empty(n, dtype=torch.bfloat16, device="cuda").normal_()
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": 2 * n, "copy_bytes_written": 2 * n, "launches": 3}), flush=True)


def cpu_baseline(host, cfg, top_p, budget_s):
    """The fp64 oracle as it stands, timed on the host on a bounded sample of
    the same layer, scaled to the metric's unit.

    Sample (one head, head 0): k-means++ for the first m picks of each side
    (time per pick x n picks), one Lloyd round per side (x rounds), the full
    permutation / selection / un-permutation of the head, and block attention
    for Q-clusters taken in order until the attention budget is spent (time
    per query-key pair x the head's pairs).  The head's time x heads is the
    extrapolated layer time; value = the layer's attention flops / that time.
    """
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    X = {x: host[x][0].double().numpy() for x in "qkv"}
    N, d = X["q"].shape
    scale = 1.0 / math.sqrt(d)
    T = {}
    t = time.perf_counter()
    m = 8
    sq = oracle.kmeanspp(X["q"], m, seed=1)
    sk = oracle.kmeanspp(X["k"], m, seed=2)
    per_pick = (time.perf_counter() - t) / (2 * m)
    T["kmeanspp"] = per_pick * (cfg.n_q + cfg.n_k)
    t = time.perf_counter()
    rng = np.random.default_rng(0)
    cq0 = X["q"][rng.choice(N, cfg.n_q, replace=False)]
    ck0 = X["k"][rng.choice(N, cfg.n_k, replace=False)]
    kq = oracle.kmeans(X["q"], cfg.n_q, 1, init=cq0)
    kk = oracle.kmeans(X["k"], cfg.n_k, 1, init=ck0)
    T["lloyd"] = (time.perf_counter() - t) * cfg.iters
    t = time.perf_counter()
    pq, oq, _ = oracle.counting_sort(kq.labels, cfg.n_q)
    pk, ok, _ = oracle.counting_sort(kk.labels, cfg.n_k)
    qp, kp, vp = oracle.permute_rows(X["q"], pq), oracle.permute_rows(X["k"], pk), oracle.permute_rows(X["v"], pk)
    P = oracle.centroid_probs(kq.centroids, kk.centroids, kk.counts, scale)
    sel = oracle.select_topp(P, kk.counts, float(np.float32(top_p)))
    T["permute_select"] = time.perf_counter() - t
    head_pairs = oracle.pair_count(sel.lists, kq.counts, kk.counts)
    t = time.perf_counter()
    done_pairs, clusters = 0, []
    for i in range(cfg.n_q):
        if time.perf_counter() - t > 0.6 * budget_s:
            break
        oracle.block_attention(qp, kp, vp, oq, ok, sel.lists, scale, q_clusters=[i])
        done_pairs += int(kq.counts[i]) * int(np.sum(kk.counts[sel.lists[i]]))
        clusters.append(i)
    t_attn = time.perf_counter() - t
    T["attention"] = t_attn / max(done_pairs, 1) * head_pairs
    t = time.perf_counter()
    oracle.unpermute_rows(qp, pq)
    T["unpermute"] = time.perf_counter() - t
    head_s = sum(T.values())
    layer_s = head_s * cfg.bh
    layer_flops = 4.0 * d * head_pairs * cfg.bh
    return {"value": round(layer_flops / layer_s / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"head 0 of {cfg.bh}: k-means++ {m} picks per side, 1 Lloyd round per side, full "
                       f"permute/select/un-permute, attention on {len(clusters)} of {cfg.n_q} Q-clusters "
                       f"({done_pairs} of {head_pairs} pairs); extrapolated x{cfg.bh} heads"),
            "layer_s_extrapolated": round(layer_s, 2),
            "stage_s_per_head": {k_: round(v_, 3) for k_, v_ in T.items()}}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path shards by head with no "
              "exchange and is not run on several GPUs here.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from sparse_attention_video_head_amd import binding as B
    from sparse_attention_video_head_amd import synth
    from sparse_attention_video_head_amd.pipeline import SVG2Layer

    cfg = synth.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    log(f"libsvg2 {B.version()}; config {cfg.name}: bh={cfg.bh} N={cfg.n_tokens} d={cfg.head_dim} "
        f"{cfg.dtype} n_q={cfg.n_q} n_k={cfg.n_k}")
    t0 = time.time()
    data = synth.make_layer(cfg)
    log(f"generated inputs in {time.time() - t0:.1f}s")
    q, k, v = (data[x].to(dev) for x in "qkv")
    host = data
    layer = SVG2Layer(cfg.bh, cfg.n_tokens, cfg.head_dim, cfg.torch_dtype, cfg.n_q, cfg.n_k, device=dev)
    seeds = dict(seed_q=(cfg.seed << 8) | 0, seed_k=(cfg.seed << 8) | 1)

    # ---- top-p: config value, or bisected on the cold-start clustering
    layer.kmeans(q, k, cfg.iters, False, **seeds)
    layer.permute(q, k, v)
    if args.top_p is not None:
        top_p = args.top_p
    elif cfg.top_p[0] is not None:
        top_p = cfg.top_p[0]
    else:
        lo, hi = 0.01, 1.0
        top_p = 0.5
        for _ in range(30):
            top_p = 0.5 * (lo + hi)
            layer.select(top_p)
            dens = layer.density()
            if abs(dens - args.density) <= 0.005:
                break
            if dens > args.density:
                hi = top_p
            else:
                lo = top_p
    layer.select(top_p)
    density = layer.density()
    log(f"top_p {top_p:.5f} -> density {density:.4f}")

    E = lambda: torch.cuda.Event(enable_timing=True)

    def step(warm: bool, iters: int, ev=None):
        if ev:
            ev[0].record()
        layer.kmeans(q, k, iters, warm, **seeds)
        if ev:
            ev[1].record()
        layer.permute(q, k, v)
        if ev:
            ev[2].record()
        layer.select(top_p)
        if ev:
            ev[3].record()
        layer.attend()
        if ev:
            ev[4].record()
        layer.unpermute()
        if ev:
            ev[5].record()

    def timed(warm: bool, iters: int, steps: int):
        evs = [[E() for _ in range(6)] for _ in range(steps)]
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        for i in range(steps):
            step(warm, iters, evs[i])
        torch.cuda.synchronize()
        wall = (time.perf_counter() - w0) * 1e3 / steps
        st = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(5)] for i in range(steps)])
        tot = np.array([evs[i][0].elapsed_time(evs[i][5]) for i in range(steps)])
        return st.mean(0), float(tot.mean()), wall

    for _ in range(args.warmup):
        step(False, cfg.iters)
    torch.cuda.synchronize()
    log("warm-up done")
    cold_stage, cold_ms, cold_wall = timed(False, cfg.iters, args.steps)
    log(f"cold step {cold_ms:.2f} ms (wall {cold_wall:.2f}); stages {np.round(cold_stage, 3).tolist()}")
    # warm start: centroid cache from the previous step, fewer Lloyd rounds
    step(True, args.warm_iters)
    warm_stage, warm_ms, _ = timed(True, args.warm_iters, args.steps)
    log(f"warm step {warm_ms:.2f} ms; stages {np.round(warm_stage, 3).tolist()}")
    # k-means rounds without seeding: iterations per second of the layer (Q and K)
    km = []
    for it in (1, 5):
        a, b = E(), E()
        torch.cuda.synchronize()
        a.record()
        layer.kmeans(q, k, it, True, **seeds)
        b.record()
        torch.cuda.synchronize()
        km.append(a.elapsed_time(b))
    ms_per_iter = (km[1] - km[0]) / 4.0
    seeding_ms = cold_stage[0] - cfg.iters * ms_per_iter

    dense_ms = None
    if not args.no_dense:
        layer.dense(q, k, v)
        a, b = E(), E()
        torch.cuda.synchronize()
        a.record()
        layer.dense(q, k, v)
        b.record()
        torch.cuda.synchronize()
        dense_ms = a.elapsed_time(b)
        log(f"dense attention {dense_ms:.2f} ms")

    pairs = int(layer.pairs.sum().item())
    attn_flops = 4.0 * cfg.head_dim * pairs
    attn_ms = float(cold_stage[3])
    attn_tflops = attn_flops / (attn_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    value = attn_flops / (cold_ms * 1e-3) / 1e12
    dense_flops = 4.0 * cfg.head_dim * cfg.bh * float(cfg.n_tokens) ** 2

    e = 2 if cfg.dtype == "bf16" else 4
    N, d, bhn = cfg.n_tokens, cfg.head_dim, cfg.bh
    permute_bytes = bhn * (6.0 * N * d * e + 8.0 * N)      # Q, K, V read + written, labels, perm
    unpermute_bytes = bhn * (2.0 * N * d * e + 4.0 * N)
    traffic = attn_traffic_per_launch()
    res = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(cold_ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}-layer", "heads": cfg.bh, "n_tokens": cfg.n_tokens,
                   "head_dim": cfg.head_dim, "n_q": cfg.n_q, "n_k": cfg.n_k, "kmeans_iters": cfg.iters,
                   "start": "cold (k-means++)", "top_p": round(top_p, 6), "density": round(density, 5)},
        "layer_ms_cold": round(cold_ms, 3),
        "layer_ms_warm": round(warm_ms, 3),
        "warm_iters": args.warm_iters,
        "stage_ms_cold": dict(zip(["kmeans", "permute", "select", "attention", "unpermute"],
                                  [round(float(x), 4) for x in cold_stage])),
        "stage_ms_warm": dict(zip(["kmeans", "permute", "select", "attention", "unpermute"],
                                  [round(float(x), 4) for x in warm_stage])),
        "attn_tflops": round(attn_tflops, 2),
        "kmeans_ms_per_iter": round(ms_per_iter, 4),
        "kmeans_iters_per_s": round(1e3 / ms_per_iter, 1) if ms_per_iter > 0 else None,
        "kmeanspp_seeding_ms": round(float(seeding_ms), 3),
        "dense_ms": round(dense_ms, 3) if dense_ms else None,
        "dense_tflops": round(dense_flops / (dense_ms * 1e-3) / 1e12, 2) if dense_ms else None,
        "speedup_vs_dense_cold": round(dense_ms / cold_ms, 3) if dense_ms else None,
        "speedup_vs_dense_warm": round(dense_ms / warm_ms, 3) if dense_ms else None,
        "permute_gbps": round(permute_bytes / (cold_stage[1] * 1e-3) / 1e9, 1),
        "unpermute_gbps": round(unpermute_bytes / (cold_stage[4] * 1e-3) / 1e9, 1),
        "roofline": {"bound": "mfma", "kernel": "k_attn_bf16" if cfg.dtype == "bf16" else "k_attn_f32",
                     "achieved": round(attn_tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / peak, 4), "traffic": traffic,
                     "flops_per_launch": attn_flops},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(host, cfg, top_p, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
