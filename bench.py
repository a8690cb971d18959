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
# timed stages of one layer step (the permutation rides on the last Lloyd
# round, the inverse permutation on the attention's stores)
STAGES = ["kmeans_permute", "select", "attention"]
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (256 CU x 2.4 GHz)
PEAK_F32_TFLOPS = 157.3
PEAK_FP8_TFLOPS = 5033.2       # MI355X dense fp8 MFMA


PEAK_CLOCK_MHZ = 2400.0         # the clock the published peaks assume


class ClockSampler:
    """Samples the shader clock every ~0.2 s between start() and stop(), read
    in-process from the amdgpu driver's ``pp_dpm_sclk`` file (the level marked
    ``*`` is the current one); under sustained matrix-core load the clock drops
    well below the one the published peak assumes.  No child process is
    started, so the sampler is also safe under a profiler that preloads itself."""

    def __init__(self):
        self.mhz, self._stop, self._th = [], False, None
        self._path = self._find()

    @staticmethod
    def _find():
        import glob
        for p in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
            try:
                with open(p) as f:
                    if "*" in f.read():
                        return p
            except OSError:
                continue
        return None

    def _run(self):
        import re
        while not self._stop and self._path:
            try:
                with open(self._path) as f:
                    for line in f:
                        if "*" in line:
                            m = re.search(r"(\d+)\s*Mhz", line, re.IGNORECASE)
                            if m:
                                self.mhz.append(int(m.group(1)))
            except OSError:
                return
            time.sleep(0.2)

    def start(self):
        import threading
        self._th = threading.Thread(target=self._run, daemon=True)
        self._th.start()

    def stop(self):
        self._stop = True
        if self._th:
            self._th.join(timeout=15)
        if not self.mhz:
            return None
        v = sorted(self.mhz)
        return {"samples": len(v), "min": v[0], "median": v[len(v) // 2], "max": v[-1]}


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
    ap.add_argument("--cpu-budget", type=float, default=30.0, help="seconds of oracle work in the CPU leg")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (counter calibration)")
    ap.add_argument("--denoise", action="store_true",
                    help="warm-start study on the denoising sequence instead of the layer step")
    ap.add_argument("--agree-heads", type=int, default=4,
                    help="--denoise: heads whose labels are compared (ARI, matched agreement)")
    ap.add_argument("--driver", action="store_true",
                    help="the denoising run through the driver (dense warm-up, cold, warm) against dense "
                         "attention on every step")
    ap.add_argument("--dense-fraction", type=float, default=0.1, help="--driver: leading dense share of the steps")
    ap.add_argument("--fp8", action="store_true",
                    help="the layer step with FP8 (E4M3) attention; the bf16 step is the default")
    ap.add_argument("--recall", action="store_true",
                    help="identification study: softmax mass recalled vs density, semantic clusters vs fixed "
                         "128-token blocks")
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
            # "- key: value" lines; the hash key itself holds a colon ("[:16]")
            if ": " in line and line.startswith("- "):
                k, v = line[2:].split(": ", 1)
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

    Sample (one head, head 0): k-means++ for the first 100 picks of each side
    (time per pick x n picks), all Lloyd rounds of both sides, the full
    permutation / selection / un-permutation of the head, and block attention
    for Q-clusters taken in order until the remaining budget is spent (every
    Q-cluster when it allows; else time per query-key pair x the head's
    pairs).  The head's time x heads is the extrapolated layer time; value =
    the layer's attention flops / that time.
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
    t_start = time.perf_counter()
    t = t_start
    m = min(100, cfg.n_q, cfg.n_k)
    sq = oracle.kmeanspp(X["q"], m, seed=1)
    sk = oracle.kmeanspp(X["k"], m, seed=2)
    per_pick = (time.perf_counter() - t) / (2 * m)
    T["kmeanspp"] = per_pick * (cfg.n_q + cfg.n_k)
    t = time.perf_counter()
    rng = np.random.default_rng(0)
    cq0 = X["q"][rng.choice(N, cfg.n_q, replace=False)]
    ck0 = X["k"][rng.choice(N, cfg.n_k, replace=False)]
    kq = oracle.kmeans(X["q"], cfg.n_q, cfg.iters, init=cq0)
    kk = oracle.kmeans(X["k"], cfg.n_k, cfg.iters, init=ck0)
    T["lloyd"] = time.perf_counter() - t
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
    attn_budget = max(budget_s - (t - t_start), 0.3 * budget_s)
    for i in range(cfg.n_q):
        if time.perf_counter() - t > attn_budget:
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
            "sample": (f"head 0 of {cfg.bh}: k-means++ {m} picks per side (scaled to {cfg.n_q} + {cfg.n_k}), "
                       f"all {cfg.iters} Lloyd rounds per side, full permute/select/un-permute, attention on "
                       f"{len(clusters)} of {cfg.n_q} Q-clusters ({done_pairs} of {head_pairs} pairs); "
                       f"extrapolated x{cfg.bh} heads"),
            "sample_s": round(time.perf_counter() - t_start, 2),
            "layer_s_extrapolated": round(layer_s, 2),
            "stage_s_per_head": {k_: round(v_, 3) for k_, v_ in T.items()}}


def padding_ratios(layer):
    """Computed work over real query-key pairs for the current selection:
    fixed 128-token blocks (every selected (Q-cluster, K-cluster) block padded
    to multiples of 128 in both dimensions) and this kernel's own padding
    (rows to 32 per Q-cluster, keys to 32 per concatenated key list)."""
    import torch
    szq = (layer.off_q[:, 1:] - layer.off_q[:, :-1]).to(torch.int64)
    szk = (layer.off_k[:, 1:] - layer.off_k[:, :-1]).to(torch.int64)
    n_q, n_k = szq.shape[1], szk.shape[1]
    valid = torch.arange(n_k, device=szk.device)[None, None, :] < layer.sel_count[:, :, None]
    idx = layer.sel_idx.clamp(0, n_k - 1).to(torch.int64)
    ksel = torch.gather(szk[:, None, :].expand(-1, n_q, -1), 2, idx) * valid
    keys = ksel.sum(2)
    keys128 = ((ksel + 127) // 128 * 128).sum(2)
    pairs = float((szq * keys).sum().item())
    fixed = float((((szq + 127) // 128 * 128) * keys128).sum().item())
    own = float((((szq + 31) // 32 * 32) * ((keys + 31) // 32 * 32)).sum().item())
    return fixed / pairs, own / pairs


def _match_agreement(a, b, n):
    """Fraction of tokens whose labels agree under the best one-to-one matching
    of the two labelings' clusters (Hungarian method on the contingency table)."""
    import numpy as np
    from scipy.optimize import linear_sum_assignment
    cont = np.zeros((n, n), dtype=np.int64)
    np.add.at(cont, (a, b), 1)
    r, c = linear_sum_assignment(-cont)
    return float(cont[r, c].sum()) / len(a)


def _objective(x, labels, cent):
    """sum_t ||x_t - c_{label(t)}||^2 over every head (fp32, per head)."""
    import torch
    tot = 0.0
    for h in range(x.shape[0]):
        c = cent[h].index_select(0, labels[h].long())
        tot += float(((x[h].float() - c) ** 2).sum().item())
    return tot


def denoise_run(args):
    """Warm start along the denoising sequence: step 0 clusters cold (k-means++
    and the config's rounds); every later step warm-starts from the previous
    step's centroids with --warm-iters rounds, and is compared with a cold start
    on the same step (time, objective, labels, output)."""
    import numpy as np
    import torch
    from sklearn.metrics import adjusted_rand_score
    from sparse_attention_video_head_amd import binding as B
    from sparse_attention_video_head_amd import synth
    from sparse_attention_video_head_amd.pipeline import SVG2Layer

    cfg = synth.CONFIGS["denoise"]
    dev = torch.device("cuda:0")
    log(f"libsvg2 {B.version()}; denoising sequence: {cfg.steps} steps, bh={cfg.bh} N={cfg.n_tokens} "
        f"d={cfg.head_dim} n_q={cfg.n_q} n_k={cfg.n_k}, warm {args.warm_iters} rounds")
    mk = lambda: SVG2Layer(cfg.bh, cfg.n_tokens, cfg.head_dim, cfg.torch_dtype, cfg.n_q, cfg.n_k, device=dev)
    warm_l, cold_l = mk(), mk()
    seeds = dict(seed_q=(cfg.seed << 8) | 0, seed_k=(cfg.seed << 8) | 1)
    E = lambda: torch.cuda.Event(enable_timing=True)

    def timed_layer(layer, x, warm, iters, top_p):
        ev = [E() for _ in range(3)]
        torch.cuda.synchronize()
        ev[0].record()
        layer.kmeans(x["q"], x["k"], iters, warm, **seeds)
        ev[1].record()
        layer.permute(x["q"], x["k"], x["v"])
        layer.select(top_p)
        out = layer.attend_unpermute()
        ev[2].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]), ev[0].elapsed_time(ev[2]), out

    steps, keep, top_p = [], {}, args.top_p
    t_gen = 0.0
    gen = synth.denoise_sequence(cfg, workers=min(16, os.cpu_count() or 1))
    for s in range(cfg.steps):
        t0 = time.time()
        host = next(gen)
        t_gen += time.time() - t0
        x = {c: host[c].to(dev) for c in "qkv"}
        if s == 0:
            # clustering and top-p of the sequence's first step (cold); warm-up launches first
            warm_l.kmeans(x["q"], x["k"], cfg.iters, False, **seeds)
            warm_l.permute(x["q"], x["k"], x["v"])
            if top_p is None:
                lo, hi = 0.01, 1.0
                for _ in range(30):
                    top_p = 0.5 * (lo + hi)
                    warm_l.select(top_p)
                    dens = warm_l.density()
                    if abs(dens - args.density) <= 0.005:
                        break
                    lo, hi = (lo, top_p) if dens > args.density else (top_p, hi)
            km, lay, _ = timed_layer(warm_l, x, False, cfg.iters, top_p)
            steps.append({"step": 0, "kmeans_ms": round(km, 3), "layer_ms": round(lay, 3), "start": "cold"})
            log(f"step 0 cold: k-means {km:.2f} ms, layer {lay:.2f} ms, top_p {top_p:.5f}")
            if not args.no_cpu_baseline:
                keep["q0"] = host["q"][0].clone()
            continue
        km_w, lay_w, out_w = timed_layer(warm_l, x, True, args.warm_iters, top_p)
        out_w = out_w.clone()
        if s == 1 and not args.no_cpu_baseline:
            keep.update(q1=host["q"][0].clone(), labels1=warm_l.labels_q[0].cpu().numpy(),
                        cent1=warm_l.cq[0].cpu().double().numpy())
        km_c, lay_c, out_c = timed_layer(cold_l, x, False, cfg.iters, top_p)
        J = {}
        for side, xs in (("q", x["q"]), ("k", x["k"])):
            lw, lc = getattr(warm_l, f"labels_{side}"), getattr(cold_l, f"labels_{side}")
            cw, cc = getattr(warm_l, f"c{side}"), getattr(cold_l, f"c{side}")
            J[side] = _objective(xs, lw, cw) / _objective(xs, lc, cc)
        ari, agree = [], []
        for side, n in (("q", cfg.n_q), ("k", cfg.n_k)):
            lw = getattr(warm_l, f"labels_{side}")[: args.agree_heads].cpu().numpy()
            lc = getattr(cold_l, f"labels_{side}")[: args.agree_heads].cpu().numpy()
            for h in range(lw.shape[0]):
                ari.append(adjusted_rand_score(lc[h], lw[h]))
                agree.append(_match_agreement(lc[h], lw[h], n))
        rel = float(torch.linalg.vector_norm((out_w.float() - out_c.float())).item()
                    / torch.linalg.vector_norm(out_c.float()).item())
        rec = {"step": s, "kmeans_ms_warm": round(km_w, 3), "kmeans_ms_cold": round(km_c, 3),
               "layer_ms_warm": round(lay_w, 3), "layer_ms_cold": round(lay_c, 3),
               "J_warm_over_cold_q": round(J["q"], 5), "J_warm_over_cold_k": round(J["k"], 5),
               "ari_mean": round(float(np.mean(ari)), 4), "matched_agreement_mean": round(float(np.mean(agree)), 4),
               "rel_l2_out_warm_vs_cold": round(rel, 5)}
        steps.append(rec)
        log(f"step {s}: k-means warm {km_w:.2f} / cold {km_c:.2f} ms; J ratio q {J['q']:.4f} k {J['k']:.4f}; "
            f"ARI {np.mean(ari):.3f}; agreement {np.mean(agree):.3f}; rel-L2(O) {rel:.4f}")
    warm_steps = steps[1:]
    mean = lambda key: float(np.mean([r[key] for r in warm_steps]))
    km_ratio = mean("kmeans_ms_cold") / mean("kmeans_ms_warm")
    res = {
        "metric": "k-means time saved by centroid caching along the denoising sequence (cold / warm)",
        "value": round(km_ratio, 3),
        "unit": "x",
        "n_gpus": 1,
        "higher_is_better": True,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": "denoise-hunyuan720p", "heads": cfg.bh, "n_tokens": cfg.n_tokens,
                   "head_dim": cfg.head_dim, "n_q": cfg.n_q, "n_k": cfg.n_k, "steps": cfg.steps,
                   "drift": cfg.drift, "cold_iters": cfg.iters, "warm_iters": args.warm_iters,
                   "top_p": round(top_p, 6), "agree_heads": args.agree_heads},
        "layer_ms_warm_mean": round(mean("layer_ms_warm"), 3),
        "layer_ms_cold_mean": round(mean("layer_ms_cold"), 3),
        "J_warm_over_cold_q_mean": round(mean("J_warm_over_cold_q"), 5),
        "J_warm_over_cold_k_mean": round(mean("J_warm_over_cold_k"), 5),
        "ari_mean": round(mean("ari_mean"), 4),
        "matched_agreement_mean": round(mean("matched_agreement_mean"), 4),
        "rel_l2_out_warm_vs_cold_mean": round(mean("rel_l2_out_warm_vs_cold"), 5),
        "input_generation_s": round(t_gen, 1),
        "steps_detail": steps,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = denoise_cpu_baseline(keep, cfg, args)
    print(json.dumps(res), flush=True)


def denoise_cpu_baseline(keep, cfg, args):
    """The fp64 oracle as it stands on head 0, Q side: a cold k-means of step 0
    (k-means++ and the config's rounds), a warm start of step 1 from those
    centroids (--warm-iters rounds) and a cold k-means of step 1, timed.  Value
    = the oracle's own cold / warm k-means time on step 1.  The cold step-1
    result is also the reference for the GPU's warm-started labels of that
    head (ARI, matched agreement, objective ratio)."""
    import numpy as np
    import oracle
    from sklearn.metrics import adjusted_rand_score
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    seed_q = (cfg.seed << 8) | 0
    x0, x1 = keep["q0"].double().numpy(), keep["q1"].double().numpy()
    c0 = oracle.kmeans(x0, cfg.n_q, cfg.iters, seed=seed_q, problem=0)
    t = time.perf_counter()
    oracle.kmeans(x1, cfg.n_q, args.warm_iters, init=c0.centroids)
    t_warm = time.perf_counter() - t
    t = time.perf_counter()
    c1 = oracle.kmeans(x1, cfg.n_q, cfg.iters, seed=seed_q, problem=0)
    t_cold = time.perf_counter() - t
    gl = keep["labels1"].astype(np.int64)
    j_gpu = oracle.objective(x1, keep["cent1"], gl)
    j_orc = oracle.objective(x1, c1.centroids, c1.labels)
    return {"value": round(t_cold / t_warm, 3), "unit": "x", "cores": threads, "kind": "oracle",
            "sample": (f"head 0, Q side (n={cfg.n_q}): fp64 cold k-means of step 0, warm start of step 1 "
                       f"({args.warm_iters} rounds), cold k-means of step 1"),
            "oracle_cold_s": round(t_cold, 2), "oracle_warm_s": round(t_warm, 2),
            "gpu_warm_vs_oracle_cold_ari": round(float(adjusted_rand_score(c1.labels, gl)), 4),
            "gpu_warm_vs_oracle_cold_matched_agreement": round(_match_agreement(c1.labels, gl, cfg.n_q), 4),
            "gpu_warm_J_over_oracle_cold_J": round(j_gpu / j_orc, 5)}


def driver_run(args):
    """The denoising run around the path: the Hunyuan-shaped layer over the
    drifting 10-step sequence through DenoiseDriver (the leading
    --dense-fraction of the steps dense, then a cold start, then warm starts
    from the centroid cache), against the library's dense attention on every
    step.  Per-step HIP-event times; the whole run is also extrapolated to 50
    steps from the per-mode means."""
    import numpy as np
    import torch
    from sparse_attention_video_head_amd import binding as B
    from sparse_attention_video_head_amd import synth
    from sparse_attention_video_head_amd.driver import DenoiseDriver, dense_steps

    cfg = synth.CONFIGS["denoise"]
    dev = torch.device("cuda:0")
    log(f"libsvg2 {B.version()}; driver over {cfg.steps} steps, bh={cfg.bh} N={cfg.n_tokens} d={cfg.head_dim} "
        f"n_q={cfg.n_q} n_k={cfg.n_k}, dense share {args.dense_fraction}, warm {args.warm_iters} rounds")
    drv = DenoiseDriver(cfg.bh, cfg.n_tokens, cfg.head_dim, cfg.torch_dtype, cfg.n_q, cfg.n_k, cfg.steps,
                        top_p=1.0, dense_fraction=args.dense_fraction, cold_iters=cfg.iters,
                        warm_iters=args.warm_iters, seed=cfg.seed, device=dev)
    e = drv.engine
    E = lambda: torch.cuda.Event(enable_timing=True)

    def timed(fn):
        a, b = E(), E()
        torch.cuda.synchronize()
        a.record()
        r = fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b), r

    gen = synth.denoise_sequence(cfg, workers=min(16, os.cpu_count() or 1))
    t0 = time.time()
    seq = [next(gen)]
    top_p = args.top_p
    rows, dense_out = [], torch.empty(cfg.bh, cfg.n_tokens, cfg.head_dim, dtype=cfg.torch_dtype, device=dev)
    for s in range(cfg.steps):
        host = seq[-1] if s == 0 else next(gen)
        x = [host[c].to(dev) for c in "qkv"]
        if s == 0:
            log(f"inputs of step 0 in {time.time() - t0:.1f}s")
            # warm-up launches, and top-p bisected on a cold clustering of step 0
            e.dense(*x, out=dense_out)
            e.kmeans(x[0], x[1], cfg.iters, False, 1, 2)
            e.permute(*x)
            if top_p is None:
                lo, hi = 0.01, 1.0
                for _ in range(30):
                    top_p = 0.5 * (lo + hi)
                    e.select(top_p)
                    dens = e.density()
                    if abs(dens - args.density) <= 0.005:
                        break
                    lo, hi = (lo, top_p) if dens > args.density else (top_p, hi)
            drv.top_p = top_p
            drv.reset()
        mode = drv.mode(0, s)
        ms, out = timed(lambda: drv(0, s, *x))
        out = out.clone()
        dms, _ = timed(lambda: e.dense(*x, out=dense_out))
        rel = float(torch.linalg.vector_norm(out.float() - dense_out.float()).item()
                    / torch.linalg.vector_norm(dense_out.float()).item())
        rows.append({"step": s, "mode": mode, "ms": round(ms, 3), "dense_ms": round(dms, 3),
                     "rel_l2_vs_dense": round(rel, 5)})
        log(f"step {s} {mode}: {ms:.2f} ms (dense {dms:.2f} ms), rel-L2 vs dense {rel:.4f}")
    run_ms = sum(r["ms"] for r in rows)
    dense_ms = sum(r["dense_ms"] for r in rows)
    mean = lambda m: float(np.mean([r["ms"] for r in rows if r["mode"] == m]))
    d50 = dense_steps(50, args.dense_fraction)
    dense_mean = float(np.mean([r["dense_ms"] for r in rows]))
    run50 = d50 * dense_mean + mean("cold") + (50 - d50 - 1) * mean("warm")
    res = {
        "metric": "attention time over a denoising run, all-dense / this driver",
        "value": round(dense_ms / run_ms, 3), "unit": "x", "n_gpus": 1, "higher_is_better": True,
        "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": "denoise-hunyuan720p-driver", "heads": cfg.bh, "n_tokens": cfg.n_tokens,
                   "head_dim": cfg.head_dim, "n_q": cfg.n_q, "n_k": cfg.n_k, "steps": cfg.steps,
                   "dense_fraction": args.dense_fraction, "cold_iters": cfg.iters, "warm_iters": args.warm_iters,
                   "top_p": round(top_p, 6)},
        "run_ms": round(run_ms, 3), "all_dense_ms": round(dense_ms, 3),
        "mean_ms": {m: round(mean(m), 3) for m in ("dense", "cold", "warm") if any(r["mode"] == m for r in rows)},
        "extrapolated_50_steps": {"dense_steps": d50, "run_ms": round(run50, 1),
                                  "all_dense_ms": round(50 * dense_mean, 1),
                                  "speedup": round(50 * dense_mean / run50, 3)},
        "steps_detail": rows,
    }
    print(json.dumps(res), flush=True)


RECALL_TOP_P = (0.05, 0.1, 0.2, 0.3, 0.5, 0.7, 0.8, 0.9, 0.95, 0.98, 0.99, 0.995, 0.998, 0.999, 0.9999)


def recall_run(args):
    """Identification accuracy at the layer's shape: for a sweep of top-p, the
    density and the mean share of each query row's exact softmax mass that
    the selection keeps, for the method's semantic clusters and for fixed
    128-token blocks with mean-pooled representatives."""
    import numpy as np
    import torch
    from sparse_attention_video_head_amd import binding as B
    from sparse_attention_video_head_amd import synth
    from sparse_attention_video_head_amd.study import IdentificationStudy

    cfg = synth.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    t0 = time.time()
    data = synth.make_layer(cfg)
    log(f"libsvg2 {B.version()}; recall study {cfg.name}: bh={cfg.bh} N={cfg.n_tokens}; inputs {time.time() - t0:.1f}s")
    q, k, v = (data[c].to(dev) for c in "qkv")
    st = IdentificationStudy(cfg.bh, cfg.n_tokens, cfg.head_dim, cfg.torch_dtype, cfg.n_q, cfg.n_k, block=128,
                             device=dev)
    seeds = dict(seed_q=(cfg.seed << 8) | 0, seed_k=(cfg.seed << 8) | 1)
    N2 = cfg.bh * float(cfg.n_tokens) ** 2
    t1 = time.time()
    curves = {}
    for name, rows in (("semantic", st.semantic(q, k, v, RECALL_TOP_P, iters=cfg.iters, **seeds)),
                       ("positional_128", st.positional(q, k, v, RECALL_TOP_P))):
        pts = [{"top_p": r["top_p"], "density": round(float(r["pairs"].sum().item()) / N2, 5),
                "recall": round(float(r["recall"].mean().item()), 5)} for r in rows]
        curves[name] = pts
        for pt in pts:
            log(f"{name:15s} p={pt['top_p']:<7} density {pt['density']:.4f} recall {pt['recall']:.4f}")
    torch.cuda.synchronize()
    elapsed = time.time() - t1

    def at(name, dens):
        pts = sorted((p["density"], p["recall"]) for p in curves[name])
        xs, ys = [p[0] for p in pts], [p[1] for p in pts]
        return round(float(np.interp(dens, xs, ys)), 5) if xs[0] <= dens <= xs[-1] else None

    res = {
        "metric": "share of the exact softmax mass recalled at 25% density, semantic clusters (fixed 128-token "
                  "blocks beside it)",
        "value": at("semantic", 0.25), "unit": "fraction", "n_gpus": 1, "higher_is_better": True,
        "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": f"{cfg.name}-identification", "heads": cfg.bh, "n_tokens": cfg.n_tokens,
                   "head_dim": cfg.head_dim, "n_q": cfg.n_q, "n_k": cfg.n_k, "kmeans_iters": cfg.iters,
                   "block": 128},
        "recall_at_density": {name: {f"{d:.2f}": at(name, d) for d in (0.05, 0.10, 0.25, 0.50)} for name in curves},
        "curves": curves, "sweep_s": round(elapsed, 2),
    }
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path shards by head with no "
              "exchange and is not run on several GPUs here.", file=sys.stderr)
        sys.exit(2)
    if args.denoise:
        denoise_run(args)
        return
    if args.driver:
        driver_run(args)
        return
    if args.recall:
        recall_run(args)
        return

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
    layer = SVG2Layer(cfg.bh, cfg.n_tokens, cfg.head_dim, cfg.torch_dtype, cfg.n_q, cfg.n_k, device=dev,
                      fp8_attention=args.fp8)
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
        # k-means of Q and K; the last Lloyd round also writes Q', K', V'
        layer.cluster(q, k, v, iters, warm, **seeds)
        if ev:
            ev[1].record()
        layer.select(top_p)
        if ev:
            ev[2].record()
        # the inverse permutation is fused into the attention's stores (FP8:
        # the last Lloyd round already stored Q', K', V' as E4M3)
        layer.attend_unpermute()
        if ev:
            ev[3].record()

    def timed(warm: bool, iters: int, steps: int):
        evs = [[E() for _ in range(4)] for _ in range(steps)]
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        for i in range(steps):
            step(warm, iters, evs[i])
        torch.cuda.synchronize()
        wall = (time.perf_counter() - w0) * 1e3 / steps
        st = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(3)] for i in range(steps)])
        tot = np.array([evs[i][0].elapsed_time(evs[i][3]) for i in range(steps)])
        return st.mean(0), float(tot.mean()), wall

    for _ in range(args.warmup):
        step(False, cfg.iters)
    torch.cuda.synchronize()
    log("warm-up done")
    clock = ClockSampler()
    clock.start()
    cold_stage, cold_ms, cold_wall = timed(False, cfg.iters, args.steps)
    log(f"cold step {cold_ms:.2f} ms (wall {cold_wall:.2f}); stages {np.round(cold_stage, 3).tolist()}")
    # work of the cold steps' selection (the layer keeps only the last select)
    cold_pairs = int(layer.pairs.sum().item())
    pad_fixed128, pad_own = padding_ratios(layer)
    # warm start: centroid cache from the previous step, fewer Lloyd rounds
    step(True, args.warm_iters)
    warm_stage, warm_ms, _ = timed(True, args.warm_iters, args.steps)
    gpu_clock = clock.stop()
    log(f"warm step {warm_ms:.2f} ms; stages {np.round(warm_stage, 3).tolist()}; shader clock MHz {gpu_clock}")
    warm_pairs = int(layer.pairs.sum().item())
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
    # a cold k-means alone (no rows moved): seeding, and what the moves in
    # the last round add
    a, b = E(), E()
    torch.cuda.synchronize()
    a.record()
    layer.kmeans(q, k, cfg.iters, False, **seeds)
    b.record()
    torch.cuda.synchronize()
    kmeans_cold_ms = a.elapsed_time(b)
    # k-means++ alone (both sides, no Lloyd round)
    a, b = E(), E()
    torch.cuda.synchronize()
    a.record()
    layer.kmeans(q, k, 0, False, **seeds)
    b.record()
    torch.cuda.synchronize()
    seeding_ms = a.elapsed_time(b)
    fused_move_ms = float(cold_stage[0]) - kmeans_cold_ms
    # the stand-alone permutation (sort + row gather of Q, K and V)
    def median_ms(fn, runs=3):
        fn()
        ts = []
        for _ in range(runs):
            a, b = E(), E()
            torch.cuda.synchronize()
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    permute_ms = median_ms(lambda: layer.permute(q, k, v, quantize=False))
    # the stand-alone inverse permutation (the layer fuses it into the
    # attention's stores, where it costs no pass of its own)
    unpermute_ms = median_ms(layer.unpermute)
    # a plain device copy of one K-sized tensor: what one read-and-write pass
    # over HBM reaches on this device, beside the 8 TB/s published peak
    k_copy = torch.empty_like(k)
    copy_ms = median_ms(lambda: k_copy.copy_(k))
    del k_copy
    # the Lloyd round's kernels one side at a time (one stream, final labels):
    # the update alone (counting sort + segmented mean) and a whole round
    # (centroid halves + assignment + update); the assignment is the difference
    lloyd_rows = {}
    for side, x, n, lab, cent in (("q", q, cfg.n_q, layer.labels_q, layer.cq),
                                  ("k", k, cfg.n_k, layer.labels_k, layer.ck)):
        bhn_, N_, d_ = x.shape
        means, cnt = torch.empty_like(cent), torch.empty(bhn_, n, dtype=torch.int32, device=x.device)
        c_out, lab_out = torch.empty_like(cent), torch.empty_like(lab)
        ws_m = torch.empty(B.lib().svg2_cluster_means_workspace_size(bhn_, N_, d_, n), dtype=torch.uint8,
                           device=x.device)
        ws_k = torch.empty(B.lib().svg2_kmeans_workspace_size(bhn_, N_, d_, n), dtype=torch.uint8, device=x.device)
        upd = median_ms(lambda: B.cluster_means(x, lab, n, means=means, counts=cnt, workspace=ws_m))
        rnd = median_ms(lambda: B.kmeans(x, n, 1, init=cent, centroids=c_out, labels=lab_out, counts=cnt,
                                         workspace=ws_k))
        e_ = x.element_size()
        upd_bytes = bhn_ * (N_ * (d_ * e_ + 12.0) + n * d_ * 4.0)
        asg_flops = 2.0 * bhn_ * N_ * n * d_
        lloyd_rows[side] = {"update_ms": round(upd, 4), "update_gbps": round(upd_bytes / (upd * 1e-3) / 1e9, 1),
                            "round_ms": round(rnd, 4), "assign_ms": round(rnd - upd, 4),
                            "assign_tflops": round(asg_flops / ((rnd - upd) * 1e-3) / 1e12, 2)}
    log(f"Lloyd kernels per side: {lloyd_rows}")

    dense_ms = rel_dense = None
    if not args.no_dense:
        layer.dense(q, k, v)
        a, b = E(), E()
        torch.cuda.synchronize()
        a.record()
        o_dense = layer.dense(q, k, v)
        b.record()
        torch.cuda.synchronize()
        dense_ms = a.elapsed_time(b)
        # the cold step's sparse output (last timed step) against dense attention
        step(False, cfg.iters)
        torch.cuda.synchronize()
        rel_dense = float(torch.linalg.vector_norm(layer.out.float() - o_dense.float()).item()
                          / torch.linalg.vector_norm(o_dense.float()).item())
        del o_dense
        log(f"dense attention {dense_ms:.2f} ms; sparse vs dense rel-L2 {rel_dense:.4f}")

    attn_flops = 4.0 * cfg.head_dim * cold_pairs
    attn_ms = float(cold_stage[2])
    attn_tflops = attn_flops / (attn_ms * 1e-3) / 1e12
    peak = PEAK_FP8_TFLOPS if args.fp8 else (PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS)
    value = attn_flops / (cold_ms * 1e-3) / 1e12
    dense_flops = 4.0 * cfg.head_dim * cfg.bh * float(cfg.n_tokens) ** 2

    e = 2 if cfg.dtype == "bf16" else 4
    N, d, bhn = cfg.n_tokens, cfg.head_dim, cfg.bh
    permute_bytes = bhn * (6.0 * N * d * e + 8.0 * N)      # Q, K, V read + written, labels, perm
    unpermute_bytes = bhn * (2.0 * N * d * e + 4.0 * N)
    # the committed counters cover the bf16 kernel at the default Hunyuan-shaped workload only
    same_workload = args.config == "hunyuan720p" and args.top_p is None and not args.fp8
    traffic = attn_traffic_per_launch() if same_workload else None
    # Lloyd distance contraction: 2 d N (n_Q + n_K) flop per head and round
    # (the matrix core issues twice that for the hi/lo centroid halves)
    lloyd_flops = 2.0 * d * N * (cfg.n_q + cfg.n_k) * bhn
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
        "dtype": "fp8" if args.fp8 else cfg.dtype,
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}-layer" + ("-fp8-attention" if args.fp8 else ""), "heads": cfg.bh, "n_tokens": cfg.n_tokens,
                   "head_dim": cfg.head_dim, "n_q": cfg.n_q, "n_k": cfg.n_k, "kmeans_iters": cfg.iters,
                   "start": "cold (k-means++)", "top_p": round(top_p, 6), "density": round(density, 5)},
        "layer_ms_cold": round(cold_ms, 3),
        "layer_ms_warm": round(warm_ms, 3),
        "warm_iters": args.warm_iters,
        "stage_ms_cold": dict(zip(STAGES, [round(float(x), 4) for x in cold_stage])),
        "stage_ms_warm": dict(zip(STAGES, [round(float(x), 4) for x in warm_stage])),
        "attn_tflops": round(attn_tflops, 2),
        "attn_tflops_warm": round(4.0 * cfg.head_dim * warm_pairs / (float(warm_stage[2]) * 1e-3) / 1e12, 2),
        "pairs_cold": cold_pairs,
        "pairs_warm": warm_pairs,
        "kmeans_ms_per_iter": round(ms_per_iter, 4),
        "kmeans_iters_per_s": round(1e3 / ms_per_iter, 1) if ms_per_iter > 0 else None,
        "kmeanspp_seeding_ms": round(float(seeding_ms), 3),
        "kmeans_cold_ms": round(kmeans_cold_ms, 3),
        "permute_in_last_round_ms": round(fused_move_ms, 3),
        "dense_ms": round(dense_ms, 3) if dense_ms else None,
        "dense_tflops": round(dense_flops / (dense_ms * 1e-3) / 1e12, 2) if dense_ms else None,
        "speedup_vs_dense_cold": round(dense_ms / cold_ms, 3) if dense_ms else None,
        "speedup_vs_dense_warm": round(dense_ms / warm_ms, 3) if dense_ms else None,
        "lloyd_round_distance_tflops": round(lloyd_flops / (ms_per_iter * 1e-3) / 1e12, 2) if ms_per_iter > 0 else None,
        # per side on one stream: update = counting sort + segmented mean (HBM-bound,
        # N (d e + 12) + n d 4 bytes per problem); assign = the rest of a round
        # (centroid halves + distance contraction, 2 N n d flop per problem, twice that issued for bf16)
        "lloyd_kernels_per_side": lloyd_rows,
        "select_share_of_dense": round(float(cold_stage[1]) / dense_ms, 5) if dense_ms else None,
        "rel_l2_sparse_vs_dense": round(rel_dense, 5) if rel_dense is not None else None,
        "padding_ratio_fixed128_blocks": round(pad_fixed128, 4),
        "padding_ratio_this_kernel": round(pad_own, 4),
        "permute_ms_standalone": round(permute_ms, 4),
        "permute_gbps": round(permute_bytes / (permute_ms * 1e-3) / 1e9, 1),
        "unpermute_gbps": round(unpermute_bytes / (unpermute_ms * 1e-3) / 1e9, 1),
        "device_copy_gbps": round(2 * k.numel() * k.element_size() / (copy_ms * 1e-3) / 1e9, 1),
        "roofline": {"bound": "mfma",
                     "kernel": "k_attn_fp8" if args.fp8 else ("k_attn_bf16" if cfg.dtype == "bf16" else "k_attn_f32"),
                     "achieved": round(attn_tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / peak, 4), "traffic": traffic,
                     "flops_per_launch": attn_flops},
        # shader clock over the timed steps, and the peak scaled to its median
        "gpu_clock_mhz": gpu_clock,
        "peak_at_measured_clock": (round(peak * gpu_clock["median"] / PEAK_CLOCK_MHZ, 1) if gpu_clock else None),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(host, cfg, top_p, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
