"""Seeded synthetic Q/K/V generators shaped like video-DiT attention layers.

This module only draws data. It holds none of the method's arithmetic (no
clustering, no scoring, no attention), so that both the fp64 oracle and the
HIP path can be fed the very same inputs from it.

The pages measure whole video generations of HunyuanVideo-T2V-13B and
Wan 2.1 at 720p ("Sparse VideoGen2" wiki summary, Results; Key claims,
[Table 1]). Weights and prompts are not available, so seeded Gaussian
mixtures with the layers' shapes stand in for their attention activations:

* tokens of a head carry a component label ``z``; ``q = mu_z + 0.3 eps``,
  ``k = mu_z + 0.3 eps'`` with independent noise, so Q and K of one token
  share a component (the semantic similarity the method clusters on);
* video-shaped configs place labels on the latent grid (frames x height x
  width) as a 3-D Voronoi field of ``2C`` random sites, then relabel 20% of
  tokens at random, so clusters are spatially correlated but scattered;
* the two 720p configs draw component weights from a Zipf law (exponent
  1.1), which makes cluster sizes heavy-tailed.

Every random stream is ``numpy.random.SeedSequence([base, head, stream])``;
values are drawn in fp64 and rounded once to the config dtype.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np
import torch

# stream ids inside one head
_S_CENTERS, _S_FIELD, _S_Q, _S_K, _S_V, _S_DRIFT = 0, 1, 2, 3, 4, 5


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    batch: int
    heads: int
    n_tokens: int
    head_dim: int
    dtype: str                 # "f32" or "bf16"
    n_centers: int             # mixture components per head
    weights: str               # "uniform" or "zipf"
    field: str                 # "iid" or "voronoi"
    grid: Optional[tuple]      # (frames, height, width) for "voronoi"
    v_kind: str                # "mixture" (same mixture as Q/K) or "normal"
    n_q: int                   # query clusters
    n_k: int                   # key clusters
    iters: int                 # cold-start Lloyd iterations
    top_p: tuple               # top-p values to run (None entries: tuned)
    seed: int                  # seed base
    noise: float = 0.3
    relabel: float = 0.2
    zipf_alpha: float = 1.1
    steps: int = 1             # denoising steps (warm-start sequence)
    drift: float = 0.05        # relative per-step drift of the sequence
    warm_iters: int = 2

    @property
    def bh(self) -> int:
        return self.batch * self.heads

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


CONFIGS = {
    "tiny": LayerConfig("tiny", 1, 1, 4096, 64, "f32", 48, "uniform", "iid", None,
                        "mixture", 32, 64, 5, (0.9,), 0),
    "small": LayerConfig("small", 1, 4, 16384, 128, "bf16", 200, "uniform", "voronoi",
                         (8, 32, 64), "normal", 100, 250, 5, (0.9,), 1),
    "wan720p": LayerConfig("wan720p", 1, 40, 75600, 128, "bf16", 600, "zipf", "voronoi",
                           (21, 45, 80), "normal", 400, 1000, 5, (0.8, 0.9, 0.95), 2),
    "hunyuan720p": LayerConfig("hunyuan720p", 1, 24, 118800, 128, "bf16", 800, "zipf",
                               "voronoi", (33, 45, 80), "normal", 400, 1000, 5, (None,), 3),
    "denoise": LayerConfig("denoise", 1, 24, 118800, 128, "bf16", 800, "zipf", "voronoi",
                           (33, 45, 80), "normal", 400, 1000, 5, (None,), 4, steps=10),
}


def _rng(cfg: LayerConfig, head: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cfg.seed, head, stream]))


def _component_weights(cfg: LayerConfig) -> np.ndarray:
    if cfg.weights == "uniform":
        w = np.ones(cfg.n_centers)
    else:
        w = (np.arange(cfg.n_centers) + 1.0) ** (-cfg.zipf_alpha)
    return w / w.sum()


def _labels(cfg: LayerConfig, head: int) -> np.ndarray:
    """Component label of every token of one head (raster order on the grid)."""
    rng = _rng(cfg, head, _S_FIELD)
    w = _component_weights(cfg)
    if cfg.field == "iid":
        return rng.choice(cfg.n_centers, size=cfg.n_tokens, p=w)
    from scipy.spatial import cKDTree
    f, hh, ww = cfg.grid
    assert f * hh * ww == cfg.n_tokens
    n_sites = 2 * cfg.n_centers
    sites = rng.uniform(0.0, 1.0, size=(n_sites, 3)) * np.array([f, hh, ww], dtype=np.float64)
    site_label = rng.choice(cfg.n_centers, size=n_sites, p=w)
    tt, yy, xx = np.meshgrid(np.arange(f), np.arange(hh), np.arange(ww), indexing="ij")
    pts = np.stack([tt.ravel(), yy.ravel(), xx.ravel()], axis=1).astype(np.float64)
    _, nearest = cKDTree(sites).query(pts, k=1)
    lab = site_label[nearest]
    flip = rng.random(cfg.n_tokens) < cfg.relabel
    lab[flip] = rng.choice(cfg.n_centers, size=int(flip.sum()), p=w)
    return lab


def head_master(cfg: LayerConfig, head: int):
    """fp64 master (q, k, v, labels) of one head, before rounding."""
    centers = _rng(cfg, head, _S_CENTERS).standard_normal((cfg.n_centers, cfg.head_dim))
    lab = _labels(cfg, head)
    mu = centers[lab]
    q = mu + cfg.noise * _rng(cfg, head, _S_Q).standard_normal(mu.shape)
    k = mu + cfg.noise * _rng(cfg, head, _S_K).standard_normal(mu.shape)
    if cfg.v_kind == "mixture":
        v = mu + cfg.noise * _rng(cfg, head, _S_V).standard_normal(mu.shape)
    else:
        v = _rng(cfg, head, _S_V).standard_normal(mu.shape)
    return q, k, v, lab


def drift_step(cfg: LayerConfig, head: int, step: int, x: np.ndarray, which: int) -> np.ndarray:
    """One denoising step of drift on an fp64 master: x + drift * rms(x) * eps."""
    rng = np.random.default_rng(np.random.SeedSequence([cfg.seed, head, _S_DRIFT, step, which]))
    rms = float(np.sqrt(np.mean(x * x)))
    return x + cfg.drift * rms * rng.standard_normal(x.shape)


def _round(a: np.ndarray, dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype)


def make_layer(cfg, heads: Optional[Sequence[int]] = None, step: int = 0):
    """Rounded inputs of one layer: dict(q, k, v, labels).

    q, k, v are CPU tensors ``[len(heads), N, d]`` in the config dtype
    (contiguous, batch folded into heads); ``labels`` is int64 ``[len(heads), N]``
    (the generator's component labels, for diagnostics only).  ``step > 0``
    applies ``step`` drift steps of the denoising sequence to the fp64 masters.
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    if heads is None:
        heads = range(cfg.bh)
    heads = list(heads)
    dt = cfg.torch_dtype
    qs, ks, vs, ls = [], [], [], []
    for h in heads:
        q, k, v, lab = head_master(cfg, h)
        for s in range(1, step + 1):
            q = drift_step(cfg, h, s, q, 0)
            k = drift_step(cfg, h, s, k, 1)
            v = drift_step(cfg, h, s, v, 2)
        qs.append(_round(q, dt))
        ks.append(_round(k, dt))
        vs.append(_round(v, dt))
        ls.append(torch.from_numpy(lab.astype(np.int64)))
    return dict(q=torch.stack(qs), k=torch.stack(ks), v=torch.stack(vs),
                labels=torch.stack(ls), cfg=cfg, heads=heads)


def _head_sequence(args):
    """Rounded (q, k, v) of one head for steps 0..steps-1 (fp64 masters kept)."""
    cfg, h, steps = args
    q, k, v, lab = head_master(cfg, h)
    m = [q, k, v]
    out = []
    for s in range(steps):
        if s > 0:
            for which in range(3):
                m[which] = drift_step(cfg, h, s, m[which], which)
        out.append(tuple(_round(x, cfg.torch_dtype) for x in m))
    return out, torch.from_numpy(lab.astype(np.int64))


def denoise_sequence(cfg, heads: Optional[Sequence[int]] = None, steps: Optional[int] = None,
                     workers: int = 0):
    """The denoising sequence step by step: yields ``make_layer(cfg, heads, s)``
    for s = 0, 1, ..., steps - 1 (default ``cfg.steps``), keeping the fp64
    masters between steps so that each step costs one drift pass.  With
    ``workers > 0`` the heads are generated in that many processes (the whole
    sequence is then produced before the first step is yielded)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    if heads is None:
        heads = range(cfg.bh)
    heads = list(heads)
    steps = cfg.steps if steps is None else steps
    if workers > 0:
        import multiprocessing
        from concurrent.futures import ProcessPoolExecutor
        # fresh interpreters: a forked copy of a process that already ran torch
        # can deadlock on its thread pools
        ctx = multiprocessing.get_context("spawn")
        with ProcessPoolExecutor(max_workers=min(workers, len(heads)), mp_context=ctx) as ex:
            per_head = list(ex.map(_head_sequence, [(cfg, h, steps) for h in heads]))
        for s in range(steps):
            yield dict(q=torch.stack([ph[0][s][0] for ph in per_head]),
                       k=torch.stack([ph[0][s][1] for ph in per_head]),
                       v=torch.stack([ph[0][s][2] for ph in per_head]),
                       labels=torch.stack([ph[1] for ph in per_head]), cfg=cfg, heads=heads, step=s)
        return
    dt = cfg.torch_dtype
    masters = [list(head_master(cfg, h)) for h in heads]
    for s in range(steps):
        if s > 0:
            for h, m in zip(heads, masters):
                for which in range(3):
                    m[which] = drift_step(cfg, h, s, m[which], which)
        yield dict(q=torch.stack([_round(m[0], dt) for m in masters]),
                   k=torch.stack([_round(m[1], dt) for m in masters]),
                   v=torch.stack([_round(m[2], dt) for m in masters]),
                   labels=torch.stack([torch.from_numpy(m[3].astype(np.int64)) for m in masters]),
                   cfg=cfg, heads=heads, step=s)


def uniform_rows(n_rows: int, n_cols: int, seed: int, dtype=torch.float32) -> torch.Tensor:
    """Plain N(0,1) matrix, used for data-movement tests (permute / unpermute)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0, 99]))
    return _round(rng.standard_normal((n_rows, n_cols)), dtype)


def random_labels(n: int, n_clusters: int, seed: int, skew: float = 0.0) -> np.ndarray:
    """Cluster labels in [0, n_clusters); skew > 0 makes sizes Zipf-like and leaves
    some clusters empty."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 1, 98]))
    if skew <= 0:
        return rng.integers(0, n_clusters, size=n).astype(np.int32)
    w = (np.arange(n_clusters) + 1.0) ** (-skew)
    w = w / w.sum()
    perm = rng.permutation(n_clusters)
    return perm[rng.choice(n_clusters, size=n, p=w)].astype(np.int32)


def gaussian_centroids(n: int, d: int, seed: int, spread: float = 1.0) -> np.ndarray:
    """fp32-valued centroid sets for stand-alone selection / assignment tests."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 2, 97]))
    return (spread * rng.standard_normal((n, d))).astype(np.float32)
