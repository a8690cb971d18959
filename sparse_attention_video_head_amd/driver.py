"""SVG2 attention along a denoising run ("Sparse VideoGen2" wiki summary,
Method, stage (1) and the dense warm-up paragraph; Key claims, §4.3 / Fig. 7(a)).

Around the per-layer path the method keeps three pieces of state and policy:

* **Dense warm-up.**  The first ~10% of the denoising steps run plain dense
  attention; sparse attention hurts most early in the trajectory.  Here the
  leading ``ceil(dense_fraction * steps)`` steps are dense.
* **Centroid cache.**  Each (layer, head, side) keeps its final fp32 centroids.
  A layer's first sparse step clusters cold (k-means++ then ``cold_iters``
  Lloyd rounds); every later step warm-starts from the cached centroids with
  ``warm_iters`` rounds, and the cache takes the new centroids.
* **Top-p schedule.**  ``top_p`` is one value for every step or a callable
  ``step -> p``.

One :class:`SVG2Layer` holds the per-call buffers (permuted Q/K/V, output,
workspaces) and is shared by every layer; only the centroid caches are per
layer (``bh * (n_q + n_k) * head_dim * 4`` bytes each).  Dense steps use the
library's own attention with every key selected.  Q, K, V are ``[bh, N, d]``
contiguous device tensors.
"""
from __future__ import annotations

import math
from typing import Callable, Dict, Optional, Tuple, Union

import torch

from .pipeline import SVG2Layer


def dense_steps(steps: int, dense_fraction: float) -> int:
    """Number of leading dense steps: the first ``dense_fraction`` of ``steps``,
    rounded up (a guard keeps 0.1 * 50 = 5 from rounding to 6)."""
    if steps <= 0 or dense_fraction <= 0.0:
        return 0
    return min(steps, int(math.ceil(dense_fraction * steps - 1e-9)))


class DenoiseDriver:
    def __init__(self, bh: int, n_tokens: int, head_dim: int, dtype: torch.dtype, n_q: int, n_k: int,
                 steps: int, top_p: Union[float, Callable[[int], float]] = 0.9, dense_fraction: float = 0.1,
                 cold_iters: int = 5, warm_iters: int = 2, seed: int = 0, device="cuda",
                 two_streams: bool = True):
        if steps < 1:
            raise ValueError("steps must be >= 1")
        if cold_iters < 1 or warm_iters < 1:
            raise ValueError("cold_iters and warm_iters must be >= 1 (the permutation needs the labels "
                             "of a Lloyd round)")
        self.steps, self.n_dense = steps, dense_steps(steps, dense_fraction)
        self.top_p = top_p
        self.cold_iters, self.warm_iters, self.seed = cold_iters, warm_iters, seed
        self.engine = SVG2Layer(bh, n_tokens, head_dim, dtype, n_q, n_k, device=device, two_streams=two_streams)
        self.cache: Dict[int, Tuple[torch.Tensor, torch.Tensor]] = {}
        self.last_mode: Optional[str] = None

    def p_at(self, step: int) -> float:
        return float(self.top_p(step)) if callable(self.top_p) else float(self.top_p)

    def seeds(self, layer: int) -> Tuple[int, int]:
        """k-means++ seeds of a layer's cold start, one per side."""
        base = (self.seed << 16) | (layer << 1)
        return base, base | 1

    def mode(self, layer: int, step: int) -> str:
        if step < self.n_dense:
            return "dense"
        return "warm" if layer in self.cache else "cold"

    def __call__(self, layer: int, step: int, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """Attention of ``layer`` at denoising ``step``; returns ``[bh, N, d]`` in
        the input's token order: ``out`` if given, else the engine's output
        buffer, which the next call overwrites."""
        if not 0 <= step < self.steps:
            raise ValueError(f"step {step} outside [0, {self.steps})")
        e = self.engine
        mode = self.mode(layer, step)
        self.last_mode = mode
        if mode == "dense":
            return e.dense(q, k, v, out=e.out if out is None else out)
        if mode == "cold":
            cq = torch.empty_like(e.cq)
            ck = torch.empty_like(e.ck)
            self.cache[layer] = (cq, ck)
        # the engine's centroid buffers are this layer's cache
        e.cq, e.ck = self.cache[layer]
        seed_q, seed_k = self.seeds(layer)
        iters = self.cold_iters if mode == "cold" else self.warm_iters
        e.cluster(q, k, v, iters, mode == "warm", seed_q, seed_k)
        e.select(self.p_at(step))
        return e.attend_unpermute(out)

    def reset(self):
        """Forget every cached centroid (a new generation starts cold)."""
        self.cache.clear()
