"""Identification accuracy of critical tokens, beside the path ("Sparse
VideoGen2" wiki summary, Key claims, §3.1 / Fig. 3; §3.2, Figs. 3-4; §5.3).

For a selection, the recall of a query row is the share of its exact softmax
mass that falls on the keys the selection gives it, exp(lse_sel - lse_all).
Two ways to form the blocks that the same centroid estimate and top-p then
select are compared at matched density:

* **semantic**: k-means clusters of Q and of K, permuted into contiguous
  blocks (the method's own path);
* **positional**: fixed blocks of ``block`` consecutive tokens in the original
  order, each represented by the mean of its rows (the prior methods' block
  representation).

Every step runs in the library: k-means, permutation, cluster means, top-p,
attention with its log-sum-exp, and the recall reduction.  Q, K, V are
``[bh, N, d]`` contiguous device tensors.
"""
from __future__ import annotations

import math
from typing import List, Sequence

import torch

from . import binding as B
from .pipeline import SVG2Layer


class IdentificationStudy:
    def __init__(self, bh: int, n_tokens: int, head_dim: int, dtype: torch.dtype, n_q: int, n_k: int,
                 block: int = 128, device="cuda"):
        self.bh, self.N, self.d, self.block = bh, n_tokens, head_dim, block
        self.layer = SVG2Layer(bh, n_tokens, head_dim, dtype, n_q, n_k, device=device)
        dev = self.layer.dev
        nb = (n_tokens + block - 1) // block
        self.n_blocks = nb
        i32 = lambda *s: torch.empty(*s, dtype=torch.int32, device=dev)
        self.block_labels = (torch.arange(n_tokens, device=dev, dtype=torch.int32) // block).repeat(bh, 1).contiguous()
        off = torch.clamp(torch.arange(nb + 1, device=dev, dtype=torch.int32) * block, max=n_tokens)
        self.block_off = off.repeat(bh, 1).contiguous()
        self.cq_b = torch.zeros(bh, nb, head_dim, dtype=torch.float32, device=dev)
        self.ck_b = torch.zeros_like(self.cq_b)
        self.nq_b, self.nk_b = i32(bh, nb), i32(bh, nb)
        self.sel_count_b, self.sel_idx_b = i32(bh, nb), i32(bh, nb, nb)
        self.pairs_b = torch.empty(bh, dtype=torch.int64, device=dev)
        self.lse_all = torch.empty(bh, n_tokens, dtype=torch.float32, device=dev)
        self.lse_sel = torch.empty_like(self.lse_all)
        self.o = torch.empty(bh, n_tokens, head_dim, dtype=dtype, device=dev)
        self.scale = 1.0 / math.sqrt(head_dim)
        lib = B.lib()
        u8 = lambda n: torch.empty(max(int(n), 1), dtype=torch.uint8, device=dev)
        self.ws_sel_b = u8(lib.svg2_select_topp_workspace_size(bh, nb, nb))
        self.ws_attn_b = u8(lib.svg2_varblock_attn_workspace_size(bh, n_tokens, nb, nb, head_dim))

    def _dense_lse(self, q, k, v):
        L = self.layer
        B.varblock_attn(q, k, v, L.dense_off, L.dense_off, L.dense_cnt, L.dense_sel, scale=self.scale,
                        out=self.o, workspace=L.ws_dense, lse=self.lse_all)

    def semantic(self, q, k, v, top_ps: Sequence[float], iters: int = 5, seed_q: int = 0,
                 seed_k: int = 1) -> List[dict]:
        """Cold k-means of Q and K, then per p: density and mean recall per problem."""
        L = self.layer
        L.kmeans(q, k, iters, False, seed_q, seed_k)
        L.permute(q, k, v)
        self._dense_lse(L.qp, L.kp, L.vp)
        out = []
        for p in top_ps:
            L.select(p)
            B.varblock_attn(L.qp, L.kp, L.vp, L.off_q, L.off_k, L.sel_count, L.sel_idx, scale=self.scale,
                            out=self.o, workspace=L.ws_attn, lse=self.lse_sel)
            rec = B.recall_mass(self.lse_sel, self.lse_all)
            out.append({"top_p": float(p), "pairs": L.pairs.clone(), "recall": rec})
        return out

    def positional(self, q, k, v, top_ps: Sequence[float]) -> List[dict]:
        """Fixed blocks with mean-pooled representatives, then per p as above."""
        L = self.layer
        B.cluster_means(q, self.block_labels, self.n_blocks, means=self.cq_b, counts=self.nq_b)
        B.cluster_means(k, self.block_labels, self.n_blocks, means=self.ck_b, counts=self.nk_b)
        self._dense_lse(q, k, v)
        out = []
        for p in top_ps:
            B.select_topp(self.cq_b, self.nq_b, self.ck_b, self.nk_b, p, scale=self.scale,
                          sel_count=self.sel_count_b, sel_idx=self.sel_idx_b, pair_count=self.pairs_b,
                          workspace=self.ws_sel_b)
            B.varblock_attn(q, k, v, self.block_off, self.block_off, self.sel_count_b, self.sel_idx_b,
                            scale=self.scale, out=self.o, workspace=self.ws_attn_b, lse=self.lse_sel)
            rec = B.recall_mass(self.lse_sel, self.lse_all)
            out.append({"top_p": float(p), "pairs": self.pairs_b.clone(), "recall": rec})
        return out
