"""One SVG2 sparse-attention layer on the GPU: the five library calls chained
("Sparse VideoGen2" wiki summary, Method, stages (1)-(4)):

    k-means(Q), k-means(K)  ->  permute Q by P_Q, K and V by P_K
    (the permutation rides on the last Lloyd round's centroid update)
    ->  centroid scores + top-p  ->  variable-block attention  ->  un-permute

Buffers (outputs and workspaces) are allocated once per shape, so repeated
calls launch kernels only.  The Q side's k-means and permutation may run on a
second stream, beside the K side's.  The centroid cache of the method is the ``centroids_q`` /
``centroids_k`` state: ``run(..., warm=True)`` warm-starts from it.
"""
from __future__ import annotations

import math
from typing import Optional

import torch

from . import binding as B


class SVG2Layer:
    def __init__(self, bh: int, n_tokens: int, head_dim: int, dtype: torch.dtype, n_q: int, n_k: int,
                 device="cuda", two_streams: bool = True, fp8_attention: bool = False):
        self.bh, self.N, self.d, self.dtype = bh, n_tokens, head_dim, dtype
        self.n_q, self.n_k = n_q, n_k
        self.scale = 1.0 / math.sqrt(head_dim)
        dev = torch.device(device)
        self.dev = dev
        L = B.lib()
        e = lambda *s, dt=torch.int32: torch.empty(*s, dtype=dt, device=dev)
        self.cq = e(bh, n_q, head_dim, dt=torch.float32)
        self.ck = e(bh, n_k, head_dim, dt=torch.float32)
        self.labels_q, self.labels_k = e(bh, n_tokens), e(bh, n_tokens)
        self.counts_q, self.counts_k = e(bh, n_q), e(bh, n_k)
        self.qp = e(bh, n_tokens, head_dim, dt=dtype)
        self.kp = e(bh, n_tokens, head_dim, dt=dtype)
        self.vp = e(bh, n_tokens, head_dim, dt=dtype)
        self.op = e(bh, n_tokens, head_dim, dt=dtype)
        self.out = e(bh, n_tokens, head_dim, dt=dtype)
        self.perm_q, self.perm_k = e(bh, n_tokens), e(bh, n_tokens)
        self.off_q, self.off_k = e(bh, n_q + 1), e(bh, n_k + 1)
        self.sel_count, self.sel_idx = e(bh, n_q), e(bh, n_q, n_k)
        self.pairs = e(bh, dt=torch.int64)
        u8 = lambda n: torch.empty(max(int(n), 1), dtype=torch.uint8, device=dev)
        self.ws_kq = u8(L.svg2_kmeans_workspace_size(bh, n_tokens, head_dim, n_q))
        self.ws_kk = u8(L.svg2_kmeans_workspace_size(bh, n_tokens, head_dim, n_k))
        self.ws_pq = u8(L.svg2_permute_workspace_size(bh, n_tokens, n_q))
        self.ws_pk = u8(L.svg2_permute_workspace_size(bh, n_tokens, n_k))
        self.ws_sel = u8(L.svg2_select_topp_workspace_size(bh, n_q, n_k))
        self.ws_attn = u8(L.svg2_varblock_attn_workspace_size(bh, n_tokens, n_q, n_k, head_dim))
        # dense baseline: one cluster holding every token, selecting itself
        self.dense_off = torch.tensor([0, n_tokens], dtype=torch.int32, device=dev).repeat(bh, 1).contiguous()
        self.dense_cnt = torch.ones(bh, 1, dtype=torch.int32, device=dev)
        self.dense_sel = torch.zeros(bh, 1, 1, dtype=torch.int32, device=dev)
        self.ws_dense = u8(L.svg2_varblock_attn_workspace_size(bh, n_tokens, 1, 1, head_dim))
        self.side = torch.cuda.Stream(device=dev) if two_streams else None
        # FP8 attention: E4M3 copies of Q', K', V' with per-problem scales
        self.fp8 = fp8_attention
        if fp8_attention:
            if dtype != torch.bfloat16 or head_dim != 128:
                raise ValueError("FP8 attention takes bf16 inputs with head_dim 128")
            self.q8, self.k8, self.v8 = (e(bh, n_tokens, head_dim, dt=torch.uint8) for _ in range(3))
            self.s8 = e(3, bh, dt=torch.float32)
            self.ws_q8 = u8(L.svg2_quantize_fp8_workspace_size(bh))

    # ------------------------------------------------------------ steps
    def kmeans(self, q, k, iters: int, warm: bool, seed_q: int, seed_k: int):
        def side_q():
            B.kmeans(q, self.n_q, iters, init=self.cq if warm else None, seed=seed_q, centroids=self.cq,
                     labels=self.labels_q, counts=self.counts_q, workspace=self.ws_kq)

        def side_k():
            B.kmeans(k, self.n_k, iters, init=self.ck if warm else None, seed=seed_k, centroids=self.ck,
                     labels=self.labels_k, counts=self.counts_k, workspace=self.ws_kk)

        if self.side is None:
            side_q()
            side_k()
            return
        main = torch.cuda.current_stream(self.dev)
        self.side.wait_stream(main)
        with torch.cuda.stream(self.side):
            side_k()
        side_q()
        main.wait_stream(self.side)

    def permute(self, q, k, v, quantize: bool = True):
        def side_q():
            B.permute(self.labels_q, self.n_q, q, outs=[self.qp], perm=self.perm_q, offsets=self.off_q,
                      workspace=self.ws_pq)

        def side_k():
            B.permute(self.labels_k, self.n_k, k, v, outs=[self.kp, self.vp], perm=self.perm_k,
                      offsets=self.off_k, workspace=self.ws_pk)

        if self.side is None:
            side_q()
            side_k()
        else:
            # the Q side on the second stream: its small sort kernels overlap the K/V row moves
            main = torch.cuda.current_stream(self.dev)
            self.side.wait_stream(main)
            with torch.cuda.stream(self.side):
                side_q()
            side_k()
            main.wait_stream(self.side)
        if self.fp8 and quantize:
            self.quantize()

    def cluster(self, q, k, v, iters: int, warm: bool, seed_q: int, seed_k: int):
        """k-means of Q and K with the permutation fused into the last Lloyd
        round: Q' from Q's clusters, K' and V' from K's."""
        if iters < 1:
            self.kmeans(q, k, iters, warm, seed_q, seed_k)
            self.permute(q, k, v)
            return

        # FP8 attention: the moved rows are stored as E4M3 directly
        f8 = self.fp8
        qo, ko, vo = (self.q8, self.k8, self.v8) if f8 else (self.qp, self.kp, self.vp)
        sq, sk, sv = (self.s8[0], self.s8[1], self.s8[2]) if f8 else (None, None, None)

        def side_q():
            B.kmeans_permute(q, self.n_q, iters, init=self.cq if warm else None, seed=seed_q, centroids=self.cq,
                             labels=self.labels_q, counts=self.counts_q, x_out=qo, perm=self.perm_q,
                             offsets=self.off_q, workspace=self.ws_kq, fp8=f8, x_scale=sq)

        def side_k():
            B.kmeans_permute(k, self.n_k, iters, y=v, init=self.ck if warm else None, seed=seed_k,
                             centroids=self.ck, labels=self.labels_k, counts=self.counts_k, x_out=ko,
                             y_out=vo, perm=self.perm_k, offsets=self.off_k, workspace=self.ws_kk, fp8=f8,
                             x_scale=sk, y_scale=sv)

        if self.side is None:
            side_q()
            side_k()
            return
        main = torch.cuda.current_stream(self.dev)
        self.side.wait_stream(main)
        with torch.cuda.stream(self.side):
            side_k()
        side_q()
        main.wait_stream(self.side)

    def select(self, top_p: float):
        B.select_topp(self.cq, self.counts_q, self.ck, self.counts_k, top_p, scale=self.scale,
                      sel_count=self.sel_count, sel_idx=self.sel_idx, pair_count=self.pairs,
                      workspace=self.ws_sel)

    def quantize(self):
        """E4M3 copies of Q', K', V' with per-problem scales (FP8 attention;
        ``cluster`` writes them directly, ``permute`` calls this)."""
        for x, x8, sc in ((self.qp, self.q8, self.s8[0]), (self.kp, self.k8, self.s8[1]),
                          (self.vp, self.v8, self.s8[2])):
            B.quantize_fp8(x, x8, sc, workspace=self.ws_q8)

    def attend(self):
        if self.fp8:
            B.varblock_attn_fp8(self.q8, self.k8, self.v8, self.s8[0], self.s8[1], self.s8[2], self.off_q,
                                self.off_k, self.sel_count, self.sel_idx, scale=self.scale, out=self.op,
                                workspace=self.ws_attn)
            return
        B.varblock_attn(self.qp, self.kp, self.vp, self.off_q, self.off_k, self.sel_count, self.sel_idx,
                        scale=self.scale, out=self.op, workspace=self.ws_attn)

    def unpermute(self, out: Optional[torch.Tensor] = None):
        return B.unpermute(self.op, self.perm_q, out=self.out if out is None else out)

    def attend_unpermute(self, out: Optional[torch.Tensor] = None):
        """Attention with the inverse permutation fused into its stores (one
        pass less over the output)."""
        dst = self.out if out is None else out
        if self.fp8:
            B.varblock_attn_fp8_unpermute(self.q8, self.k8, self.v8, self.s8[0], self.s8[1], self.s8[2],
                                          self.off_q, self.off_k, self.sel_count, self.sel_idx, self.perm_q,
                                          scale=self.scale, out=dst, workspace=self.ws_attn)
            return dst
        B.varblock_attn_unpermute(self.qp, self.kp, self.vp, self.off_q, self.off_k, self.sel_count, self.sel_idx,
                                  self.perm_q, scale=self.scale, out=dst, workspace=self.ws_attn)
        return dst

    # ------------------------------------------------------------ layer
    def run(self, q, k, v, top_p: float, iters: int = 5, warm: bool = False, seed_q: int = 0,
            seed_k: int = 1, out: Optional[torch.Tensor] = None):
        """Whole layer; returns the output in the original token order."""
        self.cluster(q, k, v, iters, warm, seed_q, seed_k)
        self.select(top_p)
        return self.attend_unpermute(out)

    def dense(self, q, k, v, out: Optional[torch.Tensor] = None):
        """This library's own dense attention (one block, every key selected)."""
        o = out if out is not None else torch.empty_like(q)
        B.varblock_attn(q, k, v, self.dense_off, self.dense_off, self.dense_cnt, self.dense_sel,
                        scale=self.scale, out=o, workspace=self.ws_dense)
        return o

    def density(self) -> float:
        return float(self.pairs.sum().item()) / (self.bh * float(self.N) ** 2)
