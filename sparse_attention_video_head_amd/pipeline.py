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


def _problem_parts(bh: int, split: bool):
    """Problem ranges [lo, hi) run as separate calls: [0, s) and [s, bh) with s
    the largest power of two below bh, so that every range starts at 0 or at a
    power of two at least as large as the range (see _part_seed)."""
    if not split or bh < 2:
        return [(0, bh)]
    s = 1 << ((bh - 1).bit_length() - 1)
    return [(0, s), (s, bh)]


def _part_seed(seed: int, lo: int) -> int:
    """The seed under which problem i of a call on problems [lo, hi) draws the
    k-means++ numbers that problem lo + i of one call on every problem draws:
    the generator's state is seed XOR (problem * 2^32 + pick), and with lo a
    power of two larger than every i (or 0), lo XOR i = lo + i."""
    return (seed ^ (lo << 32)) & ((1 << 64) - 1)


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
        # k-means runs per side in problem ranges, each on a stream of its own:
        # the dependent launches of one range (two per k-means++ pick) leave
        # gaps that the other ranges' launches fill
        self.parts = _problem_parts(bh, two_streams)
        self.ws_kq = [u8(L.svg2_kmeans_workspace_size(hi - lo, n_tokens, head_dim, n_q)) for lo, hi in self.parts]
        self.ws_kk = [u8(L.svg2_kmeans_workspace_size(hi - lo, n_tokens, head_dim, n_k)) for lo, hi in self.parts]
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
        self.streams = [torch.cuda.Stream(device=dev) for _ in range(2 * len(self.parts) - 1)] if two_streams else []
        # FP8 attention: E4M3 copies of Q', K', V' with per-problem scales
        self.fp8 = fp8_attention
        if fp8_attention:
            if dtype != torch.bfloat16 or head_dim != 128:
                raise ValueError("FP8 attention takes bf16 inputs with head_dim 128")
            self.q8, self.k8, self.v8 = (e(bh, n_tokens, head_dim, dt=torch.uint8) for _ in range(3))
            self.s8 = e(3, bh, dt=torch.float32)
            self.ws_q8 = u8(L.svg2_quantize_fp8_workspace_size(bh))

    # ------------------------------------------------------------ steps
    def _run_parts(self, jobs):
        """Runs the callables on the current stream and the side streams, one
        each, after the work queued so far; the current stream waits for all."""
        if not self.streams:
            for job in jobs:
                job()
            return
        main = torch.cuda.current_stream(self.dev)
        for st, job in zip(self.streams, jobs[1:]):
            st.wait_stream(main)
            with torch.cuda.stream(st):
                job()
        jobs[0]()
        for st in self.streams[:len(jobs) - 1]:
            main.wait_stream(st)

    def kmeans(self, q, k, iters: int, warm: bool, seed_q: int, seed_k: int):
        jobs = []
        for side, x, n, c, lab, cnt, ws, seed in (("k", k, self.n_k, self.ck, self.labels_k, self.counts_k,
                                                   self.ws_kk, seed_k),
                                                  ("q", q, self.n_q, self.cq, self.labels_q, self.counts_q,
                                                   self.ws_kq, seed_q)):
            for (lo, hi), w in zip(self.parts, ws):
                def job(x=x, n=n, c=c, lab=lab, cnt=cnt, w=w, seed=seed, lo=lo, hi=hi):
                    B.kmeans(x[lo:hi], n, iters, init=c[lo:hi] if warm else None, seed=_part_seed(seed, lo),
                             centroids=c[lo:hi], labels=lab[lo:hi], counts=cnt[lo:hi], workspace=w)
                jobs.append(job)
        self._run_parts(jobs)

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
        jobs = []
        for (lo, hi), w in zip(self.parts, self.ws_kk):
            def job_k(lo=lo, hi=hi, w=w):
                r = slice(lo, hi)
                B.kmeans_permute(k[r], self.n_k, iters, y=v[r], init=self.ck[r] if warm else None,
                                 seed=_part_seed(seed_k, lo), centroids=self.ck[r], labels=self.labels_k[r],
                                 counts=self.counts_k[r], x_out=ko[r], y_out=vo[r], perm=self.perm_k[r],
                                 offsets=self.off_k[r], workspace=w, fp8=f8, x_scale=sk[r] if f8 else None,
                                 y_scale=sv[r] if f8 else None)
            jobs.append(job_k)
        for (lo, hi), w in zip(self.parts, self.ws_kq):
            def job_q(lo=lo, hi=hi, w=w):
                r = slice(lo, hi)
                B.kmeans_permute(q[r], self.n_q, iters, init=self.cq[r] if warm else None,
                                 seed=_part_seed(seed_q, lo), centroids=self.cq[r], labels=self.labels_q[r],
                                 counts=self.counts_q[r], x_out=qo[r], perm=self.perm_q[r], offsets=self.off_q[r],
                                 workspace=w, fp8=f8, x_scale=sq[r] if f8 else None)
            jobs.append(job_q)
        self._run_parts(jobs)

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
