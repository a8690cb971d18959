"""Python binding of libsvg2 (ctypes).

Argument marshalling only: these wrappers check shapes and dtypes, allocate
outputs and workspace with torch on the tensors' device, and pass raw device
pointers plus torch's current HIP stream to the C ABI declared in
include/svg2.h.  Every step of the computation runs in the library's HIP
kernels; nothing here computes, and there is no fallback: without the built
library every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

import torch

# SVG2_LIBRARY points the binding at another build of the same library (the
# host-sanitizer build of the CPU tests); by default the in-tree one.
_LIB_PATH = os.environ.get("SVG2_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsvg2.so")
_lib = None

F32, BF16 = 0, 1
_c_int, _c_i64, _c_u64, _c_sz, _c_p = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_size_t, ctypes.c_void_p

EXPORTED = [
    "svg2_version", "svg2_status_string", "svg2_last_hip_error",
    "svg2_kmeans_workspace_size", "svg2_kmeans", "svg2_kmeans_permute", "svg2_kmeans_permute_fp8",
    "svg2_permute_workspace_size", "svg2_permute",
    "svg2_select_topp_workspace_size", "svg2_select_topp",
    "svg2_varblock_attn_workspace_size", "svg2_varblock_attn", "svg2_varblock_attn_unpermute",
    "svg2_unpermute",
    "svg2_cluster_means_workspace_size", "svg2_cluster_means", "svg2_recall_mass",
    "svg2_quantize_fp8_workspace_size", "svg2_quantize_fp8", "svg2_varblock_attn_fp8",
    "svg2_varblock_attn_fp8_unpermute",
    "svg2_varblock_attn_noalloc_max_scratch", "svg2_varblock_attn_noalloc",
]


class Svg2Error(RuntimeError):
    pass


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """Loads libsvg2.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise Svg2Error(f"{_LIB_PATH} is missing: build it with "
                        "`python -m sparse_attention_video_head_amd.build`")
    L = ctypes.CDLL(_LIB_PATH)
    L.svg2_version.restype = ctypes.c_char_p
    L.svg2_status_string.restype = ctypes.c_char_p
    L.svg2_status_string.argtypes = [ctypes.c_int]
    L.svg2_last_hip_error.restype = ctypes.c_int
    L.svg2_kmeans_workspace_size.restype = _c_sz
    L.svg2_kmeans_workspace_size.argtypes = [_c_int] * 4
    L.svg2_kmeans.restype = ctypes.c_int
    L.svg2_kmeans.argtypes = [_c_p, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_p, _c_u64,
                              _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_sz, _c_p]
    L.svg2_kmeans_permute.restype = ctypes.c_int
    L.svg2_kmeans_permute.argtypes = [_c_p, _c_p, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_p, _c_u64,
                                      _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_sz, _c_p]
    L.svg2_kmeans_permute_fp8.restype = ctypes.c_int
    L.svg2_kmeans_permute_fp8.argtypes = [_c_p, _c_p, _c_int, _c_int, _c_int, _c_int, _c_int, _c_p, _c_u64, _c_p,
                                          _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_sz, _c_p]
    L.svg2_permute_workspace_size.restype = _c_sz
    L.svg2_permute_workspace_size.argtypes = [_c_int] * 3
    L.svg2_permute.restype = ctypes.c_int
    L.svg2_permute.argtypes = [_c_p, _c_int, _c_int, _c_int, _c_int, _c_p, _c_int, _c_i64, _c_i64, _c_i64,
                               _c_p, _c_int, _c_int, _c_p, _c_p, _c_p, _c_sz, _c_p]
    L.svg2_select_topp_workspace_size.restype = _c_sz
    L.svg2_select_topp_workspace_size.argtypes = [_c_int] * 3
    L.svg2_select_topp.restype = ctypes.c_int
    L.svg2_select_topp.argtypes = [_c_p, _c_p, _c_int, _c_p, _c_p, _c_int, _c_int, _c_int, ctypes.c_float,
                                   ctypes.c_float, _c_p, _c_p, _c_p, _c_p, _c_p, _c_sz, _c_p]
    L.svg2_varblock_attn_workspace_size.restype = _c_sz
    L.svg2_varblock_attn_workspace_size.argtypes = [_c_int] * 5
    L.svg2_varblock_attn.restype = ctypes.c_int
    L.svg2_varblock_attn.argtypes = [_c_p, _c_p, _c_p, _c_int, _c_int, _c_int, _c_int, _c_p, _c_int, _c_p,
                                     _c_int, _c_p, _c_p, ctypes.c_float, _c_p, _c_p, _c_p, _c_sz, _c_p]
    L.svg2_varblock_attn_unpermute.restype = ctypes.c_int
    L.svg2_varblock_attn_unpermute.argtypes = [_c_p, _c_p, _c_p, _c_int, _c_int, _c_int, _c_int, _c_p, _c_int,
                                               _c_p, _c_int, _c_p, _c_p, ctypes.c_float, _c_p, _c_p, _c_int,
                                               _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_sz, _c_p]
    L.svg2_unpermute.restype = ctypes.c_int
    L.svg2_unpermute.argtypes = [_c_p, _c_int, _c_int, _c_int, _c_int, _c_p, _c_p, _c_int, _c_i64, _c_i64,
                                 _c_i64, _c_p]
    L.svg2_cluster_means_workspace_size.restype = _c_sz
    L.svg2_cluster_means_workspace_size.argtypes = [_c_int] * 4
    L.svg2_cluster_means.restype = ctypes.c_int
    L.svg2_cluster_means.argtypes = [_c_p, _c_int, _c_int, _c_int, _c_int, _c_p, _c_int, _c_p, _c_p, _c_p, _c_sz,
                                     _c_p]
    L.svg2_recall_mass.restype = ctypes.c_int
    L.svg2_recall_mass.argtypes = [_c_p, _c_p, _c_int, _c_int, _c_p, _c_p]
    L.svg2_quantize_fp8_workspace_size.restype = _c_sz
    L.svg2_quantize_fp8_workspace_size.argtypes = [_c_int]
    L.svg2_quantize_fp8.restype = ctypes.c_int
    L.svg2_quantize_fp8.argtypes = [_c_p, _c_int, _c_int, _c_int, _c_p, _c_p, _c_p, _c_sz, _c_p]
    L.svg2_varblock_attn_fp8.restype = ctypes.c_int
    L.svg2_varblock_attn_fp8.argtypes = [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_int, _c_int, _c_int, _c_p, _c_int,
                                         _c_p, _c_int, _c_p, _c_p, ctypes.c_float, _c_p, _c_p, _c_p, _c_sz, _c_p]
    L.svg2_varblock_attn_fp8_unpermute.restype = ctypes.c_int
    L.svg2_varblock_attn_fp8_unpermute.argtypes = [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_int, _c_int, _c_int, _c_p,
                                                   _c_int, _c_p, _c_int, _c_p, _c_p, ctypes.c_float, _c_p, _c_p,
                                                   _c_int, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_sz, _c_p]
    L.svg2_varblock_attn_noalloc_max_scratch.restype = _c_sz
    L.svg2_varblock_attn_noalloc_max_scratch.argtypes = []
    L.svg2_varblock_attn_noalloc.restype = ctypes.c_int
    L.svg2_varblock_attn_noalloc.argtypes = [_c_p, _c_p, _c_p, _c_int, _c_int, _c_int, _c_int, _c_p, _c_int, _c_p,
                                             _c_int, _c_p, _c_p, ctypes.c_float, _c_p, _c_p, _c_p]
    _lib = L
    return L


def version() -> str:
    return lib().svg2_version().decode()


def _check(status: int, what: str):
    if status != 0:
        L = lib()
        msg = L.svg2_status_string(status).decode()
        raise Svg2Error(f"{what}: {msg} (status {status}, hip error {L.svg2_last_hip_error()})")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise Svg2Error(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise Svg2Error("svg2 operates on GPU tensors only")


def _same_device(dev: torch.device, *ts):
    """Every given tensor lives on ``dev``, the device of the call's first
    input (which _need_cuda has already required to be a GPU)."""
    for t in ts:
        if t is not None and t.device != dev:
            raise Svg2Error(f"every tensor of one call must be on {dev} (got {t.device})")


def _need_out(t: Optional[torch.Tensor], shape, dtype: torch.dtype, dev: torch.device, what: str):
    """A caller-supplied output or in/out buffer: on ``dev``, of ``dtype``, of
    exactly ``shape`` and contiguous, since the kernels write through its raw
    pointer at that size."""
    if t is None:
        return
    _same_device(dev, t)
    if t.dtype != dtype:
        raise Svg2Error(f"{what} must be {dtype} (got {t.dtype})")
    if tuple(t.shape) != tuple(shape):
        raise Svg2Error(f"{what} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise Svg2Error(f"{what} must be contiguous")


def _workspace(nbytes: int, dev, workspace: Optional[torch.Tensor]):
    """The caller's workspace (on ``dev``, contiguous, at least ``nbytes``) or
    a new one when none is given."""
    if nbytes == 0:
        return None
    if workspace is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _same_device(dev, workspace)
    if not workspace.is_contiguous():
        raise Svg2Error("the workspace must be contiguous")
    if workspace.numel() * workspace.element_size() < nbytes:
        raise Svg2Error(f"the workspace holds {workspace.numel() * workspace.element_size()} bytes, "
                        f"{nbytes} are needed")
    return workspace


def _lists(bh: int, dev: torch.device, q_offsets, k_offsets, sel_count, sel_idx):
    """Checks the attention's cluster offsets and selection lists against bh
    problems; returns (n_q, n_k)."""
    for t, name in ((q_offsets, "q_offsets"), (k_offsets, "k_offsets")):
        if t.dim() != 2 or t.shape[0] != bh or t.shape[1] < 2:
            raise Svg2Error(f"{name} must be [bh, n + 1] with bh = {bh} and n >= 1")
    n_q = q_offsets.shape[1] - 1
    n_k = k_offsets.shape[1] - 1
    _need_out(q_offsets, (bh, n_q + 1), torch.int32, dev, "q_offsets")
    _need_out(k_offsets, (bh, n_k + 1), torch.int32, dev, "k_offsets")
    _need_out(sel_count, (bh, n_q), torch.int32, dev, "sel_count")
    _need_out(sel_idx, (bh, n_q, n_k), torch.int32, dev, "sel_idx")
    return n_q, n_k


def _lse_buffer(lse, bh: int, N: int, dev: torch.device):
    """``lse`` is a flag (allocate or not) or the caller's fp32 [bh, N] tensor."""
    if isinstance(lse, torch.Tensor):
        _need_out(lse, (bh, N), torch.float32, dev, "lse")
        return lse
    return torch.empty(bh, N, dtype=torch.float32, device=dev) if lse else None


# ---------------------------------------------------------------- kmeans
def kmeans(x: torch.Tensor, n_clusters: int, n_iters: int, init: Optional[torch.Tensor] = None,
           seed: int = 0, min_dist: bool = False, seed_index: bool = False,
           centroids: Optional[torch.Tensor] = None, labels: Optional[torch.Tensor] = None,
           counts: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """k-means of x [bh, N, d] (contiguous).  Returns dict(centroids [bh,n,d] fp32,
    labels [bh,N] int32, counts [bh,n] int32, min_dist, seed_index)."""
    _need_cuda(x, init)
    if x.dim() != 3 or not x.is_contiguous():
        raise Svg2Error("x must be a contiguous [bh, N, d] tensor")
    bh, N, d = x.shape
    dev = x.device
    _need_out(init, (bh, n_clusters, d), torch.float32, dev, "init")
    _need_out(centroids, (bh, n_clusters, d), torch.float32, dev, "centroids")
    _need_out(labels, (bh, N), torch.int32, dev, "labels")
    _need_out(counts, (bh, n_clusters), torch.int32, dev, "counts")
    if centroids is None:
        centroids = torch.empty(bh, n_clusters, d, dtype=torch.float32, device=dev)
    if labels is None and n_iters > 0:
        labels = torch.empty(bh, N, dtype=torch.int32, device=dev)
    if counts is None and n_iters > 0:
        counts = torch.empty(bh, n_clusters, dtype=torch.int32, device=dev)
    md = torch.empty(bh, N, dtype=torch.float32, device=dev) if min_dist else None
    si = torch.empty(bh, n_clusters, dtype=torch.int32, device=dev) if seed_index else None
    L = lib()
    ws_n = L.svg2_kmeans_workspace_size(bh, N, d, n_clusters)
    ws = _workspace(ws_n, dev, workspace)
    st = L.svg2_kmeans(_ptr(x), _dtype_code(x), bh, N, d, n_clusters, n_iters, _ptr(init),
                       ctypes.c_uint64(seed & ((1 << 64) - 1)), _ptr(centroids), _ptr(labels),
                       _ptr(counts), _ptr(md), _ptr(si), _ptr(ws), ws_n, _stream(dev))
    _check(st, "svg2_kmeans")
    return dict(centroids=centroids, labels=labels, counts=counts, min_dist=md, seed_index=si)


def kmeans_permute(x: torch.Tensor, n_clusters: int, n_iters: int, y: Optional[torch.Tensor] = None,
                   init: Optional[torch.Tensor] = None, seed: int = 0, centroids: Optional[torch.Tensor] = None,
                   labels: Optional[torch.Tensor] = None, counts: Optional[torch.Tensor] = None,
                   x_out: Optional[torch.Tensor] = None, y_out: Optional[torch.Tensor] = None,
                   perm: Optional[torch.Tensor] = None, offsets: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None, fp8: bool = False,
                   x_scale: Optional[torch.Tensor] = None, y_scale: Optional[torch.Tensor] = None):
    """k-means of x [bh, N, d] (n_iters >= 1) with the rows of x, and of y when
    given, gathered into the final clusters' order in the last round.  With
    ``fp8`` (bf16 inputs) the gathered rows are E4M3 (uint8) with [bh] fp32
    scales, as quantize_fp8 of the bf16 rows.  Returns dict(centroids, labels,
    counts, x_perm, y_perm, perm, offsets, x_scale, y_scale)."""
    _need_cuda(x, y, init)
    if x.dim() != 3 or not x.is_contiguous():
        raise Svg2Error("x must be a contiguous [bh, N, d] tensor")
    bh, N, d = x.shape
    dev = x.device
    _need_out(y, x.shape, x.dtype, dev, "y")
    _need_out(init, (bh, n_clusters, d), torch.float32, dev, "init")
    _need_out(centroids, (bh, n_clusters, d), torch.float32, dev, "centroids")
    _need_out(labels, (bh, N), torch.int32, dev, "labels")
    _need_out(counts, (bh, n_clusters), torch.int32, dev, "counts")
    _need_out(perm, (bh, N), torch.int32, dev, "perm")
    _need_out(offsets, (bh, n_clusters + 1), torch.int32, dev, "offsets")
    e = lambda *sh, dt=torch.int32: torch.empty(*sh, dtype=dt, device=dev)
    centroids = e(bh, n_clusters, d, dt=torch.float32) if centroids is None else centroids
    labels = e(bh, N) if labels is None else labels
    counts = e(bh, n_clusters) if counts is None else counts
    if fp8 and x.dtype != torch.bfloat16:
        raise Svg2Error("E4M3 rows are made from bf16 inputs")
    odt = torch.uint8 if fp8 else x.dtype
    x_out = torch.empty(x.shape, dtype=odt, device=dev) if x_out is None else x_out
    if y is not None and y_out is None:
        y_out = torch.empty(x.shape, dtype=odt, device=dev)
    _need_out(x_out, x.shape, odt, dev, "x_out")
    _need_out(y_out, x.shape, odt, dev, "y_out")
    perm = e(bh, N) if perm is None else perm
    offsets = e(bh, n_clusters + 1) if offsets is None else offsets
    L = lib()
    ws_n = L.svg2_kmeans_workspace_size(bh, N, d, n_clusters)
    ws = _workspace(ws_n, dev, workspace)
    if fp8:
        x_scale = e(bh, dt=torch.float32) if x_scale is None else x_scale
        if y is not None and y_scale is None:
            y_scale = e(bh, dt=torch.float32)
        _need_out(x_scale, (bh,), torch.float32, dev, "x_scale")
        _need_out(y_scale, (bh,), torch.float32, dev, "y_scale")
        st = L.svg2_kmeans_permute_fp8(_ptr(x), _ptr(y), bh, N, d, n_clusters, n_iters, _ptr(init),
                                       ctypes.c_uint64(seed & ((1 << 64) - 1)), _ptr(centroids), _ptr(labels),
                                       _ptr(counts), _ptr(x_out), _ptr(x_scale), _ptr(y_out),
                                       _ptr(y_scale if y is not None else None), _ptr(perm), _ptr(offsets),
                                       _ptr(ws), ws_n, _stream(dev))
        _check(st, "svg2_kmeans_permute_fp8")
        return dict(centroids=centroids, labels=labels, counts=counts, x_perm=x_out, y_perm=y_out, perm=perm,
                    offsets=offsets, x_scale=x_scale, y_scale=y_scale if y is not None else None)
    st = L.svg2_kmeans_permute(_ptr(x), _ptr(y), _dtype_code(x), bh, N, d, n_clusters, n_iters, _ptr(init),
                               ctypes.c_uint64(seed & ((1 << 64) - 1)), _ptr(centroids), _ptr(labels),
                               _ptr(counts), None, None, _ptr(x_out), _ptr(y_out), _ptr(perm), _ptr(offsets),
                               _ptr(ws), ws_n, _stream(dev))
    _check(st, "svg2_kmeans_permute")
    return dict(centroids=centroids, labels=labels, counts=counts, x_perm=x_out, y_perm=y_out, perm=perm,
                offsets=offsets, x_scale=None, y_scale=None)


# ---------------------------------------------------------------- permute
def _strided_view(t: torch.Tensor):
    """(bh, N, d, heads, sb, sh, st) of a [bh,N,d] or [B,H,N,d] view whose
    last dimension is contiguous."""
    if t.stride(-1) != 1:
        raise Svg2Error("the head dimension must be contiguous")
    if t.dim() == 3:
        bh, N, d = t.shape
        return bh, N, d, 1, t.stride(0), 0, t.stride(1)
    if t.dim() == 4:
        B, H, N, d = t.shape
        return B * H, N, d, H, t.stride(0), t.stride(1), t.stride(2)
    raise Svg2Error("expected a [bh, N, d] or [B, H, N, d] tensor")


def permute(labels: torch.Tensor, n_clusters: int, *tensors: torch.Tensor,
            outs: Optional[Sequence[torch.Tensor]] = None, perm: Optional[torch.Tensor] = None,
            offsets: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Gathers rows of 1 or 2 tensors into cluster order.  Returns
    (list of contiguous [bh, N, d] tensors, perm [bh,N] int32, offsets [bh,n+1] int32)."""
    _need_cuda(labels, *tensors)
    if not 1 <= len(tensors) <= 2:
        raise Svg2Error("permute takes one or two tensors")
    views = [_strided_view(t) for t in tensors]
    if len(set(views)) != 1 or len({t.dtype for t in tensors}) != 1:
        raise Svg2Error("permuted tensors must share shape, strides and dtype")
    bh, N, d, heads, sb, sh, st = views[0]
    if labels.dtype != torch.int32 or not labels.is_contiguous() or tuple(labels.shape) != (bh, N):
        raise Svg2Error("labels must be contiguous int32 [bh, N]")
    dev = labels.device
    _same_device(dev, *tensors)
    if outs is None:
        outs = [torch.empty(bh, N, d, dtype=tensors[0].dtype, device=dev) for _ in tensors]
    if len(outs) != len(tensors):
        raise Svg2Error("one output per permuted tensor")
    for o in outs:
        _need_out(o, (bh, N, d), tensors[0].dtype, dev, "permute output")
    _need_out(perm, (bh, N), torch.int32, dev, "perm")
    _need_out(offsets, (bh, n_clusters + 1), torch.int32, dev, "offsets")
    if perm is None:
        perm = torch.empty(bh, N, dtype=torch.int32, device=dev)
    if offsets is None:
        offsets = torch.empty(bh, n_clusters + 1, dtype=torch.int32, device=dev)
    L = lib()
    ws_n = L.svg2_permute_workspace_size(bh, N, n_clusters)
    ws = _workspace(ws_n, dev, workspace)
    src = (ctypes.c_void_p * 2)(*[t.data_ptr() for t in tensors], *([0] * (2 - len(tensors))))
    dst = (ctypes.c_void_p * 2)(*[t.data_ptr() for t in outs], *([0] * (2 - len(outs))))
    s = L.svg2_permute(_ptr(labels), bh, N, n_clusters, len(tensors), src, heads, sb, sh, st, dst,
                       _dtype_code(tensors[0]), d, _ptr(perm), _ptr(offsets), _ptr(ws), ws_n, _stream(dev))
    _check(s, "svg2_permute")
    return outs, perm, offsets


# ---------------------------------------------------------------- select
def select_topp(q_centroids: torch.Tensor, q_counts: torch.Tensor, k_centroids: torch.Tensor,
                k_counts: torch.Tensor, top_p: float, scale: Optional[float] = None,
                probs: bool = False, sel_count: Optional[torch.Tensor] = None,
                sel_idx: Optional[torch.Tensor] = None, pair_count: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None):
    """Top-p K-cluster selection per Q-cluster.  Returns dict(sel_count [bh,n_q],
    sel_idx [bh,n_q,n_k], probs, pair_count [bh] int64)."""
    _need_cuda(q_centroids, q_counts, k_centroids, k_counts)
    if q_centroids.dim() != 3 or k_centroids.dim() != 3:
        raise Svg2Error("centroids must be [bh, n, d] tensors")
    bh, n_q, d = q_centroids.shape
    n_k = k_centroids.shape[1]
    for t, dt in ((q_centroids, torch.float32), (k_centroids, torch.float32), (q_counts, torch.int32),
                  (k_counts, torch.int32)):
        if t.dtype != dt or not t.is_contiguous():
            raise Svg2Error("centroids must be contiguous fp32, counts contiguous int32")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dev = q_centroids.device
    _need_out(q_counts, (bh, n_q), torch.int32, dev, "q_counts")
    _need_out(k_centroids, (bh, n_k, d), torch.float32, dev, "k_centroids")
    _need_out(k_counts, (bh, n_k), torch.int32, dev, "k_counts")
    _need_out(sel_count, (bh, n_q), torch.int32, dev, "sel_count")
    _need_out(sel_idx, (bh, n_q, n_k), torch.int32, dev, "sel_idx")
    _need_out(pair_count, (bh,), torch.int64, dev, "pair_count")
    if sel_count is None:
        sel_count = torch.empty(bh, n_q, dtype=torch.int32, device=dev)
    if sel_idx is None:
        sel_idx = torch.empty(bh, n_q, n_k, dtype=torch.int32, device=dev)
    pr = torch.empty(bh, n_q, n_k, dtype=torch.float32, device=dev) if probs else None
    pairs = pair_count if pair_count is not None else torch.empty(bh, dtype=torch.int64, device=dev)
    L = lib()
    ws_n = L.svg2_select_topp_workspace_size(bh, n_q, n_k)
    ws = _workspace(ws_n, dev, workspace)
    s = L.svg2_select_topp(_ptr(q_centroids), _ptr(q_counts), n_q, _ptr(k_centroids), _ptr(k_counts), n_k,
                           bh, d, ctypes.c_float(scale), ctypes.c_float(top_p), _ptr(sel_count),
                           _ptr(sel_idx), _ptr(pr), _ptr(pairs), _ptr(ws), ws_n, _stream(dev))
    _check(s, "svg2_select_topp")
    return dict(sel_count=sel_count, sel_idx=sel_idx, probs=pr, pair_count=pairs)


# ---------------------------------------------------------------- attention
def varblock_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_offsets: torch.Tensor,
                  k_offsets: torch.Tensor, sel_count: torch.Tensor, sel_idx: torch.Tensor,
                  scale: Optional[float] = None, lse=False, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None):
    """Variable-block sparse attention on permuted contiguous [bh, N, d]
    tensors.  Returns (out [bh,N,d], lse [bh,N] fp32 or None); ``lse`` is a
    flag or a contiguous fp32 [bh, N] tensor to write it into."""
    _need_cuda(q, k, v, q_offsets, k_offsets, sel_count, sel_idx)
    if q.dim() != 3:
        raise Svg2Error("q, k, v must be contiguous [bh, N, d] tensors of one dtype")
    bh, N, d = q.shape
    dev = q.device
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need_out(t, q.shape, q.dtype, dev, name)
    n_q, n_k = _lists(bh, dev, q_offsets, k_offsets, sel_count, sel_idx)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _need_out(out, q.shape, q.dtype, dev, "out")
    if out is None:
        out = torch.empty_like(q)
    ls = _lse_buffer(lse, bh, N, dev)
    L = lib()
    ws_n = L.svg2_varblock_attn_workspace_size(bh, N, n_q, n_k, d)
    ws = _workspace(ws_n, dev, workspace)
    s = L.svg2_varblock_attn(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), bh, N, d, _ptr(q_offsets), n_q,
                             _ptr(k_offsets), n_k, _ptr(sel_count), _ptr(sel_idx), ctypes.c_float(scale),
                             _ptr(out), _ptr(ls), _ptr(ws), ws_n, _stream(dev))
    _check(s, "svg2_varblock_attn")
    return out, ls


def varblock_attn_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_offsets: torch.Tensor,
                          k_offsets: torch.Tensor, sel_count: torch.Tensor, sel_idx: torch.Tensor,
                          out: torch.Tensor, lse: Optional[torch.Tensor] = None, scale: Optional[float] = None):
    """varblock_attn through svg2_varblock_attn_noalloc: no workspace, the
    library's fixed scratch array instead; ``out`` (and ``lse``) must be given,
    so that nothing on this path allocates."""
    _need_cuda(q, k, v, q_offsets, k_offsets, sel_count, sel_idx, out, lse)
    if q.dim() != 3:
        raise Svg2Error("q, k, v must be contiguous [bh, N, d] tensors of one dtype")
    bh, N, d = q.shape
    dev = q.device
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _need_out(t, q.shape, q.dtype, dev, name)
    n_q, n_k = _lists(bh, dev, q_offsets, k_offsets, sel_count, sel_idx)
    _need_out(lse, (bh, N), torch.float32, dev, "lse")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    s = lib().svg2_varblock_attn_noalloc(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), bh, N, d, _ptr(q_offsets), n_q,
                                         _ptr(k_offsets), n_k, _ptr(sel_count), _ptr(sel_idx), ctypes.c_float(scale),
                                         _ptr(out), _ptr(lse), _stream(dev))
    _check(s, "svg2_varblock_attn_noalloc")
    return out, lse


def varblock_attn_unpermute(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_offsets: torch.Tensor,
                            k_offsets: torch.Tensor, sel_count: torch.Tensor, sel_idx: torch.Tensor,
                            perm: torch.Tensor, scale: Optional[float] = None, lse=False,
                            out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """varblock_attn with the inverse permutation fused into its stores: out
    row perm[i] = attention output row i (original token order).  ``out`` may be
    a strided [bh,N,d] or [B,H,N,d] view (default: new contiguous tensor);
    ``lse`` (flag or fp32 [bh, N] tensor) is in the original order too."""
    _need_cuda(q, k, v, q_offsets, k_offsets, sel_count, sel_idx, perm, out)
    if q.dim() != 3:
        raise Svg2Error("q, k, v must be contiguous [bh, N, d] tensors of one dtype")
    bh, N, d = q.shape
    dev = q.device
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need_out(t, q.shape, q.dtype, dev, name)
    n_q, n_k = _lists(bh, dev, q_offsets, k_offsets, sel_count, sel_idx)
    _need_out(perm, (bh, N), torch.int32, dev, "perm")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _same_device(dev, out)
    obh, oN, od, heads, sb, sh, st = _strided_view(out)
    if (obh, oN, od) != (bh, N, d) or out.dtype != q.dtype:
        raise Svg2Error("out does not match q")
    ls = _lse_buffer(lse, bh, N, dev)
    L = lib()
    ws_n = L.svg2_varblock_attn_workspace_size(bh, N, n_q, n_k, d)
    ws = _workspace(ws_n, dev, workspace)
    s = L.svg2_varblock_attn_unpermute(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), bh, N, d, _ptr(q_offsets), n_q,
                                       _ptr(k_offsets), n_k, _ptr(sel_count), _ptr(sel_idx), ctypes.c_float(scale),
                                       _ptr(perm), _ptr(out), heads, sb, sh, st, _ptr(ls), _ptr(ws), ws_n,
                                       _stream(dev))
    _check(s, "svg2_varblock_attn_unpermute")
    return out, ls


# ---------------------------------------------------------------- unpermute
def unpermute(src: torch.Tensor, perm: torch.Tensor, out: Optional[torch.Tensor] = None):
    """Scatters rows back: out row perm[i] = src row i.  ``out`` may be a
    strided [bh,N,d] or [B,H,N,d] view (default: new contiguous tensor)."""
    _need_cuda(src, perm, out)
    if src.dim() != 3 or not src.is_contiguous():
        raise Svg2Error("src must be a contiguous [bh, N, d] tensor")
    bh, N, d = src.shape
    if perm.dtype != torch.int32 or not perm.is_contiguous() or tuple(perm.shape) != (bh, N):
        raise Svg2Error("perm must be contiguous int32 [bh, N]")
    _same_device(src.device, perm)
    if out is None:
        out = torch.empty_like(src)
    _same_device(src.device, out)
    obh, oN, od, heads, sb, sh, st = _strided_view(out)
    if (obh, oN, od) != (bh, N, d) or out.dtype != src.dtype:
        raise Svg2Error("out does not match src")
    s = lib().svg2_unpermute(_ptr(src), _dtype_code(src), bh, N, d, _ptr(perm), _ptr(out), heads, sb, sh, st,
                             _stream(src.device))
    _check(s, "svg2_unpermute")
    return out


# ------------------------------------------------------- identification study
def cluster_means(x: torch.Tensor, labels: torch.Tensor, n_clusters: int, means: Optional[torch.Tensor] = None,
                  counts: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Count and fp32 mean row of every label of each problem (the Lloyd update
    alone).  Returns (means [bh, n, d] fp32, counts [bh, n] int32); a label with
    no row keeps the value ``means`` held."""
    _need_cuda(x, labels, means, counts)
    if x.dim() != 3 or not x.is_contiguous():
        raise Svg2Error("x must be a contiguous [bh, N, d] tensor")
    bh, N, d = x.shape
    if labels.dtype != torch.int32 or tuple(labels.shape) != (bh, N) or not labels.is_contiguous():
        raise Svg2Error("labels must be contiguous int32 [bh, N]")
    dev = x.device
    _same_device(dev, labels)
    _need_out(means, (bh, n_clusters, d), torch.float32, dev, "means")
    _need_out(counts, (bh, n_clusters), torch.int32, dev, "counts")
    if means is None:
        means = torch.zeros(bh, n_clusters, d, dtype=torch.float32, device=dev)
    if counts is None:
        counts = torch.empty(bh, n_clusters, dtype=torch.int32, device=dev)
    L = lib()
    ws_n = L.svg2_cluster_means_workspace_size(bh, N, d, n_clusters)
    ws = _workspace(ws_n, dev, workspace)
    st = L.svg2_cluster_means(_ptr(x), _dtype_code(x), bh, N, d, _ptr(labels), n_clusters, _ptr(means),
                              _ptr(counts), _ptr(ws), ws_n, _stream(dev))
    _check(st, "svg2_cluster_means")
    return means, counts


def recall_mass(lse_sel: torch.Tensor, lse_all: torch.Tensor, out: Optional[torch.Tensor] = None):
    """Per problem, the mean over rows of exp(lse_sel - lse_all): the share of
    each row's softmax mass that a selection keeps.  Returns [bh] fp64."""
    _need_cuda(lse_sel, lse_all, out)
    for t in (lse_sel, lse_all):
        if t.dtype != torch.float32 or t.dim() != 2 or not t.is_contiguous() or t.shape != lse_sel.shape:
            raise Svg2Error("lse_sel and lse_all must be contiguous fp32 [bh, N] tensors of one shape")
    bh, N = lse_sel.shape
    _same_device(lse_sel.device, lse_all)
    _need_out(out, (bh,), torch.float64, lse_sel.device, "out")
    if out is None:
        out = torch.empty(bh, dtype=torch.float64, device=lse_sel.device)
    L = lib()
    st = L.svg2_recall_mass(_ptr(lse_sel), _ptr(lse_all), bh, N, _ptr(out), _stream(lse_sel.device))
    _check(st, "svg2_recall_mass")
    return out


# ------------------------------------------------------------------ fp8 attention
def quantize_fp8(x: torch.Tensor, x8: Optional[torch.Tensor] = None, scale: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None):
    """E4M3 copy of a contiguous bf16 [bh, N, d] tensor with one fp32 scale per
    problem (max|x| / 448).  Returns (x8 uint8 [bh, N, d], scale [bh] fp32)."""
    _need_cuda(x, x8, scale)
    if x.dim() != 3 or not x.is_contiguous() or x.dtype != torch.bfloat16:
        raise Svg2Error("x must be a contiguous bf16 [bh, N, d] tensor")
    bh, N, d = x.shape
    dev = x.device
    _need_out(x8, (bh, N, d), torch.uint8, dev, "x8")
    _need_out(scale, (bh,), torch.float32, dev, "scale")
    if x8 is None:
        x8 = torch.empty(bh, N, d, dtype=torch.uint8, device=dev)
    if scale is None:
        scale = torch.empty(bh, dtype=torch.float32, device=dev)
    L = lib()
    ws_n = L.svg2_quantize_fp8_workspace_size(bh)
    ws = _workspace(ws_n, dev, workspace)
    st = L.svg2_quantize_fp8(_ptr(x), bh, N, d, _ptr(x8), _ptr(scale), _ptr(ws), ws_n, _stream(dev))
    _check(st, "svg2_quantize_fp8")
    return x8, scale


def varblock_attn_fp8(q8: torch.Tensor, k8: torch.Tensor, v8: torch.Tensor, q_scale: torch.Tensor,
                      k_scale: torch.Tensor, v_scale: torch.Tensor, q_offsets: torch.Tensor, k_offsets: torch.Tensor,
                      sel_count: torch.Tensor, sel_idx: torch.Tensor, scale: Optional[float] = None, lse=False,
                      out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """svg2_varblock_attn on E4M3 inputs (uint8 [bh, N, 128] with [bh] fp32
    scales).  Returns (out bf16 [bh, N, 128], lse or None)."""
    _need_cuda(q8, k8, v8, q_scale, k_scale, v_scale, q_offsets, k_offsets, sel_count, sel_idx)
    if q8.dim() != 3:
        raise Svg2Error("q8, k8, v8 must be contiguous uint8 [bh, N, d] tensors of one shape")
    bh, N, d = q8.shape
    dev = q8.device
    for t, name in ((q8, "q8"), (k8, "k8"), (v8, "v8")):
        _need_out(t, q8.shape, torch.uint8, dev, name)
    for t, name in ((q_scale, "q_scale"), (k_scale, "k_scale"), (v_scale, "v_scale")):
        _need_out(t, (bh,), torch.float32, dev, name)
    n_q, n_k = _lists(bh, dev, q_offsets, k_offsets, sel_count, sel_idx)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _need_out(out, (bh, N, d), torch.bfloat16, dev, "out")
    if out is None:
        out = torch.empty(bh, N, d, dtype=torch.bfloat16, device=dev)
    ls = _lse_buffer(lse, bh, N, dev)
    L = lib()
    ws_n = L.svg2_varblock_attn_workspace_size(bh, N, n_q, n_k, d)
    ws = _workspace(ws_n, dev, workspace)
    st = L.svg2_varblock_attn_fp8(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale), bh, N,
                                  d, _ptr(q_offsets), n_q, _ptr(k_offsets), n_k, _ptr(sel_count), _ptr(sel_idx),
                                  ctypes.c_float(scale), _ptr(out), _ptr(ls), _ptr(ws), ws_n, _stream(dev))
    _check(st, "svg2_varblock_attn_fp8")
    return out, ls


def varblock_attn_fp8_unpermute(q8: torch.Tensor, k8: torch.Tensor, v8: torch.Tensor, q_scale: torch.Tensor,
                                k_scale: torch.Tensor, v_scale: torch.Tensor, q_offsets: torch.Tensor,
                                k_offsets: torch.Tensor, sel_count: torch.Tensor, sel_idx: torch.Tensor,
                                perm: torch.Tensor, scale: Optional[float] = None, lse=False,
                                out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """varblock_attn_fp8 with the inverse permutation fused into its stores:
    out row perm[i] = attention output row i.  ``out`` is a bf16 [bh,N,d] or
    [B,H,N,d] view; ``lse`` (flag or fp32 [bh, N] tensor) in the original order."""
    _need_cuda(q8, k8, v8, q_scale, k_scale, v_scale, q_offsets, k_offsets, sel_count, sel_idx, perm, out)
    if q8.dim() != 3:
        raise Svg2Error("q8, k8, v8 must be contiguous uint8 [bh, N, d] tensors of one shape")
    bh, N, d = q8.shape
    dev = q8.device
    for t, name in ((q8, "q8"), (k8, "k8"), (v8, "v8")):
        _need_out(t, q8.shape, torch.uint8, dev, name)
    for t, name in ((q_scale, "q_scale"), (k_scale, "k_scale"), (v_scale, "v_scale")):
        _need_out(t, (bh,), torch.float32, dev, name)
    n_q, n_k = _lists(bh, dev, q_offsets, k_offsets, sel_count, sel_idx)
    _need_out(perm, (bh, N), torch.int32, dev, "perm")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty(bh, N, d, dtype=torch.bfloat16, device=dev)
    _same_device(dev, out)
    obh, oN, od, heads, sb, sh, st = _strided_view(out)
    if (obh, oN, od) != (bh, N, d) or out.dtype != torch.bfloat16:
        raise Svg2Error("out must be a bf16 view of shape [bh, N, d]")
    ls = _lse_buffer(lse, bh, N, dev)
    L = lib()
    ws_n = L.svg2_varblock_attn_workspace_size(bh, N, n_q, n_k, d)
    ws = _workspace(ws_n, dev, workspace)
    s = L.svg2_varblock_attn_fp8_unpermute(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(q_scale), _ptr(k_scale),
                                           _ptr(v_scale), bh, N, d, _ptr(q_offsets), n_q, _ptr(k_offsets), n_k,
                                           _ptr(sel_count), _ptr(sel_idx), ctypes.c_float(scale), _ptr(perm),
                                           _ptr(out), heads, sb, sh, st, _ptr(ls), _ptr(ws), ws_n, _stream(dev))
    _check(s, "svg2_varblock_attn_fp8_unpermute")
    return out, ls
