// C ABI of libsvg2: argument validation (always before any HIP call),
// workspace carving and kernel dispatch.  The operations are specified in
// include/svg2.h.
#include "svg2.h"

#include <math.h>
#include <string.h>

#include "internal.hpp"

using namespace svg2;

namespace {

thread_local int g_last_hip_error = 0;

// below 2^24 so that one head's rows at d = 128 (N x 256 bytes) stay under the
// 4 GiB a buffer resource's 32-bit record count covers
constexpr int kMaxTokens = (1 << 24) - 1;
constexpr size_t kAlign = 256;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return SVG2_OK;
  g_last_hip_error = (int)e;
  return SVG2_ERR_HIP;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
bool dtype_ok(int32_t dt) { return dt == SVG2_F32 || dt == SVG2_BF16; }
int esize(int32_t dt) { return dt == SVG2_F32 ? 4 : 2; }
bool dim_ok(int32_t d) { return d == 64 || d == 128; }

// Bump allocator over the caller's workspace; with base == nullptr it only
// measures.
struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(size_t count) {
    off = (off + kAlign - 1) / kAlign * kAlign;
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

struct KmeansWs {
  double* d2;
  int32_t* near;      // bh * N ints of space: the 16-bit nearest pick of each token
  int32_t* picks;
  double* cc;
  double* bsum;
  uint16_t* c_hi;
  uint16_t* c_lo;
  float* c_norm;
  int32_t* hist;
  int32_t* perm;
  int32_t* offsets;
  double* partial;    // bh * (n + mean_chunks(N)) * d: per-chunk centroid sums
  uint32_t* amax;     // 2 bh: max|x|, max|y| per problem (E4M3 row moves)
  AsgFixWs fix;       // near ties of the bf16 assignment (count bh; token, dmin bh * N)
};

KmeansWs carve_kmeans(Carve& c, int bh, int N, int d, int n) {
  KmeansWs w;
  const size_t bN = (size_t)bh * N;
  w.d2 = c.take<double>(bN);
  w.near = c.take<int32_t>(bN);
  w.picks = c.take<int32_t>((size_t)bh * n);
  w.cc = c.take<double>((size_t)bh * n);
  w.bsum = c.take<double>((size_t)bh * ((N + 255) / 256));
  w.c_hi = c.take<uint16_t>((size_t)bh * centroid_rows(n) * d);
  w.c_lo = c.take<uint16_t>((size_t)bh * centroid_rows(n) * d);
  w.c_norm = c.take<float>((size_t)bh * centroid_rows(n));
  w.hist = c.take<int32_t>((size_t)bh * sort_chunks(N) * n);
  w.perm = c.take<int32_t>(bN);
  w.offsets = c.take<int32_t>((size_t)bh * (n + 1));
  w.partial = c.take<double>((size_t)bh * (n + mean_chunks(N)) * d);
  w.amax = c.take<uint32_t>((size_t)2 * bh);
  w.fix.count = c.take<int32_t>((size_t)bh);
  w.fix.token = c.take<int32_t>(bN);
  w.fix.dmin = c.take<float>(bN);
  w.fix.hist = w.hist;
  return w;
}

bool shape_ok(int32_t bh, int32_t N, int32_t n) {
  return bh >= 1 && N >= 1 && N <= kMaxTokens && n >= 1 && n <= kMaxClusters && n <= N;
}

bool strides_ok(int32_t heads, int32_t bh, int64_t sb, int64_t sh, int64_t st, int es) {
  if (heads < 1 || bh % heads != 0) return false;
  const int64_t q = 16 / es;
  if (sb < 0 || sh < 0 || st < 0) return false;
  return sb % q == 0 && sh % q == 0 && st % q == 0;
}

// Attention work lists; the fp32 kernel uses the smaller row block, hence the
// larger per-head item list.
AttnWs carve_attn(Carve& c, int bh, int N, int n_q) {
  const int bm = attn_block_rows(false) < attn_block_rows(true) ? attn_block_rows(false) : attn_block_rows(true);
  const size_t mx = (size_t)attn_max_items(N, n_q, attn_block_rows(true));
  AttnWs w;
  w.tiles = c.take<int32_t>((size_t)bh * n_q);
  w.item_count = c.take<int32_t>((size_t)bh);
  w.items = c.take<int32_t>((size_t)bh * attn_max_items(N, n_q, bm));
  w.xitems = c.take<int32_t>((size_t)bh * kAttnXcds * mx);
  w.xcount = c.take<int32_t>((size_t)bh * kAttnXcds);
  w.queue = c.take<int32_t>(2 * kAttnXcds);
  w.flat = c.take<int32_t>((size_t)kAttnXcds * bh * mx * 2);
  w.kmax = c.take<uint32_t>((size_t)bh);
  return w;
}

// svg2_kmeans, and with mv.x_out set, svg2_kmeans_permute(_fp8): the last
// round's sort writes perm / offsets and its centroid update also moves the
// rows (as E4M3 when fp8, with max|.| taken from the inputs first).
int kmeans_run(const void* x, int32_t dtype, int32_t bh, int32_t n_tokens, int32_t head_dim,
               int32_t n_clusters, int32_t n_iters, const float* init_centroids, uint64_t seed,
               float* centroids, int32_t* labels, int32_t* counts, float* min_dist, int32_t* seed_index,
               MeanMove mv, bool fp8, int32_t* perm_out, int32_t* offsets_out, void* workspace,
               size_t workspace_bytes, hipStream_t stream) {
  if (!dtype_ok(dtype)) return SVG2_ERR_INVALID_ARG;
  if (!shape_ok(bh, n_tokens, n_clusters)) return SVG2_ERR_INVALID_ARG;
  if (!dim_ok(head_dim)) return SVG2_ERR_UNSUPPORTED;
  if (n_iters < 0 || n_iters > 100) return SVG2_ERR_INVALID_ARG;
  if (!x || !aligned(x, 16) || !centroids || !aligned(centroids, 16)) return SVG2_ERR_INVALID_ARG;
  if (init_centroids && !aligned(init_centroids, 16)) return SVG2_ERR_INVALID_ARG;
  if (n_iters > 0 && (!labels || !counts)) return SVG2_ERR_INVALID_ARG;
  if ((labels && !aligned(labels, 4)) || (counts && !aligned(counts, 4)) ||
      (min_dist && !aligned(min_dist, 4)) || (seed_index && !aligned(seed_index, 4)))
    return SVG2_ERR_INVALID_ARG;
  const size_t need = svg2_kmeans_workspace_size(bh, n_tokens, head_dim, n_clusters);
  if (workspace_bytes < need || (need && !workspace)) return SVG2_ERR_WORKSPACE;
  if (!aligned(workspace, kAlign)) return SVG2_ERR_INVALID_ARG;

  Carve c(workspace);
  const KmeansWs w = carve_kmeans(c, bh, n_tokens, head_dim, n_clusters);
  const bool bf16 = dtype == SVG2_BF16;
  const int N = n_tokens, n = n_clusters, d = head_dim;
  int st;
  if (fp8) {
    mv.amax = w.amax;
    st = hip_status(launch_amax_bf16(x, bh, N, d, w.amax, stream));
    if (st) return st;
    if (mv.y) {
      st = hip_status(launch_amax_bf16(mv.y, bh, N, d, w.amax + bh, stream));
      if (st) return st;
    }
  }
  if (!init_centroids) {
    st = hip_status(launch_kmeanspp(x, bf16, bh, N, d, n, seed, w.d2, w.near, centroids, seed_index,
                                    w.picks, w.cc, w.bsum, stream));
    if (st) return st;
  } else if (init_centroids != centroids) {
    st = hip_status(hipMemcpyAsync(centroids, init_centroids, (size_t)bh * n * d * sizeof(float),
                                   hipMemcpyDeviceToDevice, stream));
    if (st) return st;
  }
  for (int it = 0; it < n_iters; ++it) {
    // After k-means++ the first round's labels are the seeding's nearest picks
    // (the same exact decision), unless that round must also report min_dist.
    const bool from_seeds = !init_centroids && it == 0 && !(it == n_iters - 1 && min_dist);
    if (from_seeds) {
      st = hip_status(launch_labels_from_seeding(w.near, bh, N, labels, stream));
      if (st) return st;
    } else {
      if (bf16) {
        const SortStart ss{w.fix.count, w.hist, (size_t)bh * sort_chunks(N) * n};
        st = hip_status(launch_prep_centroids(centroids, bh, n, d, w.c_hi, w.c_lo, w.c_norm, ss, stream));
        if (st) return st;
      }
      st = hip_status(launch_assign(x, bf16, bh, N, d, n, centroids, w.c_hi, w.c_lo, w.c_norm, labels,
                                    it == n_iters - 1 ? min_dist : nullptr, w.fix, stream));
      if (st) return st;
    }
    const bool last = it == n_iters - 1 && mv.x_out;
    int32_t* pm = last ? perm_out : w.perm;
    int32_t* of = last ? offsets_out : w.offsets;
    // the bf16 assignment adds the sort's label histograms as it writes the labels
    const bool have_hist = bf16 && !from_seeds;
    st = hip_status(launch_counting_sort(labels, bh, N, n, w.hist, have_hist, pm, of, counts, stream));
    if (st) return st;
    st = hip_status(launch_centroid_mean(x, bf16, bh, N, d, n, pm, of, w.partial, centroids, stream,
                                         last ? mv : MeanMove{}));
    if (st) return st;
  }
  return SVG2_OK;
}

// the FP8 attention's checks and launch; om maps output rows (identity, or
// token perm[row] through strides)
int attn_fp8_run(const void* q8, const void* k8, const void* v8, const float* q_scale, const float* k_scale,
                 const float* v_scale, int32_t bh, int32_t n_tokens, int32_t head_dim, const int32_t* q_offsets,
                 int32_t n_q, const int32_t* k_offsets, int32_t n_k, const int32_t* sel_count,
                 const int32_t* sel_idx, float scale, void* out, float* lse, const OutMap& om, void* workspace,
                 size_t workspace_bytes, hipStream_t stream) {
  if (n_q < 1 || n_q > kMaxClusters || n_k < 1 || n_k > kMaxClusters) return SVG2_ERR_INVALID_ARG;
  if (!(isfinite(scale) && scale > 0.f)) return SVG2_ERR_INVALID_ARG;
  if (!q8 || !k8 || !v8 || !out || !aligned(q8, 16) || !aligned(k8, 16) || !aligned(v8, 16) || !aligned(out, 16))
    return SVG2_ERR_INVALID_ARG;
  if (!q_scale || !k_scale || !v_scale || !aligned(q_scale, 4) || !aligned(k_scale, 4) || !aligned(v_scale, 4))
    return SVG2_ERR_INVALID_ARG;
  if (!q_offsets || !k_offsets || !sel_count || !sel_idx || !aligned(q_offsets, 4) ||
      !aligned(k_offsets, 4) || !aligned(sel_count, 4) || !aligned(sel_idx, 4) || (lse && !aligned(lse, 4)))
    return SVG2_ERR_INVALID_ARG;
  const size_t need = svg2_varblock_attn_workspace_size(bh, n_tokens, n_q, n_k, head_dim);
  if (workspace_bytes < need || !workspace) return SVG2_ERR_WORKSPACE;
  if (!aligned(workspace, kAlign)) return SVG2_ERR_INVALID_ARG;
  Carve c(workspace);
  const AttnWs ws = carve_attn(c, bh, n_tokens, n_q);
  return hip_status(launch_varblock_attn_fp8(q8, k8, v8, q_scale, k_scale, v_scale, bh, n_tokens, q_offsets, n_q,
                                             k_offsets, n_k, sel_count, sel_idx, scale, out, lse, om, ws, stream));
}

}  // namespace

namespace svg2 {
void record_hip_error(int e) { g_last_hip_error = e; }
}  // namespace svg2

extern "C" {

const char* svg2_version(void) { return "svg2-mi355x 0.1.0 (gfx950)"; }

const char* svg2_status_string(int status) {
  switch (status) {
    case SVG2_OK: return "ok";
    case SVG2_ERR_INVALID_ARG: return "invalid argument";
    case SVG2_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case SVG2_ERR_WORKSPACE: return "workspace too small";
    case SVG2_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

int svg2_last_hip_error(void) { return g_last_hip_error; }

// ------------------------------------------------------------------ kmeans
size_t svg2_kmeans_workspace_size(int32_t bh, int32_t n_tokens, int32_t head_dim, int32_t n_clusters) {
  if (!shape_ok(bh, n_tokens, n_clusters) || !dim_ok(head_dim)) return 0;
  Carve c(nullptr);
  carve_kmeans(c, bh, n_tokens, head_dim, n_clusters);
  return c.off;
}

int svg2_kmeans(const void* x, int32_t dtype, int32_t bh, int32_t n_tokens, int32_t head_dim,
                int32_t n_clusters, int32_t n_iters, const float* init_centroids, uint64_t seed,
                float* centroids, int32_t* labels, int32_t* counts, float* min_dist,
                int32_t* seed_index, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return kmeans_run(x, dtype, bh, n_tokens, head_dim, n_clusters, n_iters, init_centroids, seed, centroids,
                    labels, counts, min_dist, seed_index, MeanMove{}, false, nullptr, nullptr, workspace,
                    workspace_bytes, stream);
}

int svg2_kmeans_permute(const void* x, const void* y, int32_t dtype, int32_t bh, int32_t n_tokens,
                        int32_t head_dim, int32_t n_clusters, int32_t n_iters, const float* init_centroids,
                        uint64_t seed, float* centroids, int32_t* labels, int32_t* counts, float* min_dist,
                        int32_t* seed_index, void* x_perm, void* y_perm, int32_t* perm, int32_t* offsets,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (n_iters < 1) return SVG2_ERR_INVALID_ARG;
  if (!x_perm || !aligned(x_perm, 16) || !perm || !aligned(perm, 4) || !offsets || !aligned(offsets, 4))
    return SVG2_ERR_INVALID_ARG;
  if ((y == nullptr) != (y_perm == nullptr)) return SVG2_ERR_INVALID_ARG;
  if (y && (!aligned(y, 16) || !aligned(y_perm, 16))) return SVG2_ERR_INVALID_ARG;
  if (x_perm == x || (y && (y_perm == y || y_perm == x || x_perm == y || y_perm == x_perm)))
    return SVG2_ERR_INVALID_ARG;
  MeanMove mv;
  mv.x_out = x_perm;
  mv.y = y;
  mv.y_out = y_perm;
  return kmeans_run(x, dtype, bh, n_tokens, head_dim, n_clusters, n_iters, init_centroids, seed, centroids,
                    labels, counts, min_dist, seed_index, mv, false, perm, offsets, workspace, workspace_bytes,
                    stream);
}

int svg2_kmeans_permute_fp8(const void* x, const void* y, int32_t bh, int32_t n_tokens, int32_t head_dim,
                            int32_t n_clusters, int32_t n_iters, const float* init_centroids, uint64_t seed,
                            float* centroids, int32_t* labels, int32_t* counts, void* x8_perm, float* x_scale,
                            void* y8_perm, float* y_scale, int32_t* perm, int32_t* offsets, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  if (n_iters < 1) return SVG2_ERR_INVALID_ARG;
  if (!x8_perm || !aligned(x8_perm, 16) || !x_scale || !aligned(x_scale, 4) || !perm || !aligned(perm, 4) ||
      !offsets || !aligned(offsets, 4))
    return SVG2_ERR_INVALID_ARG;
  if ((y == nullptr) != (y8_perm == nullptr) || (y == nullptr) != (y_scale == nullptr)) return SVG2_ERR_INVALID_ARG;
  if (y && (!aligned(y, 16) || !aligned(y8_perm, 16) || !aligned(y_scale, 4))) return SVG2_ERR_INVALID_ARG;
  if (x8_perm == x || (y && (y8_perm == y || y8_perm == x || x8_perm == y || y8_perm == x8_perm)))
    return SVG2_ERR_INVALID_ARG;
  MeanMove mv;
  mv.x_out = x8_perm;
  mv.y = y;
  mv.y_out = y8_perm;
  mv.x_scale = x_scale;
  mv.y_scale = y_scale;
  return kmeans_run(x, SVG2_BF16, bh, n_tokens, head_dim, n_clusters, n_iters, init_centroids, seed, centroids,
                    labels, counts, nullptr, nullptr, mv, true, perm, offsets, workspace, workspace_bytes, stream);
}

// ------------------------------------------------------------------ permute
size_t svg2_permute_workspace_size(int32_t bh, int32_t n_tokens, int32_t n_clusters) {
  if (!shape_ok(bh, n_tokens, n_clusters)) return 0;
  Carve c(nullptr);
  c.take<int32_t>((size_t)bh * sort_chunks(n_tokens) * n_clusters);
  c.take<int32_t>((size_t)bh * n_clusters);
  return c.off;
}

int svg2_permute(const int32_t* labels, int32_t bh, int32_t n_tokens, int32_t n_clusters,
                 int32_t n_tensors, const void* const* src, int32_t heads, int64_t src_b_stride,
                 int64_t src_h_stride, int64_t src_token_stride, void* const* dst, int32_t dtype,
                 int32_t head_dim, int32_t* perm, int32_t* offsets, void* workspace,
                 size_t workspace_bytes, hipStream_t stream) {
  if (!dtype_ok(dtype)) return SVG2_ERR_INVALID_ARG;
  if (!shape_ok(bh, n_tokens, n_clusters)) return SVG2_ERR_INVALID_ARG;
  if (!dim_ok(head_dim)) return SVG2_ERR_UNSUPPORTED;
  if (n_tensors < 1 || n_tensors > 2 || !src || !dst) return SVG2_ERR_INVALID_ARG;
  if (!labels || !aligned(labels, 4) || !perm || !aligned(perm, 4) || !offsets || !aligned(offsets, 4))
    return SVG2_ERR_INVALID_ARG;
  for (int t = 0; t < n_tensors; ++t)
    if (!src[t] || !dst[t] || !aligned(src[t], 16) || !aligned(dst[t], 16)) return SVG2_ERR_INVALID_ARG;
  if (!strides_ok(heads, bh, src_b_stride, src_h_stride, src_token_stride, esize(dtype)))
    return SVG2_ERR_INVALID_ARG;
  const size_t need = svg2_permute_workspace_size(bh, n_tokens, n_clusters);
  if (workspace_bytes < need || !workspace) return SVG2_ERR_WORKSPACE;
  if (!aligned(workspace, kAlign)) return SVG2_ERR_INVALID_ARG;

  Carve c(workspace);
  int32_t* hist = c.take<int32_t>((size_t)bh * sort_chunks(n_tokens) * n_clusters);
  int32_t* counts = c.take<int32_t>((size_t)bh * n_clusters);
  int st = hip_status(launch_counting_sort(labels, bh, n_tokens, n_clusters, hist, false, perm, offsets, counts,
                                           stream));
  if (st) return st;
  return hip_status(launch_gather_rows(n_tensors, src, dst, esize(dtype), head_dim, bh, n_tokens, heads,
                                       src_b_stride, src_h_stride, src_token_stride, perm, stream));
}

// ------------------------------------------------------------------ select
size_t svg2_select_topp_workspace_size(int32_t bh, int32_t n_q, int32_t n_k) {
  if (bh < 1 || n_q < 1 || n_q > kMaxClusters || n_k < 1 || n_k > kMaxClusters) return 0;
  Carve c(nullptr);
  c.take<int64_t>((size_t)bh * n_q);
  c.take<double>((size_t)bh * n_q * n_k);
  return c.off;
}

int svg2_select_topp(const float* q_centroids, const int32_t* q_counts, int32_t n_q,
                     const float* k_centroids, const int32_t* k_counts, int32_t n_k, int32_t bh,
                     int32_t head_dim, float scale, float top_p, int32_t* sel_count, int32_t* sel_idx,
                     float* probs, int64_t* pair_count, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
  if (bh < 1 || n_q < 1 || n_q > kMaxClusters || n_k < 1 || n_k > kMaxClusters) return SVG2_ERR_INVALID_ARG;
  if (!dim_ok(head_dim)) return SVG2_ERR_UNSUPPORTED;
  if (!(isfinite(scale) && scale > 0.f)) return SVG2_ERR_INVALID_ARG;
  if (!(isfinite(top_p) && top_p > 0.f && top_p <= 1.f)) return SVG2_ERR_INVALID_ARG;
  if (!q_centroids || !k_centroids || !q_counts || !k_counts || !sel_count || !sel_idx)
    return SVG2_ERR_INVALID_ARG;
  if (!aligned(q_centroids, 16) || !aligned(k_centroids, 16) || !aligned(q_counts, 4) ||
      !aligned(k_counts, 4) || !aligned(sel_count, 4) || !aligned(sel_idx, 4) ||
      (probs && !aligned(probs, 4)) || (pair_count && !aligned(pair_count, 8)))
    return SVG2_ERR_INVALID_ARG;
  const size_t need = svg2_select_topp_workspace_size(bh, n_q, n_k);
  if (workspace_bytes < need || !workspace) return SVG2_ERR_WORKSPACE;
  if (!aligned(workspace, kAlign)) return SVG2_ERR_INVALID_ARG;
  Carve c(workspace);
  int64_t* row_pairs = c.take<int64_t>((size_t)bh * n_q);
  double* logits = c.take<double>((size_t)bh * n_q * n_k);
  return hip_status(launch_select_topp(q_centroids, q_counts, n_q, k_centroids, k_counts, n_k, bh, head_dim,
                                       (double)scale, (double)top_p, sel_count, sel_idx, probs, row_pairs,
                                       logits, pair_count, stream));
}

// ------------------------------------------------------------------ attention
size_t svg2_varblock_attn_workspace_size(int32_t bh, int32_t n_tokens, int32_t n_q, int32_t n_k,
                                         int32_t head_dim) {
  if (bh < 1 || n_tokens < 1 || n_tokens > kMaxTokens || n_q < 1 || n_q > kMaxClusters || n_k < 1 ||
      n_k > kMaxClusters || !dim_ok(head_dim))
    return 0;
  Carve c(nullptr);
  carve_attn(c, bh, n_tokens, n_q);
  return c.off;
}

int svg2_varblock_attn(const void* q, const void* k, const void* v, int32_t dtype, int32_t bh,
                       int32_t n_tokens, int32_t head_dim, const int32_t* q_offsets, int32_t n_q,
                       const int32_t* k_offsets, int32_t n_k, const int32_t* sel_count,
                       const int32_t* sel_idx, float scale, void* out, float* lse, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  if (!dtype_ok(dtype)) return SVG2_ERR_INVALID_ARG;
  if (bh < 1 || n_tokens < 1 || n_tokens > kMaxTokens) return SVG2_ERR_INVALID_ARG;
  if (n_q < 1 || n_q > kMaxClusters || n_k < 1 || n_k > kMaxClusters) return SVG2_ERR_INVALID_ARG;
  if (!dim_ok(head_dim)) return SVG2_ERR_UNSUPPORTED;
  if (!(isfinite(scale) && scale > 0.f)) return SVG2_ERR_INVALID_ARG;
  if (!q || !k || !v || !out || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return SVG2_ERR_INVALID_ARG;
  if (!q_offsets || !k_offsets || !sel_count || !sel_idx || !aligned(q_offsets, 4) ||
      !aligned(k_offsets, 4) || !aligned(sel_count, 4) || !aligned(sel_idx, 4) || (lse && !aligned(lse, 4)))
    return SVG2_ERR_INVALID_ARG;
  const size_t need = svg2_varblock_attn_workspace_size(bh, n_tokens, n_q, n_k, head_dim);
  if (workspace_bytes < need || !workspace) return SVG2_ERR_WORKSPACE;
  if (!aligned(workspace, kAlign)) return SVG2_ERR_INVALID_ARG;
  Carve c(workspace);
  const AttnWs ws = carve_attn(c, bh, n_tokens, n_q);
  return hip_status(launch_varblock_attn(q, k, v, dtype == SVG2_BF16, bh, n_tokens, head_dim, q_offsets, n_q,
                                         k_offsets, n_k, sel_count, sel_idx, scale, out, lse,
                                         contiguous_out(n_tokens, head_dim), ws, stream));
}

int svg2_varblock_attn_unpermute(const void* q, const void* k, const void* v, int32_t dtype, int32_t bh,
                                 int32_t n_tokens, int32_t head_dim, const int32_t* q_offsets, int32_t n_q,
                                 const int32_t* k_offsets, int32_t n_k, const int32_t* sel_count,
                                 const int32_t* sel_idx, float scale, const int32_t* perm, void* dst,
                                 int32_t heads, int64_t dst_b_stride, int64_t dst_h_stride,
                                 int64_t dst_token_stride, float* lse, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  if (!dtype_ok(dtype)) return SVG2_ERR_INVALID_ARG;
  if (bh < 1 || n_tokens < 1 || n_tokens > kMaxTokens) return SVG2_ERR_INVALID_ARG;
  if (n_q < 1 || n_q > kMaxClusters || n_k < 1 || n_k > kMaxClusters) return SVG2_ERR_INVALID_ARG;
  if (!dim_ok(head_dim)) return SVG2_ERR_UNSUPPORTED;
  if (!(isfinite(scale) && scale > 0.f)) return SVG2_ERR_INVALID_ARG;
  if (!q || !k || !v || !dst || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(dst, 16))
    return SVG2_ERR_INVALID_ARG;
  if (!q_offsets || !k_offsets || !sel_count || !sel_idx || !perm || !aligned(q_offsets, 4) ||
      !aligned(k_offsets, 4) || !aligned(sel_count, 4) || !aligned(sel_idx, 4) || !aligned(perm, 4) ||
      (lse && !aligned(lse, 4)))
    return SVG2_ERR_INVALID_ARG;
  if (!strides_ok(heads, bh, dst_b_stride, dst_h_stride, dst_token_stride, esize(dtype)))
    return SVG2_ERR_INVALID_ARG;
  const size_t need = svg2_varblock_attn_workspace_size(bh, n_tokens, n_q, n_k, head_dim);
  if (workspace_bytes < need || !workspace) return SVG2_ERR_WORKSPACE;
  if (!aligned(workspace, kAlign)) return SVG2_ERR_INVALID_ARG;
  Carve c(workspace);
  const AttnWs ws = carve_attn(c, bh, n_tokens, n_q);
  const OutMap om{perm, heads, dst_b_stride, dst_h_stride, dst_token_stride};
  return hip_status(launch_varblock_attn(q, k, v, dtype == SVG2_BF16, bh, n_tokens, head_dim, q_offsets, n_q,
                                         k_offsets, n_k, sel_count, sel_idx, scale, dst, lse, om, ws, stream));
}

// ------------------------------------------------------------------ unpermute
int svg2_unpermute(const void* src, int32_t dtype, int32_t bh, int32_t n_tokens, int32_t head_dim,
                   const int32_t* perm, void* dst, int32_t heads, int64_t dst_b_stride,
                   int64_t dst_h_stride, int64_t dst_token_stride, hipStream_t stream) {
  if (!dtype_ok(dtype)) return SVG2_ERR_INVALID_ARG;
  if (bh < 1 || n_tokens < 1 || n_tokens > kMaxTokens) return SVG2_ERR_INVALID_ARG;
  if (!dim_ok(head_dim)) return SVG2_ERR_UNSUPPORTED;
  if (!src || !dst || !perm || !aligned(src, 16) || !aligned(dst, 16) || !aligned(perm, 4))
    return SVG2_ERR_INVALID_ARG;
  if (!strides_ok(heads, bh, dst_b_stride, dst_h_stride, dst_token_stride, esize(dtype)))
    return SVG2_ERR_INVALID_ARG;
  return hip_status(launch_scatter_rows(src, dst, esize(dtype), head_dim, bh, n_tokens, heads, dst_b_stride,
                                        dst_h_stride, dst_token_stride, perm, stream));
}

// ------------------------------------------------------------------ fp8 attention
size_t svg2_quantize_fp8_workspace_size(int32_t bh) {
  if (bh < 1) return 0;
  Carve c(nullptr);
  c.take<uint32_t>((size_t)bh);
  return c.off;
}

int svg2_quantize_fp8(const void* x, int32_t bh, int32_t n_tokens, int32_t head_dim, void* x8, float* scale,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (bh < 1 || n_tokens < 1 || n_tokens > kMaxTokens) return SVG2_ERR_INVALID_ARG;
  if (!dim_ok(head_dim)) return SVG2_ERR_UNSUPPORTED;
  if (!x || !x8 || !scale || !aligned(x, 16) || !aligned(x8, 16) || !aligned(scale, 4)) return SVG2_ERR_INVALID_ARG;
  const size_t need = svg2_quantize_fp8_workspace_size(bh);
  if (workspace_bytes < need || !workspace) return SVG2_ERR_WORKSPACE;
  if (!aligned(workspace, kAlign)) return SVG2_ERR_INVALID_ARG;
  return hip_status(launch_quantize_fp8(x, bh, n_tokens, head_dim, static_cast<uint8_t*>(x8), scale,
                                        static_cast<uint32_t*>(workspace), stream));
}

int svg2_varblock_attn_fp8(const void* q8, const void* k8, const void* v8, const float* q_scale,
                           const float* k_scale, const float* v_scale, int32_t bh, int32_t n_tokens,
                           int32_t head_dim, const int32_t* q_offsets, int32_t n_q,
                           const int32_t* k_offsets, int32_t n_k, const int32_t* sel_count,
                           const int32_t* sel_idx, float scale, void* out, float* lse, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  if (bh < 1 || n_tokens < 1 || n_tokens > kMaxTokens) return SVG2_ERR_INVALID_ARG;
  if (head_dim != 128) return SVG2_ERR_UNSUPPORTED;
  return attn_fp8_run(q8, k8, v8, q_scale, k_scale, v_scale, bh, n_tokens, head_dim, q_offsets, n_q, k_offsets,
                      n_k, sel_count, sel_idx, scale, out, lse, contiguous_out(n_tokens, head_dim), workspace,
                      workspace_bytes, stream);
}

int svg2_varblock_attn_fp8_unpermute(const void* q8, const void* k8, const void* v8, const float* q_scale,
                                     const float* k_scale, const float* v_scale, int32_t bh, int32_t n_tokens,
                                     int32_t head_dim, const int32_t* q_offsets, int32_t n_q,
                                     const int32_t* k_offsets, int32_t n_k, const int32_t* sel_count,
                                     const int32_t* sel_idx, float scale, const int32_t* perm, void* dst,
                                     int32_t heads, int64_t dst_b_stride, int64_t dst_h_stride,
                                     int64_t dst_token_stride, float* lse, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  if (bh < 1 || n_tokens < 1 || n_tokens > kMaxTokens) return SVG2_ERR_INVALID_ARG;
  if (head_dim != 128) return SVG2_ERR_UNSUPPORTED;
  if (!perm || !aligned(perm, 4)) return SVG2_ERR_INVALID_ARG;
  if (!strides_ok(heads, bh, dst_b_stride, dst_h_stride, dst_token_stride, 2)) return SVG2_ERR_INVALID_ARG;
  const OutMap om{perm, heads, dst_b_stride, dst_h_stride, dst_token_stride};
  return attn_fp8_run(q8, k8, v8, q_scale, k_scale, v_scale, bh, n_tokens, head_dim, q_offsets, n_q, k_offsets,
                      n_k, sel_count, sel_idx, scale, dst, lse, om, workspace, workspace_bytes, stream);
}

// ------------------------------------------------------- identification study
size_t svg2_cluster_means_workspace_size(int32_t bh, int32_t n_tokens, int32_t head_dim, int32_t n_clusters) {
  if (!shape_ok(bh, n_tokens, n_clusters) || !dim_ok(head_dim)) return 0;
  Carve c(nullptr);
  c.take<int32_t>((size_t)bh * sort_chunks(n_tokens) * n_clusters);
  c.take<int32_t>((size_t)bh * n_tokens);
  c.take<int32_t>((size_t)bh * (n_clusters + 1));
  c.take<double>((size_t)bh * (n_clusters + mean_chunks(n_tokens)) * head_dim);
  return c.off;
}

int svg2_cluster_means(const void* x, int32_t dtype, int32_t bh, int32_t n_tokens, int32_t head_dim,
                       const int32_t* labels, int32_t n_clusters, float* means, int32_t* counts,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!dtype_ok(dtype)) return SVG2_ERR_INVALID_ARG;
  if (!shape_ok(bh, n_tokens, n_clusters)) return SVG2_ERR_INVALID_ARG;
  if (!dim_ok(head_dim)) return SVG2_ERR_UNSUPPORTED;
  if (!x || !labels || !means || !counts || !aligned(x, 16) || !aligned(labels, 4) || !aligned(means, 4) ||
      !aligned(counts, 4))
    return SVG2_ERR_INVALID_ARG;
  const size_t need = svg2_cluster_means_workspace_size(bh, n_tokens, head_dim, n_clusters);
  if (workspace_bytes < need || !workspace) return SVG2_ERR_WORKSPACE;
  if (!aligned(workspace, kAlign)) return SVG2_ERR_INVALID_ARG;
  Carve c(workspace);
  int32_t* hist = c.take<int32_t>((size_t)bh * sort_chunks(n_tokens) * n_clusters);
  int32_t* perm = c.take<int32_t>((size_t)bh * n_tokens);
  int32_t* offsets = c.take<int32_t>((size_t)bh * (n_clusters + 1));
  double* partial = c.take<double>((size_t)bh * (n_clusters + mean_chunks(n_tokens)) * head_dim);
  int st = hip_status(launch_counting_sort(labels, bh, n_tokens, n_clusters, hist, false, perm, offsets, counts,
                                           stream));
  if (st) return st;
  return hip_status(launch_centroid_mean(x, dtype == SVG2_BF16, bh, n_tokens, head_dim, n_clusters, perm, offsets,
                                         partial, means, stream));
}

int svg2_recall_mass(const float* lse_sel, const float* lse_all, int32_t bh, int32_t n_tokens,
                     double* mean_recall, hipStream_t stream) {
  if (bh < 1 || n_tokens < 1 || n_tokens > kMaxTokens) return SVG2_ERR_INVALID_ARG;
  if (!lse_sel || !lse_all || !mean_recall || !aligned(lse_sel, 4) || !aligned(lse_all, 4) ||
      !aligned(mean_recall, 8))
    return SVG2_ERR_INVALID_ARG;
  return hip_status(launch_recall_mass(lse_sel, lse_all, bh, n_tokens, mean_recall, stream));
}

}  // extern "C"
