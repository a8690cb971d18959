/*
 * svg2.h - C ABI of the SVG2 semantic-aware-permutation sparse attention path
 * for AMD Instinct MI355X (gfx950).
 *
 * The operations follow the method as the page "Sparse VideoGen2: Accelerate
 * Video Generation with Sparse Attention via Semantic-Aware Permutation" (a
 * paper-wiki summary) states it, per attention head and layer:
 *   svg2_kmeans        k-means on the Q tokens or the K tokens, seeded by
 *                      k-means++ or warm-started from cached centroids
 *                      [Method, stage (1); Key claims, §4.1, §4.3 / Fig. 7(a)]
 *   svg2_permute       reorder rows into contiguous cluster blocks; K and V
 *                      share one permutation   [Method, stage (2)]
 *   svg2_select_topp   centroid-based score estimate weighted by cluster
 *                      size, top-p K-cluster selection per Q-cluster
 *                      [Method, stage (3); Key claims, §4.2, Eq. 1, Eq. 2]
 *   svg2_varblock_attn attention over variable-sized cluster blocks with no
 *                      padding to a fixed block size
 *                      [Method, stage (4); Key claims, §4.3 / Fig. 7(b)]
 *   svg2_unpermute     the inverse permutation of the output rows
 *                      [Method, stage (2)]
 * an FP8 variant of the attention (svg2_quantize_fp8, svg2_varblock_attn_fp8),
 * and, beside the path, two analysis calls (cluster means of given labels,
 * and the attention mass a selection recalls) for the identification study.
 *
 * Conventions shared by every call
 *   - Tensor arguments are DEVICE pointers allocated by the caller, 16-byte
 *     aligned.  Head_dim is innermost.  "bh" is batch * heads: the calls
 *     batch independent (batch, head) problems.
 *   - Ownership: every buffer belongs to the caller; the library keeps no
 *     pointer after a call returns and holds no state between calls.
 *   - Every call is asynchronous on `stream` (0 = the null stream); none
 *     allocates device memory, frees or synchronises.  Buffers must stay
 *     alive until the queued work has finished.
 *   - Errors: a call returns SVG2_OK or an error status.  All arguments are
 *     validated on the host before any HIP call; on an error nothing is
 *     enqueued.  A failing kernel launch returns SVG2_ERR_HIP and
 *     svg2_last_hip_error() gives the hipError_t (per thread).
 *   - Workspace: calls that need scratch memory take (workspace,
 *     workspace_bytes); svg2_*_workspace_size gives the minimum.  Its content
 *     on entry does not matter and on exit is unspecified.
 *   - Results are bitwise reproducible run to run (no floating-point atomics).
 *   - Supported: head_dim 64 or 128; dtype fp32 or bf16; 1 <= n_clusters <=
 *     min(n_tokens, 4096); 1 <= n_tokens < 2^24.
 */
#ifndef SVG2_H
#define SVG2_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum svg2_status {
  SVG2_OK = 0,
  SVG2_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, size out of range  */
  SVG2_ERR_UNSUPPORTED = 2,   /* valid but unsupported shape or dtype        */
  SVG2_ERR_WORKSPACE = 3,     /* workspace smaller than *_workspace_size()   */
  SVG2_ERR_HIP = 4            /* a HIP call failed; see svg2_last_hip_error  */
} svg2_status;

typedef enum svg2_dtype {
  SVG2_F32 = 0,               /* IEEE binary32                               */
  SVG2_BF16 = 1               /* bfloat16 (upper half of a binary32)         */
} svg2_dtype;

const char* svg2_version(void);
const char* svg2_status_string(int status);
int svg2_last_hip_error(void);

/* ------------------------------------------------------------------------
 * svg2_kmeans - k-means of the rows of x, independently for each of the bh
 * problems  [Method, stage (1); Key claims, §4.3 / Fig. 7(a)].
 *
 *   x               [bh, n_tokens, head_dim] dtype, contiguous.
 *   init_centroids  [bh, n_clusters, head_dim] fp32 (warm start, the centroid
 *                   cache of the previous denoising step), or NULL: cold start
 *                   by k-means++ (first centre floor(u_0 N), each further
 *                   centre the smallest token t whose running sum of D^2
 *                   exceeds u_k * sum D^2, D^2 = squared distance to the
 *                   nearest chosen centre; u_k = top 53 bits of
 *                   splitmix64(seed ^ (problem * 2^32 + k)) * 2^-53).
 *   n_iters         T in [0, 100] Lloyd rounds, each = assign every token to
 *                   its nearest centroid (squared Euclidean, ties to the lowest
 *                   index), then set every non-empty centroid to the mean of
 *                   its members (an empty one keeps its value).  T = 0 only
 *                   seeds (or copies init_centroids).
 *   centroids       out [bh, n_clusters, head_dim] fp32; may alias
 *                   init_centroids (in-place cache update).
 *   labels          out [bh, n_tokens] int32: labels of the T-th assignment
 *                   (not written when T = 0; may then be NULL).
 *   counts          out [bh, n_clusters] int32: member counts of those labels
 *                   (not written when T = 0; may then be NULL).
 *   min_dist        out [bh, n_tokens] fp32 or NULL: ||x - c_label||^2 at the
 *                   T-th assignment.
 *   seed_index      out [bh, n_clusters] int32 or NULL: token index of each
 *                   k-means++ pick (cold start only).
 * ---------------------------------------------------------------------- */
size_t svg2_kmeans_workspace_size(int32_t bh, int32_t n_tokens, int32_t head_dim,
                                  int32_t n_clusters);
int svg2_kmeans(const void* x, int32_t dtype, int32_t bh, int32_t n_tokens,
                int32_t head_dim, int32_t n_clusters, int32_t n_iters,
                const float* init_centroids, uint64_t seed,
                float* centroids, int32_t* labels, int32_t* counts,
                float* min_dist, int32_t* seed_index,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * svg2_kmeans_permute - svg2_kmeans followed by the permutation of its
 * final labels (svg2_permute), in one call: the last Lloyd round's centroid
 * update reads every row in cluster order anyway, and stores it there too
 * [Method, stages (1) and (2)].
 *
 *   x, dtype ... seed_index   as for svg2_kmeans; n_iters must be >= 1.
 *   y               [bh, n_tokens, head_dim] dtype, contiguous, or NULL: a
 *                   second tensor permuted the same way (V beside K).
 *   x_perm          out [bh, n_tokens, head_dim]: row i = row perm[i] of x.
 *   y_perm          out, the same for y; NULL exactly when y is NULL.
 *   perm, offsets   out [bh, n_tokens] / [bh, n_clusters + 1] int32, as
 *                   svg2_permute gives them for the returned labels.
 *   workspace       svg2_kmeans_workspace_size bytes.
 * Outputs must not overlap the inputs or each other.  Every output equals,
 * bit for bit, svg2_kmeans followed by svg2_permute of its labels.
 * ---------------------------------------------------------------------- */
int svg2_kmeans_permute(const void* x, const void* y, int32_t dtype, int32_t bh,
                        int32_t n_tokens, int32_t head_dim, int32_t n_clusters,
                        int32_t n_iters, const float* init_centroids, uint64_t seed,
                        float* centroids, int32_t* labels, int32_t* counts,
                        float* min_dist, int32_t* seed_index, void* x_perm,
                        void* y_perm, int32_t* perm, int32_t* offsets,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* svg2_kmeans_permute_fp8 - svg2_kmeans_permute on bf16 inputs whose
 * permuted copies are stored as E4M3 bytes, for the FP8 attention [Method,
 * stages (1) and (2)]: x8_perm, x_scale (and y8_perm, y_scale) are, bit for
 * bit, svg2_quantize_fp8 of the bf16 rows svg2_kmeans_permute would write
 * (the per-problem max|.| does not depend on the row order, so it is taken
 * from x and y before the clustering starts).
 *
 *   x8_perm, y8_perm  out [bh, n_tokens, head_dim] uint8 (E4M3).
 *   x_scale, y_scale  out [bh] fp32 dequantization scales.
 *   y, y8_perm and y_scale are all NULL or all given.  Other arguments as for
 *   svg2_kmeans_permute (dtype is bf16; min_dist and seed_index are not
 *   offered).  Workspace: svg2_kmeans_workspace_size bytes. */
int svg2_kmeans_permute_fp8(const void* x, const void* y, int32_t bh, int32_t n_tokens,
                            int32_t head_dim, int32_t n_clusters, int32_t n_iters,
                            const float* init_centroids, uint64_t seed, float* centroids,
                            int32_t* labels, int32_t* counts, void* x8_perm, float* x_scale,
                            void* y8_perm, float* y_scale, int32_t* perm, int32_t* offsets,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * svg2_permute - build the permutation of each problem from its cluster
 * labels and gather rows into contiguous cluster blocks; with n_tensors = 2
 * the same permutation is applied to both (K and V)  [Method, stage (2)].
 *
 *   labels          [bh, n_tokens] int32 in [0, n_clusters).  A label out of
 *                   range is clamped into it (memory stays safe; the result
 *                   is then unspecified).
 *   src[t]          host array of n_tensors device pointers; element (p, i, e)
 *                   of source t is at
 *                   src[t] + (p / heads) * src_b_stride + (p % heads) *
 *                   src_h_stride + i * src_token_stride + e   (in elements),
 *                   which covers [B,H,N,d] and [B,N,H,d] layouts.
 *   dst[t]          host array of device pointers, contiguous
 *                   [bh, n_tokens, head_dim].
 *   perm            out [bh, n_tokens] int32: perm[i] = original token placed
 *                   at slot i; clusters in ascending label order, tokens of a
 *                   cluster in ascending original index.
 *   offsets         out [bh, n_clusters + 1] int32: cluster c occupies slots
 *                   [offsets[c], offsets[c+1]).
 * Strides must be multiples of 16 bytes / element size.
 * ---------------------------------------------------------------------- */
size_t svg2_permute_workspace_size(int32_t bh, int32_t n_tokens, int32_t n_clusters);
int svg2_permute(const int32_t* labels, int32_t bh, int32_t n_tokens,
                 int32_t n_clusters, int32_t n_tensors, const void* const* src,
                 int32_t heads, int64_t src_b_stride, int64_t src_h_stride,
                 int64_t src_token_stride, void* const* dst, int32_t dtype,
                 int32_t head_dim, int32_t* perm, int32_t* offsets,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * svg2_select_topp - per Q-cluster i, estimate the attention mass of every
 * K-cluster j from the centroids and choose the fewest K-clusters whose
 * estimated mass reaches top_p  [Method, stage (3); Key claims, §4.2].
 *
 *   l_ij = scale * cq_i . ck_j;  w_ij = |K_j| exp(l_ij - max_l l_il) over
 *   non-empty K-clusters;  P_ij = w_ij / sum_l w_il.  Sort by (-P, j), keep
 *   the shortest prefix whose running sum is >= top_p (top_p >= 1 keeps every
 *   non-empty cluster).  Computed in fp64.
 *
 *   q_centroids     [bh, n_q, head_dim] fp32;  q_counts [bh, n_q] int32.
 *   k_centroids     [bh, n_k, head_dim] fp32;  k_counts [bh, n_k] int32.
 *   scale           > 0 (the pipeline uses 1/sqrt(head_dim)); top_p in (0, 1].
 *   sel_count       out [bh, n_q] int32.
 *   sel_idx         out [bh, n_q, n_k] int32: row i holds the sel_count[i]
 *                   chosen K-clusters in ascending order; the rest of the row
 *                   is left unspecified.
 *   probs           out [bh, n_q, n_k] fp32 or NULL: P (0 for empty clusters).
 *   pair_count      out [bh] int64 or NULL: sum_i |Q_i| sum_{j in S_i} |K_j|.
 * ---------------------------------------------------------------------- */
size_t svg2_select_topp_workspace_size(int32_t bh, int32_t n_q, int32_t n_k);
int svg2_select_topp(const float* q_centroids, const int32_t* q_counts, int32_t n_q,
                     const float* k_centroids, const int32_t* k_counts, int32_t n_k,
                     int32_t bh, int32_t head_dim, float scale, float top_p,
                     int32_t* sel_count, int32_t* sel_idx, float* probs,
                     int64_t* pair_count, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/* ------------------------------------------------------------------------
 * svg2_varblock_attn - block-sparse attention over variable-sized cluster
 * blocks of permuted Q', K', V'  [Method, stage (4); Key claims, §4.3].
 *
 *   Row r of Q-cluster i (r in [q_offsets[i], q_offsets[i+1])) attends to the
 *   key rows of its selected K-clusters, K(i) = union over j in S_i of
 *   [k_offsets[j], k_offsets[j+1]):
 *     out_r = sum_{u in K(i)} softmax_u(scale * q_r . k_u) v_u,
 *     lse_r = log sum_{u in K(i)} exp(scale * q_r . k_u)   (natural log).
 *   A row whose selection holds no key gets out = 0, lse = -inf.
 *   bf16: products on bf16 matrix cores with fp32 accumulation, softmax in
 *   fp32, probabilities rounded to bf16 before the P.V product, output
 *   rounded to bf16.  fp32: fp32 throughout.
 *
 *   q, k, v         [bh, n_tokens, head_dim] dtype, contiguous (permuted).
 *   q_offsets       [bh, n_q + 1], k_offsets [bh, n_k + 1] int32 (monotone,
 *                   0 .. n_tokens).
 *   sel_count       [bh, n_q] int32; sel_idx [bh, n_q, n_k] int32 (indices in
 *                   [0, n_k); order is free; a repeated index is attended twice).
 *   out             out [bh, n_tokens, head_dim] dtype, permuted order.
 *   lse             out [bh, n_tokens] fp32 or NULL.
 * Dense attention is the special case n_q = n_k = 1, offsets {0, N}, sel {0}.
 * ---------------------------------------------------------------------- */
size_t svg2_varblock_attn_workspace_size(int32_t bh, int32_t n_tokens, int32_t n_q,
                                         int32_t n_k, int32_t head_dim);
int svg2_varblock_attn(const void* q, const void* k, const void* v, int32_t dtype,
                       int32_t bh, int32_t n_tokens, int32_t head_dim,
                       const int32_t* q_offsets, int32_t n_q,
                       const int32_t* k_offsets, int32_t n_k,
                       const int32_t* sel_count, const int32_t* sel_idx, float scale,
                       void* out, float* lse, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* ------------------------------------------------------------------------
 * svg2_varblock_attn_unpermute - svg2_varblock_attn with the inverse
 * permutation fused into its output stores  [Method, stages (2) and (4)]:
 * the same values as svg2_varblock_attn into a buffer followed by
 * svg2_unpermute of that buffer, without the pass over it.
 *
 *   Output row r of problem p (permuted order) goes to token t = perm[p, r]:
 *   element e at dst + (p / heads) * dst_b_stride + (p % heads) *
 *   dst_h_stride + t * dst_token_stride + e (strides in elements, multiples of
 *   16 bytes; heads divides bh); lse, if not NULL, [bh, n_tokens] fp32 at
 *   p * n_tokens + t.  perm is [bh, n_tokens] int32, a permutation of
 *   0..n_tokens-1 (a row whose index is out of range is not written).
 *   The other arguments and the workspace are those of svg2_varblock_attn.
 * ---------------------------------------------------------------------- */
int svg2_varblock_attn_unpermute(const void* q, const void* k, const void* v, int32_t dtype,
                                 int32_t bh, int32_t n_tokens, int32_t head_dim,
                                 const int32_t* q_offsets, int32_t n_q,
                                 const int32_t* k_offsets, int32_t n_k,
                                 const int32_t* sel_count, const int32_t* sel_idx, float scale,
                                 const int32_t* perm, void* dst, int32_t heads,
                                 int64_t dst_b_stride, int64_t dst_h_stride,
                                 int64_t dst_token_stride, float* lse, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * svg2_varblock_attn_noalloc - svg2_varblock_attn with no workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, serving loops that must not call hipMalloc, harnesses that
 * forbid it.  Same arguments (minus workspace), same results, same kernels.
 *
 *   Scratch: a fixed array of svg2_varblock_attn_noalloc_max_scratch() bytes
 *   (16 MiB) inside the library, one per GPU, held until the process ends;
 *   its device address is resolved on the first call on each device.  The
 *   call allocates and frees nothing.
 *   Limit: a problem whose svg2_varblock_attn_workspace_size exceeds that
 *   size returns SVG2_ERR_WORKSPACE before any HIP call (at head_dim 128 and
 *   400 / 1000 clusters: 24 x 118,800 tokens needs 3.2 MiB, 40 x 75,600
 *   needs 3.9 MiB).  Argument errors are those of svg2_varblock_attn.
 *   Concurrency: every call on one GPU uses that GPU's one array, so calls
 *   that overlap on one GPU (several streams or threads) race; calls queued
 *   in order on one stream are safe.  Nothing needs clearing between calls.
 * ---------------------------------------------------------------------- */
size_t svg2_varblock_attn_noalloc_max_scratch(void);
int svg2_varblock_attn_noalloc(const void* q, const void* k, const void* v, int32_t dtype,
                               int32_t bh, int32_t n_tokens, int32_t head_dim,
                               const int32_t* q_offsets, int32_t n_q,
                               const int32_t* k_offsets, int32_t n_k,
                               const int32_t* sel_count, const int32_t* sel_idx, float scale,
                               void* out, float* lse, hipStream_t stream);

/* ------------------------------------------------------------------------
 * svg2_unpermute - scatter rows back to the original token order:
 * dst row perm[i] = src row i  [Method, stage (2)].
 *
 *   src             [bh, n_tokens, head_dim] dtype, contiguous.
 *   perm            [bh, n_tokens] int32, a permutation of 0..n_tokens-1 (an
 *                   index out of range is skipped).
 *   dst             element (p, t, e) at dst + (p / heads) * dst_b_stride +
 *                   (p % heads) * dst_h_stride + t * dst_token_stride + e.
 * ---------------------------------------------------------------------- */
int svg2_unpermute(const void* src, int32_t dtype, int32_t bh, int32_t n_tokens,
                   int32_t head_dim, const int32_t* perm, void* dst, int32_t heads,
                   int64_t dst_b_stride, int64_t dst_h_stride, int64_t dst_token_stride,
                   hipStream_t stream);

/* ------------------------------------------------------------------------
 * FP8 attention (the project README's open-source plan, "Support FP8
 * attention"): E4M3 copies of the permuted Q', K', V' with one scale per
 * problem and tensor, then the variable-block attention on them.
 *
 * svg2_quantize_fp8 - x8 = E4M3(x * r_p) with r_p = 448 / max|x_p| and the
 * dequantization scale[p] = max|x_p| / 448 (both correctly rounded fp32; 1
 * for an all-zero problem).  The product is taken in fp32 and clamped to
 * +-448, the conversion rounds to nearest even (OCP E4M3: bias 7, largest
 * finite 448, subnormals kept).
 *
 *   x               [bh, n_tokens, head_dim] bf16, contiguous.
 *   x8              out [bh, n_tokens, head_dim] E4M3 bytes.
 *   scale           out [bh] fp32.
 *   workspace       svg2_quantize_fp8_workspace_size(bh) bytes.
 * ---------------------------------------------------------------------- */
size_t svg2_quantize_fp8_workspace_size(int32_t bh);
int svg2_quantize_fp8(const void* x, int32_t bh, int32_t n_tokens, int32_t head_dim, void* x8, float* scale,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/* svg2_varblock_attn_fp8 - svg2_varblock_attn on E4M3 inputs, head_dim 128
 * only [Method, stage (4)]: S = (q8 . k8) * q_scale * k_scale on the fp8
 * matrix cores (fp32 accumulation), softmax in fp32, probabilities rounded
 * to E4M3 before the P.V product (they are at most 2^8), O = (P v8) *
 * v_scale / row sum (the row sum adds the fp32 probabilities), stored bf16.
 * Arguments as for svg2_varblock_attn, plus the three [bh] fp32 scales; the
 * workspace is svg2_varblock_attn_workspace_size's.  Head_dim other than 128
 * returns SVG2_ERR_UNSUPPORTED. */
int svg2_varblock_attn_fp8(const void* q8, const void* k8, const void* v8, const float* q_scale,
                           const float* k_scale, const float* v_scale, int32_t bh, int32_t n_tokens,
                           int32_t head_dim, const int32_t* q_offsets, int32_t n_q,
                           const int32_t* k_offsets, int32_t n_k, const int32_t* sel_count,
                           const int32_t* sel_idx, float scale, void* out, float* lse, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* svg2_varblock_attn_fp8_unpermute - svg2_varblock_attn_fp8 with the inverse
 * permutation fused into its output stores [Method, stages (2) and (4)]: the
 * same values as svg2_varblock_attn_fp8 followed by svg2_unpermute (bf16).
 * perm, dst, heads, the strides and lse as for svg2_varblock_attn_unpermute;
 * the other arguments as for svg2_varblock_attn_fp8. */
int svg2_varblock_attn_fp8_unpermute(const void* q8, const void* k8, const void* v8,
                                     const float* q_scale, const float* k_scale,
                                     const float* v_scale, int32_t bh, int32_t n_tokens,
                                     int32_t head_dim, const int32_t* q_offsets, int32_t n_q,
                                     const int32_t* k_offsets, int32_t n_k,
                                     const int32_t* sel_count, const int32_t* sel_idx,
                                     float scale, const int32_t* perm, void* dst,
                                     int32_t heads, int64_t dst_b_stride,
                                     int64_t dst_h_stride, int64_t dst_token_stride,
                                     float* lse, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/* ------------------------------------------------------------------------
 * Analysis calls beside the path (the identification-accuracy study:
 * [Key claims, §3.1 / Fig. 3; §3.2, Figs. 3-4; §5.3]).
 *
 * svg2_cluster_means - the Lloyd update on its own: per problem, the count
 * and the mean row of every label [Method, stage (1)].  With labels
 * t / block it gives the mean-pooled representatives of fixed position-based
 * blocks, the block representation whose mismatch with in-block semantics
 * the pages name as the first cause of misidentified critical tokens.
 *
 *   x               [bh, n_tokens, head_dim] dtype, contiguous.
 *   labels          [bh, n_tokens] int32 in [0, n_clusters) (out of range:
 *                   clamped; memory stays safe, the result is unspecified).
 *   means           out [bh, n_clusters, head_dim] fp32: the fp64 mean of
 *                   each label's rows, rounded to fp32.  A label with no row
 *                   keeps its previous value.
 *   counts          out [bh, n_clusters] int32.
 * ---------------------------------------------------------------------- */
size_t svg2_cluster_means_workspace_size(int32_t bh, int32_t n_tokens, int32_t head_dim,
                                         int32_t n_clusters);
int svg2_cluster_means(const void* x, int32_t dtype, int32_t bh, int32_t n_tokens, int32_t head_dim,
                       const int32_t* labels, int32_t n_clusters, float* means, int32_t* counts,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * svg2_recall_mass - the share of each query row's exact softmax mass that
 * a selection keeps, averaged over the rows of each problem:
 *     mean_r exp(lse_sel[r] - lse_all[r])
 * where lse_sel is the log-sum-exp over the selected keys and lse_all over
 * every key (both from svg2_varblock_attn, rows in the same order).  Rows
 * with lse_all = -inf (no key) are skipped; lse_sel = -inf counts as 0.
 * The sum runs in fp64 in a fixed order.
 *
 *   lse_sel, lse_all  [bh, n_tokens] fp32.
 *   mean_recall       out [bh] fp64 (NaN for a problem with no valid row).
 * ---------------------------------------------------------------------- */
int svg2_recall_mass(const float* lse_sel, const float* lse_all, int32_t bh, int32_t n_tokens,
                     double* mean_recall, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* SVG2_H */
