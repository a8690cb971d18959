// Host-side launchers of the SVG2 kernels (internal to libsvg2).
#pragma once
#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace svg2 {

// the thread's SVG2_ERR_HIP cause, as svg2_last_hip_error() reports it
void record_hip_error(int e);

constexpr int kMaxClusters = 4096;
constexpr int kSortChunk = 1024;             // tokens per counting-sort chunk
__host__ __device__ inline int sort_chunks(int n_tokens) { return (n_tokens + kSortChunk - 1) / kSortChunk; }

// ----------------------------------------------------------------- sort.hip
// Stable counting sort of labels [bh, N] in [0, n): perm, offsets [bh, n+1],
// counts [bh, n] (required).  hist_ws holds bh * sort_chunks(N) * n ints.
// With have_hist the chunk histograms are already in hist_ws (the bf16
// assignment adds them, after a k_prep_centroids that cleared them);
// otherwise the sort builds them.
hipError_t launch_counting_sort(const int32_t* labels, int bh, int N, int n, int32_t* hist_ws, bool have_hist,
                                int32_t* perm, int32_t* offsets, int32_t* counts, hipStream_t s);
// dst[t][p][i][:] = src[t] row perm[p][i] of problem p (strided source), t < n_tensors <= 2.
hipError_t launch_gather_rows(int n_tensors, const void* const* src, void* const* dst, int esize,
                              int d, int bh, int N, int heads, int64_t sb, int64_t sh, int64_t st,
                              const int32_t* perm, hipStream_t s);
// dst row perm[p][i] of problem p (strided) = src[p][i] (contiguous).
hipError_t launch_scatter_rows(const void* src, void* dst, int esize, int d, int bh, int N,
                               int heads, int64_t sb, int64_t sh, int64_t st, const int32_t* perm,
                               hipStream_t s);

// --------------------------------------------------------------- kmeans.hip
// k-means++ seeding (two kernels per pick).  d2_ws: bh*N doubles; near_ws:
// bh*N ints of space, holding bh*N 16-bit nearest-pick numbers; picks_ws: bh*n ints;
// cc_ws: bh*n doubles; bsum_ws: bh*ceil(N/256) doubles.  Writes centroids
// [bh,n,d] fp32 and seed_index [bh,n] (may be null).
hipError_t launch_kmeanspp(const void* x, bool bf16, int bh, int N, int d, int n, uint64_t seed,
                           double* d2_ws, int32_t* near_ws, float* centroids, int32_t* seed_index,
                           int32_t* picks_ws, double* cc_ws, double* bsum_ws, hipStream_t s);
// Labels of the first Lloyd round after seeding: each token's nearest pick,
// from near_ws as left by launch_kmeanspp.
hipError_t launch_labels_from_seeding(const int32_t* near_ws, int bh, int N, int32_t* labels, hipStream_t s);
// centroid split for the matrix-core assignment: c_hi + c_lo (bf16 pair) and ||c||^2,
// kCentroidPad-row padded per problem (padding rows: zeros, ||c||^2 = +inf)
constexpr int kCentroidPad = 32;
__host__ __device__ inline int centroid_rows(int n) { return (n + kCentroidPad - 1) / kCentroidPad * kCentroidPad; }
// What the prep clears for the round's assignment and sort: the near-tie
// counts [bh] and the chunk histograms (hist_words ints).
struct SortStart {
  int32_t* fix_count;
  int32_t* hist;
  size_t hist_words;
};
hipError_t launch_prep_centroids(const float* c, int bh, int n, int d, uint16_t* c_hi,
                                 uint16_t* c_lo, float* c_norm, const SortStart& st, hipStream_t s);
// Near ties of the bf16 assignment, decided again in fp64: count [bh], token
// and dmin [bh, N] (the listed tokens and their smallest matrix-core distance);
// hist: the counting sort's chunk histograms, which the assignment fills.
struct AsgFixWs {
  int32_t* count;
  int32_t* token;
  float* dmin;
  int32_t* hist;
};
hipError_t launch_assign(const void* x, bool bf16, int bh, int N, int d, int n, const float* c,
                         const uint16_t* c_hi, const uint16_t* c_lo, const float* c_norm,
                         int32_t* labels, float* min_dist, const AsgFixWs& fw, hipStream_t s);
// centroid c = mean of the rows perm[offsets[c] .. offsets[c+1]); empty keeps c.
// partial_ws: bh * (n + mean_chunks(N)) * d doubles.
constexpr int kMeanChunk = 512;              // sorted positions per partial-sum work-group
inline int mean_chunks(int n_tokens) { return (n_tokens + kMeanChunk - 1) / kMeanChunk; }
// Rows moved by the centroid update: row perm[r] of x (and of y, if given)
// stored to row r of x_out (y_out).  With amax set (bf16 inputs only) the
// rows are stored as E4M3 bytes scaled by 448 / max|.|, amax[p] for x and
// amax[bh + p] for y, and x_scale / y_scale[p] receive the dequantization
// scales.  x_out == nullptr: no move.
struct MeanMove {
  void* x_out = nullptr;
  const void* y = nullptr;
  void* y_out = nullptr;
  const uint32_t* amax = nullptr;
  float* x_scale = nullptr;
  float* y_scale = nullptr;
};
hipError_t launch_centroid_mean(const void* x, bool bf16, int bh, int N, int d, int n,
                                const int32_t* perm, const int32_t* offsets, double* partial_ws, float* c,
                                hipStream_t s, const MeanMove& mv = MeanMove{});
// max|x| per problem of a bf16 [bh, N, d] tensor, as float bits in amax_ws[bh]
hipError_t launch_amax_bf16(const void* x, int bh, int N, int d, uint32_t* amax_ws, hipStream_t s);

// --------------------------------------------------------------- select.hip
hipError_t launch_select_topp(const float* cq, const int32_t* q_counts, int n_q, const float* ck,
                              const int32_t* k_counts, int n_k, int bh, int d, double scale,
                              double top_p, int32_t* sel_count, int32_t* sel_idx, float* probs,
                              int64_t* row_pairs_ws, double* logits_ws, int64_t* pair_count, hipStream_t s);

// ----------------------------------------------------------------- attn.hip
int attn_block_rows(bool bf16);
inline int attn_max_items(int N, int n_q, int bm) { return (N + bm - 1) / bm + n_q; }
// Attention work lists, carved from the caller's workspace (all int32).  The
// bf16 kernel takes its items from per-XCD queues: xitems/xcount hold each
// head's items per XCD, flat the queue of each XCD (heads in order, pairs of
// (head, item)), queue each XCD's next-item counter and item total.
constexpr int kAttnXcds = 8;
struct AttnWs {
  int32_t* tiles;        // [bh, n_q] key tiles per Q-cluster
  int32_t* item_count;   // [bh] items per head
  int32_t* items;        // [bh, attn_max_items(N, n_q, smallest row block)]
  int32_t* xitems;       // [bh, kAttnXcds, attn_max_items(N, n_q, 128)]
  int32_t* xcount;       // [bh, kAttnXcds]
  int32_t* queue;        // [2 kAttnXcds]
  int32_t* flat;         // [kAttnXcds, bh * attn_max_items(N, n_q, 128), 2]
  uint32_t* kmax;        // [bh] largest squared key norm per problem (fp32 bits)
};
// Where the attention writes output row r of problem p: row t = perm[p, r]
// (r itself when perm is null) at element offset (p / heads) * bs +
// (p % heads) * hs + t * ts; lse at p * N + t.  A row with t outside
// [0, N) is not written.
struct OutMap {
  const int32_t* perm;
  int heads;
  int64_t bs, hs, ts;
};
inline OutMap contiguous_out(int N, int d) { return OutMap{nullptr, 1, (int64_t)N * d, 0, d}; }
hipError_t launch_varblock_attn(const void* q, const void* k, const void* v, bool bf16, int bh,
                                int N, int d, const int32_t* q_off, int n_q, const int32_t* k_off,
                                int n_k, const int32_t* sel_count, const int32_t* sel_idx,
                                float scale, void* out, float* lse, const OutMap& om, const AttnWs& ws,
                                hipStream_t s);

// FP8 (E4M3) Q, K, V with per-problem scales, head_dim 128, bf16 output; the
// same workspace as launch_varblock_attn (row block kAttnBM).
hipError_t launch_varblock_attn_fp8(const void* q, const void* k, const void* v, const float* q_scale,
                                    const float* k_scale, const float* v_scale, int bh, int N,
                                    const int32_t* q_off, int n_q, const int32_t* k_off, int n_k,
                                    const int32_t* sel_count, const int32_t* sel_idx, float scale, void* out,
                                    float* lse, const OutMap& om, const AttnWs& ws, hipStream_t s);

// ---------------------------------------------------------------- quant.hip
// x8 = E4M3(x / scale), scale[p] = max|x_p| / 448 (1 if all zero); x bf16
// [bh, N, d]; amax_ws: bh words.
hipError_t launch_quantize_fp8(const void* x, int bh, int N, int d, uint8_t* x8, float* scale, uint32_t* amax_ws,
                               hipStream_t s);

// --------------------------------------------------------------- recall.hip
// mean_recall[p] = mean over rows with lse_all > -inf of exp(lse_sel - lse_all).
hipError_t launch_recall_mass(const float* lse_sel, const float* lse_all, int bh, int N, double* mean_recall,
                              hipStream_t s);

}  // namespace svg2
