// Centroid-based attention-score estimation and top-p selection ("Sparse
// VideoGen2" wiki summary, Method, stage (3); Key claims, §4.2, Eq. 1, Eq. 2).
//
// One work-group per (Q-cluster, problem), all in fp64:
//   logit_j = scale * cq . ck_j, w_j = |K_j| exp(logit_j - max), P_j = w_j / sum w
// over non-empty K-clusters, a bitonic sort by (-P, j) in LDS, a prefix sum of
// the sorted P, the shortest prefix reaching top_p, and an ascending
// compaction of the chosen cluster ids.
#include <limits.h>

#include "common.hpp"
#include "internal.hpp"

namespace svg2 {

constexpr int kSelThreads = 256;

__device__ __forceinline__ bool sel_before(double pa, int ja, double pb, int jb) {
  return pa > pb || (pa == pb && ja < jb);
}

template <int D>
__global__ __launch_bounds__(kSelThreads) void k_select_topp(
    const float* __restrict__ cq, const int32_t* __restrict__ q_counts, int n_q,
    const float* __restrict__ ck, const int32_t* __restrict__ k_counts, int n_k, int npad,
    double scale, double top_p, int32_t* __restrict__ sel_count, int32_t* __restrict__ sel_idx,
    float* __restrict__ probs, int64_t* __restrict__ row_pairs) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  double* sP = reinterpret_cast<double*>(smem);                 // [npad]
  int32_t* sJ = reinterpret_cast<int32_t*>(sP + npad);          // [npad]
  uint8_t* sF = reinterpret_cast<uint8_t*>(sJ + npad);          // [npad]
  __shared__ double s_q[D];
  __shared__ double s_red[17];
  __shared__ int64_t s_ired[17];
  __shared__ int s_cut;

  const int i = blockIdx.x, p = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const float* kc = ck + (size_t)p * n_k * D;
  const int32_t* kn = k_counts + (size_t)p * n_k;
  for (int e = tid; e < D; e += kSelThreads) s_q[e] = (double)cq[((size_t)p * n_q + i) * D + e];
  if (tid == 0) s_cut = INT_MAX;
  __syncthreads();

  // ---- logits: 16 lanes per key centroid, 4 centroids per wave step
  constexpr int DPL = D / 16;
  const int sub = lane >> 4, sl = lane & 15;
  for (int j0 = wave * 4; j0 < n_k; j0 += 4 * (kSelThreads / kWave)) {
    const int j = j0 + sub;
    double acc = 0.0;
    if (j < n_k) {
      const float* r = kc + (size_t)j * D + sl * DPL;
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc += (double)r[e] * s_q[sl * DPL + e];
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
    if (sl == 0 && j < n_k) sP[j] = scale * acc;
  }
  __syncthreads();

  // ---- max over non-empty clusters
  double mx = -__builtin_inf();
  int ne_local = 0;
  for (int j = tid; j < n_k; j += kSelThreads)
    if (kn[j] > 0) {
      mx = fmax(mx, sP[j]);
      ++ne_local;
    }
  mx = wave_max(mx);
  if (lane == 0) s_red[wave] = mx;
  __syncthreads();
  mx = s_red[0];
  for (int w = 1; w < kSelThreads / kWave; ++w) mx = fmax(mx, s_red[w]);
  __syncthreads();
  const int64_t n_nonempty = block_sum<int64_t>((int64_t)ne_local, s_ired);

  // ---- size-weighted exponentials and their sum
  double wsum_local = 0.0;
  for (int j = tid; j < n_k; j += kSelThreads) {
    const double w = kn[j] > 0 ? (double)kn[j] * exp(sP[j] - mx) : 0.0;
    sP[j] = w;
    wsum_local += w;
  }
  const double wsum = block_sum(wsum_local, s_red);
  for (int j = tid; j < npad; j += kSelThreads) {
    double key;
    if (j >= n_k) key = -2.0;                       // padding: after everything
    else if (kn[j] > 0) key = sP[j] / wsum;
    else key = -1.0;                                // empty cluster
    if (probs && j < n_k) probs[((size_t)p * n_q + i) * n_k + j] = key > 0.0 ? (float)key : 0.f;
    sP[j] = key;
    sJ[j] = j < n_k ? j : INT_MAX;
    sF[j] = 0;
  }
  __syncthreads();

  // ---- bitonic sort by (-P, j)
  for (int k = 2; k <= npad; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int x = tid; x < npad / 2; x += kSelThreads) {
        const int a = 2 * jj * (x / jj) + (x % jj);
        const int b = a + jj;
        const double pa = sP[a], pb = sP[b];
        const int ja = sJ[a], jb = sJ[b];
        const bool up = (a & k) == 0;
        const bool swap = up ? sel_before(pb, jb, pa, ja) : sel_before(pa, ja, pb, jb);
        if (swap) {
          sP[a] = pb; sP[b] = pa;
          sJ[a] = jb; sJ[b] = ja;
        }
      }
      __syncthreads();
    }
  }

  // ---- shortest prefix with running sum >= top_p
  int count;
  if (top_p >= 1.0) {
    count = (int)n_nonempty;
  } else {
    const int per = npad / kSelThreads > 0 ? npad / kSelThreads : 1;
    const int a0 = min(tid * per, npad), a1 = min(a0 + per, npad);
    double loc = 0.0;
    for (int a = a0; a < a1; ++a)
      if (a < n_nonempty) loc += sP[a];
    double tot;
    double run = block_exclusive_scan(loc, s_red, &tot);
    for (int a = a0; a < a1 && a < n_nonempty; ++a) {
      run += sP[a];
      if (run >= top_p) {
        atomicMin(&s_cut, a);
        break;
      }
    }
    __syncthreads();
    count = s_cut == INT_MAX ? (int)n_nonempty : s_cut + 1;
  }
  for (int a = tid; a < count; a += kSelThreads) sF[sJ[a]] = 1;
  __syncthreads();

  // ---- ascending compaction of the chosen cluster ids
  const int per = (n_k + kSelThreads - 1) / kSelThreads;
  const int j0 = min(tid * per, n_k), j1 = min(j0 + per, n_k);
  int64_t c_loc = 0, keys_loc = 0;
  for (int j = j0; j < j1; ++j)
    if (sF[j]) {
      ++c_loc;
      keys_loc += kn[j];
    }
  int64_t c_tot;
  int64_t pos = block_exclusive_scan(c_loc, s_ired, &c_tot);
  int32_t* out = sel_idx + ((size_t)p * n_q + i) * n_k;
  for (int j = j0; j < j1; ++j)
    if (sF[j]) out[pos++] = j;
  const int64_t keys = block_sum(keys_loc, s_ired);
  if (tid == 0) {
    sel_count[(size_t)p * n_q + i] = count;
    row_pairs[(size_t)p * n_q + i] = keys * (int64_t)q_counts[(size_t)p * n_q + i];
  }
}

__global__ __launch_bounds__(256) void k_pair_sum(const int64_t* __restrict__ row_pairs, int n_q,
                                                  int64_t* __restrict__ pair_count) {
  __shared__ int64_t s_ired[17];
  const int p = blockIdx.x;
  int64_t s = 0;
  for (int i = threadIdx.x; i < n_q; i += 256) s += row_pairs[(size_t)p * n_q + i];
  s = block_sum(s, s_ired);
  if (threadIdx.x == 0) pair_count[p] = s;
}

hipError_t launch_select_topp(const float* cq, const int32_t* q_counts, int n_q, const float* ck,
                              const int32_t* k_counts, int n_k, int bh, int d, double scale,
                              double top_p, int32_t* sel_count, int32_t* sel_idx, float* probs,
                              int64_t* row_pairs_ws, int64_t* pair_count, hipStream_t s) {
  int npad = 64;
  while (npad < n_k) npad <<= 1;
  const size_t lds = (size_t)npad * (sizeof(double) + sizeof(int32_t) + 1);
  const dim3 grid(n_q, bh);
  if (d == 128)
    hipLaunchKernelGGL(k_select_topp<128>, grid, dim3(kSelThreads), lds, s, cq, q_counts, n_q, ck, k_counts,
                       n_k, npad, scale, top_p, sel_count, sel_idx, probs, row_pairs_ws);
  else
    hipLaunchKernelGGL(k_select_topp<64>, grid, dim3(kSelThreads), lds, s, cq, q_counts, n_q, ck, k_counts,
                       n_k, npad, scale, top_p, sel_count, sel_idx, probs, row_pairs_ws);
  if (pair_count) hipLaunchKernelGGL(k_pair_sum, dim3(bh), dim3(256), 0, s, row_pairs_ws, n_q, pair_count);
  return hipGetLastError();
}

}  // namespace svg2
