// Centroid-based attention-score estimation and top-p selection ("Sparse
// VideoGen2" wiki summary, Method, stage (3); Key claims, §4.2, Eq. 1, Eq. 2).
//
// All in fp64.  k_select_logits: logit_ij = scale * cq_i . ck_j for a block of
// kLogitRows Q-clusters per work-group, so each K-centroid row is read once per
// block.  k_select_topp, one work-group per (Q-cluster, problem):
//   w_j = |K_j| exp(logit_j - max), P_j = w_j / sum w
// over non-empty K-clusters, a bitonic sort by (-P, j) (sel_sort), a prefix sum of
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

// Bitonic sort of npad (key, id) pairs by sel_before, EPT consecutive entries
// per thread in registers (entry a = thread * EPT + m).  A compare-exchange of
// entries a and a ^ jj is done in registers when jj < EPT, across lanes by
// shuffles when the partner is in the same wave, and through LDS (sP, sJ,
// with two barriers) otherwise, which happens only in the last few stages.
// Each entry's slot keeps the earlier of the pair when its slot is the lower
// one of an ascending pair or the upper one of a descending pair.  Entries
// that compare equal are identical padding, so copying one over the other
// loses nothing.
template <int EPT>
__device__ __forceinline__ void sel_sort(double (&P)[EPT], int (&J)[EPT], int npad, double* sP, int32_t* sJ) {
  const int t = threadIdx.x;
  const bool live = t * EPT < npad;
  for (int k = 2; k <= npad; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      if (jj < EPT) {
#pragma unroll
        for (int m = 0; m < EPT; ++m) {
          const int m2 = m ^ jj;
          if ((m & jj) == 0 && m2 < EPT) {
            const bool asc = ((t * EPT + m) & k) == 0;
            if (asc ? sel_before(P[m2], J[m2], P[m], J[m]) : sel_before(P[m], J[m], P[m2], J[m2])) {
              const double tp = P[m]; P[m] = P[m2]; P[m2] = tp;
              const int tj = J[m]; J[m] = J[m2]; J[m2] = tj;
            }
          }
        }
      } else if (jj < kWave * EPT) {
        const int lm = jj / EPT;
#pragma unroll
        for (int m = 0; m < EPT; ++m) {
          const double pp = __shfl_xor(P[m], lm);
          const int pj = __shfl_xor(J[m], lm);
          const int a = t * EPT + m;
          const bool want_first = ((a & jj) == 0) == ((a & k) == 0);
          if (want_first != sel_before(P[m], J[m], pp, pj)) {
            P[m] = pp;
            J[m] = pj;
          }
        }
      } else {
        if (live)
#pragma unroll
          for (int m = 0; m < EPT; ++m) {
            sP[t * EPT + m] = P[m];
            sJ[t * EPT + m] = J[m];
          }
        __syncthreads();
        if (live)
#pragma unroll
          for (int m = 0; m < EPT; ++m) {
            const int a = t * EPT + m;
            const double pp = sP[a ^ jj];
            const int pj = sJ[a ^ jj];
            const bool want_first = ((a & jj) == 0) == ((a & k) == 0);
            if (want_first != sel_before(P[m], J[m], pp, pj)) {
              P[m] = pp;
              J[m] = pj;
            }
          }
        __syncthreads();
      }
    }
  }
  if (live)
#pragma unroll
    for (int m = 0; m < EPT; ++m) {
      sP[t * EPT + m] = P[m];
      sJ[t * EPT + m] = J[m];
    }
  __syncthreads();
}

// The same network with every compare-exchange through LDS (npad / 2 pairs
// per stage, a barrier after each stage), for lists longer than the register
// version holds.
__device__ __noinline__ void sel_sort_shared(int npad, double* sP, int32_t* sJ) {
  for (int k = 2; k <= npad; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int x = threadIdx.x; x < npad / 2; x += kSelThreads) {
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
}

template <int EPT>
__device__ __forceinline__ void sel_sort_lds(int npad, double* sP, int32_t* sJ) {
  double P[EPT];
  int J[EPT];
  const int t = threadIdx.x;
#pragma unroll
  for (int m = 0; m < EPT; ++m) {
    const int a = t * EPT + m;
    P[m] = a < npad ? sP[a] : -2.0;
    J[m] = a < npad ? sJ[a] : INT_MAX;
  }
  sel_sort<EPT>(P, J, npad, sP, sJ);
}

// Logits of kLogitRows Q-clusters against every K-cluster of problem p.  The
// dot product is summed in one fixed order: 16 chunks of D/16 consecutive
// elements, each a running sum from its first product (the products of fp32
// values are exact in fp64), then the chunk sums pairwise as a butterfly
// (chunk k with k + 8, then the results 4 apart, 2 apart, 1 apart):
//   A_k = p_k + p_{k+8},  dot = ((A0 + A4) + (A2 + A6)) + ((A1 + A5) + (A3 + A7)).
// Lane (key row, Q row): the kLogitRows lanes of one key row read the same
// addresses, so each K-centroid row is fetched once per work-group.
constexpr int kLogitRows = 8;

template <int D>
__global__ __launch_bounds__(kSelThreads) void k_select_logits(const float* __restrict__ cq, int n_q,
                                                               const float* __restrict__ ck, int n_k,
                                                               double scale, double* __restrict__ logits) {
  constexpr int C = D / 16;                          // elements per chunk
  // rows padded by 16 bytes: the kLogitRows rows read at one offset fall in
  // different LDS banks
  __shared__ double s_q[kLogitRows][D + 2];
  const int i0 = blockIdx.x * kLogitRows, p = blockIdx.y;
  const int rows = min(kLogitRows, n_q - i0);
  for (int e = threadIdx.x; e < kLogitRows * D; e += kSelThreads) {
    const int r = e / D, c = e % D;
    s_q[r][c] = r < rows ? (double)cq[((size_t)p * n_q + i0 + r) * D + c] : 0.0;
  }
  __syncthreads();
  const int r = threadIdx.x % kLogitRows;
  const double* q = s_q[r];
  for (int j = threadIdx.x / kLogitRows; j < n_k; j += kSelThreads / kLogitRows) {
    const float* kr = ck + ((size_t)p * n_k + j) * D;
    auto A = [&](int k) {                            // p_k + p_{k+8}
      double lo = 0.0, hi = 0.0;
#pragma unroll
      for (int e = 0; e < C; ++e) {
        lo = fma((double)kr[k * C + e], q[k * C + e], lo);
        hi = fma((double)kr[(k + 8) * C + e], q[(k + 8) * C + e], hi);
      }
      return lo + hi;
    };
    const double a0 = A(0), a4 = A(4), a2 = A(2), a6 = A(6);
    const double c0 = (a0 + a4) + (a2 + a6);
    const double a1 = A(1), a5 = A(5), a3 = A(3), a7 = A(7);
    const double c1 = (a1 + a5) + (a3 + a7);
    if (r < rows) logits[((size_t)p * n_q + i0 + r) * n_k + j] = scale * (c0 + c1);
  }
}

__global__ __launch_bounds__(kSelThreads) void k_select_topp(
    const double* __restrict__ logits, const int32_t* __restrict__ q_counts, int n_q,
    const int32_t* __restrict__ k_counts, int n_k, int npad, double top_p,
    int32_t* __restrict__ sel_count, int32_t* __restrict__ sel_idx, float* __restrict__ probs,
    int64_t* __restrict__ row_pairs) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  double* sP = reinterpret_cast<double*>(smem);                 // [npad]
  int32_t* sJ = reinterpret_cast<int32_t*>(sP + npad);          // [npad]
  uint8_t* sF = reinterpret_cast<uint8_t*>(sJ + npad);          // [npad]
  __shared__ double s_red[17];
  __shared__ int64_t s_ired[17];
  __shared__ int s_cut;

  const int i = blockIdx.x, p = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int32_t* kn = k_counts + (size_t)p * n_k;
  const double* lg = logits + ((size_t)p * n_q + i) * n_k;
  if (tid == 0) s_cut = INT_MAX;
  for (int j = tid; j < n_k; j += kSelThreads) sP[j] = lg[j];
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
  switch (npad / kSelThreads) {
    case 0:
    case 1: sel_sort_lds<1>(npad, sP, sJ); break;
    case 2: sel_sort_lds<2>(npad, sP, sJ); break;
    case 4: sel_sort_lds<4>(npad, sP, sJ); break;
    default: sel_sort_shared(npad, sP, sJ); break;   // more than 1024 K-clusters
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
                              int64_t* row_pairs_ws, double* logits_ws, int64_t* pair_count, hipStream_t s) {
  int npad = 64;
  while (npad < n_k) npad <<= 1;
  const size_t lds = (size_t)npad * (sizeof(double) + sizeof(int32_t) + 1);
  const dim3 lgrid((n_q + kLogitRows - 1) / kLogitRows, bh);
  if (d == 128)
    hipLaunchKernelGGL(k_select_logits<128>, lgrid, dim3(kSelThreads), 0, s, cq, n_q, ck, n_k, scale, logits_ws);
  else
    hipLaunchKernelGGL(k_select_logits<64>, lgrid, dim3(kSelThreads), 0, s, cq, n_q, ck, n_k, scale, logits_ws);
  hipLaunchKernelGGL(k_select_topp, dim3(n_q, bh), dim3(kSelThreads), lds, s, logits_ws, q_counts, n_q, k_counts,
                     n_k, npad, top_p, sel_count, sel_idx, probs, row_pairs_ws);
  if (pair_count) hipLaunchKernelGGL(k_pair_sum, dim3(bh), dim3(256), 0, s, row_pairs_ws, n_q, pair_count);
  return hipGetLastError();
}

}  // namespace svg2
