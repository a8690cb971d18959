// Identification study, beside the path: the share of each query row's exact
// softmax mass that a selection keeps ("Sparse VideoGen2" wiki summary, Key
// claims, §3.1 / Fig. 3 and §3.2, Figs. 3-4).  With lse_sel the log-sum-exp
// over the selected keys and lse_all over every key, a row keeps
// exp(lse_sel - lse_all) of its mass.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace svg2 {

constexpr int kRecallThreads = 1024;

// One work-group per problem: fp64 sum over the rows in a fixed order (each
// thread's rows in index order, then the block sum), divided by the number of
// rows that have any key.
__global__ __launch_bounds__(kRecallThreads) void k_recall_mass(const float* __restrict__ lse_sel,
                                                                const float* __restrict__ lse_all, int N,
                                                                double* __restrict__ mean_recall) {
  __shared__ double s_sum[17];
  __shared__ int s_cnt[17];
  const int p = blockIdx.x;
  const float* a = lse_sel + (size_t)p * N;
  const float* b = lse_all + (size_t)p * N;
  double sum = 0.0;
  int rows = 0;
  for (int t = threadIdx.x; t < N; t += blockDim.x) {
    const float all = b[t];
    if (!(all > -INFINITY)) continue;          // no key (or NaN): not counted
    ++rows;
    const float sel = a[t];
    if (sel > -INFINITY) sum += exp((double)sel - (double)all);
  }
  const double total = block_sum(sum, s_sum);
  const int n = block_sum(rows, s_cnt);
  if (threadIdx.x == 0) mean_recall[p] = n > 0 ? total / (double)n : (double)NAN;
}

hipError_t launch_recall_mass(const float* lse_sel, const float* lse_all, int bh, int N, double* mean_recall,
                              hipStream_t s) {
  hipLaunchKernelGGL(k_recall_mass, dim3(bh), dim3(kRecallThreads), 0, s, lse_sel, lse_all, N, mean_recall);
  return hipGetLastError();
}

}  // namespace svg2
