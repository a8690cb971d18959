// Semantic-aware permutation: stable counting sort of cluster labels and the
// row gathers / scatters that move Q, K, V into contiguous cluster blocks and
// the output back ("Sparse VideoGen2" wiki summary, Method, stage (2)).
//
// Sort: (1) per-chunk label histograms in LDS, (2) one work-group per problem
// turns them into cluster offsets and per-(chunk, cluster) start slots,
// (3) one wave per chunk walks its tokens in order and places each at
// start[label] + rank, the rank among equal labels coming from wave ballots.
// Integer only: results are exact and deterministic.
#include "common.hpp"
#include "internal.hpp"

namespace svg2 {

__global__ __launch_bounds__(256) void k_sort_hist(const int32_t* __restrict__ labels, int N, int n,
                                                   int nchunks, int32_t* __restrict__ hist) {
  extern __shared__ int32_t sh[];
  const int chunk = blockIdx.x, p = blockIdx.y;
  for (int c = threadIdx.x; c < n; c += blockDim.x) sh[c] = 0;
  __syncthreads();
  const int32_t* lab = labels + (size_t)p * N;
  const int t0 = chunk * kSortChunk, t1 = min(N, t0 + kSortChunk);
  for (int t = t0 + threadIdx.x; t < t1; t += blockDim.x) atomicAdd(&sh[clampi(lab[t], 0, n - 1)], 1);
  __syncthreads();
  int32_t* h = hist + ((size_t)p * nchunks + chunk) * n;
  for (int c = threadIdx.x; c < n; c += blockDim.x) h[c] = sh[c];
}

// One work-group of 1024 threads per problem; thread i owns clusters 4i..4i+3.
__global__ __launch_bounds__(1024) void k_sort_scan(int N, int n, int nchunks, int32_t* __restrict__ hist,
                                                    int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ counts) {
  __shared__ int32_t scratch[17];
  const int p = blockIdx.x;
  int32_t* h = hist + (size_t)p * nchunks * n;
  int tot[4];
  int local = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int c = 4 * threadIdx.x + e;
    int s = 0;
    if (c < n)
      for (int ch = 0; ch < nchunks; ++ch) s += h[(size_t)ch * n + c];
    tot[e] = s;
    local += s;
  }
  int total;
  int run = block_exclusive_scan(local, scratch, &total);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int c = 4 * threadIdx.x + e;
    if (c < n) {
      offsets[(size_t)p * (n + 1) + c] = run;
      if (counts) counts[(size_t)p * n + c] = tot[e];
      int base = run;
      for (int ch = 0; ch < nchunks; ++ch) {
        const int v = h[(size_t)ch * n + c];
        h[(size_t)ch * n + c] = base;
        base += v;
      }
      run += tot[e];
    }
  }
  if (threadIdx.x == 0) offsets[(size_t)p * (n + 1) + n] = total;
}

// One wave per chunk: stable placement.  `start` (the rewritten histogram)
// gives the first slot of each cluster inside this chunk.
__global__ __launch_bounds__(64) void k_sort_place(const int32_t* __restrict__ labels, int N, int n,
                                                   int nchunks, int nbits,
                                                   const int32_t* __restrict__ start,
                                                   int32_t* __restrict__ perm) {
  extern __shared__ int32_t cnt[];
  const int chunk = blockIdx.x, p = blockIdx.y;
  const int lane = threadIdx.x;
  const int32_t* st = start + ((size_t)p * nchunks + chunk) * n;
  for (int c = lane; c < n; c += kWave) cnt[c] = st[c];
  __syncthreads();
  const int32_t* lab = labels + (size_t)p * N;
  int32_t* out = perm + (size_t)p * N;
  const int t0 = chunk * kSortChunk, t1 = min(N, t0 + kSortChunk);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = t0; base < t1; base += kWave) {
    const int t = base + lane;
    const bool valid = t < t1;
    const int l = valid ? clampi(lab[t], 0, n - 1) : 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (l >> b) & 1;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const int rank = __popcll(peers & below);
    int pos = 0;
    if (valid) pos = cnt[l] + rank;
    // every lane has read its count before the group's last lane bumps it
    __builtin_amdgcn_wave_barrier();
    if (valid && (peers >> lane) == 1ull) cnt[l] += __popcll(peers);
    __builtin_amdgcn_wave_barrier();
    if (valid) out[pos] = t;
  }
}

hipError_t launch_counting_sort(const int32_t* labels, int bh, int N, int n, int32_t* hist_ws,
                                int32_t* perm, int32_t* offsets, int32_t* counts, hipStream_t s) {
  const int nchunks = sort_chunks(N);
  int nbits = 0;
  while ((1 << nbits) < n) ++nbits;
  const size_t lds = (size_t)n * sizeof(int32_t);
  hipLaunchKernelGGL(k_sort_hist, dim3(nchunks, bh), dim3(256), lds, s, labels, N, n, nchunks, hist_ws);
  hipLaunchKernelGGL(k_sort_scan, dim3(bh), dim3(1024), 0, s, N, n, nchunks, hist_ws, offsets, counts);
  hipLaunchKernelGGL(k_sort_place, dim3(nchunks, bh), dim3(64), lds, s, labels, N, n, nchunks, nbits,
                     hist_ws, perm);
  return hipGetLastError();
}

// ---------------------------------------------------------------- row moves
// Rows are moved as 16-byte vectors; V = row bytes / 16 lanes cooperate on a
// row, so reads and writes of a row are contiguous.
struct RowMove {
  const char* src[2];
  char* dst[2];
};

template <int NT, bool GATHER>
__global__ __launch_bounds__(256) void k_move_rows(RowMove mv, int vec_per_row, int vec_shift, int bh,
                                                   int N, int heads, int64_t sb, int64_t sh,
                                                   int64_t st, const int32_t* __restrict__ perm) {
  // sb/sh/st are strided-side strides in BYTES; the contiguous side is [bh, N, row]
  const int64_t row_bytes = (int64_t)vec_per_row * 16;
  const int64_t total = (int64_t)bh * N * vec_per_row;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total;
       g += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = g >> vec_shift;             // p * N + i
    const int v = (int)(g & (vec_per_row - 1));
    const int p = (int)(row / N);
    const int j = perm[row];
    if ((unsigned)j >= (unsigned)N) continue;
    const int64_t strided = (int64_t)(p / heads) * sb + (int64_t)(p % heads) * sh + (int64_t)j * st + v * 16;
    const int64_t packed = row * row_bytes + v * 16;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (GATHER) {
        const u32x4_t val = *reinterpret_cast<const u32x4_t*>(mv.src[t] + strided);
        *reinterpret_cast<u32x4_t*>(mv.dst[t] + packed) = val;
      } else {
        const u32x4_t val = *reinterpret_cast<const u32x4_t*>(mv.src[t] + packed);
        *reinterpret_cast<u32x4_t*>(mv.dst[t] + strided) = val;
      }
    }
  }
}

static int grid_for(int64_t work) {
  int64_t blocks = (work + 255) / 256;
  const int64_t cap = 256 * 64;     // enough resident waves to saturate HBM
  return (int)(blocks < cap ? (blocks < 1 ? 1 : blocks) : cap);
}

hipError_t launch_gather_rows(int n_tensors, const void* const* src, void* const* dst, int esize,
                              int d, int bh, int N, int heads, int64_t sb, int64_t sh, int64_t st,
                              const int32_t* perm, hipStream_t s) {
  RowMove mv{};
  for (int t = 0; t < n_tensors; ++t) {
    mv.src[t] = static_cast<const char*>(src[t]);
    mv.dst[t] = static_cast<char*>(dst[t]);
  }
  const int vpr = d * esize / 16;
  int shift = 0;
  while ((1 << shift) < vpr) ++shift;
  const int64_t work = (int64_t)bh * N * vpr;
  sb *= esize; sh *= esize; st *= esize;
  if (n_tensors == 1)
    hipLaunchKernelGGL((k_move_rows<1, true>), dim3(grid_for(work)), dim3(256), 0, s, mv, vpr, shift,
                       bh, N, heads, sb, sh, st, perm);
  else
    hipLaunchKernelGGL((k_move_rows<2, true>), dim3(grid_for(work)), dim3(256), 0, s, mv, vpr, shift,
                       bh, N, heads, sb, sh, st, perm);
  return hipGetLastError();
}

hipError_t launch_scatter_rows(const void* src, void* dst, int esize, int d, int bh, int N,
                               int heads, int64_t sb, int64_t sh, int64_t st, const int32_t* perm,
                               hipStream_t s) {
  RowMove mv{};
  mv.src[0] = static_cast<const char*>(src);
  mv.dst[0] = static_cast<char*>(dst);
  const int vpr = d * esize / 16;
  int shift = 0;
  while ((1 << shift) < vpr) ++shift;
  const int64_t work = (int64_t)bh * N * vpr;
  sb *= esize; sh *= esize; st *= esize;
  hipLaunchKernelGGL((k_move_rows<1, false>), dim3(grid_for(work)), dim3(256), 0, s, mv, vpr, shift, bh,
                     N, heads, sb, sh, st, perm);
  return hipGetLastError();
}

}  // namespace svg2
