// Semantic-aware permutation: stable counting sort of cluster labels and the
// row gathers / scatters that move Q, K, V into contiguous cluster blocks and
// the output back ("Sparse VideoGen2" wiki summary, Method, stage (2)).
//
// Sort: (1) per-chunk label histograms in LDS, (2) per cluster (one thread
// each) the column of chunk counts becomes the chunk-relative start slots and
// the cluster total, (3) one work-group per problem scans the totals into
// cluster offsets, (4) one wave per chunk walks its tokens in order and places
// each at offset[label] + start[chunk][label] + rank, the rank among equal
// labels coming from wave ballots.
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

// One thread per (problem, cluster): the cluster's counts in every chunk are
// replaced by the number of its tokens in the earlier chunks; the total goes
// to `counts`.  Consecutive threads read consecutive clusters of a chunk row.
__global__ __launch_bounds__(256) void k_sort_columns(int n, int nchunks, int32_t* __restrict__ hist,
                                                      int32_t* __restrict__ counts) {
  const int p = blockIdx.y;
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= n) return;
  int32_t* h = hist + (size_t)p * nchunks * n + c;
  int run = 0;
  int ch = 0;
  for (; ch + 4 <= nchunks; ch += 4) {
    const int v0 = h[(size_t)ch * n], v1 = h[(size_t)(ch + 1) * n];
    const int v2 = h[(size_t)(ch + 2) * n], v3 = h[(size_t)(ch + 3) * n];
    h[(size_t)ch * n] = run;
    h[(size_t)(ch + 1) * n] = run + v0;
    h[(size_t)(ch + 2) * n] = run + v0 + v1;
    h[(size_t)(ch + 3) * n] = run + v0 + v1 + v2;
    run += v0 + v1 + v2 + v3;
  }
  for (; ch < nchunks; ++ch) {
    const int v = h[(size_t)ch * n];
    h[(size_t)ch * n] = run;
    run += v;
  }
  counts[(size_t)p * n + c] = run;
}

// One work-group of 1024 threads per problem: exclusive scan of the cluster
// totals (thread i owns clusters 4i..4i+3).
__global__ __launch_bounds__(1024) void k_sort_offsets(int n, const int32_t* __restrict__ counts,
                                                       int32_t* __restrict__ offsets) {
  __shared__ int32_t scratch[17];
  const int p = blockIdx.x;
  int tot[4];
  int local = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int c = 4 * threadIdx.x + e;
    tot[e] = c < n ? counts[(size_t)p * n + c] : 0;
    local += tot[e];
  }
  int total;
  int run = block_exclusive_scan(local, scratch, &total);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int c = 4 * threadIdx.x + e;
    if (c < n) offsets[(size_t)p * (n + 1) + c] = run;
    run += tot[e];
  }
  if (threadIdx.x == 0) offsets[(size_t)p * (n + 1) + n] = total;
}

// One wave per chunk: stable placement.  The first slot of each cluster inside
// this chunk is its offset plus its count in the earlier chunks.
__global__ __launch_bounds__(64) void k_sort_place(const int32_t* __restrict__ labels, int N, int n,
                                                   int nchunks, int nbits,
                                                   const int32_t* __restrict__ start,
                                                   const int32_t* __restrict__ offsets,
                                                   int32_t* __restrict__ perm) {
  extern __shared__ int32_t cnt[];
  const int chunk = blockIdx.x, p = blockIdx.y;
  const int lane = threadIdx.x;
  const int32_t* st = start + ((size_t)p * nchunks + chunk) * n;
  const int32_t* off = offsets + (size_t)p * (n + 1);
  for (int c = lane; c < n; c += kWave) cnt[c] = off[c] + st[c];
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
  hipLaunchKernelGGL(k_sort_columns, dim3((n + 255) / 256, bh), dim3(256), 0, s, n, nchunks, hist_ws, counts);
  hipLaunchKernelGGL(k_sort_offsets, dim3(bh), dim3(1024), 0, s, n, counts, offsets);
  hipLaunchKernelGGL(k_sort_place, dim3(nchunks, bh), dim3(64), lds, s, labels, N, n, nchunks, nbits,
                     hist_ws, offsets, perm);
  return hipGetLastError();
}

// ---------------------------------------------------------------- row moves
// Rows are moved as 16-byte vectors: V = row bytes / 16 lanes cooperate on a
// row, so reads and writes of a row are contiguous.  A work-group takes
// kMoveRows consecutive rows of one problem (grid y = problem) and each lane
// keeps kMoveUnroll rows' loads in flight before storing them.
constexpr int kMoveRows = 128;
constexpr int kMoveUnroll = 4;

struct RowMove {
  const char* src[2];
  char* dst[2];
};

template <int NT, bool GATHER>
__global__ __launch_bounds__(256) void k_move_rows(RowMove mv, int vec_per_row, int vec_shift, int N,
                                                   int heads, int64_t sb, int64_t sh, int64_t st,
                                                   const int32_t* __restrict__ perm) {
  // sb/sh/st are strided-side strides in BYTES; the contiguous side is [bh, N, row]
  const int p = blockIdx.y;
  const int64_t row_bytes = (int64_t)vec_per_row * 16;
  const int sub = threadIdx.x & (vec_per_row - 1);
  const int r0 = threadIdx.x >> vec_shift;
  const int rows_per_pass = blockDim.x >> vec_shift;
  const int64_t sbase = (int64_t)(p / heads) * sb + (int64_t)(p % heads) * sh + sub * 16;
  const int64_t pbase = (int64_t)p * N * row_bytes + sub * 16;
  const int32_t* pp = perm + (size_t)p * N;
  const int i_end = min(N, (int)(blockIdx.x + 1) * kMoveRows);
  for (int i0 = blockIdx.x * kMoveRows + r0; i0 < i_end; i0 += rows_per_pass * kMoveUnroll) {
    int j[kMoveUnroll];
    u32x4_t val[kMoveUnroll][NT];
#pragma unroll
    for (int u = 0; u < kMoveUnroll; ++u) {
      const int i = i0 + u * rows_per_pass;
      j[u] = i < i_end ? pp[i] : -1;
      if ((unsigned)j[u] >= (unsigned)N) j[u] = -1;
    }
#pragma unroll
    for (int u = 0; u < kMoveUnroll; ++u) {
      if (j[u] < 0) continue;
      const int i = i0 + u * rows_per_pass;
      const int64_t from = GATHER ? sbase + (int64_t)j[u] * st : pbase + (int64_t)i * row_bytes;
#pragma unroll
      for (int t = 0; t < NT; ++t) val[u][t] = *reinterpret_cast<const u32x4_t*>(mv.src[t] + from);
    }
#pragma unroll
    for (int u = 0; u < kMoveUnroll; ++u) {
      if (j[u] < 0) continue;
      const int i = i0 + u * rows_per_pass;
      const int64_t to = GATHER ? pbase + (int64_t)i * row_bytes : sbase + (int64_t)j[u] * st;
#pragma unroll
      for (int t = 0; t < NT; ++t) *reinterpret_cast<u32x4_t*>(mv.dst[t] + to) = val[u][t];
    }
  }
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
  sb *= esize; sh *= esize; st *= esize;
  const dim3 grid((N + kMoveRows - 1) / kMoveRows, bh);
  if (n_tensors == 1)
    hipLaunchKernelGGL((k_move_rows<1, true>), grid, dim3(256), 0, s, mv, vpr, shift, N, heads, sb, sh, st,
                       perm);
  else
    hipLaunchKernelGGL((k_move_rows<2, true>), grid, dim3(256), 0, s, mv, vpr, shift, N, heads, sb, sh, st,
                       perm);
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
  sb *= esize; sh *= esize; st *= esize;
  const dim3 grid((N + kMoveRows - 1) / kMoveRows, bh);
  hipLaunchKernelGGL((k_move_rows<1, false>), grid, dim3(256), 0, s, mv, vpr, shift, N, heads, sb, sh, st,
                     perm);
  return hipGetLastError();
}

}  // namespace svg2
