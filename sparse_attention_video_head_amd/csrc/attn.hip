// Block-sparse attention over variable-sized cluster blocks ("Sparse
// VideoGen2" wiki summary, Method, stage (4); Key claims, §4.3 / Fig. 7(b)).
//
// Work item = (problem, Q-cluster i, 128-row slab of that cluster).  The key
// list of item i is the concatenation of the key ranges of its selected
// K-clusters; it is walked in tiles of 32 keys (bf16; 64 for FP8) that may
// straddle cluster boundaries, so the only padding is the tail of the whole
// list (and of the query slab), not a round-up of every cluster to a fixed
// block size.
//
// bf16 kernel, one wave = 32 query rows, 4 waves share each K/V tile in LDS:
//   S^T = K Q^T        v_mfma_f32_32x32x16_bf16, K tile from LDS, Q in registers
//   online softmax     fp32, base 2 (scale * log2 e folded in), per lane: one
//                      query, 16 of the tile's keys; one cross-half exchange
//                      for the max; the row sum adds the bf16-rounded P that
//                      weight V, so the normaliser is the sum of the weights.
//                      Where the Cauchy-Schwarz bound of a wave's scores is
//                      small, the reference is fixed at that bound and no
//                      maximum is taken (k_key_norm_max gives max ||k||).
//   O^T += V^T P^T     P re-used straight from the S accumulator (no shuffle):
//                      the key order inside each 16-key MFMA step is permuted,
//                      and V^T is staged in LDS in the same permuted order.
#include <math.h>

#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace svg2 {

constexpr int kAttnBM = 128;     // query rows per work item (bf16 kernel)
constexpr int kAttnBN = 32;      // keys per tile (bf16 kernel)
constexpr int kAttnF32BM = 64;   // query rows per work item (fp32 kernel)

int attn_block_rows(bool bf16) { return bf16 ? kAttnBM : kAttnF32BM; }

// ---------------------------------------------------------------- planning
// The items of one problem differ in length by orders of magnitude (a Q-cluster
// may select a handful of keys or nearly all of them), and the launch ends
// with its slowest work-group.  The plan therefore hands out the items of each
// problem longest key list first, so that the short ones fill the tail.
//
// Key tiles per Q-cluster: one wave per cluster, capped at kSortTilesMax for
// the sort key.
constexpr int kSortTilesMax = (1 << 19) - 1;

__global__ __launch_bounds__(256) void k_attn_lengths(const int32_t* __restrict__ k_off, int n_k, int N,
                                                      const int32_t* __restrict__ sel_count,
                                                      const int32_t* __restrict__ sel_idx, int n_q,
                                                      int tile, int32_t* __restrict__ tiles,
                                                      uint32_t* __restrict__ kmax) {
  const int p = blockIdx.y;
  if (kmax && blockIdx.x == 0 && threadIdx.x == 0) kmax[p] = 0u;    // for k_key_norm_max
  const int i = blockIdx.x * (blockDim.x / kWave) + (int)(threadIdx.x / kWave);
  if (i >= n_q) return;
  const int lane = lane_id();
  const int32_t* ko = k_off + (size_t)p * (n_k + 1);
  const int32_t* sel = sel_idx + ((size_t)p * n_q + i) * n_k;
  const int cnt = clampi(sel_count[(size_t)p * n_q + i], 0, n_k);
  long long keys = 0;
  for (int j = lane; j < cnt; j += kWave) {
    const int c = sel[j];
    if ((unsigned)c < (unsigned)n_k) {
      const int a = clampi(ko[c], 0, N);
      keys += clampi(ko[c + 1], a, N) - a;
    }
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) keys += __shfl_xor(keys, o);
  if (lane == 0) tiles[(size_t)p * n_q + i] = (int32_t)min((keys + tile - 1) / tile, (long long)kSortTilesMax);
}

// Largest squared key norm of each problem, for the bf16 kernel's fixed
// softmax reference (below): 2048 rows per work-group, D/8 lanes per row
// (16 bytes each), 8 rows' loads in flight per lane, fp32 sums of the squares,
// the work-group's maximum in LDS, then one atomic max per work-group on the
// value's bits (non-negative floats order like their bit patterns).  Atomics
// on one address are served one at a time, so there are few of them.
constexpr int kNormRows = 2048;

template <int D>
__global__ __launch_bounds__(256) void k_key_norm_max(const uint16_t* __restrict__ K, int N,
                                                      uint32_t* __restrict__ kmax) {
  constexpr int LPR = D / 8;                 // lanes per row
  constexpr int RPP = 256 / LPR;             // rows per pass of the work-group
  const int p = blockIdx.y;
  const int sub = threadIdx.x % LPR;
  const uint16_t* Kp = K + (size_t)p * N * D;
  float best = 0.f;
  const int rb = blockIdx.x * kNormRows + (int)threadIdx.x / LPR;
#pragma unroll 8
  for (int it = 0; it < kNormRows / RPP; ++it) {
    const int r = rb + it * RPP;
    u32x4_t w = {0u, 0u, 0u, 0u};
    if (r < N) w = *reinterpret_cast<const u32x4_t*>(Kp + (size_t)r * D + sub * 8);
    float s2 = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = bf16_lo(w[e]), b = bf16_hi(w[e]);
      s2 = fmaf(a, a, s2);
      s2 = fmaf(b, b, s2);
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) s2 += __shfl_xor(s2, m);
    best = fmaxf(best, s2);
  }
#pragma unroll
  for (int m = kWave / 2; m >= 1; m >>= 1) best = fmaxf(best, __shfl_xor(best, m));
  __shared__ float s_best[256 / kWave];
  if (lane_id() == 0) s_best[threadIdx.x / kWave] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 256 / kWave; ++w) best = fmaxf(best, s_best[w]);
    atomicMax(kmax + p, __float_as_uint(best));
  }
}

// Clusters of problem p in decreasing order of key tiles (ties: lower cluster
// index first): a bitonic sort in LDS of (tiles << 12 | 4095 - cluster); the
// padding entries (0) end up past n_q because every real entry is positive.
__device__ __forceinline__ void sort_clusters(uint32_t* order, const int32_t* tiles_p, int n_q) {
  int P = 64;
  while (P < n_q) P <<= 1;
  for (int i = threadIdx.x; i < P; i += blockDim.x)
    order[i] = i < n_q ? ((uint32_t)tiles_p[i] << 12) | (uint32_t)(kMaxClusters - 1 - i) : 0u;
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int t = threadIdx.x; t < P / 2; t += blockDim.x) {
        const int a = 2 * t - (t & (j - 1));
        const int b = a + j;
        const uint32_t x = order[a], y = order[b];
        const bool first_larger = (a & k) == 0;
        if (first_larger ? x < y : x > y) {
          order[a] = y;
          order[b] = x;
        }
      }
      __syncthreads();
    }
  }
}

// One work-group per problem: the list of (cluster, slab) items, clusters in
// decreasing order of key tiles.
__global__ __launch_bounds__(1024) void k_attn_plan(const int32_t* __restrict__ q_off, int n_q, int N,
                                                    int bm, int max_items,
                                                    const int32_t* __restrict__ tiles,
                                                    int32_t* __restrict__ item_count,
                                                    int32_t* __restrict__ items) {
  __shared__ int32_t scratch[17];
  __shared__ uint32_t order[kMaxClusters];
  const int p = blockIdx.x;
  const int32_t* qo = q_off + (size_t)p * (n_q + 1);
  sort_clusters(order, tiles + (size_t)p * n_q, n_q);
  int nb[4], cl[4];
  int local = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int s = 4 * threadIdx.x + e;
    nb[e] = 0;
    cl[e] = 0;
    if (s < n_q) {
      const int i = kMaxClusters - 1 - (int)(order[s] & (kMaxClusters - 1));
      const int a = clampi(qo[i], 0, N), b = clampi(qo[i + 1], a, N);
      nb[e] = (b - a + bm - 1) / bm;
      cl[e] = i;
    }
    local += nb[e];
  }
  int total;
  int base = block_exclusive_scan(local, scratch, &total);
  int32_t* it = items + (size_t)p * max_items;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    for (int r = 0; r < nb[e] && base < max_items; ++r, ++base) it[base] = cl[e] | (r << 12);
  if (threadIdx.x == 0) item_count[p] = min(total, max_items);
}

// Per-XCD work lists.  Each XCD has its own L2, and the slabs of one Q-cluster
// read the same key list, so a Q-cluster's slabs go to one XCD, where they run
// side by side and share that list through the L2.  Work of an item in tiles:
// its key tiles plus a fixed cost for its start (Q rows, the first tiles'
// latency) and end.
constexpr int kItemOverheadTiles = 4;

// One work-group per problem: clusters longest first, each to the least
// loaded XCD so far (all its slabs), the items kept in that order per XCD.
// The greedy pass is sequential (one wave, in registers); the slab counts
// before it and the item writes after it are parallel.
__global__ __launch_bounds__(1024) void k_attn_plan_xcd(const int32_t* __restrict__ q_off, int n_q, int N,
                                                        int bm, int max_items,
                                                        const int32_t* __restrict__ tiles,
                                                        int32_t* __restrict__ xcount,
                                                        int32_t* __restrict__ xitems) {
  __shared__ uint32_t order[kMaxClusters];
  __shared__ int s_nb[kMaxClusters];            // slabs of sorted cluster s, then its XCD and first slot
  const int p = blockIdx.x;
  const int32_t* qo = q_off + (size_t)p * (n_q + 1);
  sort_clusters(order, tiles + (size_t)p * n_q, n_q);
  for (int s = threadIdx.x; s < n_q; s += blockDim.x) {
    const int i = kMaxClusters - 1 - (int)(order[s] & (kMaxClusters - 1));
    const int a = clampi(qo[i], 0, N), b = clampi(qo[i + 1], a, N);
    s_nb[s] = (b - a + bm - 1) / bm;
  }
  __syncthreads();
  if (threadIdx.x < kWave) {
    // wave 0: the greedy pass over 64 clusters at a time, their slab and tile
    // counts read from the lanes; the XCD loads and counts stay in registers
    const int lane = threadIdx.x;
    long long load[kAttnXcds];
    int cnt[kAttnXcds];
#pragma unroll
    for (int y = 0; y < kAttnXcds; ++y) {
      load[y] = 0;
      cnt[y] = 0;
    }
    for (int s0 = 0; s0 < n_q; s0 += kWave) {
      const int sl = s0 + lane;
      const int nb_l = sl < n_q ? s_nb[sl] : 0;
      const int t_l = sl < n_q ? (int)(order[sl] >> 12) : 0;
      int code_l = -1;
      const int m = min(kWave, n_q - s0);
      for (int j = 0; j < m; ++j) {
        const int nb = __builtin_amdgcn_readlane(nb_l, j);
        const int t = __builtin_amdgcn_readlane(t_l, j);
        int x = 0;
        long long lx = load[0];
#pragma unroll
        for (int y = 1; y < kAttnXcds; ++y)
          if (load[y] < lx) {
            lx = load[y];
            x = y;
          }
        int first = 0;
#pragma unroll
        for (int y = 0; y < kAttnXcds; ++y)
          if (y == x) {
            first = cnt[y];
            if (nb > 0) load[y] += (long long)nb * (t + kItemOverheadTiles);
            cnt[y] = min(first + nb, max_items);
          }
        if (lane == j) code_l = nb > 0 ? (x << 24) | first : -1;   // first < max_items < 2^24
      }
      if (sl < n_q) s_nb[sl] = code_l;
    }
    if (lane == 0) {
#pragma unroll
      for (int y = 0; y < kAttnXcds; ++y) xcount[p * kAttnXcds + y] = cnt[y];
    }
  }
  __syncthreads();
  int32_t* out = xitems + (size_t)p * kAttnXcds * max_items;
  for (int s = threadIdx.x; s < n_q; s += blockDim.x) {
    const int code = s_nb[s];
    if (code < 0) continue;
    const int i = kMaxClusters - 1 - (int)(order[s] & (kMaxClusters - 1));
    const int a = clampi(qo[i], 0, N), b = clampi(qo[i + 1], a, N);
    const int nb = (b - a + bm - 1) / bm;
    const int x = code >> 24, first = code & 0xffffff;
    for (int r = 0; r < nb && first + r < max_items; ++r) out[(size_t)x * max_items + first + r] = i | (r << 12);
  }
}

// One work-group per XCD: that XCD's queue, the problems' lists in problem
// order as (problem, item) pairs, so that all XCDs work through the problems
// together (one problem's K and V stay in the last-level cache); resets the
// queue's counter and sets its item total.
__global__ __launch_bounds__(256) void k_attn_flatten(const int32_t* __restrict__ xcount,
                                                      const int32_t* __restrict__ xitems, int bh, int max_items,
                                                      int32_t* __restrict__ flat, int32_t* __restrict__ queue) {
  const int x = blockIdx.x;
  int32_t* f = flat + (size_t)x * bh * max_items * 2;
  int off = 0;
  for (int p = 0; p < bh; ++p) {
    const int c = xcount[p * kAttnXcds + x];
    const int32_t* src = xitems + ((size_t)p * kAttnXcds + x) * max_items;
    for (int k = threadIdx.x; k < c; k += blockDim.x) {
      f[2 * (size_t)(off + k)] = p;
      f[2 * (size_t)(off + k) + 1] = src[k];
    }
    off += c;
  }
  if (threadIdx.x == 0) {
    queue[x] = 0;
    queue[kAttnXcds + x] = off;
  }
}

// Walks the concatenated key ranges of the selected clusters; all threads of a
// work-group advance the same cursor (uniform control flow).
struct KeyCursor {
  const int32_t* sel;
  const int32_t* koff;
  int nsel, n_k, N;
  int next, pos, rem;

  __device__ __forceinline__ void init(const int32_t* s, const int32_t* ko, int ns, int nk, int n) {
    sel = s; koff = ko; nsel = ns; n_k = nk; N = n;
    next = 0; pos = 0; rem = 0;
  }
  __device__ __forceinline__ void open_ranges() {
    while (rem == 0 && next < nsel) {
      const int j = sel[next++];
      if ((unsigned)j >= (unsigned)n_k) continue;
      const int a = clampi(koff[j], 0, N);
      pos = a;
      rem = clampi(koff[j + 1], a, N) - a;
    }
  }
  // Fills up to `tile` keys; slot_of[e] (this thread's slots) get key indices
  // or -1.  Returns the number of keys in the tile; *contiguous tells that the
  // tile is full and inside one key range (key = first key + slot).
  template <int NS>
  __device__ __forceinline__ int fill(int tile, const int (&slot_of)[NS], int (&key)[NS], bool* contiguous) {
    open_ranges();
    if (rem >= tile) {
#pragma unroll
      for (int e = 0; e < NS; ++e) key[e] = slot_of[e] >= 0 ? pos + slot_of[e] : -1;
      pos += tile;
      rem -= tile;
      *contiguous = true;
      return tile;
    }
    *contiguous = false;
#pragma unroll
    for (int e = 0; e < NS; ++e) key[e] = -1;
    int filled = 0;
    while (filled < tile) {
      if (rem == 0) {
        if (next >= nsel) break;
        const int j = sel[next++];
        if ((unsigned)j >= (unsigned)n_k) continue;
        const int a = clampi(koff[j], 0, N);
        const int b = clampi(koff[j + 1], a, N);
        pos = a;
        rem = b - a;
        continue;
      }
      const int take = min(rem, tile - filled);
#pragma unroll
      for (int e = 0; e < NS; ++e) {
        const int s = slot_of[e] - filled;
        if (s >= 0 && s < take) key[e] = pos + s;
      }
      filled += take;
      pos += take;
      rem -= take;
    }
    return filled;
  }
};

// ---------------------------------------------------------------- bf16
// Lazy rescaling: the exponentials use a reference max m_ref that only moves
// when a tile's max exceeds it by more than kLazyTau (log2 units), so P stays
// <= 2^kLazyTau and O / l are rescaled rarely.  The result is the same
// softmax; only the intermediate scaling differs.
constexpr float kLazyTau = 8.f;
// Largest score bound (log2 units) at which the bf16 kernel fixes a query's
// reference instead of tracking the running maximum.
constexpr float kFixedBound = 32.f;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) uint16_t lds_u16_t;
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// Work-group barrier for the tile loop.  The direct-to-LDS tile loads are
// ordered by explicit vmcnt waits before it; a fenced __syncthreads would also
// wait for the loads that are meant to stay in flight.  This waits for the
// wave's own LDS accesses (lgkmcnt 0) and then meets the other waves; the asm
// statement's memory clobber keeps the compiler from moving memory accesses
// across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);            // lgkmcnt(0); vmcnt, expcnt not waited for
  asm volatile("s_barrier" ::: "memory");
}

template <typename Tp>
__device__ __forceinline__ lds_u16_t* to_lds(Tp* p) {
  return (lds_u16_t*)(lds_void_t*)(void*)p;
}

// K and V tiles sit row-major in LDS, keys x D, with the 16-byte chunks of
// each row XOR-swizzled (no padding, so they can be filled by direct
// global -> LDS loads).  LDS serves a 16-byte read 16 lanes at a time and an
// 8-byte transposing read 32 lanes at a time, over 64 banks of 4 bytes:
//   K: chunk c of row r at c ^ (r % 16): the 16 rows of one pass hit 16
//      different chunk positions;
//   V: a transposing read covers 4 rows x 4 chunks per 16 lanes and two such
//      groups (columns 16 apart) per pass.  At D = 128 a row spans all 64
//      banks, so chunk c of row r sits at c ^ 4 (r % 4) and the 4 rows use 4
//      disjoint blocks of 4 chunks; at D = 64 two rows share the banks and
//      c ^ 2 (r % 4) separates rows r and r + 2.
template <int D> struct TileGeom {
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static __device__ __forceinline__ int k_chunk(int r, int c) { return c ^ (r & (CPR - 1) & 15); }
  static __device__ __forceinline__ int v_chunk(int r, int c) {
    return c ^ ((CPR == 16 ? 4 : 2) * (r & 3));
  }
};

// Key ranges of the selected K-clusters, staged in LDS this many at a time.
constexpr int kRangeChunk = 512;

// Walks the concatenated key ranges of the selected clusters from an LDS copy
// of (first key, length) per cluster.  Every thread of the work-group runs the
// same cursor on the same data (uniform control flow); staging the next chunk
// of ranges synchronises the group.
struct LdsCursor {
  const int32_t* sel;
  const int32_t* koff;
  int* s_start;
  int* s_len;
  int nsel, n_k, N;
  int base, nst, r, pos, rem;

  __device__ __forceinline__ void stage() {
    for (int i = threadIdx.x; i < nst; i += blockDim.x) {
      const int j = sel[base + i];
      int a = 0, l = 0;
      if ((unsigned)j < (unsigned)n_k) {
        a = clampi(koff[j], 0, N);
        l = clampi(koff[j + 1], a, N) - a;
      }
      s_start[i] = a;
      s_len[i] = l;
    }
    __syncthreads();
  }
  __device__ __forceinline__ void init(const int32_t* s, const int32_t* ko, int ns, int nk, int n, int* ss,
                                       int* sl) {
    sel = s; koff = ko; nsel = ns; n_k = nk; N = n; s_start = ss; s_len = sl;
    base = 0; nst = min(ns, kRangeChunk); r = 0; pos = 0; rem = 0;
    stage();
  }
  // Leaves rem > 0 unless every range has been consumed.
  __device__ __forceinline__ void open() {
    while (rem == 0) {
      if (r == nst) {
        if (base + nst >= nsel) return;
        __syncthreads();                       // all reads of this chunk are done
        base += nst;
        nst = min(nsel - base, kRangeChunk);
        r = 0;
        stage();
      }
      pos = s_start[r];
      rem = s_len[r];
      ++r;
    }
  }
  // Keys of the next tile of `tile` slots: slot_of[e] (this thread's slots)
  // get key indices or -1.  Returns the number of keys in the tile.
  template <int NS>
  __device__ __forceinline__ int fill(int tile, const int (&slot_of)[NS], int (&key)[NS]) {
    open();
    if (rem >= tile) {
#pragma unroll
      for (int e = 0; e < NS; ++e) key[e] = slot_of[e] >= 0 ? pos + slot_of[e] : -1;
      pos += tile;
      rem -= tile;
      return tile;
    }
#pragma unroll
    for (int e = 0; e < NS; ++e) key[e] = -1;
    int filled = 0;
    while (filled < tile) {
      open();
      if (rem == 0) break;
      const int take = min(rem, tile - filled);
#pragma unroll
      for (int e = 0; e < NS; ++e) {
        const int s = slot_of[e] - filled;
        if (s >= 0 && s < take) key[e] = pos + s;
      }
      filled += take;
      pos += take;
      rem -= take;
    }
    return filled;
  }
  // The next tile of `tile` rows, for a lane that loads tile rows row[q]:
  // when the tile is one run of consecutive keys inside one range, *first is
  // its first key (rkey[] is left alone), else *first = -1 and rkey[q] is the
  // key of row row[q], or -1 past the end of the list.  Returns the number of
  // keys in the tile.  The range walk is uniform (scalar); per range piece a
  // lane spends two vector ops per row.
  template <int NR>
  __device__ __forceinline__ int fill_rows(int tile, const int (&row)[NR], int (&rkey)[NR], int* first) {
    open();
    if (rem >= tile) {
      *first = pos;
      pos += tile;
      rem -= tile;
      return tile;
    }
    *first = -1;
    int c[NR];                                   // key - row of the piece holding each row
#pragma unroll
    for (int q = 0; q < NR; ++q) c[q] = 0;
    int filled = 0;
    while (filled < tile) {
      open();
      if (rem == 0) break;
      const int take = min(rem, tile - filled);
      const int cj = pos - filled;
#pragma unroll
      for (int q = 0; q < NR; ++q) c[q] = row[q] >= filled ? cj : c[q];
      filled += take;
      pos += take;
      rem -= take;
    }
#pragma unroll
    for (int q = 0; q < NR; ++q) rkey[q] = row[q] < filled ? row[q] + c[q] : -1;
    return filled;
  }
};

// One tile = 32 rows of K (or V).  Each wave fills 8 rows with direct-to-LDS
// buffer loads of 16 bytes per lane: lane -> row RPI q + lane/CPR of the
// wave's 8, 16-byte slot lane%CPR of the row (swizzled); the hardware writes
// lane i's 16 bytes at m0 + 16 i.  The buffer descriptor spans one head's rows
// (at most 2^32 bytes: N <= 2^24, D <= 128), the byte offset is 32-bit.
//
// The loads are inline assembly.  As compiler-visible loads into LDS, a
// global load would make the compiler wait for every LDS read in flight
// wherever it waits for one, and either kind makes it wait for the loads
// themselves before reads of buffers it cannot tell apart.  The kernel orders
// these loads itself: an explicit vmcnt wait for the tile, then a barrier.
typedef int i32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4_t head_rsrc(const void* base, int N, int D) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  const uint64_t bytes = (uint64_t)N * (uint64_t)D * 2u;
  i32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));   // stride 0
  r[2] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(bytes > 0xffffffffu ? 0xffffffffu : bytes));
  r[3] = 0x00020000;                                                               // raw 32-bit data
  return r;
}

// 16 bytes per lane from buffer offset voff + soff to LDS byte address
// lds + 16 * lane (lds and soff uniform).  m0 carries the LDS address; it is
// saved and restored around the load (the compiler keeps m0 for itself), and
// the load waits one cycle after m0 is written.
__device__ __forceinline__ void lds_dma16(i32x4_t rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[lds]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[vo], %[rs], %[so] offen lds\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved)
      : [lds] "s"(lds), [vo] "v"(voff), [rs] "s"(rsrc), [so] "s"(soff)
      : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// Per wave and 32-key tile the work is two matrix-core phases, S^T = K Q^T
// (D/16 MFMAs) and O^T += V^T P^T (D/16 MFMAs), with the softmax of the tile
// between them on the vector ALU.  Three work-groups share a CU (52 KB of LDS
// and at most 168 registers each), so every SIMD holds three waves and the
// matrix core of one overlaps the softmax of another.  K and V tiles go
// through a ring of 3 LDS slots (tile j in slot j % 3), loaded 2 tiles ahead:
//   step t:  load K, V of tile t+2 -> slot (t+2) % 3
//            S[t] = K[t] Q^T;  softmax;  O += V[t]^T P[t]^T
//            wait for the loads of tiles <= t+1, barrier
// The SIMD issues one instruction per cycle for its waves, and an MFMA takes
// half of its matrix-core time in issue cycles, so the vector work beside the
// MFMAs bounds the kernel: per step it is kept to the softmax itself (operand
// addresses are per-lane constants with the slot in the instructions'
// immediate offsets; a tile inside one key range is loaded with a scalar row
// offset).
// The grid is persistent (three work-groups per CU); each work-group takes
// items from its XCD's queue (a Q-cluster's slabs on one XCD, clusters longest
// first, problems in order) until every queue is empty.
template <int D>
__global__ __launch_bounds__(256, 3) void k_attn_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    int N, const int32_t* __restrict__ q_off, int n_q, const int32_t* __restrict__ k_off, int n_k,
    const int32_t* __restrict__ sel_count, const int32_t* __restrict__ sel_idx, float scale_log2,
    uint16_t* __restrict__ O, float* __restrict__ lse, OutMap om, const int32_t* __restrict__ flat,
    int32_t* __restrict__ queue, size_t cap, const uint32_t* __restrict__ kmax) {
  constexpr int BN = kAttnBN;
  constexpr int KS = D / 16;           // 16-wide k-steps of Q.K
  constexpr int DT = D / 32;           // 32-row tiles of O^T
  constexpr int CPR = D / 8;
  constexpr int RPI = kWave / CPR;
  constexpr int INS = 8 / RPI;
  constexpr int ROWB = D * 2;          // bytes per K or V row
  constexpr int SLOT = 2 * BN * ROWB;  // bytes per ring slot: K tile, then V tile
  static_assert(BN == 32 && INS >= 1 && INS <= 4, "tile geometry");
  // s_waitcnt immediates: vmcnt = the loads of one tile; expcnt and lgkmcnt
  // left at their maxima (not waited for)
  constexpr int kWaitTile = 0xF70 | (2 * INS);
  __shared__ __attribute__((aligned(16))) uint16_t sT[3 * 2 * BN * D];
  __shared__ int s_rs[kRangeChunk], s_rl[kRangeChunk];
  __shared__ int s_job[2];

  // Work items come from the queue of the XCD this work-group runs on (hardware
  // register XCC_ID), then, once it is empty, from the other XCDs' queues.
  const int xcc = __builtin_amdgcn_s_getreg((3 << 11) | 20) & (kAttnXcds - 1);
  for (int qx = 0; qx < kAttnXcds; ++qx) {
    const int x = (xcc + qx) & (kAttnXcds - 1);
    const int total_x = queue[kAttnXcds + x];
    for (;;) {
      __syncthreads();                               // the previous item is done with LDS
      if (threadIdx.x == 0) {
        const int j = atomicAdd(&queue[x], 1);
        int pj = -1, ij = 0;
        if (j < total_x) {
          pj = flat[2 * ((size_t)x * cap + j)];
          ij = flat[2 * ((size_t)x * cap + j) + 1];
        }
        s_job[0] = pj;
        s_job[1] = ij;
      }
      __syncthreads();
      const int p = s_job[0];
      if (p < 0) break;
      const int item = s_job[1];
      const int ci = item & 0xfff, rb = item >> 12;
      const int32_t* qo = q_off + (size_t)p * (n_q + 1);
      const int qa = clampi(qo[ci], 0, N), qb = clampi(qo[ci + 1], qa, N);
      const int tid = threadIdx.x, lane = tid & (kWave - 1);
      const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
      const int col = lane & 31, half = lane >> 5;
      const int row0 = qa + rb * kAttnBM + wave * 32;
      const bool active = row0 < qb;                 // this wave has query rows
      const int row = row0 + col;
      const bool row_ok = row < qb;
      const size_t base = (size_t)p * N * D;
      const i32x4_t Kr = head_rsrc(K + base, N, D);
      const i32x4_t Vr = head_rsrc(V + base, N, D);

      bf16x8_t qf[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (row_ok) v = *reinterpret_cast<const u32x4_t*>(Q + base + (size_t)row * D + ks * 16 + half * 8);
        qf[ks] = __builtin_bit_cast(bf16x8_t, v);
      }

      // this lane's tile rows (one per direct-to-LDS load)
      int trow[INS];
#pragma unroll
      for (int q = 0; q < INS; ++q) trow[q] = 8 * wave + RPI * q + lane / CPR;

      LdsCursor cur;
      cur.init(sel_idx + ((size_t)p * n_q + ci) * n_k, k_off + (size_t)p * (n_k + 1),
               clampi(sel_count[(size_t)p * n_q + ci], 0, n_k), n_k, N, s_rs, s_rl);
      // The Q rows have landed by now; saying so here, before any tile load is in
      // flight, keeps the compiler from waiting for every load (the tile loads
      // included) at the first use of Q in each step.
      __builtin_amdgcn_s_waitcnt(0xF70);

      // Softmax state.  m_ref is the reference max (log2 units); thr is the raw
      // score above which a tile moves it: (m_ref + kLazyTau) / scale_log2, kept
      // in raw units so the common path needs no multiply.  The row sum adds the
      // bf16-rounded P that feed the P.V product (two dot2 accumulators over the
      // packed pairs), so the normaliser is the sum of the weights actually used.
      float m_ref = -__builtin_inff();
      float thr = -__builtin_inff();
      const float inv_scale_log2 = 1.f / scale_log2;
      float l_a = 0.f, l_b = 0.f;                    // this lane's share of the row sum
      // Fixed reference.  Every score of this query lies in [-sbound, sbound]
      // after the scale, sbound = scale_log2 * ||q|| * max ||k|| (Cauchy-Schwarz,
      // with a margin for the matrix core's fp32 sums).  So with the reference
      // at sbound the weights 2^(s * scale_log2 - sbound) are at most 1, and the
      // largest weight of the row is at least 2^(-2 sbound).  When sbound is at
      // most kFixedBound for every query of the wave, the reference is fixed
      // there for the whole key list and the per-tile maximum is not computed
      // (the largest weight then stays above 2^-64, far from underflow).
      bool fixed_ref;
      {
        float qn = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const u32x4_t w = __builtin_bit_cast(u32x4_t, qf[ks]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float a = bf16_lo(w[e]), b = bf16_hi(w[e]);
            qn = fmaf(a, a, qn);
            qn = fmaf(b, b, qn);
          }
        }
        const auto sq = __builtin_amdgcn_permlane32_swap(__float_as_uint(qn), __float_as_uint(qn), false, false);
        qn = __uint_as_float(sq[0]) + __uint_as_float(sq[1]);
        const float sbound = scale_log2 * sqrtf(qn * __uint_as_float(kmax[p])) * (1.f + 0x1p-10f) + 0x1p-20f;
        fixed_ref = __ballot(!(sbound <= kFixedBound)) == 0ull;
        if (fixed_ref) m_ref = sbound;
      }
      f32x16_t o[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;

      // LDS byte addresses (slot 0) of the operand reads; the asm statements hide
      // their range from the compiler, which would otherwise turn the slot's add
      // into a vector op per read instead of the reads' immediate offset
      //   K (S^T = K Q^T): row col, chunk 2 ks + half
      //   V^T (transposing read): rows 4 half + (lane%16)/4 (+ 16 kk, + 8),
      //   columns dt*32 + 16 ((lane/16)%2) + 4 (lane%4); the swizzle depends on
      //   the row only through row % 4, which the added rows keep
      const uint32_t lds0 = lds_addr(sT);
      uint32_t kaddr[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        kaddr[ks] = lds0 + (uint32_t)(col * ROWB + TileGeom<D>::k_chunk(col, 2 * ks + half) * 16);
        asm volatile("" : "+v"(kaddr[ks]));
      }
      const int vr = (lane & 15) >> 2;
      const int vcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      uint32_t vaddr[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int r = 4 * half + vr, c0 = dt * 32 + vcol;
        vaddr[dt] = lds0 + (uint32_t)(BN * ROWB + r * ROWB + TileGeom<D>::v_chunk(r, c0 >> 3) * 16 + (c0 & 7) * 2);
        asm volatile("" : "+v"(vaddr[dt]));
      }
      // this lane's source offsets for its tile rows: within the tile (a run of
      // consecutive keys from a scalar first key), and the swizzled 16-byte slot
      // within the row (a tile assembled from several key ranges)
      uint32_t kl_off[INS], vl_off[INS], krun[INS], vrun[INS];
#pragma unroll
      for (int q = 0; q < INS; ++q) {
        const int r = 8 * wave + RPI * q + lane / CPR;
        kl_off[q] = (uint32_t)TileGeom<D>::k_chunk(r, lane % CPR) * 16u;
        vl_off[q] = (uint32_t)TileGeom<D>::v_chunk(r, lane % CPR) * 16u;
        krun[q] = (uint32_t)r * ROWB + kl_off[q];
        vrun[q] = (uint32_t)r * ROWB + vl_off[q];
      }
      // Loads of one tile into ring slot `s` (compile-time): 2 INS instructions
      // per wave on every path, so that the vmcnt waits count the same loads.
      auto load_tile = [&](int s, int first, const int (&key)[INS]) __attribute__((always_inline)) {
        const uint32_t kdst = lds0 + (uint32_t)(s * SLOT + 8 * wave * ROWB);
        if (first >= 0) {
          const uint32_t so = (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)first * ROWB));   // uniform
#pragma unroll
          for (int q = 0; q < INS; ++q) {
            lds_dma16(Kr, kdst + (uint32_t)(RPI * q * ROWB), krun[q], so);
            lds_dma16(Vr, kdst + (uint32_t)(BN * ROWB + RPI * q * ROWB), vrun[q], so);
          }
        } else {
#pragma unroll
          for (int q = 0; q < INS; ++q) {
            const uint32_t ro = (uint32_t)max(key[q], 0) * ROWB;
            lds_dma16(Kr, kdst + (uint32_t)(RPI * q * ROWB), ro + kl_off[q], 0u);
            lds_dma16(Vr, kdst + (uint32_t)(BN * ROWB + RPI * q * ROWB), ro + vl_off[q], 0u);
          }
        }
      };
      auto kread = [&](int s, int ks) __attribute__((always_inline)) {
        return *(const __attribute__((address_space(3))) bf16x8_t*)(uintptr_t)(kaddr[ks] + (uint32_t)(s * SLOT));
      };
      auto vread = [&](int s, int j) __attribute__((always_inline)) {
        const int kk = j / DT, dt = j % DT;
        const uint32_t a = vaddr[dt] + (uint32_t)(s * SLOT + 16 * kk * ROWB);
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(uintptr_t)a);
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(uintptr_t)(a + 8 * ROWB));
        return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };

      // S^T for the 32 keys of the K tile in slot s; lane holds query `col` and
      // keys (i/4)*8 + half*4 + i%4.  The K fragments are read kAhead k-steps
      // ahead of their MFMA, so the LDS latency overlaps the matrix core instead
      // of sitting before every step.  The scheduling groups pin that order (mask
      // 0x100: LDS reads, 0x008: MFMA); left alone, the scheduler pairs each read
      // with its MFMA and waits on it.
      auto scores = [&](int s, f32x16_t& sc) __attribute__((always_inline)) {
        constexpr int kAhead = KS < 2 ? KS : 2;
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[i] = 0.f;
        bf16x8_t a[KS];
#pragma unroll
        for (int ks = 0; ks < kAhead; ++ks) a[ks] = kread(s, ks);
        // raised issue priority while the wave feeds the matrix core, so that
        // the other waves' softmax work fills in around its MFMAs (lowered
        // again after each MFMA run)
        __builtin_amdgcn_s_setprio(1);
        __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if (ks + kAhead < KS) a[ks + kAhead] = kread(s, ks + kAhead);
          sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], qf[ks], sc, 0, 0, 0);
          if (ks + kAhead < KS) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          } else {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          }
        }
      };
      // Scores, softmax and O^T += V^T P^T of the tile in slot s.
      auto step = [&](int s, int filled, auto fixed_c) __attribute__((always_inline)) {
        f32x16_t sc;
        scores(s, sc);
        __builtin_amdgcn_s_setprio(0);
        if (filled < BN) {
          // key of score i: (i/4)*8 + 4*half + i%4; compared against the list end
          // shifted by this lane's half, so every compare takes an inline constant
          const int lim = filled - 4 * half;
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if ((i >> 2) * 8 + (i & 3) >= lim) sc[i] = -__builtin_inff();
        }
        if constexpr (!decltype(fixed_c)::value) {
          // raw max of the tile's scores for this query (v_maximum3: scores are
          // never NaN, and the NaN-propagating maximum needs no canonicalising)
          float mx = sc[0];
#pragma unroll
          for (int i = 1; i < 16; ++i) mx = __builtin_elementwise_maximum(mx, sc[i]);
          {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            mx = __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
          }
          if (mx > thr) {
            const float m_new = mx * scale_log2;
            const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
            l_a *= alpha;
            l_b *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
              for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
            m_ref = m_new;
            thr = (m_new + kLazyTau) * inv_scale_log2;
          }
        }
        const float neg = -m_ref;
        const bf16x2_t ones = __builtin_bit_cast(bf16x2_t, 0x3F803F80u);
        u32x4_t pw[2];
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[i], scale_log2, neg));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[i + 1], scale_log2, neg));
          const uint32_t w = pack_bf16x2(p0, p1);
          pw[i >> 3][(i & 7) >> 1] = w;
          if (i & 2)
            l_b = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), ones, l_b, false);
          else
            l_a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), ones, l_a, false);
        }
        // V^T fragments: two transposing reads per MFMA, issued kAhead MFMAs early
        constexpr int NV = 2 * DT;
        constexpr int kAhead = NV < 2 ? NV : 2;
        bf16x8_t va[NV];
#pragma unroll
        for (int j = 0; j < kAhead; ++j) va[j] = vread(s, j);
        __builtin_amdgcn_s_setprio(1);
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAhead, 0);
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          if (j + kAhead < NV) va[j + kAhead] = vread(s, j + kAhead);
          const int kk = j / DT, dt = j % DT;
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[j], __builtin_bit_cast(bf16x8_t, pw[kk]), o[dt], 0, 0, 0);
          if (j + kAhead < NV) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_s_setprio(0);
      };

      // tiles 0 and 1 -> slots 0 and 1.  The loads are issued even past the end
      // of the key list (all rows then read key 0 and the tile is never used), so
      // that every step has the same loads in flight.
      int key[INS];
      int first;
      int f0 = cur.fill_rows<INS>(BN, trow, key, &first);
      load_tile(0, first, key);
      int f1 = 0;
      if (f0 > 0) {
        f1 = cur.fill_rows<INS>(BN, trow, key, &first);
      } else {
        first = -1;
#pragma unroll
        for (int q = 0; q < INS; ++q) key[q] = -1;
      }
      load_tile(1, first, key);
      __builtin_amdgcn_s_waitcnt(kWaitTile);         // tile 0 has landed
      lds_barrier();

      // step t (tile t in slot s = t % 3, compile-time): load tile t+2 into slot
      // (s+2) % 3, compute tile t, wait for tile t+1, barrier
      auto iter = [&](auto sc_, auto fixed_c) __attribute__((always_inline)) -> bool {
        constexpr int s = decltype(sc_)::value;
        int f2 = 0;
        if (f1 > 0) {
          f2 = cur.fill_rows<INS>(BN, trow, key, &first);
        } else {
          first = -1;
#pragma unroll
          for (int q = 0; q < INS; ++q) key[q] = -1;
        }
        load_tile((s + 2) % 3, first, key);
        if (active) step(s, f0, fixed_c);
        __builtin_amdgcn_s_waitcnt(kWaitTile);       // tiles <= t+1 have landed
        lds_barrier();
        f0 = f1;
        f1 = f2;
        return f0 > 0;
      };
      // one loop per reference mode, so that neither carries the other's
      // registers; a work-group's waves may run different ones (the loops take
      // the same barriers in the same order)
      if (f0 > 0) {
        if (fixed_ref) {
          const std::true_type fx;
          while (iter(std::integral_constant<int, 0>{}, fx) && iter(std::integral_constant<int, 1>{}, fx) &&
                 iter(std::integral_constant<int, 2>{}, fx)) {
          }
        } else {
          const std::false_type fx;
          while (iter(std::integral_constant<int, 0>{}, fx) && iter(std::integral_constant<int, 1>{}, fx) &&
                 iter(std::integral_constant<int, 2>{}, fx)) {
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0xF70);             // no tile load outlives the loop

      // lanes i and i+32 hold the two halves of query col's keys
      float l_tot;
      {
        const float l_part = l_a + l_b;
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_part), __float_as_uint(l_part), false, false);
        l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      }
      const int tout = row_ok ? (om.perm ? om.perm[(size_t)p * N + row] : row) : -1;
      if (row_ok && (unsigned)tout < (unsigned)N) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        uint16_t* orow = O + (p / om.heads) * om.bs + (p % om.heads) * om.hs + (int64_t)tout * om.ts;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            uint2 w;
            w.x = pack_bf16x2(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv);
            w.y = pack_bf16x2(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv);
            *reinterpret_cast<uint2*>(orow + dt * 32 + g * 8 + half * 4) = w;
          }
        if (lse && half == 0)
          lse[(size_t)p * N + tout] = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * 0.69314718055994531f
                                                 : -__builtin_inff();
      }
    }  // items of queue x
  }  // queues
}

// ---------------------------------------------------------------- fp8
// FP8 (OCP E4M3) Q, K, V with one scale per problem and tensor, head_dim 128
// (the project README's open-source plan, "Support FP8 attention").  The
// same work items, key walk, LDS ring and barriers as the bf16 kernel, with
// 64-key tiles and the gfx950 matrix-core op v_mfma_*_32x32x64_f8f6f4:
//   S^T = K Q^T     two 32-key blocks x two 64-dim steps (4 MFMAs per tile)
//   softmax         fp32, as in the bf16 kernel; P rounded to E4M3 (P <= 2^8)
//   O^T += V^T P^T  one MFMA per 32-dim block of O (4 per tile)
// Lane layout of the f8 MFMA operands: lane m + 32 h holds row (or column) m
// and k = 32 h + j in byte j of its eight registers.  The P operand takes the
// S accumulators as they lie: byte 16 t + i of lane (n, h) is the probability
// of key 32 t + 8 (i / 4) + 4 h + i % 4, and the V^T operand is read in that
// key order with transposing byte reads (ds_read_b64_tr_b8: in each group of
// 16 lanes, lane i gets byte i % 8 of the 8-byte chunk addressed by lane
// 2 r + i / 8, r = 0..7).
// Rows of a tile are 128 bytes (8 chunks of 16 B); chunk c of row r sits at
// c ^ f(r), f(r) = 4 ((r >> 1) & 1) | ((r >> 2) & 3): the 16 rows of a
// 16-byte read and the 8 rows x 2 chunks of a 32-lane transposing read then
// fall on distinct banks.
constexpr int kAttnF8BN = 64;
constexpr int kAttnF8D = 128;

__device__ __forceinline__ int f8_swz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;

__device__ __forceinline__ f32x16_t mfma_f8(const i32x8_t& a, const i32x8_t& b, const f32x16_t& c) {
  // formats E4M3 x E4M3, unit block scales (exponent 127)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__global__ __launch_bounds__(256, 3) void k_attn_fp8(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
    const float* __restrict__ q_scale, const float* __restrict__ k_scale, const float* __restrict__ v_scale,
    int N, const int32_t* __restrict__ q_off, int n_q,
    const int32_t* __restrict__ k_off, int n_k, const int32_t* __restrict__ sel_count,
    const int32_t* __restrict__ sel_idx, float scale_log2, uint16_t* __restrict__ O, float* __restrict__ lse,
    OutMap om, const int32_t* __restrict__ flat, int32_t* __restrict__ queue, size_t cap) {
  constexpr int BN = kAttnF8BN;
  constexpr int D = kAttnF8D;
  constexpr int ROW = D;                         // bytes per tile row
  constexpr int kWaitTile = 0xF70 | 4;           // vmcnt: the 4 loads of one tile
  constexpr int kWaitAll = 0xF70;
  __shared__ __attribute__((aligned(16))) uint8_t sT0[2 * BN * ROW], sT1[2 * BN * ROW], sT2[2 * BN * ROW];
  __shared__ int s_rs[kRangeChunk], s_rl[kRangeChunk];
  __shared__ int s_job[2];

  // Work items come from the queue of the XCD this work-group runs on (hardware
  // register XCC_ID), then, once it is empty, from the other XCDs' queues.
  const int xcc = __builtin_amdgcn_s_getreg((3 << 11) | 20) & (kAttnXcds - 1);
  for (int qx = 0; qx < kAttnXcds; ++qx) {
    const int x = (xcc + qx) & (kAttnXcds - 1);
    const int total_x = queue[kAttnXcds + x];
    for (;;) {
      __syncthreads();                               // the previous item is done with LDS
      if (threadIdx.x == 0) {
        const int j = atomicAdd(&queue[x], 1);
        int pj = -1, ij = 0;
        if (j < total_x) {
          pj = flat[2 * ((size_t)x * cap + j)];
          ij = flat[2 * ((size_t)x * cap + j) + 1];
        }
        s_job[0] = pj;
        s_job[1] = ij;
      }
      __syncthreads();
      const int p = s_job[0];
      if (p < 0) break;
      const int item = s_job[1];
      const int ci = item & 0xfff, rb = item >> 12;
      const int32_t* qo = q_off + (size_t)p * (n_q + 1);
      const int qa = clampi(qo[ci], 0, N), qb = clampi(qo[ci + 1], qa, N);
      const int tid = threadIdx.x, lane = tid & (kWave - 1);
      const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
      const int col = lane & 31, half = lane >> 5;
      const int row0 = qa + rb * kAttnBM + wave * 32;
      const bool active = row0 < qb;
      const int row = row0 + col;
      const bool row_ok = row < qb;
      const size_t base = (size_t)p * N * D;
      const uint8_t* Kp = K + base;
      const uint8_t* Vp = V + base;
      const float sq = q_scale[p], sk = k_scale[p], sv = v_scale[p];
      const float sl2 = scale_log2 * sq * sk;

      // Q operand of S^T = K Q^T: lane (n, h) holds dims 64 kd + 32 h + 0..31 of query n
      i32x8_t qf[2];
#pragma unroll
      for (int kd = 0; kd < 2; ++kd) {
        u32x4_t a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
        if (row_ok) {
          const u32x4_t* src = reinterpret_cast<const u32x4_t*>(Q + base + (size_t)row * D + 64 * kd + 32 * half);
          a = src[0];
          b = src[1];
        }
        qf[kd] = (i32x8_t){(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
      }

      // this lane's tile rows for the direct-to-LDS loads: 16 rows per wave, 8 per load
      int slot_of[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) slot_of[q] = 16 * wave + 8 * q + lane / 8;
      uint32_t l_off[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) l_off[q] = (uint32_t)(((lane & 7) ^ f8_swz(slot_of[q])) * 16);

      LdsCursor cur;
      cur.init(sel_idx + ((size_t)p * n_q + ci) * n_k, k_off + (size_t)p * (n_k + 1),
               clampi(sel_count[(size_t)p * n_q + ci], 0, n_k), n_k, N, s_rs, s_rl);

      // softmax state as in the bf16 kernel: reference max m_ref (log2 units),
      // the raw score thr that moves it, two row-sum accumulators
      float m_ref = -__builtin_inff();
      float thr = -__builtin_inff();
      const float inv_sl2 = 1.f / sl2;
      float l_a = 0.f, l_b = 0.f;
      f32x16_t o[4];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;

      // K operand: lane (m, h) reads row 32 t + m, chunks 4 kd + 2 h + {0, 1}
      const int fc = f8_swz(col);
      uint32_t koff[2][2];
#pragma unroll
      for (int kd = 0; kd < 2; ++kd)
#pragma unroll
        for (int u = 0; u < 2; ++u) koff[kd][u] = (uint32_t)(col * ROW + ((4 * kd + 2 * half + u) ^ fc) * 16);
      // V^T operand, read q of 4 (bytes 8 q .. 8 q + 7 of the lane's operand): the
      // lane addresses row key(q, r, h) = 16 q + 8 (r / 4) + 4 h + r % 4, r = (lane % 16) / 2,
      // dims 32 dt + 16 g + 8 s .. + 8, g = (lane / 16) % 2, s = lane % 2
      const int vr = (lane & 15) >> 1, vs = lane & 1, vg = (lane >> 4) & 1;
      const int vrow = 8 * (vr >> 2) + 4 * half + (vr & 3);
      const int fv = f8_swz(vrow);
      uint32_t voff[4];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) voff[dt] = (uint32_t)(vrow * ROW + ((2 * dt + vg) ^ fv) * 16 + 8 * vs);

      auto step = [&](const uint8_t* kt, const uint8_t* vt, int filled) __attribute__((always_inline)) {
        const __attribute__((address_space(3))) uint8_t* kb = (const __attribute__((address_space(3))) uint8_t*)(
            const __attribute__((address_space(3))) void*)(const void*)kt;
        const __attribute__((address_space(3))) uint8_t* vb = (const __attribute__((address_space(3))) uint8_t*)(
            const __attribute__((address_space(3))) void*)(const void*)vt;
        f32x16_t sc[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
          for (int i = 0; i < 16; ++i) sc[t][i] = 0.f;
#pragma unroll
          for (int kd = 0; kd < 2; ++kd) {
            const u32x4_t a0 = *(const lds_u32x4_t*)(kb + t * 32 * ROW + koff[kd][0]);
            const u32x4_t a1 = *(const lds_u32x4_t*)(kb + t * 32 * ROW + koff[kd][1]);
            const i32x8_t a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                               (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
            sc[t] = mfma_f8(a, qf[kd], sc[t]);
          }
        }
        if (filled < BN) {
          const int lim = filled - 4 * half;
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i)
              if (32 * t + (i >> 2) * 8 + (i & 3) >= lim) sc[t][i] = -__builtin_inff();
        }
        // raw tile max (v_maximum3: no canonicalising of the MFMA results)
        float mx = sc[0][0];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = (t == 0 ? 1 : 0); i < 16; ++i) mx = __builtin_elementwise_maximum(mx, sc[t][i]);
        {
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
          mx = __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        if (mx > thr) {
          const float m_new = mx * sl2;
          const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
          l_a *= alpha;
          l_b *= alpha;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
          m_ref = m_new;
          thr = (m_new + kLazyTau) * inv_sl2;
        }
        const float neg = -m_ref;
        i32x8_t pf;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 16; i += 4) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[t][i], sl2, neg));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[t][i + 1], sl2, neg));
            const float p2 = __builtin_amdgcn_exp2f(fmaf(sc[t][i + 2], sl2, neg));
            const float p3 = __builtin_amdgcn_exp2f(fmaf(sc[t][i + 3], sl2, neg));
            if (i & 4)
              l_b += (p0 + p1) + (p2 + p3);
            else
              l_a += (p0 + p1) + (p2 + p3);
            int w = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
            w = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, w, true);
            pf[4 * t + (i >> 2)] = w;
          }
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          i32x8_t a;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const i32x2_t r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)(vb + q * 16 * ROW + voff[dt]));
            a[2 * q] = r[0];
            a[2 * q + 1] = r[1];
          }
          o[dt] = mfma_f8(a, pf, o[dt]);
        }
      };

      uint8_t* k0 = sT0;
      uint8_t* k1 = sT1;
      uint8_t* k2 = sT2;
      uint8_t* v0 = k0 + BN * ROW;
      uint8_t* v1 = k1 + BN * ROW;
      uint8_t* v2 = k2 + BN * ROW;
      auto dma = [&](const uint8_t* src, uint8_t* dst, const int (&key)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const uint32_t off = (uint32_t)max(key[q], 0) * (uint32_t)ROW + l_off[q];
          __builtin_amdgcn_global_load_lds((const void*)(src + off), (lds_void_t*)(void*)(dst + (16 * wave + 8 * q) * ROW),
                                           16, 0, 0);
        }
      };

      int key[2];
      int f0 = cur.fill<2>(BN, slot_of, key);
      if (f0 > 0) {
        dma(Kp, k0, key);
        dma(Vp, v0, key);
      }
      int f1 = f0 > 0 ? cur.fill<2>(BN, slot_of, key) : 0;
      if (f1 > 0) {
        dma(Kp, k1, key);
        dma(Vp, v1, key);
        __builtin_amdgcn_s_waitcnt(kWaitTile);
      } else {
        __builtin_amdgcn_s_waitcnt(kWaitAll);
      }
      lds_barrier();

      auto iter = [&](auto late, const uint8_t* kc, const uint8_t* vc, uint8_t* kd, uint8_t* vd)
          __attribute__((always_inline)) -> bool {
        int f2 = 0;
        if (f1 > 0) {
          f2 = cur.fill<2>(BN, slot_of, key);
        } else {
          key[0] = key[1] = -1;
        }
        if constexpr (!decltype(late)::value) {
          dma(Kp, kd, key);
          dma(Vp, vd, key);
        }
        if (active) step(kc, vc, f0);
        if constexpr (decltype(late)::value) {
          dma(Kp, kd, key);
          dma(Vp, vd, key);
        }
        __builtin_amdgcn_s_waitcnt(kWaitTile);
        lds_barrier();
        f0 = f1;
        f1 = f2;
        return f0 > 0;
      };
      if (f0 > 0) {
        constexpr std::true_type late{};
        constexpr std::false_type early{};
        while (iter(late, k0, v0, k2, v2) && iter(early, k1, v1, k0, v0) && iter(early, k2, v2, k1, v1)) {
        }
      }
      // the last iterations' loads (of key row 0 past the list's end) must land
      // before the next item's loads reuse the ring
      __builtin_amdgcn_s_waitcnt(kWaitAll);

      float l_tot;
      {
        const float l_part = l_a + l_b;
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_part), __float_as_uint(l_part), false, false);
        l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      }
      // output row: row itself, or token perm[row] through the destination's strides
      const int tout = row_ok ? (om.perm ? om.perm[(size_t)p * N + row] : row) : -1;
      if (row_ok && (unsigned)tout < (unsigned)N) {
        const float inv = l_tot > 0.f ? sv / l_tot : 0.f;
        uint16_t* orow = O + (p / om.heads) * om.bs + (p % om.heads) * om.hs + (int64_t)tout * om.ts;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            uint2 w;
            w.x = pack_bf16x2(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv);
            w.y = pack_bf16x2(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv);
            *reinterpret_cast<uint2*>(orow + dt * 32 + g * 8 + half * 4) = w;
          }
        if (lse && half == 0)
          lse[(size_t)p * N + tout] = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * 0.69314718055994531f
                                                 : -__builtin_inff();
      }
    }
  }
}

// ---------------------------------------------------------------- fp32
// fp32 inputs: two threads per query row (each owns half of the head dim),
// keys staged 32 at a time in LDS, exact fp32 online softmax per key.
template <int D>
__global__ __launch_bounds__(128) void k_attn_f32(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V, int N,
    const int32_t* __restrict__ q_off, int n_q, const int32_t* __restrict__ k_off, int n_k,
    const int32_t* __restrict__ sel_count, const int32_t* __restrict__ sel_idx, float scale,
    float* __restrict__ O, float* __restrict__ lse, OutMap om, const int32_t* __restrict__ item_count,
    const int32_t* __restrict__ items, int max_items) {
  constexpr int BN = 32;
  constexpr int H = D / 2;
  __shared__ float sK[BN * D];
  __shared__ float sV[BN * D];
  const int p = blockIdx.y;
  if ((int)blockIdx.x >= item_count[p]) return;
  const int item = items[(size_t)p * max_items + blockIdx.x];
  const int ci = item & 0xfff, rb = item >> 12;
  const int32_t* qo = q_off + (size_t)p * (n_q + 1);
  const int qa = clampi(qo[ci], 0, N), qb = clampi(qo[ci + 1], qa, N);
  const int tid = threadIdx.x;
  const int row = qa + rb * kAttnF32BM + tid / 2;
  const int hh = tid & 1;
  const bool row_ok = row < qb;
  const size_t base = (size_t)p * N * D;
  float q[H], o[H];
#pragma unroll
  for (int e = 0; e < H; ++e) {
    q[e] = row_ok ? Q[base + (size_t)row * D + hh * H + e] : 0.f;
    o[e] = 0.f;
  }
  // each thread loads BN*D/128 floats of K and of V per tile
  constexpr int PER = BN * D / 128;
  int slot_of[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) slot_of[e] = (tid + 128 * e) / D;
  KeyCursor cur;
  cur.init(sel_idx + ((size_t)p * n_q + ci) * n_k, k_off + (size_t)p * (n_k + 1),
           clampi(sel_count[(size_t)p * n_q + ci], 0, n_k), n_k, N);
  float m_run = -__builtin_inff(), l_run = 0.f;
  for (;;) {
    int key[PER];
    bool contiguous;
    const int filled = cur.fill<PER>(BN, slot_of, key, &contiguous);
    if (filled == 0) break;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int f = tid + 128 * e;
      const int c = f % D;
      sK[f] = key[e] >= 0 ? K[base + (size_t)key[e] * D + c] : 0.f;
      sV[f] = key[e] >= 0 ? V[base + (size_t)key[e] * D + c] : 0.f;
    }
    __syncthreads();
    for (int j = 0; j < filled; ++j) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < H; ++e) part = fmaf(q[e], sK[j * D + hh * H + e], part);
      const float sc = (part + __shfl_xor(part, 1)) * scale;
      const float m_new = fmaxf(m_run, sc);
      const float corr = expf(m_run - m_new);
      const float pe = expf(sc - m_new);
      l_run = l_run * corr + pe;
#pragma unroll
      for (int e = 0; e < H; ++e) o[e] = fmaf(pe, sV[j * D + hh * H + e], o[e] * corr);
      m_run = m_new;
    }
  }
  const int trow = row_ok ? (om.perm ? om.perm[(size_t)p * N + row] : row) : -1;
  if (row_ok && (unsigned)trow < (unsigned)N) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    float* orow = O + (p / om.heads) * om.bs + (p % om.heads) * om.hs + (int64_t)trow * om.ts;
#pragma unroll
    for (int e = 0; e < H; ++e) orow[hh * H + e] = o[e] * inv;
    if (lse && hh == 0) lse[(size_t)p * N + trow] = l_run > 0.f ? m_run + logf(l_run) : -__builtin_inff();
  }
}

// Resident work-groups of the bf16 kernel: three per CU, a multiple of the
// XCD count.
static int attn_persistent_grid() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                               hipSuccess || cus < 1)
    cus = 256;
  const int g = cus * 3 / kAttnXcds * kAttnXcds;
  return g < kAttnXcds ? kAttnXcds : g;
}

hipError_t launch_varblock_attn(const void* q, const void* k, const void* v, bool bf16, int bh,
                                int N, int d, const int32_t* q_off, int n_q, const int32_t* k_off,
                                int n_k, const int32_t* sel_count, const int32_t* sel_idx,
                                float scale, void* out, float* lse, const OutMap& om, const AttnWs& ws,
                                hipStream_t s) {
  const int bm = attn_block_rows(bf16);
  const int max_items = attn_max_items(N, n_q, bm);
  hipLaunchKernelGGL(k_attn_lengths, dim3((n_q + 3) / 4, bh), dim3(256), 0, s, k_off, n_k, N, sel_count,
                     sel_idx, n_q, bf16 ? kAttnBN : 32, ws.tiles, ws.kmax);
  if (bf16) {
    const dim3 gk((N + kNormRows - 1) / kNormRows, bh);
    if (d == 128)
      hipLaunchKernelGGL(k_key_norm_max<128>, gk, dim3(256), 0, s, static_cast<const uint16_t*>(k), N, ws.kmax);
    else
      hipLaunchKernelGGL(k_key_norm_max<64>, gk, dim3(256), 0, s, static_cast<const uint16_t*>(k), N, ws.kmax);
    hipLaunchKernelGGL(k_attn_plan_xcd, dim3(bh), dim3(1024), 0, s, q_off, n_q, N, bm, max_items, ws.tiles,
                       ws.xcount, ws.xitems);
    hipLaunchKernelGGL(k_attn_flatten, dim3(kAttnXcds), dim3(256), 0, s, ws.xcount, ws.xitems, bh, max_items,
                       ws.flat, ws.queue);
    const float sl2 = scale * 1.4426950408889634f;
    const size_t cap = (size_t)bh * max_items;
    const dim3 grid_p(attn_persistent_grid());
#define SVG2_ATTN(D)                                                                                  \
  hipLaunchKernelGGL(k_attn_bf16<D>, grid_p, dim3(256), 0, s, static_cast<const uint16_t*>(q),        \
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), N, q_off, n_q, \
                     k_off, n_k, sel_count, sel_idx, sl2, static_cast<uint16_t*>(out), lse, om, ws.flat, \
                     ws.queue, cap, ws.kmax)
    if (d == 128) SVG2_ATTN(128); else SVG2_ATTN(64);
#undef SVG2_ATTN
  } else {
    hipLaunchKernelGGL(k_attn_plan, dim3(bh), dim3(1024), 0, s, q_off, n_q, N, bm, max_items, ws.tiles,
                       ws.item_count, ws.items);
    const dim3 grid(max_items, bh);
#define SVG2_ATTN(D)                                                                                   \
  hipLaunchKernelGGL(k_attn_f32<D>, grid, dim3(128), 0, s, static_cast<const float*>(q),               \
                     static_cast<const float*>(k), static_cast<const float*>(v), N, q_off, n_q, k_off, \
                     n_k, sel_count, sel_idx, scale, static_cast<float*>(out), lse, om, ws.item_count, \
                     ws.items, max_items)
    if (d == 128) SVG2_ATTN(128); else SVG2_ATTN(64);
#undef SVG2_ATTN
  }
  return hipGetLastError();
}

hipError_t launch_varblock_attn_fp8(const void* q, const void* k, const void* v, const float* q_scale,
                                    const float* k_scale, const float* v_scale, int bh, int N,
                                    const int32_t* q_off, int n_q, const int32_t* k_off, int n_k,
                                    const int32_t* sel_count, const int32_t* sel_idx, float scale, void* out,
                                    float* lse, const OutMap& om, const AttnWs& ws, hipStream_t s) {
  const int max_items = attn_max_items(N, n_q, kAttnBM);
  hipLaunchKernelGGL(k_attn_lengths, dim3((n_q + 3) / 4, bh), dim3(256), 0, s, k_off, n_k, N, sel_count, sel_idx,
                     n_q, kAttnF8BN, ws.tiles, nullptr);
  hipLaunchKernelGGL(k_attn_plan_xcd, dim3(bh), dim3(1024), 0, s, q_off, n_q, N, kAttnBM, max_items, ws.tiles,
                     ws.xcount, ws.xitems);
  hipLaunchKernelGGL(k_attn_flatten, dim3(kAttnXcds), dim3(256), 0, s, ws.xcount, ws.xitems, bh, max_items,
                     ws.flat, ws.queue);
  const size_t cap = (size_t)bh * max_items;
  hipLaunchKernelGGL(k_attn_fp8, dim3(attn_persistent_grid()), dim3(256), 0, s,
                     static_cast<const uint8_t*>(q), static_cast<const uint8_t*>(k), static_cast<const uint8_t*>(v),
                     q_scale, k_scale, v_scale, N, q_off, n_q, k_off, n_k, sel_count, sel_idx,
                     scale * 1.4426950408889634f, static_cast<uint16_t*>(out), lse, om, ws.flat, ws.queue, cap);
  return hipGetLastError();
}

}  // namespace svg2
